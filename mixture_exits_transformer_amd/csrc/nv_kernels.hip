// HIP kernels of the N-vium decode step for gfx950 (CDNA4, wave64).
//
// Layer arithmetic follows the LLaMA-2 pre-norm block named in section 4 of the
// gist.science technical summary of N-vium; exits follow section 2, part
// "Architektur" (router w_k, stick-breaking p_k, per-exit distribution pi_k);
// causal chunks of deferred rows follow section 2, part "Inferenz: Piggybacking".
#include "nv_internal.h"
#include "nv_device.h"

#include <hip/hip_ext.h>
#include <limits.h>
#include <math.h>
#include <stdio.h>

namespace nv {

// Measurement events for the next launches (set by the runtime's timing mode).  The
// dispatch packet itself stamps them, so they bracket the kernel's execution only.
static thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void set_launch_events(hipEvent_t start, hipEvent_t stop) {
    t_ev_start = start;
    t_ev_stop = stop;
}

static thread_local unsigned long long* t_stamp = nullptr;

void set_launch_stamp(unsigned long long* stamps) { t_stamp = stamps; }
unsigned long long* current_launch_stamp() { return t_stamp; }
void current_launch_events(hipEvent_t* start, hipEvent_t* stop) {
    *start = t_ev_start;
    *stop = t_ev_stop;
}

// 16-byte load with the nontemporal hint, for data read once per launch whose next use is
// beyond every cache level (a decode step's weights, the K/V cache).
typedef unsigned int stream_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load16(const void* p) {
    const stream_u4 v = __builtin_nontemporal_load((const stream_u4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Symbol of the last kernel a launch wrapper issued while timing (as profilers print it).
static thread_local char t_name[160];

const char* last_launch_name() { return t_name; }

// Most blocks of any launch since the last take_launch_blocks() (the stamp entries written).
static thread_local int t_blocks = 0;

int take_launch_blocks() {
    const int n = t_blocks;
    t_blocks = 0;
    return n;
}

void note_launch_blocks(int n) {
    if (n > t_blocks) t_blocks = n;
}

#define NV_LAUNCH(K, G, B, SHM, ST, ...)                                                     \
    do {                                                                                     \
        {                                                                                    \
            const dim3 g_ = (G);                                                             \
            const int nb_ = (int)(g_.x * g_.y * g_.z);                                       \
            if (nb_ > t_blocks) t_blocks = nb_;                                              \
        }                                                                                    \
        if (t_ev_stop) {                                                                     \
            hipExtLaunchKernelGGL((K), G, B, SHM, ST, t_ev_start, t_ev_stop, 0, __VA_ARGS__);  \
            t_ev_start = nullptr;                                                            \
        } else {                                                                             \
            hipLaunchKernelGGL((K), G, B, SHM, ST, __VA_ARGS__);                             \
        }                                                                                    \
    } while (0)

// ------------------------------------------------------------------------------------------
// RoPE table: cs[pos][i] = (cos, sin)(pos * base^(-2i/hd)), computed in float64.
// ------------------------------------------------------------------------------------------

__global__ void k_rope_table(float* cs, int max_ctx, int hd, double base) {
    const int half = hd / 2;
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)max_ctx * half) return;
    int pos = (int)(idx / half), i = (int)(idx % half);
    double theta = pow(base, -2.0 * (double)i / (double)hd);
    double ang = (double)pos * theta;
    cs[2 * idx] = (float)cos(ang);
    cs[2 * idx + 1] = (float)sin(ang);
}

hipError_t launch_rope_table(float* cs, int max_ctx, int hd, float base, hipStream_t st) {
    int64_t n = (int64_t)max_ctx * (hd / 2);
    NV_LAUNCH(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cs, max_ctx, hd,
                       (double)base);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// embedding gather: hidden row = E[token]
// ------------------------------------------------------------------------------------------

__global__ void k_embed(const int* tokens, const RowInfo* rows, int n, const void* E, int wbf16, float* Hs,
                        int d, int by_seq) {
    int r = blockIdx.x;
    if (r >= n) return;
    int64_t src = (int64_t)tokens[by_seq ? rows[r].seq : r] * d;
    float* dst = Hs + (int64_t)rows[r].hrow * d;
    for (int k = threadIdx.x; k < d; k += blockDim.x)
        dst[k] = wbf16 ? __uint_as_float(((uint32_t)((const uint16_t*)E)[src + k]) << 16)
                       : ((const float*)E)[src + k];
}

hipError_t launch_embed(const int* tokens, const RowInfo* rows, int n, const void* E, int wbf16, float* Hs, int d,
                        hipStream_t st, int by_seq) {
    if (n <= 0) return hipSuccess;
    NV_LAUNCH(k_embed, dim3(n), dim3(256), 0, st, tokens, rows, n, E, wbf16, Hs, d, by_seq);
    return hipGetLastError();
}


// ------------------------------------------------------------------------------------------
// Epilogue for a pair of adjacent output columns (n, n+1), n even, of row `row`.
// ------------------------------------------------------------------------------------------

template <int EPI>
__device__ __forceinline__ void epi_pair_t(const GemmArgs& a, int row, int n, float v0, float v1) {
    if constexpr (EPI == EPI_SWIGLU) {
        const int orow = a.o_rows ? a.o_rows[row].hrow : row;
        const float y = v0 / (1.0f + expf(-v0)) * v1;
        if (a.out_bf16) a.out_bf16[(int64_t)orow * a.ldo + (n >> 1)] = f2bf(y);
        else a.out[(int64_t)orow * a.ldo + (n >> 1)] = y;
        return;
    }
    if constexpr (EPI == EPI_QKV) {
        // columns n, n+1 hold rotation partners j and j + hd/2 of one head of q, k or v
        const RowInfo ri = a.a_rows[row];
        const LayerDims& D = a.D;
        const int half = D.hd >> 1;
        const int p = n >> 1;
        const int part = p / (D.d >> 1);
        const int pp = p - part * (D.d >> 1);
        const int h = pp / half, j = pp - h * half;
        if (part == 2) {
            const int64_t b = kv_base(D, ri.seq, a.layer, 1, h) + (int64_t)ri.pos * D.hd;
            kv_store(a.kv, D.kv_bf16, b + j, v0);
            kv_store(a.kv, D.kv_bf16, b + j + half, v1);
            return;
        }
        const float c = a.rope[((int64_t)ri.pos * half + j) * 2];
        const float s = a.rope[((int64_t)ri.pos * half + j) * 2 + 1];
        const float r0 = v0 * c - v1 * s, r1 = v1 * c + v0 * s;
        if (part == 0) {
            float* q = a.q_out + (int64_t)row * D.d + h * D.hd;
            q[j] = r0;
            q[j + half] = r1;
        } else {
            const int64_t b = kv_base(D, ri.seq, a.layer, 0, h) + (int64_t)ri.pos * D.hd;
            kv_store(a.kv, D.kv_bf16, b + j, r0);
            kv_store(a.kv, D.kv_bf16, b + j + half, r1);
        }
        return;
    }
    if constexpr (EPI == EPI_STORE || EPI == EPI_SILU || EPI == EPI_RESID) {
        const int orow = a.o_rows ? a.o_rows[row].hrow : row;
        float* o = a.out + (int64_t)orow * a.ldo + n;
        if constexpr (EPI == EPI_STORE) {
            o[0] = v0;
            o[1] = v1;
        } else if constexpr (EPI == EPI_SILU) {
            o[0] = v0 / (1.0f + expf(-v0));
            o[1] = v1 / (1.0f + expf(-v1));
        } else {
            o[0] += v0;
            o[1] += v1;
        }
    }
}

__device__ __forceinline__ void epi_pair(const GemmArgs& a, int row, int n, float v0, float v1) {
    switch (a.epi) {
        case EPI_SWIGLU: epi_pair_t<EPI_SWIGLU>(a, row, n, v0, v1); break;
        case EPI_QKV: epi_pair_t<EPI_QKV>(a, row, n, v0, v1); break;
        case EPI_STORE: epi_pair_t<EPI_STORE>(a, row, n, v0, v1); break;
        case EPI_SILU: epi_pair_t<EPI_SILU>(a, row, n, v0, v1); break;
        default: epi_pair_t<EPI_RESID>(a, row, n, v0, v1); break;
    }
}



// (first start, last end) over the block stamps of one launch into rec[0..1]; the stamp
// slots are reset to (max, 0) for the next launch.
__global__ __launch_bounds__(1024) void k_stamp_reduce(unsigned long long* stamps, int n, unsigned long long* rec) {
    __shared__ unsigned long long lo[1024], hi[1024];
    unsigned long long a = ~0ull, b = 0ull;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        a = min(a, stamps[2 * i]);
        b = max(b, stamps[2 * i + 1]);
        stamps[2 * i] = ~0ull;
        stamps[2 * i + 1] = 0ull;
    }
    lo[threadIdx.x] = a;
    hi[threadIdx.x] = b;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            lo[threadIdx.x] = min(lo[threadIdx.x], lo[threadIdx.x + s]);
            hi[threadIdx.x] = max(hi[threadIdx.x], hi[threadIdx.x + s]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        rec[0] = lo[0];
        rec[1] = hi[0];
    }
}

hipError_t launch_stamp_reduce(unsigned long long* stamps, int n, unsigned long long* rec, hipStream_t st) {
    hipLaunchKernelGGL(k_stamp_reduce, dim3(1), dim3(1024), 0, st, stamps, n, rec);
    return hipGetLastError();
}

// What the epilogue of one (row, column pair) needs from memory, fetched early so the
// epilogue itself issues no dependent loads.
struct EpiCtx {
    int orow;      // output row (hidden-state row for EPI_RESID)
    int seq, pos;  // EPI_QKV: sequence and position of the row
    float c, s;    // EPI_QKV: RoPE cos / sin for this pair
    float r0, r1;  // EPI_RESID with has_res: the residual values of columns n, n+1
    bool has_res;
};

// E: the epilogue kind when fixed at compile time, or -1 to read a.epi (each decode product's
// kernel then holds only its own epilogue, and no load of another kind's path can hold up
// this one's registers).
template <int E>
__device__ __forceinline__ int epi_kind(const GemmArgs& a) { return E >= 0 ? E : a.epi; }

template <int E = -1>
__device__ __forceinline__ EpiCtx epi_prepare(const GemmArgs& a, int row, int n) {
    EpiCtx e{};
    if (epi_kind<E>(a) == EPI_QKV) {
        const RowInfo ri = a.a_rows[row];
        e.seq = ri.seq;
        e.pos = ri.pos;
        const int half = a.D.hd >> 1;
        const int p = n >> 1;
        const int pp = p % (a.D.d >> 1);
        const int j = pp % half;
        e.c = a.rope[((int64_t)ri.pos * half + j) * 2];
        e.s = a.rope[((int64_t)ri.pos * half + j) * 2 + 1];
    } else {
        e.orow = a.o_rows ? a.o_rows[row].hrow : row;
    }
    return e;
}

// The same context for a contiguous chunk (GemmArgs::contig): every address is known without
// a table load, so these loads can be issued after the weight loads; the residual values
// of EPI_RESID are fetched here too (only this thread writes them).
template <int E = -1>
__device__ __forceinline__ EpiCtx epi_prefetch(const GemmArgs& a, int row, int n) {
    EpiCtx e{};
    const int epi = epi_kind<E>(a);
    if (epi == EPI_QKV) {
        e.seq = a.seq0;
        e.pos = a.pos0 + row;
        const int half = a.D.hd >> 1;
        const int pp = (n >> 1) % (a.D.d >> 1);
        const int j = pp % half;
        const float2 cs = *(const float2*)(a.rope + ((int64_t)e.pos * half + j) * 2);
        e.c = cs.x;
        e.s = cs.y;
    } else {
        e.orow = a.o_rows ? a.o_row0 + row : row;
        if (epi == EPI_RESID) {
            const float2 r = *(const float2*)(a.out + (int64_t)e.orow * a.ldo + n);
            e.r0 = r.x;
            e.r1 = r.y;
            e.has_res = true;
        }
    }
    return e;
}

template <int E = -1>
__device__ __forceinline__ void epi_apply(const GemmArgs& a, const EpiCtx& e, int row, int n, float v0, float v1) {
    const int epi = epi_kind<E>(a);
    if (epi == EPI_SWIGLU) {
        a.out[(int64_t)e.orow * a.ldo + (n >> 1)] = v0 / (1.0f + expf(-v0)) * v1;
    } else if (epi == EPI_QKV) {
        const LayerDims& D = a.D;
        const int half = D.hd >> 1;
        const int p = n >> 1;
        const int part = p / (D.d >> 1);
        const int pp = p - part * (D.d >> 1);
        const int h = pp / half, j = pp - h * half;
        if (part == 2) {
            const int64_t b = kv_base(D, e.seq, a.layer, 1, h) + (int64_t)e.pos * D.hd;
            kv_store(a.kv, D.kv_bf16, b + j, v0);
            kv_store(a.kv, D.kv_bf16, b + j + half, v1);
            return;
        }
        const float r0 = v0 * e.c - v1 * e.s, r1 = v1 * e.c + v0 * e.s;
        if (part == 0) {
            float* q = a.q_out + (int64_t)row * D.d + h * D.hd;
            q[j] = r0;
            q[j + half] = r1;
        } else {
            const int64_t b = kv_base(D, e.seq, a.layer, 0, h) + (int64_t)e.pos * D.hd;
            kv_store(a.kv, D.kv_bf16, b + j, r0);
            kv_store(a.kv, D.kv_bf16, b + j + half, r1);
        }
    } else {
        float* o = a.out + (int64_t)e.orow * a.ldo + n;
        if (epi == EPI_STORE) {
            o[0] = v0;
            o[1] = v1;
        } else if (epi == EPI_SILU) {
            o[0] = v0 / (1.0f + expf(-v0));
            o[1] = v1 / (1.0f + expf(-v1));
        } else if (e.has_res) {
            o[0] = e.r0 + v0;
            o[1] = e.r1 + v1;
        } else {
            o[0] += v0;
            o[1] += v1;
        }
    }
}

// ------------------------------------------------------------------------------------------
// GEMV-shaped products (R <= GV_RMAX rows) on the vector ALUs.  Each wave owns CPW adjacent
// output columns; lanes span K in 16-byte chunks (chunk c of a row is read by lane c % 64,
// so one instruction reads 1 KB of a weight row, fully coalesced).  All of a wave's
// weight loads are issued before the activation rows are staged (RMSNormed, fp32) into
// LDS, so the weight stream is in flight while the prologue runs.  Each (row, column) dot
// product ends with a wavefront reduction.
// ------------------------------------------------------------------------------------------

constexpr int GV_RMAX = 8;

template <bool WBF, int CPW, int CH, int HEAD>
__global__ __launch_bounds__(256) void k_gemv(GemmArgs a) {
    extern __shared__ float sm[];
    constexpr int EPC = WBF ? 8 : 4;
    constexpr int ESZ = WBF ? 2 : 4;
    const int K = a.K, R = a.R;
    const int nch = K / EPC;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = (blockIdx.x * 4 + wave) * CPW;
    float* As = sm;
    float* inv = sm + R * K;

    uint4 w[CPW][CH];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const uint4* wp = (const uint4*)((const char*)a.W + (size_t)(n0 + c) * K * ESZ);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int ch = lane + 64 * j;
            w[c][j] = ch < nch ? wp[ch] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    for (int r = wave; r < R; r += 4) {
        const int ar = a.a_rows ? a.a_rows[r].hrow : r;
        const float* src = a.A + (int64_t)ar * a.lda;
        float ss = 0.f;
        if (a.norm_w) {
            for (int k = lane; k < K; k += 64) ss += src[k] * src[k];
            ss = wave_sum(ss);
        }
        if (lane == 0) inv[r] = a.norm_w ? 1.0f / sqrtf(ss / (float)K + a.eps) : 1.0f;
    }
    __syncthreads();
    for (int idx = threadIdx.x * 4; idx < R * K; idx += blockDim.x * 4) {
        const int r = idx / K, k = idx - r * K;      // K % 4 == 0: a float4 stays in one row
        const int ar = a.a_rows ? a.a_rows[r].hrow : r;
        float4 v = *(const float4*)(a.A + (int64_t)ar * a.lda + k);
        const float iv = inv[r];
        v.x *= iv; v.y *= iv; v.z *= iv; v.w *= iv;
        if (a.norm_w) {
            const float4 g = *(const float4*)(a.norm_w + k);
            v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
        }
        *(float4*)(As + idx) = v;
    }
    __syncthreads();

    float acc[CPW][GV_RMAX];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int r = 0; r < GV_RMAX; ++r) acc[c][r] = 0.f;

#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int ch = lane + 64 * j;
        if (ch < nch) {
            float wf[CPW][EPC];
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const uint32_t u[4] = {w[c][j].x, w[c][j].y, w[c][j].z, w[c][j].w};
                if constexpr (WBF) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        wf[c][2 * e] = bf_lo(u[e]);
                        wf[c][2 * e + 1] = bf_hi(u[e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) wf[c][e] = __uint_as_float(u[e]);
                }
            }
#pragma unroll
            for (int r = 0; r < GV_RMAX; ++r) {
                if (r < R) {
                    float av[EPC];
                    const float4* ap = (const float4*)(As + r * K + ch * EPC);
#pragma unroll
                    for (int e = 0; e < EPC / 4; ++e) {
                        const float4 t = ap[e];
                        av[4 * e] = t.x; av[4 * e + 1] = t.y; av[4 * e + 2] = t.z; av[4 * e + 3] = t.w;
                    }
#pragma unroll
                    for (int c = 0; c < CPW; ++c)
#pragma unroll
                        for (int e = 0; e < EPC; ++e) acc[c][r] = fmaf(wf[c][e], av[e], acc[c][r]);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < GV_RMAX; ++r) {
        if (r < R) {
            float v[CPW];
#pragma unroll
            for (int c = 0; c < CPW; ++c) v[c] = wave_sum(acc[c][r]);
            if (lane == 0) {
#pragma unroll
                for (int c = 0; c < CPW; c += 2) epi_pair(a, r, n0 + c, v[c], v[c + 1]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Row-tiled GEMM on the vector ALUs (fp32 weights or no matrix-core shape), any R.  Each block owns GV_COLS consecutive output columns,
// two per wave (so a SwiGLU gate/up pair stays in one wave).  Lanes span K with 16-byte
// weight loads (a wave reads 1 KB of a weight row per instruction, fully coalesced), the
// activation tile (RMSNormed, fp32) sits in LDS, and each (row, column) dot product is
// finished by a wavefront reduction.  Rows are processed in tiles of rt rows.
// ------------------------------------------------------------------------------------------

constexpr int GV_COLS = 8;
constexpr int GV_RT_MAX = 8;

__host__ __device__ inline int gv_row_tile(int K) {
    int rt = 16000 / K;   // activation tile + inverse norms stay under 64 KB of LDS
    return rt < 1 ? 1 : (rt > GV_RT_MAX ? GV_RT_MAX : rt);
}

template <bool WBF, int HEAD>
__global__ __launch_bounds__(256) void k_gemm_valu(GemmArgs a) {
    extern __shared__ float sm[];
    const int K = a.K;
    const int rt = gv_row_tile(K);
    float* As = sm;
    float* inv = sm + rt * K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * GV_COLS + wave * 2;
    constexpr int EPC = WBF ? 8 : 4;  // elements per 16-byte chunk
    const int nchunk = K / EPC;
    const size_t esz = WBF ? 2 : 4;
    const char* W0 = (const char*)a.W + (size_t)n0 * K * esz;
    const char* W1 = W0 + (size_t)K * esz;

    for (int rt0 = 0; rt0 < a.R; rt0 += rt) {
        const int nr = min(rt, a.R - rt0);
        for (int r = wave; r < nr; r += 4) {
            const int ar = a.a_rows ? a.a_rows[rt0 + r].hrow : rt0 + r;
            const float* src = a.A + (int64_t)ar * a.lda;
            float ss = 0.f;
            if (a.norm_w) {
                for (int k = lane; k < K; k += 64) ss += src[k] * src[k];
                ss = wave_sum(ss);
            }
            if (lane == 0) inv[r] = a.norm_w ? 1.0f / sqrtf(ss / (float)K + a.eps) : 1.0f;
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nr * K; idx += blockDim.x) {
            const int r = idx / K, k = idx - r * K;
            const int ar = a.a_rows ? a.a_rows[rt0 + r].hrow : rt0 + r;
            float v = a.A[(int64_t)ar * a.lda + k] * inv[r];
            if (a.norm_w) v *= a.norm_w[k];
            As[idx] = v;
        }
        __syncthreads();

        float acc0[GV_RT_MAX], acc1[GV_RT_MAX];
#pragma unroll
        for (int r = 0; r < GV_RT_MAX; ++r) acc0[r] = acc1[r] = 0.f;

        for (int ch = lane; ch < nchunk; ch += 64) {
            const uint4 q0 = *(const uint4*)(W0 + (size_t)ch * 16);
            const uint4 q1 = *(const uint4*)(W1 + (size_t)ch * 16);
            float w0[EPC], w1[EPC];
            if constexpr (WBF) {
                const uint32_t u0[4] = {q0.x, q0.y, q0.z, q0.w}, u1[4] = {q1.x, q1.y, q1.z, q1.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w0[2 * e] = bf_lo(u0[e]);
                    w0[2 * e + 1] = bf_hi(u0[e]);
                    w1[2 * e] = bf_lo(u1[e]);
                    w1[2 * e + 1] = bf_hi(u1[e]);
                }
            } else {
                w0[0] = __uint_as_float(q0.x); w0[1] = __uint_as_float(q0.y);
                w0[2] = __uint_as_float(q0.z); w0[3] = __uint_as_float(q0.w);
                w1[0] = __uint_as_float(q1.x); w1[1] = __uint_as_float(q1.y);
                w1[2] = __uint_as_float(q1.z); w1[3] = __uint_as_float(q1.w);
            }
#pragma unroll
            for (int r = 0; r < GV_RT_MAX; ++r) {
                if (r < nr) {
                    const float* ap = As + r * K + ch * EPC;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        acc0[r] = fmaf(w0[e], ap[e], acc0[r]);
                        acc1[r] = fmaf(w1[e], ap[e], acc1[r]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < GV_RT_MAX; ++r) {
            if (r < nr) {
                const float g = wave_sum(acc0[r]);
                const float u = wave_sum(acc1[r]);
                if (lane == 0) epi_pair(a, rt0 + r, n0, g, u);
            }
        }
        __syncthreads();
    }
}


// ------------------------------------------------------------------------------------------
// Skinny / tall GEMM on the matrix cores (bf16 weights, rows >= a threshold).
// Block = 4 waves, tile 64 rows x BN columns, K in stages of 64 staged through LDS
// (double-buffered).  Activations are RMSNormed (inverse RMS precomputed per row),
// rounded to bf16 and held in LDS; wave w owns rows 16w..16w+15 of the tile and all
// BN/16 column tiles, accumulating with v_mfma_f32_16x16x32_bf16:
//   A operand: lane l holds A[l%16][8*(l/16) .. +8]; B operand: lane l holds
//   W[n = l%16][8*(l/16) .. +8]; result: lane l holds D[4*(l/16) + i][l%16].
// BN = 16 spreads decode-sized chunks over many blocks; BN = 64 reuses each weight
// tile across 64 rows per block for long prompts.
// ------------------------------------------------------------------------------------------

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
// Staging registers use the compiler's own vector type: arrays of HIP's uint4 (a struct)
// are not promoted to registers, which parks every prefetched tile in scratch.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int MF_BM = 64, MF_BK = 64, MF_LDK = MF_BK + 8;

__global__ __launch_bounds__(256) void k_row_rms(const float* A, int64_t lda, const RowInfo* rows, int R, int K,
                                                 float eps, float* inv) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = blockIdx.x * 4 + wave;
    if (r >= R) return;
    const float* src = A + (int64_t)(rows ? rows[r].hrow : r) * lda;
    float ss = 0.f;
    for (int k = lane; k < K; k += 64) ss += src[k] * src[k];
    ss = wave_sum(ss);
    if (lane == 0) inv[r] = 1.0f / sqrtf(ss / (float)K + eps);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return cvt_bf2(lo, hi); }

template <int BN, int HEAD>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs a) {
    constexpr int NT = BN / 16;
    __shared__ __align__(16) uint16_t As[2][MF_BM * MF_LDK];
    __shared__ __align__(16) uint16_t Ws[2][BN * MF_LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * MF_BM;
    const int K = a.K;
    // global -> LDS assignment: thread handles 16 consecutive k of one row
    const int lr = tid >> 2, lk = (tid & 3) * 16;
    const int grow = m0 + lr;
    const bool a_ok = grow < a.R;
    const float* Arow = a.A + (int64_t)(a_ok ? (a.a_rows ? a.a_rows[grow].hrow : grow) : 0) * a.lda;
    const float rs = (a_ok && a.norm_w) ? a.rms_ws[grow] : 1.0f;
    const bool w_on = lr < BN;
    const uint16_t* Wrow = (const uint16_t*)a.W + (int64_t)(n0 + (w_on ? lr : 0)) * K;

    f32x4_t ar[4];
    u32x4 wr[2];
    auto gload = [&](int k0) __attribute__((always_inline)) {
        if (a_ok) {
#pragma unroll
            for (int j = 0; j < 4; ++j) ar[j] = *(const f32x4_t*)(Arow + k0 + lk + 4 * j);
        }
        if (w_on) {
            wr[0] = *(const u32x4*)(Wrow + k0 + lk);
            wr[1] = *(const u32x4*)(Wrow + k0 + lk + 8);
        }
    };
    auto lstore = [&](int buf, int k0) __attribute__((always_inline)) {
        uint32_t p[8];
        if (a_ok) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float x0 = ar[j >> 1][(2 * j) & 3] * rs, x1 = ar[j >> 1][(2 * j + 1) & 3] * rs;
                if (a.norm_w) {
                    x0 *= a.norm_w[k0 + lk + 2 * j];
                    x1 *= a.norm_w[k0 + lk + 2 * j + 1];
                }
                p[j] = pack_bf2(x0, x1);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = 0u;
        }
        uint4* dst = (uint4*)&As[buf][lr * MF_LDK + lk];
        dst[0] = make_uint4(p[0], p[1], p[2], p[3]);
        dst[1] = make_uint4(p[4], p[5], p[6], p[7]);
        if (w_on) {
            u32x4* wd = (u32x4*)&Ws[buf][lr * MF_LDK + lk];
            wd[0] = wr[0];
            wd[1] = wr[1];
        }
    };

    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    const int nk = K / MF_BK;
    gload(0);
    lstore(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * MF_BK);
#pragma unroll
        for (int ks = 0; ks < MF_BK; ks += 32) {
            const uint4 au = *(const uint4*)&As[buf][(wave * 16 + (lane & 15)) * MF_LDK + ks + 8 * (lane >> 4)];
            const bf16x8_t af = __builtin_bit_cast(bf16x8_t, au);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint4 bu = *(const uint4*)&Ws[buf][(t * 16 + (lane & 15)) * MF_LDK + ks + 8 * (lane >> 4)];
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8_t, bu), acc[t], 0, 0,
                                                                 0);
            }
        }
        if (kt + 1 < nk) lstore(buf ^ 1, (kt + 1) * MF_BK);
        __syncthreads();
    }

#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int col = n0 + t * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wave * 16 + 4 * (lane >> 4) + i;
            const float v = acc[t][i];
            const float u = __shfl_xor(v, 1, 64);     // partner column (n ^ 1), same row
            if (row < a.R && (col & 1) == 0) epi_pair(a, row, col, v, u);
        }
    }
}


// ------------------------------------------------------------------------------------------
// Long-chunk products on bf16 activations.  k_rows_bf16 writes each row of A once as bf16
// (RMSNormed and scaled by the norm weight when norm_w is set) into a contiguous [R][K]
// scratch; k_gemm_bf16 then computes 128-row x BN-column tiles with eight waves in a 4x2
// layout (32 x BN/2 each), K in 64-wide steps through two or three LDS stages filled by
// direct global-to-LDS loads, on v_mfma_f32_16x16x32_bf16 (lane layout as in
// k_gemm_mfma).  Epilogues as for the other products (row i of the chunk keeps its
// a_rows / o_rows entries).
// ------------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_rows_bf16(const float* A, int64_t lda, const RowInfo* rows, int R, int K,
                                                   const float* norm_w, float eps, uint16_t* out) {
    const int r = blockIdx.x;
    if (r >= R) return;
    const float* src = A + (int64_t)(rows ? rows[r].hrow : r) * lda;
    __shared__ float red[4];
    float inv = 1.0f;
    if (norm_w) {
        float ss = 0.f;
        for (int k = threadIdx.x * 4; k < K; k += 1024) {
            const float4 v = *(const float4*)(src + k);
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
        __syncthreads();
        inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)K + eps);
    }
    uint16_t* dst = out + (int64_t)r * K;
    for (int k = threadIdx.x * 4; k < K; k += 1024) {
        float4 v = *(const float4*)(src + k);
        if (norm_w) {
            const float4 g = *(const float4*)(norm_w + k);
            v = make_float4(v.x * inv * g.x, v.y * inv * g.y, v.z * inv * g.z, v.w * inv * g.w);
        }
        *(uint2*)(dst + k) = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
    }
}

// The same pass with one wave per row and the whole row in registers (K = 256 NPL): one
// load per element, the sum of squares reduced inside the wave, no block barrier.
template <int NPL>
__global__ __launch_bounds__(256) void k_rows_bf16_w(const float* A, int64_t lda, const RowInfo* rows, int R, int K,
                                                     const float* norm_w, float eps, uint16_t* out) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R) return;
    // the norm weights do not depend on the row: they are loaded first, beside the row
    // table lookup, so that only the row's own load follows it
    float4 g[NPL];
    if (norm_w) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) g[j] = *(const float4*)(norm_w + 4 * (lane + 64 * j));
    }
    const float* src = A + (int64_t)(rows ? rows[r].hrow : r) * lda;
    float4 v[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) v[j] = *(const float4*)(src + 4 * (lane + 64 * j));
    float inv = 1.0f;
    if (norm_w) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NPL; ++j) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
        ss = wave_sum(ss);
        inv = 1.0f / sqrtf(ss / (float)K + eps);
    }
    uint16_t* dst = out + (int64_t)r * K;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int k = 4 * (lane + 64 * j);
        float4 x = v[j];
        if (norm_w) x = make_float4(x.x * inv * g[j].x, x.y * inv * g[j].y, x.z * inv * g[j].z, x.w * inv * g[j].w);
        *(uint2*)(dst + k) = make_uint2(pack_bf2(x.x, x.y), pack_bf2(x.z, x.w));
    }
}

static void launch_rows_bf16_any(const GemmArgs& a, hipStream_t st) {
    const int npl = a.K / 256;
    if (a.K % 256 != 0 || npl < 1 || npl > 16) {
        NV_LAUNCH(k_rows_bf16, dim3(a.R), dim3(256), 0, st, a.A, a.lda, a.a_rows, a.R, a.K, a.norm_w, a.eps, a.abf);
        return;
    }
    const dim3 grid((a.R + 3) / 4), block(256);
#define NV_RW(NPLV) NV_LAUNCH(HIP_KERNEL_NAME(k_rows_bf16_w<NPLV>), grid, block, 0, st, a.A, a.lda, a.a_rows, a.R, \
                              a.K, a.norm_w, a.eps, a.abf)
    switch (npl) {
        case 1: NV_RW(1); break;
        case 2: NV_RW(2); break;
        case 3: NV_RW(3); break;
        case 4: NV_RW(4); break;
        case 5: NV_RW(5); break;
        case 6: NV_RW(6); break;
        case 7: NV_RW(7); break;
        case 8: NV_RW(8); break;
        case 9: NV_RW(9); break;
        case 10: NV_RW(10); break;
        case 11: NV_RW(11); break;
        case 12: NV_RW(12); break;
        case 13: NV_RW(13); break;
        case 14: NV_RW(14); break;
        case 15: NV_RW(15); break;
        default: NV_RW(16); break;
    }
#undef NV_RW
}

constexpr int GB_BM = 128, GB_BK = 64, GB_LDK = GB_BK;
// 16-byte chunk j of tile row r is stored at chunk j ^ gb_swz(r): the 8 lanes storing one
// row and the 16 lanes reading one k-chunk of 16 rows then cover every LDS bank once.
__device__ __forceinline__ int gb_swz(int r) { return (r >> 1) & 7; }
constexpr int GB_MIN_ROWS = 33;    // chunks of at least this many rows use k_gemm_bf16

// Direct global -> LDS loads (global_load_lds_dwordx4): lane l of a wave writes its 16
// bytes at ldsbase + 16 l, so a tile is laid out by choosing which global chunk each lane
// fetches.  The loads count on vmcnt; the K loop waits for them with explicit counts and
// meets at a bare s_barrier, because a fenced barrier would wait for every load in flight.
#define NV_LDS(p) ((__attribute__((address_space(3))) void*)(p))
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");      // keeps the compiler from moving LDS accesses across
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Eight waves per block (NW/2 x 2, each 32 rows x BN/2 columns): against four waves of
// 64 rows, twice the waves per CU to cover latency for a third more fragment reads.
constexpr int GB_NW = 8;

template <int BN, int HEAD, int EPI, int ST, int NW = GB_NW, int BM = GB_BM>
__global__ __launch_bounds__(64 * NW) void k_gemm_bf16(GemmArgs a) {
    constexpr int NTH = 64 * NW;                      // threads
    constexpr int WN = BN / 2;                        // columns per wave (waves in NW/2 x 2)
    constexpr int NT = WN / 16;
    constexpr int WR = BM / (NW / 2);              // rows per wave
    constexpr int MT = WR / 16;
    constexpr int ACH = BM * GB_BK / 8 / NTH;      // 16-byte chunks per thread per tile
    constexpr int WCH = BN * GB_BK / 8 / NTH;
    static_assert(ACH * NTH * 8 == BM * GB_BK && WCH * NTH * 8 == BN * GB_BK, "tile chunks per thread");
    constexpr int NL = ACH + WCH;                     // loads per thread per tile
    constexpr int A_EL = BM * GB_LDK, W_EL = BN * GB_LDK;
    constexpr int CLD = BN + 4;                       // fp32 output tile row stride
    constexpr int OPER_B = ST * (A_EL + W_EL) * 2, OUT_B = BM * CLD * 4;
    static_assert(ST == 2 || ST == 3, "two or three operand stages");
    __shared__ __align__(16) unsigned char smem[OPER_B > OUT_B ? OPER_B : OUT_B];
    uint16_t* const As = (uint16_t*)smem;             // [ST][BM][GB_LDK]
    uint16_t* const Ws = As + ST * A_EL;              // [ST][BN][GB_LDK]
    float* const Cs = (float*)smem;                   // [BM][CLD] after the last product
    const unsigned long long t_begin = stamp_begin(a.stamp);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int K = a.K;
    const uint16_t* Ab = a.abf;
    const uint16_t* Wb = (const uint16_t*)a.W;
    // tile kt into stage s: load j of a wave fills chunk slots p0 .. p0 + 63 of the stage
    // (p0 = 64 NW j + 64 wave); slot p is row p / 8, position p % 8, which holds the row's
    // k-chunk (p % 8) ^ gb_swz(row)
    auto issue = [&](int kt, int s) __attribute__((always_inline)) {
        const int k0 = kt * GB_BK;
        uint16_t* const Ad = As + s * A_EL;
        uint16_t* const Wd = Ws + s * W_EL;
#pragma unroll
        for (int j = 0; j < ACH; ++j) {
            const int p0 = NTH * j + 64 * wave, p = p0 + lane, row = p >> 3;
            const int grow = min(m0 + row, a.R - 1);   // rows past R are computed and dropped
            const int g = (p & 7) ^ gb_swz(row);
            __builtin_amdgcn_global_load_lds((const void*)(Ab + (int64_t)grow * K + k0 + 8 * g), NV_LDS(Ad + 8 * p0),
                                             16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < WCH; ++j) {
            const int p0 = NTH * j + 64 * wave, p = p0 + lane, row = p >> 3;
            const int g = (p & 7) ^ gb_swz(row);
            __builtin_amdgcn_global_load_lds((const void*)(Wb + (int64_t)(n0 + row) * K + k0 + 8 * g),
                                             NV_LDS(Wd + 8 * p0), 16, 0, 0);
        }
    };
    f32x4_t acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    const int nk = K / GB_BK;
#pragma unroll
    for (int s = 0; s < ST - 1; ++s)
        if (s < nk) issue(s, s);
    int cs = 0;                                        // stage holding tile kt
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's loads of tile kt are done once at most the later tiles' are in flight
        if constexpr (ST == 3) {
            if (kt + 1 < nk) wait_vmcnt<NL>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        wait_lgkmcnt0();                               // and its reads of tile kt - 1 have returned
        barrier_nofence();                             // every wave's part of tile kt is in LDS
        if (kt + ST - 1 < nk) issue(kt + ST - 1, cs == 0 ? ST - 1 : cs - 1);   // the stage of tile kt - 1
        const uint16_t* Ab_l = As + cs * A_EL;
        const uint16_t* Wb_l = Ws + cs * W_EL;
        // every operand fragment of the 64-wide step is read in one burst (one LDS latency
        // per step instead of one per 32-wide half and per re-read), then the products
        bf16x8_t af[2][MT], bfr[2][NT];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kch = 4 * h + (lane >> 4);          // 16-byte k-chunk of this lane
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int row = wm * WR + i * 16 + (lane & 15);
                af[h][i] = __builtin_bit_cast(bf16x8_t,
                                              *(const u32x4*)&Ab_l[row * GB_LDK + ((kch ^ gb_swz(row)) << 3)]);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int row = wn * WN + t * 16 + (lane & 15);
                bfr[h][t] = __builtin_bit_cast(bf16x8_t,
                                               *(const u32x4*)&Wb_l[row * GB_LDK + ((kch ^ gb_swz(row)) << 3)]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);             // keep the scheduler from sinking the reads
        // the first half's products need only its own reads (the compiler may still wait
        // for all of them while direct-to-LDS loads are in flight)
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | ((MT + NT) << 8));
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][i], bfr[0][t], acc[i][t], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1][i], bfr[1][t], acc[i][t], 0, 0, 0);
        cs = cs + 1 == ST ? 0 : cs + 1;
    }
    __syncthreads();                                   // all reads of the last stage are done
    // residual epilogue: the tile's output rows, fetched once while the tile goes to LDS
    const int rows = min(BM, a.R - m0);
    static_assert(BM <= NTH, "one thread per row of the tile");
    __shared__ int s_orow[EPI == EPI_RESID && HEAD == 0 ? BM : 1];
    int orow_t = 0;
    if constexpr (EPI == EPI_RESID && HEAD == 0) {
        if (tid < rows) orow_t = a.o_rows ? a.o_rows[m0 + tid].hrow : m0 + tid;
    }
    // the output tile goes through LDS (the operand buffers are free now), so that the
    // epilogue runs as one compact loop with coalesced stores
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Cs[(wm * WR + i * 16 + 4 * (lane >> 4) + e) * CLD + wn * WN + t * 16 + (lane & 15)] = acc[i][t][e];
    if constexpr (EPI == EPI_RESID && HEAD == 0) {
        if (tid < rows) s_orow[tid] = orow_t;
    }
    __syncthreads();
    if constexpr (HEAD != 0) {
        if (a.xent_part) {
            // fused cross-entropy: TPR threads per row (adjacent lanes) reduce each 64-column
            // group of the row to (max, sum of exp(z - max)); reading column q + TPR k of
            // rows 132 floats apart, the 16 rows x 4 lanes of a wave cover every bank once
            constexpr int TPR = NTH / BM;
            static_assert(TPR >= 1 && TPR <= 64 && (TPR & (TPR - 1)) == 0 && 64 % TPR == 0, "threads per row");
            const int r = tid / TPR, q = tid % TPR;
            const bool live = r < rows;
            const int ng = a.N / 64;
#pragma unroll
            for (int h = 0; h < BN / 64; ++h) {
                const float* cr = &Cs[r * CLD + 64 * h];
                float mx = -INFINITY;
                if (live) {
#pragma unroll
                    for (int c = q; c < 64; c += TPR) mx = fmaxf(mx, cr[c]);
                }
#pragma unroll
                for (int off = 1; off < TPR; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
                float sm = 0.f;
                if (live) {
#pragma unroll
                    for (int c = q; c < 64; c += TPR) sm += expf(cr[c] - mx);
                }
#pragma unroll
                for (int off = 1; off < TPR; off <<= 1) sm += __shfl_xor(sm, off, 64);
                if (live && q == 0)
                    *(float2*)&a.xent_part[2 * ((int64_t)(m0 + r) * ng + n0 / 64 + h)] = make_float2(mx, sm);
            }
            if (live && q == 0) {
                const int tc = a.xent_targets[m0 + r] - n0;
                if (tc >= 0 && tc < BN) a.xent_tgt[m0 + r] = Cs[r * CLD + tc];
            }
            stamp_end_lin(a.stamp, t_begin, STAMP_BLOCKS);
            return;
        }
    }
    if constexpr (EPI == EPI_RESID && HEAD == 0) {
        // each thread keeps one column pair (c, c + 1) and takes every RPI-th row; the
        // residual values of all its rows are loaded before the first store, so their
        // latencies overlap instead of following one another (O/down at 2047 rows:
        // 33.7 -> 30.2 us per launch)
        constexpr int PPR = BN / 2, RPI = NTH / PPR, IT = BM / RPI;
        static_assert(NTH % PPR == 0 && BM % RPI == 0, "a fixed column pair per thread");
        const int c = 2 * (tid % PPR), rt = tid / PPR, n = n0 + c;
        float2 res[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = rt + it * RPI;
            res[it] = r < rows ? *(const float2*)(a.out + (int64_t)s_orow[r] * a.ldo + n) : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = rt + it * RPI;
            if (r >= rows) break;
            const float2 v = *(const float2*)&Cs[r * CLD + c];
            *(float2*)(a.out + (int64_t)s_orow[r] * a.ldo + n) = make_float2(res[it].x + v.x, res[it].y + v.y);
        }
    } else {
        for (int idx = tid; idx < rows * (BN / 2); idx += NTH) {
            const int r = idx / (BN / 2), c = 2 * (idx - r * (BN / 2));
            const float2 v = *(const float2*)&Cs[r * CLD + c];
            epi_pair_t<EPI>(a, m0 + r, n0 + c, v.x, v.y);
        }
    }
    stamp_end_lin(a.stamp, t_begin, STAMP_BLOCKS);
}

template <int BN, int ST, int NW = GB_NW, int BM = GB_BM>
static void launch_gemm_bf16_bn(const GemmArgs& a, dim3 grid, hipStream_t st) {
    const dim3 blk(64 * NW);
    if (a.head) {
        NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_bf16<BN, 1, EPI_STORE, ST, NW, BM>), grid, blk, 0, st, a);
        return;
    }
    switch (a.epi) {
        case EPI_STORE: NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_bf16<BN, 0, EPI_STORE, ST, NW, BM>), grid, blk, 0, st, a); break;
        case EPI_RESID: NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_bf16<BN, 0, EPI_RESID, ST, NW, BM>), grid, blk, 0, st, a); break;
        case EPI_SWIGLU: NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_bf16<BN, 0, EPI_SWIGLU, ST, NW, BM>), grid, blk, 0, st, a); break;
        case EPI_QKV: NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_bf16<BN, 0, EPI_QKV, ST, NW, BM>), grid, blk, 0, st, a); break;
        default: NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_bf16<BN, 0, EPI_SILU, ST, NW, BM>), grid, blk, 0, st, a); break;
    }
}

// Whether a product takes the split-K decode path, and its slice count.
int sk_slices(const GemmArgs& a) {
    if (!a.wbf16 || a.head > 1 || a.comb || !a.sk_ws || a.mfma_min_rows <= 0 || a.sk_min_rows <= 0 || a.R < a.sk_min_rows ||
        a.R > a.sk_max_rows || a.R > SK_MAX_ROWS || a.K % SK_KC || a.N % 32 || a.out_bf16 || a.abf_ready || a.xent_part ||
        a.xd_part || a.epi < EPI_STORE || a.epi > EPI_SILU)
        return 0;
    const int ntb = a.norm_w ? (a.sk_ntb & 15) : ((a.sk_ntb >> 4) & 15);
    if ((ntb != 1 && ntb != 2) || a.N % (16 * ntb)) return 0;
    const int nks = a.K / SK_KC;
    if ((int64_t)nks * a.R * (a.N + 1) > a.sk_cap) return 0;
    return nks;
}

bool gemm_uses_bf16_rows(const GemmArgs& a) {
    return a.wbf16 && a.abf && a.mfma_min_rows > 0 && a.R >= GB_MIN_ROWS && a.N % 64 == 0 && a.K % GB_BK == 0 &&
           !a.comb && !sk_slices(a);
}

// ------------------------------------------------------------------------------------------
// Decode-sized products, K split across the waves of a block.
//
// A block owns a few output columns; wave w takes the w-th slice of K, so each lane holds
// one 16-byte chunk of K per column (chunk = 64 w + lane).  Activation chunks are loaded
// first and weight chunks after them (loads retire in order, so the activations can be
// used while the weights are still in flight); nothing waits on a barrier until the
// cross-wave reduction at the end.  RMSNorm is folded in: the product is taken on
// (x * g) and scaled by 1/rms(x) per row in the epilogue, the sum of squares coming from
// the same chunks.
// ------------------------------------------------------------------------------------------

constexpr int KS_CPB = 8;          // output columns per block (vector-ALU kernel)

// ------------------------------------------------------------------------------------------
// Exit draw.  Inverse-CDF sampling of softmax(z) in token-id order (gist.science summary,
// section 3: each exit's distribution is sampled exactly; the walk of the gates picked the
// exit).  The one-row head product (k_gemv_ks with HEAD 2) ends with the online-softmax
// step of each block: block b holds the logits of ids 8b..8b+7 and writes m_b = max z and
// s_b = sum_j exp(z_j - m_b) (float32 exponentials summed in float32 in id order).  Then one
// block (k_exit_draw) merges the partials:
//   M = max_b m_b, t_b = s_b * exp(m_b - M) (float64), Z = sum_b t_b in block order;
//   target = u * Z; b* = the block where the running sum of t_b first exceeds target;
//   token = 8 b* + the first j with target < S_b* + c_j * exp(m_b* - M), c_j the float32
//   running sum of exp(z_j - m_b*), which ends at s_b* exactly (the same operations).
// If rounding leaves target at or past the total, the token is the last id with nonzero
// mass.  The kernel boundary between the two makes the partials visible: on this chip a
// completion count across the head product's 4000 blocks costs more than that boundary.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void exit_partial(const GemmArgs& a, const float* zb) {
    __syncthreads();                                   // zb[] written by the epilogue threads
    if (threadIdx.x == 0) {
        float mb = -INFINITY;
        for (int j = 0; j < KS_CPB; ++j) mb = fmaxf(mb, zb[j]);
        float sb = 0.f;
        if (mb != -INFINITY)
            for (int j = 0; j < KS_CPB; ++j) sb += expf(zb[j] - mb);
        *(float2*)(a.xd_part + 2 * (int64_t)blockIdx.x) = make_float2(mb, sb);
    }
}

template <int PER>   // partials per thread: ceil(nb / XD_THREADS) <= PER <= XD_PER
__global__ __launch_bounds__(XD_THREADS) void k_exit_draw(const float* part, int nb, const float* logits, float u,
                                                          int* token) {
    __shared__ float s_red[XD_THREADS / 64];
    __shared__ double s_dred[XD_THREADS / 64];
    __shared__ int s_bstar, s_last;
    __shared__ double s_pre;
    __shared__ float s_mb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = XD_THREADS / 64;
    const int per = (nb + XD_THREADS - 1) / XD_THREADS;          // <= PER (checked at launch)
    const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
    if (tid == 0) {
        s_bstar = -1;
        s_last = -1;
    }
    float pm[PER], ps[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float2 v = *(const float2*)(part + 2 * (b0 + i < b1 ? b0 + i : 0));   // past the range: block 0, unused
        pm[i] = v.x;
        ps[i] = v.y;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (b0 + i < b1) mx = fmaxf(mx, pm[i]);
    mx = wave_max(mx);
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w]);
    // t_b = s_b e^(m_b - M) in float32 (each at most 8, relative error ~1e-7); this thread's
    // sum, and every running sum below, in float64 in block order
    float t[PER];
    double loc = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        t[i] = (b0 + i < b1 && pm[i] != -INFINITY) ? ps[i] * expf(pm[i] - M) : 0.f;
        loc += (double)t[i];
    }
    // exclusive prefix of the thread sums in thread order (fixed order: waves, then lanes)
    double inc = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    if (lane == 63) s_dred[wave] = inc;
    __syncthreads();
    double wpre = 0.0, Z = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (w < wave) wpre += s_dred[w];
        Z += s_dred[w];
    }
    double exc = __shfl_up(inc, 1, 64);
    if (lane == 0) exc = 0.0;
    const double lo = wpre + exc, hi = wpre + inc;   // lo of a thread == hi of the one before
    const double target = (double)u * Z;
    if (b0 < b1 && lo <= target && target < hi) {
        // the first block of this range whose running sum passes target (the last one if
        // rounding keeps the walk below it)
        double cum = lo, prev = lo, pre = lo;
        int bs = -1;
        float mbs = -INFINITY, mprev = -INFINITY;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (bs < 0 && b0 + i < b1) {
                const double nx = cum + (double)t[i];
                if (target < nx) {
                    bs = b0 + i;
                    pre = cum;
                    mbs = pm[i];
                }
                prev = cum;
                mprev = pm[i];
                cum = nx;
            }
        }
        if (bs < 0) {
            bs = b1 - 1;
            pre = prev;
            mbs = mprev;
        }
        s_bstar = bs;
        s_pre = pre;
        s_mb = mbs;
    }
    // the last block with a nonzero weight (for the fall-back)
    int lb = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (b0 + i < b1 && t[i] > 0.f) lb = b0 + i;
    if (lb >= 0) atomicMax(&s_last, lb);
    __syncthreads();
    if (tid == 0) {
        int tok = -1;
        const int bs = s_bstar;
        if (bs >= 0) {
            // the crossing block's 8 logits in one round of loads (its max came through LDS)
            static_assert(KS_CPB == 8, "a head block's logits are two float4");
            const float mb = s_mb;
            const float* zb = logits + (int64_t)bs * KS_CPB;
            float z[KS_CPB];
            if ((reinterpret_cast<uintptr_t>(zb) & 15) == 0) {
                const float4 z0 = *(const float4*)zb, z1 = *(const float4*)(zb + 4);
                z[0] = z0.x; z[1] = z0.y; z[2] = z0.z; z[3] = z0.w;
                z[4] = z1.x; z[5] = z1.y; z[6] = z1.z; z[7] = z1.w;
            } else {
#pragma unroll
                for (int j = 0; j < KS_CPB; ++j) z[j] = zb[j];
            }
            const double f = mb == -INFINITY ? 0.0 : (double)expf(mb - M);
            float c = 0.f;
            tok = bs * KS_CPB + KS_CPB - 1;
#pragma unroll
            for (int j = 0; j < KS_CPB; ++j) {
                c += expf(z[j] - mb);
                if (target < s_pre + (double)c * f) {
                    tok = bs * KS_CPB + j;
                    break;
                }
            }
        } else if (s_last >= 0) {
            // target at or past the rounded total: the last id with nonzero mass
            const int L = s_last;
            const float mb = part[2 * L];
            for (int j = KS_CPB - 1; j >= 0; --j)
                if (expf(logits[L * KS_CPB + j] - mb) > 0.f) {
                    tok = L * KS_CPB + j;
                    break;
                }
        }
        *token = tok;
    }
}

hipError_t launch_exit_draw(const float* part, int nb, const float* logits, float u, int* token, hipStream_t st) {
    if (nb < 1 || nb > XD_PER * XD_THREADS || !part || !logits || !token || !(u >= 0.0f && u < 1.0f))
        return hipErrorInvalidValue;
    if (t_ev_stop) snprintf(t_name, sizeof(t_name), "nv::k_exit_draw");
    if (nb <= 8 * XD_THREADS)
        NV_LAUNCH(HIP_KERNEL_NAME(k_exit_draw<8>), dim3(1), dim3(XD_THREADS), 0, st, part, nb, logits, u, token);
    else
        NV_LAUNCH(HIP_KERNEL_NAME(k_exit_draw<XD_PER>), dim3(1), dim3(XD_THREADS), 0, st, part, nb, logits, u, token);
    return hipGetLastError();
}

template <bool WBF, int RM, int HEAD, bool COMB = false, int EPIT = -1>
__global__ __launch_bounds__(512) void k_gemv_ks(GemmArgs a) {
    static_assert(!COMB || RM == 1, "the fused attention merge handles one row");
    static_assert(HEAD != 2 || (RM == 1 && !COMB), "the fused exit draw handles one row");
    __shared__ float xd_z[HEAD == 2 ? KS_CPB : 1];
    constexpr int EPC = WBF ? 8 : 4;
    constexpr int ESZ = WBF ? 2 : 4;
    constexpr int NV = KS_CPB * RM;     // values per lane to reduce
    __shared__ float red[8][NV];
    __shared__ float ssr[8][RM];
    const unsigned long long t_begin = stamp_begin(a.stamp);
    const int K = a.K, R = a.R;
    const int nch = K / EPC;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int n0 = blockIdx.x * KS_CPB;
    const int ch = wave * 64 + lane;
    const bool act = ch < nch;
    const int k0 = (act ? ch : nch - 1) * EPC;

    // epilogue context of the thread that will finish (row er, columns n0+ec, n0+ec+1); for a
    // contiguous chunk it is fetched after the weight loads (below)
    const bool ethr = threadIdx.x < KS_CPB / 2 * RM;
    const int er = threadIdx.x % RM, ec = 2 * (threadIdx.x / RM);
    EpiCtx ectx{};
    if (!a.contig && ethr && er < R) ectx = epi_prepare<EPIT>(a, er, n0 + ec);

    // activation chunks (rows past R repeat row R-1; their results are never written)
    float av[RM][EPC];
    const CombineInfo cmb = !COMB                       ? CombineInfo{0, 0, 1, 1}
                            : (a.contig && a.comb_ns > 0) ? CombineInfo{0, 0, a.comb_ns, 1}
                                                          : a.comb[0];
    if (!COMB || cmb.nsplit == 1) {
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const int rr = r < R ? r : R - 1;
            const int ar = !a.a_rows ? rr : a.contig ? a.a_row0 + rr : a.a_rows[rr].hrow;
            const float4* ap = (const float4*)(a.A + (int64_t)ar * a.lda + k0);
#pragma unroll
            for (int e = 0; e < EPC / 4; ++e) {
                const float4 t = ap[e];
                av[r][4 * e] = t.x; av[r][4 * e + 1] = t.y; av[r][4 * e + 2] = t.z; av[r][4 * e + 3] = t.w;
            }
        }
    }
    float gv[EPC];
    if (a.norm_w) {
        const float4* gp = (const float4*)(a.norm_w + k0);
#pragma unroll
        for (int e = 0; e < EPC / 4; ++e) {
            const float4 t = gp[e];
            gv[4 * e] = t.x; gv[4 * e + 1] = t.y; gv[4 * e + 2] = t.z; gv[4 * e + 3] = t.w;
        }
    }
    // COMB: this lane's 8 dims (e0..e0+7 of head h) of the attention output are the online
    // merge of the split partials (max m_s, sum l_s, unnormalised output o_s), 8 splits per
    // batch.  The first batch is loaded before the weights, so that its latency overlaps
    // theirs (vector loads retire in order: loaded after, it would wait for the weights).
    const bool merge = COMB && cmb.nsplit > 1;
    const int c_hd = a.D.hd, c_h = COMB ? k0 / max(c_hd, 1) : 0, c_e0 = k0 - c_h * c_hd;
    const int64_t c_base = COMB ? cmb.base + (int64_t)c_h * cmb.nsplit * cmb.nrows + cmb.off : 0;
    auto load_parts = [&](int s0, float2 (&ml)[8], float (&ob)[8][EPC]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int sp = s0 + j < cmb.nsplit ? s0 + j : cmb.nsplit - 1;
            const int64_t slot = c_base + (int64_t)sp * cmb.nrows;
            ml[j] = *(const float2*)(a.part_ml + 2 * slot);
            const float4* op = (const float4*)(a.part_o + slot * c_hd + c_e0);
#pragma unroll
            for (int q4 = 0; q4 < EPC / 4; ++q4) {
                const float4 t = op[q4];
                ob[j][4 * q4] = t.x; ob[j][4 * q4 + 1] = t.y; ob[j][4 * q4 + 2] = t.z; ob[j][4 * q4 + 3] = t.w;
            }
        }
    };
    float2 ml0[8];
    float ob0[8][EPC];
    if constexpr (COMB) {
        if (merge) load_parts(0, ml0, ob0);
    }

    uint4 w[KS_CPB];
#pragma unroll
    for (int c = 0; c < KS_CPB; ++c) w[c] = stream_load16((const char*)a.W + ((size_t)(n0 + c) * K + k0) * ESZ);
    // every weight load is issued before anything waits on the activations
    __builtin_amdgcn_sched_barrier(0);
    if (a.contig && ethr && er < R) ectx = epi_prefetch<EPIT>(a, er, n0 + ec);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (COMB) {
        if (merge) {
            const int ns = cmb.nsplit;
            float M = -INFINITY, L = 0.f, O[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) O[e] = 0.f;
            auto merge_parts = [&](int s0, const float2 (&ml)[8], const float (&ob)[8][EPC]) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (s0 + j < ns && ml[j].x != -INFINITY) {
                        const float Mn = fmaxf(M, ml[j].x);
                        const float ca = expf(M - Mn), cb = expf(ml[j].x - Mn);
                        L = ca * L + cb * ml[j].y;
#pragma unroll
                        for (int e = 0; e < EPC; ++e) O[e] = ca * O[e] + cb * ob[j][e];
                        M = Mn;
                    }
                }
            };
            merge_parts(0, ml0, ob0);
            for (int s0 = 8; s0 < ns; s0 += 8) {
                float2 ml[8];
                float ob[8][EPC];
                load_parts(s0, ml, ob);
                merge_parts(s0, ml, ob);
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) av[0][e] = O[e] / L;
        }
    }

    const float amask = act ? 1.0f : 0.0f;   // lanes past the end of K contribute nothing
    float ss[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        ss[r] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            const float x = av[r][e] * amask;
            ss[r] = fmaf(x, x, ss[r]);
            av[r][e] = a.norm_w ? x * gv[e] : x;
        }
    }
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < KS_CPB; ++c) {
        const uint32_t u[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
        float wf[EPC];
        if constexpr (WBF) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wf[2 * e] = bf_lo(u[e]);
                wf[2 * e + 1] = bf_hi(u[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) wf[e] = __uint_as_float(u[e]);
        }
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[c * RM + r] = fmaf(wf[e], av[r][e], acc[c * RM + r]);
    }
    // value index c*RM + r: row (lane / 16) holds indices [row * NV/4, (row + 1) * NV/4)
    wave_rowsum_transpose<NV>(acc);
    if ((lane & 15) == 0) {
#pragma unroll
        for (int j = 0; j < NV / 4; ++j) red[wave][(lane >> 4) * (NV / 4) + j] = acc[j];
    }
    if (a.norm_w) {
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const float t = wave_total(ss[r]);
            if (lane == 0) ssr[wave][r] = t;
        }
    }
    __syncthreads();
    if (ethr && er < R) {
        float v0 = 0.f, v1 = 0.f, sq = 0.f;
        for (int ww = 0; ww < nw; ++ww) {
            v0 += red[ww][ec * RM + er];
            v1 += red[ww][(ec + 1) * RM + er];
            if (a.norm_w) sq += ssr[ww][er];
        }
        if (a.norm_w) {
            const float inv = 1.0f / sqrtf(sq / (float)K + a.eps);
            v0 *= inv;
            v1 *= inv;
        }
        epi_apply<EPIT>(a, ectx, er, n0 + ec, v0, v1);
        if constexpr (HEAD == 2) {
            xd_z[ec] = v0;
            xd_z[ec + 1] = v1;
        }
    }
    if constexpr (HEAD == 2) exit_partial(a, xd_z);
    stamp_end(a.stamp, t_begin);
}

// Matrix-core version for 9..32 rows: the block owns 16 columns; wave w takes the w-th
// K slice in steps of 32 (one v_mfma_f32_16x16x32_bf16 per 16-row tile and step).
// Activation fragments (rows l%16 of each tile, k 8*(l/16)..) are loaded first, scaled by
// g, rounded to bf16; weight fragments W[n0 + l%16][k ...] follow.  Partial tiles of the
// waves are summed through LDS.
template <int S, int MT, int NT, bool NORM, int HEAD>
__global__ __launch_bounds__(1024) void k_gemm_mfma_ks(GemmArgs a) {
    __shared__ float red[16][MT][NT][64][4];
    __shared__ float ssr[16][MT * 16];
    const unsigned long long t_begin = stamp_begin(a.stamp);
    const int K = a.K, R = a.R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int n0 = blockIdx.x * 16 * NT;
    const int kq = 8 * (lane >> 4);
    const int kb = wave * (32 * S) + kq;   // host: K == nw * 32 * S

    // epilogue context for the rows this lane finishes (waves < MT * NT own one
    // (row tile, column tile) each)
    EpiCtx ectx[4];
    const int emt = wave / NT, ent = wave - (wave / NT) * NT;
    const int ecol = n0 + ent * 16 + (lane & 15);
    if (wave < MT * NT && (ecol & 1) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = emt * 16 + 4 * (lane >> 4) + i;
            if (row < R) ectx[i] = epi_prepare(a, row, ecol);
        }
    }
    // activation fragments: row (tile*16 + l%16), k = kb + 32 s .. +8; rows past R repeat R-1
    float x[MT][S][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int row = mt * 16 + (lane & 15);
        row = row < R ? row : R - 1;
        const float* ap = a.A + (int64_t)(a.a_rows ? a.a_rows[row].hrow : row) * a.lda + kb;
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) {
            const float4 x0 = *(const float4*)(ap + 32 * s2), x1 = *(const float4*)(ap + 32 * s2 + 4);
            x[mt][s2][0] = x0.x; x[mt][s2][1] = x0.y; x[mt][s2][2] = x0.z; x[mt][s2][3] = x0.w;
            x[mt][s2][4] = x1.x; x[mt][s2][5] = x1.y; x[mt][s2][6] = x1.z; x[mt][s2][7] = x1.w;
        }
    }
    float gn[NORM ? S : 1][8];
    if constexpr (NORM) {
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) {
            const float4 g0 = *(const float4*)(a.norm_w + kb + 32 * s2);
            const float4 g1 = *(const float4*)(a.norm_w + kb + 32 * s2 + 4);
            gn[s2][0] = g0.x; gn[s2][1] = g0.y; gn[s2][2] = g0.z; gn[s2][3] = g0.w;
            gn[s2][4] = g1.x; gn[s2][5] = g1.y; gn[s2][6] = g1.z; gn[s2][7] = g1.w;
        }
    }
    u32x4 wv[NT][S];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const uint16_t* wp = (const uint16_t*)a.W + (int64_t)(n0 + nt * 16 + (lane & 15)) * K + kb;
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) wv[nt][s2] = *(const u32x4*)(wp + 32 * s2);
    }

    float ss[MT];
    bf16x8_t af[MT][S];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        ss[mt] = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) {
            uint32_t p[4];
            if constexpr (NORM) {
#pragma unroll
                for (int e = 0; e < 8; ++e) ss[mt] = fmaf(x[mt][s2][e], x[mt][s2][e], ss[mt]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x0 = x[mt][s2][2 * e], x1 = x[mt][s2][2 * e + 1];
                if constexpr (NORM) {
                    x0 *= gn[NORM ? s2 : 0][2 * e];
                    x1 *= gn[NORM ? s2 : 0][2 * e + 1];
                }
                p[e] = pack_bf2(x0, x1);
            }
            af[mt][s2] = __builtin_bit_cast(bf16x8_t, make_uint4(p[0], p[1], p[2], p[3]));
        }
    }
    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, wv[nt][s2]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt][s2], bf, acc[mt][nt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][mt][nt][lane][i] = acc[mt][nt][i];
        float t = ss[mt];
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 32, 64);
        if (lane < 16) ssr[wave][mt * 16 + lane] = t;
    }
    __syncthreads();
    if (wave < MT * NT) {
        const int mt = emt;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        for (int ww = 0; ww < nw; ++ww)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += red[ww][mt][ent][lane][i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mt * 16 + 4 * (lane >> 4) + i;
            float y = v[i];
            if constexpr (NORM) {
                float sq = 0.f;
                for (int ww = 0; ww < nw; ++ww) sq += ssr[ww][row];
                y *= 1.0f / sqrtf(sq / (float)K + a.eps);
            }
            const float u = __shfl_xor(y, 1, 64);
            if (row < R && (ecol & 1) == 0) epi_apply(a, ectx[i], row, ecol, y, u);
        }
    }
    stamp_end(a.stamp, t_begin);
}

// Decode-sized row groups (up to 16 MT rows) on the matrix cores with K split across
// blocks.  Block (x, y) owns 16 NTB output columns and the K slice [SK_KC y, SK_KC (y + 1));
// its four waves are NTB column tiles times 4 / NTB k-parts of KPW steps of 32.  The rows'
// slice is staged once per block in LDS as bf16 (times the RMSNorm weight for NORM), the
// weight fragments stream straight into registers, the k-parts are added through LDS and
// the block stores its fp32 partial tile (column tile 0 also its rows' sums of squares).
// A 1536-column product thus runs on 96 x K/512 blocks instead of 96, so that every
// compute unit streams weights.  k_gemm_sk_reduce then adds the slices in slice order and
// applies RMSNorm's row scale and the product's epilogue.
template <int MT, int NTB, bool NORM>
__global__ __launch_bounds__(256) void k_gemm_sk(GemmArgs a, float* part, float* pss) {
    constexpr int KPARTS = 4 / NTB;
    constexpr int KPW = SK_KC / (KPARTS * 32);   // k-steps per wave
    constexpr int LDA = SK_KC + 8;               // bf16 per LDS row: rows 16 bytes apart in bank order
    constexpr int RP = 16 * MT;
    constexpr int RW = RP / 4;                   // rows staged per wave
    static_assert(SK_KC == 512, "the staging below covers 512 values per row with 64 lanes");
    __shared__ __attribute__((aligned(16))) uint16_t as[RP][LDA];
    __shared__ f32x4_t red[KPARTS - 1 > 0 ? KPARTS - 1 : 1][NTB][MT][64];
    const unsigned long long t_begin = stamp_begin(a.stamp);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nt = wave % NTB, kp = wave / NTB;
    const int K = a.K, R = a.R, N = a.N;
    const int n0 = blockIdx.x * 16 * NTB, ks = blockIdx.y, k0 = ks * SK_KC;

    // weight fragments: row n0 + 16 nt + lane % 16, k = k0 + 32 (kp KPW + s) + 8 (lane / 16)
    u32x4 wv[KPW];
    {
        const uint16_t* wp = (const uint16_t*)a.W + (int64_t)(n0 + nt * 16 + (lane & 15)) * K + k0 +
                             32 * kp * KPW + 8 * (lane >> 4);
#pragma unroll
        for (int s = 0; s < KPW; ++s) wv[s] = __builtin_nontemporal_load((const u32x4*)(wp + 32 * s));
    }
    // the rows' slice: wave w stages rows w, w + 4, ...; a lane takes floats 4 lane .. 4 lane + 3
    // and 256 + 4 lane .. 256 + 4 lane + 3 (rows past R are zero)
    float4 gv[2];
    if constexpr (NORM) {
        gv[0] = *(const float4*)(a.norm_w + k0 + 4 * lane);
        gv[1] = *(const float4*)(a.norm_w + k0 + 256 + 4 * lane);
    }
    float4 xv[RW][2];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int r = wave + 4 * i;
        if (r < R) {
            const float* ap = a.A + (int64_t)(a.a_rows ? a.a_rows[r].hrow : r) * a.lda + k0 + 4 * lane;
            xv[i][0] = *(const float4*)ap;
            xv[i][1] = *(const float4*)(ap + 256);
        } else {
            xv[i][0] = xv[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    float ss[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int r = wave + 4 * i;
        float4 x0 = xv[i][0], x1 = xv[i][1];
        if constexpr (NORM) {
            float t = x0.x * x0.x;
            t = fmaf(x0.y, x0.y, t); t = fmaf(x0.z, x0.z, t); t = fmaf(x0.w, x0.w, t);
            t = fmaf(x1.x, x1.x, t); t = fmaf(x1.y, x1.y, t); t = fmaf(x1.z, x1.z, t); t = fmaf(x1.w, x1.w, t);
            ss[i] = t;
            x0.x *= gv[0].x; x0.y *= gv[0].y; x0.z *= gv[0].z; x0.w *= gv[0].w;
            x1.x *= gv[1].x; x1.y *= gv[1].y; x1.z *= gv[1].z; x1.w *= gv[1].w;
        }
        *(uint2*)&as[r][4 * lane] = make_uint2(pack_bf2(x0.x, x0.y), pack_bf2(x0.z, x0.w));
        *(uint2*)&as[r][256 + 4 * lane] = make_uint2(pack_bf2(x1.x, x1.y), pack_bf2(x1.z, x1.w));
    }
    if constexpr (NORM) {
        if (blockIdx.x == 0) {   // one block per slice stores the slice's sums of squares
#pragma unroll
            for (int i = 0; i < RW; ++i) {
                const int r = wave + 4 * i;
                const float t = wave_total(ss[i]);
                if (lane == 0 && r < R) pss[ks * R + r] = t;
            }
        }
    }
    __syncthreads();

    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KPW; ++s) {
        const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, wv[s]);
        const int kk = 32 * (kp * KPW + s) + 8 * (lane >> 4);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const u32x4 au = *(const u32x4*)&as[mt * 16 + (lane & 15)][kk];
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, au), bf, acc[mt], 0, 0, 0);
        }
    }
    if constexpr (KPARTS > 1) {
        if (kp > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[kp - 1][nt][mt][lane] = acc[mt];
        }
        __syncthreads();
        if (kp == 0) {
#pragma unroll
            for (int q = 0; q < KPARTS - 1; ++q)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt] += red[q][nt][mt][lane];
        }
    }
    if (kp == 0) {
        // acc[mt][i] is (row mt*16 + 4 (lane / 16) + i, column lane % 16) of the tile
        const int col = n0 + nt * 16 + (lane & 15);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = mt * 16 + 4 * (lane >> 4) + i;
                if (row < R) part[((int64_t)ks * R + row) * N + col] = acc[mt][i];
            }
    }
    stamp_end_lin(a.stamp, t_begin, STAMP_BLOCKS);
}

// The slices of k_gemm_sk added in slice order, RMSNorm's row scale, then the product's
// epilogue on the column pair (col, col + 1) of one row.
template <bool NORM>
__global__ __launch_bounds__(256) void k_gemm_sk_reduce(GemmArgs a, const float* part, const float* pss, int nks) {
    const int np = a.N >> 1;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.R * np) return;
    const int row = idx / np, col = 2 * (idx - row * np);
    float y = 0.f, u = 0.f, sq = 0.f;
    for (int s0 = 0; s0 < nks; s0 += 8) {
        // eight slices' loads issued before the first add
        float2 p[8];
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = s0 + j;
            p[j] = s < nks ? *(const float2*)(part + ((int64_t)s * a.R + row) * a.N + col) : make_float2(0.f, 0.f);
            q[j] = NORM && s < nks ? pss[s * a.R + row] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (s0 + j < nks) {
                y += p[j].x;
                u += p[j].y;
                sq += q[j];
            }
        }
    }
    if constexpr (NORM) {
        const float inv = 1.0f / sqrtf(sq / (float)a.K + a.eps);
        y *= inv;
        u *= inv;
    }
    const EpiCtx e = epi_prepare(a, row, col);
    epi_apply(a, e, row, col, y, u);
}

static bool use_mfma(const GemmArgs& a) {
    return a.wbf16 && a.mfma_min_rows > 0 && a.R >= a.mfma_min_rows && a.K % MF_BK == 0 && a.N % 64 == 0 &&
           (a.norm_w == nullptr || a.rms_ws != nullptr);
}

hipError_t launch_rows_bf16(const GemmArgs& a, hipStream_t st) {
    if (!gemm_uses_bf16_rows(a)) return hipErrorInvalidValue;
    launch_rows_bf16_any(a, st);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    if (a.R <= 0) return hipSuccess;
    // the fused cross-entropy exists only in the long-chunk head product
    if (a.xent_part && (!a.head || !a.xent_tgt || !a.xent_targets || !gemm_uses_bf16_rows(a)))
        return hipErrorInvalidValue;
    const int epc = a.wbf16 ? 8 : 4;
    GemmArgs b = a;
    b.stamp = t_stamp;
    if (a.comb) {   // single row, attention output merged on the fly (vector-ALU path only)
        const int nw = (a.K / epc + 63) / 64;
        if (a.R != 1 || !a.wbf16 || a.K % epc || a.N % KS_CPB || nw > 8 || a.D.hd % 8) return hipErrorInvalidValue;
        if (a.epi != EPI_RESID) return hipErrorInvalidValue;
        if (t_ev_stop) snprintf(t_name, sizeof(t_name), "void nv::k_gemv_ks<true, 1, 0, true, %d>(nv::GemmArgs)", EPI_RESID);
        NV_LAUNCH(HIP_KERNEL_NAME(k_gemv_ks<true, 1, 0, true, EPI_RESID>), dim3(a.N / KS_CPB), dim3(64 * nw), 0, st, b);
        return hipGetLastError();
    }
    // decode-sized row groups on the matrix cores, K split across blocks
    if (const int nks = sk_slices(a)) {
        const int mt = (a.R + 15) / 16;
        const bool norm = a.norm_w != nullptr;
        const int ntb = norm ? (a.sk_ntb & 15) : ((a.sk_ntb >> 4) & 15);
        float* part = a.sk_ws;
        float* pss = part + (int64_t)nks * a.R * a.N;
        const dim3 grid(a.N / (16 * ntb), nks), block(256);
        if (t_ev_stop)
            snprintf(t_name, sizeof(t_name), "void nv::k_gemm_sk<%d, %d, %s>(nv::GemmArgs)", mt, ntb,
                     norm ? "true" : "false");
#define NV_SK2(MTV, NTV)                                                                                      \
    do {                                                                                                     \
        if (norm) NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_sk<MTV, NTV, true>), grid, block, 0, st, b, part, pss);   \
        else NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_sk<MTV, NTV, false>), grid, block, 0, st, b, part, pss);       \
    } while (0)
#define NV_SK(MTV)                                                                                            \
    do {                                                                                                     \
        if (ntb == 1) NV_SK2(MTV, 1); else NV_SK2(MTV, 2);                                                   \
    } while (0)
        if (mt == 1) NV_SK(1); else if (mt == 2) NV_SK(2); else if (mt == 3) NV_SK(3); else NV_SK(4);
#undef NV_SK
#undef NV_SK2
        // the reduction belongs to the same timed product; its blocks store no stamps
        const int stamped = t_blocks;
        const dim3 rgrid((a.R * (a.N / 2) + 255) / 256);
        if (norm) NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_sk_reduce<true>), rgrid, block, 0, st, b, part, pss, nks);
        else NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_sk_reduce<false>), rgrid, block, 0, st, b, part, pss, nks);
        t_blocks = stamped;
        return hipGetLastError();
    }
    // decode-sized rows, vector ALUs (rows <= 8, and below the matrix-core threshold)
    if (a.R <= 8 && (a.mfma_min_rows == 0 || a.R < a.mfma_min_rows || !a.wbf16) && a.K % epc == 0 &&
        a.N % KS_CPB == 0 && (a.K / epc + 63) / 64 <= 8 && a.K % 4 == 0) {
        const int nw = (a.K / epc + 63) / 64;
        const dim3 grid(a.N / KS_CPB), block(64 * nw);
        const int rm = a.R <= 1 ? 1 : a.R <= 2 ? 2 : a.R <= 4 ? 4 : 8;
        // bf16: one instance per epilogue kind (the head's is EPI_STORE); fp32: run-time kind
        const int ek = !a.wbf16 ? -1 : a.head ? (int)EPI_STORE : a.epi;
#define NV_KS_E(WB, RMV, HD, E) NV_LAUNCH(HIP_KERNEL_NAME(k_gemv_ks<WB, RMV, HD, false, E>), grid, block, 0, st, b)
#define NV_KS(RMV)                                                                                            \
    do {                                                                                                     \
        if (!a.wbf16) {                                                                                      \
            if (a.head) NV_KS_E(false, RMV, 1, -1); else NV_KS_E(false, RMV, 0, -1);                         \
        } else if (a.head) {                                                                                 \
            NV_KS_E(true, RMV, 1, EPI_STORE);                                                                \
        } else {                                                                                             \
            switch (a.epi) {                                                                                 \
                case EPI_QKV: NV_KS_E(true, RMV, 0, EPI_QKV); break;                                         \
                case EPI_RESID: NV_KS_E(true, RMV, 0, EPI_RESID); break;                                     \
                case EPI_SWIGLU: NV_KS_E(true, RMV, 0, EPI_SWIGLU); break;                                   \
                case EPI_SILU: NV_KS_E(true, RMV, 0, EPI_SILU); break;                                       \
                default: NV_KS_E(true, RMV, 0, EPI_STORE); break;                                            \
            }                                                                                                \
        }                                                                                                    \
    } while (0)
        if (a.head == 2) {
            // the head product with its softmax partials: one row
            if (a.R != 1 || !a.xd_part || a.epi != EPI_STORE || a.N / KS_CPB > XD_PER * XD_THREADS)
                return hipErrorInvalidValue;
            if (t_ev_stop) snprintf(t_name, sizeof(t_name), "void nv::k_gemv_ks<%s, 1, 2, false, %d>(nv::GemmArgs)",
                                    a.wbf16 ? "true" : "false", ek);
            if (a.wbf16) NV_KS_E(true, 1, 2, EPI_STORE);
            else NV_KS_E(false, 1, 2, -1);
            return hipGetLastError();
        }
        if (a.wbf16 && !a.head && (a.epi < EPI_STORE || a.epi > EPI_SILU)) return hipErrorInvalidValue;
        if (t_ev_stop) snprintf(t_name, sizeof(t_name), "void nv::k_gemv_ks<%s, %d, %d, false, %d>(nv::GemmArgs)",
                                a.wbf16 ? "true" : "false", rm, a.head ? 1 : 0, ek);
        if (rm == 1) NV_KS(1); else if (rm == 2) NV_KS(2); else if (rm == 4) NV_KS(4); else NV_KS(8);
#undef NV_KS
#undef NV_KS_E
        return hipGetLastError();
    }
    // decode-sized rows on the matrix cores (rows <= 32): K split across the waves, S k-steps each
    if (a.wbf16 && a.R <= 32 && a.mfma_min_rows > 0 && a.R >= a.mfma_min_rows && a.N % 16 == 0) {
        int S = 0;
        for (int cand : {3, 8, 1})
            if (a.K % (32 * cand) == 0 && a.K / (32 * cand) <= 16 && !(cand == 8 && a.norm_w)) {
                S = cand;
                break;
            }
        if (S > 0) {
            const int nw = a.K / (32 * S);
            // two column tiles per block when one tile per block would take more than one
            // round of blocks (a block of 16 waves fills a CU)
            const int ntv = (a.N % 32 == 0 && a.N / 16 > 256) ? 2 : 1;
            const dim3 grid(a.N / (16 * ntv)), block(64 * nw);
#define NV_MKS3(SV, MTV, NTV, NV_)                                                                             \
    do {                                                                                                      \
        if (a.head) NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_mfma_ks<SV, MTV, NTV, NV_, 1>), grid, block, 0, st, b); \
        else NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_mfma_ks<SV, MTV, NTV, NV_, 0>), grid, block, 0, st, b);        \
    } while (0)
#define NV_MKS2(SV, MTV, NV_)                                                                                  \
    do {                                                                                                      \
        if (ntv == 2) NV_MKS3(SV, MTV, 2, NV_); else NV_MKS3(SV, MTV, 1, NV_);                              \
    } while (0)
#define NV_MKS(SV, MTV)                                                                                        \
    do {                                                                                                      \
        if (a.norm_w) NV_MKS2(SV, MTV, true); else NV_MKS2(SV, MTV, false);                                   \
    } while (0)
            if (nw >= 2 || a.R <= 16) {
                if (t_ev_stop)
                    snprintf(t_name, sizeof(t_name), "void nv::k_gemm_mfma_ks<%d, %d, %d, %s, %d>(nv::GemmArgs)", S,
                             a.R <= 16 ? 1 : 2, ntv, a.norm_w ? "true" : "false", a.head ? 1 : 0);
                if (a.R <= 16) {
                    if (S == 3) NV_MKS(3, 1); else if (S == 8) NV_MKS2(8, 1, false); else NV_MKS(1, 1);
                } else {
                    if (S == 3) NV_MKS(3, 2); else if (S == 8) NV_MKS2(8, 2, false); else NV_MKS(1, 2);
                }
#undef NV_MKS
#undef NV_MKS2
#undef NV_MKS3
                return hipGetLastError();
            }
        }
    }
    if (gemm_uses_bf16_rows(a)) {
        if (!a.abf_ready) {
            launch_rows_bf16_any(a, st);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const unsigned mt = (unsigned)((a.R + GB_BM - 1) / GB_BM);
        // 128-column tiles (two stages, two blocks per CU) when their blocks fill at least 3/4
        // of the rounds of 512 slots they take; else 64-column tiles, with three stages
        // while at most one round of 512 is launched (the deeper prefetch pays when few
        // blocks share a CU) and two stages (three blocks per CU) above that
        const long b128 = (a.N / 128) * (long)mt, b64 = (a.N / 64) * (long)mt;
        const bool wide = a.N % 128 == 0 && 4 * b128 >= 3 * 512 * ((b128 + 511) / 512);
        const int stg = wide ? 2 : b64 <= 512 ? 3 : 2;
        // narrow products on up to 1024 rows take 64-row tiles (twice the blocks; prefill of
        // 256 rows 5.4 -> 4.8 ms at 1.5B); at 2047 rows the 128-row tiles measured faster
        const bool half = !wide && stg == 3 && mt <= 8;
        if (t_ev_stop)
            snprintf(t_name, sizeof(t_name), "%svoid nv::k_gemm_bf16<%d, %d, %d, %d, %d, %d>(nv::GemmArgs)",
                     a.abf_ready ? "" : "nv::k_rows_bf16 + ", wide ? 128 : 64, a.head ? 1 : 0,
                     a.head ? (int)EPI_STORE : a.epi, stg, GB_NW, half ? 64 : GB_BM);
        if (wide) launch_gemm_bf16_bn<128, 2>(b, dim3(a.N / 128, mt), st);
        else if (stg == 3 && half) launch_gemm_bf16_bn<64, 3, GB_NW, 64>(b, dim3(a.N / 64, (a.R + 63) / 64), st);
        else if (stg == 3) launch_gemm_bf16_bn<64, 3>(b, dim3(a.N / 64, mt), st);
        else launch_gemm_bf16_bn<64, 2>(b, dim3(a.N / 64, mt), st);
        return hipGetLastError();
    }
    if (use_mfma(a)) {
        if (a.norm_w) {
            NV_LAUNCH(k_row_rms, dim3((a.R + 3) / 4), dim3(256), 0, st, a.A, a.lda, a.a_rows, a.R, a.K, a.eps,
                               a.rms_ws);
        }
        const unsigned mt = (unsigned)((a.R + MF_BM - 1) / MF_BM);
        if (t_ev_stop)
            snprintf(t_name, sizeof(t_name), "%svoid nv::k_gemm_mfma<%d, %d>(nv::GemmArgs)",
                     a.norm_w ? "nv::k_row_rms + " : "", a.R <= MF_BM ? 16 : 64, a.head ? 1 : 0);
        if (a.R <= MF_BM) {
            if (a.head)
                NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_mfma<16, 1>), dim3(a.N / 16, mt), dim3(256), 0, st, a);
            else
                NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_mfma<16, 0>), dim3(a.N / 16, mt), dim3(256), 0, st, a);
        } else {
            if (a.head)
                NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_mfma<64, 1>), dim3(a.N / 64, mt), dim3(256), 0, st, a);
            else
                NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_mfma<64, 0>), dim3(a.N / 64, mt), dim3(256), 0, st, a);
        }
        return hipGetLastError();
    }
    {
        const int epc = a.wbf16 ? 8 : 4;
        const int need = (a.K / epc + 63) / 64;
        const int ch = need <= 1 ? 1 : need <= 2 ? 2 : need <= 3 ? 3 : need <= 4 ? 4 : need <= 8 ? 8 : 0;
        const int cpw = a.N >= 4096 ? 4 : 2;
        const size_t shm = ((size_t)a.R * a.K + GV_RMAX) * sizeof(float);
        if (a.R <= GV_RMAX && ch > 0 && a.K % epc == 0 && a.N % (4 * cpw) == 0 && shm <= 160 * 1024) {
            const dim3 grid(a.N / (4 * cpw));
#define NV_GV(WB, CP, C, HD)                                                                                  \
    NV_LAUNCH(HIP_KERNEL_NAME(k_gemv<WB, CP, C, HD>), grid, dim3(256), shm, st, a)
#define NV_GV_CH(WB, CP, HD)                                                                                  \
    switch (ch) {                                                                                            \
        case 1: NV_GV(WB, CP, 1, HD); break;                                                                 \
        case 2: NV_GV(WB, CP, 2, HD); break;                                                                 \
        case 3: NV_GV(WB, CP, 3, HD); break;                                                                 \
        case 4: NV_GV(WB, CP, 4, HD); break;                                                                 \
        default: NV_GV(WB, CP, 8, HD); break;                                                                \
    }
            if (a.wbf16) {
                if (cpw == 4) { if (a.head) { NV_GV_CH(true, 4, 1) } else { NV_GV_CH(true, 4, 0) } }
                else { if (a.head) { NV_GV_CH(true, 2, 1) } else { NV_GV_CH(true, 2, 0) } }
            } else {
                if (cpw == 4) { if (a.head) { NV_GV_CH(false, 4, 1) } else { NV_GV_CH(false, 4, 0) } }
                else { if (a.head) { NV_GV_CH(false, 2, 1) } else { NV_GV_CH(false, 2, 0) } }
            }
#undef NV_GV_CH
#undef NV_GV
            return hipGetLastError();
        }
    }
    const int rt = gv_row_tile(a.K);
    const size_t shm = ((size_t)rt * a.K + GV_RT_MAX) * sizeof(float);
    if (t_ev_stop)
        snprintf(t_name, sizeof(t_name), "void nv::k_gemm_valu<%s, %d>(nv::GemmArgs)", a.wbf16 ? "true" : "false",
                 a.head ? 1 : 0);
    dim3 grid(a.N / GV_COLS);
    if (a.wbf16) {
        if (a.head)
            NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_valu<true, 1>), grid, dim3(256), shm, st, a);
        else
            NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_valu<true, 0>), grid, dim3(256), shm, st, a);
    } else {
        if (a.head)
            NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_valu<false, 1>), grid, dim3(256), shm, st, a);
        else
            NV_LAUNCH(HIP_KERNEL_NAME(k_gemm_valu<false, 0>), grid, dim3(256), shm, st, a);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Chunked causal attention, split over the key range (partials combined afterwards).
// Block = 4 waves; a 64-key tile of K and V is staged in LDS and shared by all rows of the
// item; wave w handles rows w, w+4, ...  Lane j scores key j of the tile; each row keeps a
// running max / sum / output (online softmax) in registers.
// ------------------------------------------------------------------------------------------

constexpr int AT_TILE_MAX = 64;
constexpr int AT_MAX_ROWS = 32;     // rows per item
// keys per LDS tile: 64 for head_dim <= 64, 32 for head_dim 128 (LDS stays under 64 KB)
__host__ __device__ inline int at_tile(int hd) { return hd > 64 ? 32 : 64; }
constexpr int AT_RPW = AT_MAX_ROWS / 4;

__global__ __launch_bounds__(256) void k_attn(const AttnItem* items, const RowInfo* rows, const float* q,
                                              const void* kv, int layer, LayerDims D, float* part_ml,
                                              float* part_o, float* out) {
    extern __shared__ float sm[];
    const AttnItem it = items[blockIdx.x];
    const int hd = D.hd;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int TILE = at_tile(hd);
    float* Ks = sm;                           // [TILE][hd + 1]
    float* Vs = Ks + TILE * (hd + 1);         // [TILE][hd]
    float* Qs = Vs + TILE * hd;               // [nrows][hd], pre-scaled by 1/sqrt(hd)
    const float scale = 1.0f / sqrtf((float)hd);
    for (int idx = threadIdx.x; idx < it.nrows * hd; idx += blockDim.x) {
        const int r = idx / hd, e = idx - r * hd;
        Qs[idx] = q[(int64_t)(it.row0 + r) * D.d + it.head * hd + e] * scale;
    }
    const int seq = it.seq;
    const int64_t kb = kv_base(D, seq, layer, 0, it.head);
    const int64_t vb = kv_base(D, seq, layer, 1, it.head);

    float m[AT_RPW], l[AT_RPW], o0[AT_RPW], o1[AT_RPW];
    int qp[AT_RPW];
#pragma unroll
    for (int i = 0; i < AT_RPW; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.f;
        o0[i] = o1[i] = 0.f;
        const int r = wave + 4 * i;
        qp[i] = r < it.nrows ? rows[it.row0 + r].pos : -1;
    }
    const int d0 = lane, d1 = lane + 64;

    for (int t0 = it.lo; t0 < it.hi; t0 += TILE) {
        const int tn = min(TILE, it.hi - t0);
        __syncthreads();
        for (int idx = threadIdx.x; idx < tn * hd; idx += blockDim.x) {
            const int j = idx / hd, e = idx - j * hd;
            Ks[j * (hd + 1) + e] = kv_load(kv, D.kv_bf16, kb + (int64_t)(t0 + j) * hd + e);
            Vs[j * hd + e] = kv_load(kv, D.kv_bf16, vb + (int64_t)(t0 + j) * hd + e);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < AT_RPW; ++i) {
            const int r = wave + 4 * i;
            if (r >= it.nrows || qp[i] < t0) continue;
            float s = -INFINITY;
            if (lane < tn && t0 + lane <= qp[i]) {
                const float* qr = Qs + r * hd;
                const float* kr = Ks + lane * (hd + 1);
                float acc = 0.f;
                for (int e = 0; e < hd; ++e) acc = fmaf(qr[e], kr[e], acc);
                s = acc;
            }
            const float mt = wave_max(s);
            const float mn = fmaxf(m[i], mt);
            const float p = (s == -INFINITY) ? 0.f : expf(s - mn);
            const float alpha = expf(m[i] - mn);
            l[i] = l[i] * alpha + wave_sum(p);
            float a0 = o0[i] * alpha, a1 = o1[i] * alpha;
            for (int j = 0; j < tn; ++j) {
                const float pj = __shfl(p, j, 64);
                if (d0 < hd) a0 = fmaf(pj, Vs[j * hd + d0], a0);
                if (d1 < hd) a1 = fmaf(pj, Vs[j * hd + d1], a1);
            }
            o0[i] = a0;
            o1[i] = a1;
            m[i] = mn;
        }
    }
#pragma unroll
    for (int i = 0; i < AT_RPW; ++i) {
        const int r = wave + 4 * i;
        if (r >= it.nrows) continue;
        if (it.nsplit == 1) {      // unsplit key range: finished here, the combine pass skips the row
            float* orow = out + (int64_t)(it.row0 + r) * D.d + it.head * hd;
            if (d0 < hd) orow[d0] = o0[i] / l[i];
            if (d1 < hd) orow[d1] = o1[i] / l[i];
            continue;
        }
        const int64_t slot = it.part + r;
        if (lane == 0) {
            part_ml[2 * slot] = m[i];
            part_ml[2 * slot + 1] = l[i];
        }
        if (d0 < hd) part_o[slot * hd + d0] = o0[i];
        if (d1 < hd) part_o[slot * hd + d1] = o1[i];
    }
}

// ------------------------------------------------------------------------------------------
// Chunked causal attention on the matrix cores (bf16 KV cache), for launch groups of many
// rows.  An item is up to 16 NWA consecutive rows of one sequence, one head and one key
// range; wave w takes rows 16w..16w+15.  Per 64-key tile (K and V double-buffered in LDS,
// both with keys as rows) the wave forms the transposed scores S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16: lane l then holds the scores of query l%16 for keys
// 16t + 4(l/16) + i (t = 0..3, i = 0..3).  That is, with keys permuted inside each
// 32-key step, the B operand of O^T = V^T P^T, so the probabilities go from the
// accumulators to the second product without leaving the registers; the V^T operand is
// read from the row-major V tile by transposing LDS reads, with the same key permutation.  Every value a lane holds belongs to its one query, so the online
// softmax rescales a lane's accumulators by one factor; the row max crosses the four lane
// groups of a query once per tile, the row sum only at the end.
// Outputs: the normalised row (single split) or the (max, sum, unnormalised output)
// partials that k_attn_combine merges, as k_attn writes them.
// ------------------------------------------------------------------------------------------

constexpr int AM_KT = 64;     // keys per tile

// V operand reads: ds_read_b64_tr_b16 treats each group of 16 lanes as a 16 x 4 block of
// 16-bit values (lane j's 8 bytes are row j) and returns to lane i the values
// (row 4e + i/4, column i%4), e = 0..3.  With lane j of group g pointing at key row
// 4g + j/4 and dims 4(j%4) .. +3 of a row-major V tile, lane i receives dim i of four
// consecutive keys: exactly its slice of the transposed operand.  So V is staged like K
// (coalesced 16-byte loads, one 16-byte LDS store per chunk) and transposed by the read.
typedef short nv_s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) nv_s16x4_t*)(p)));
}

template <int HD, int NWA>
__global__ __launch_bounds__(64 * NWA) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_attn_mfma(
    const AttnItem* items, const RowInfo* rows, const float* q, const uint16_t* kv, int layer, LayerDims D,
    float* part_ml, float* part_o, float* out, unsigned long long* stamp, DecGeom dg) {
    const unsigned long long t_begin = stamp_begin(stamp);
    constexpr int KLD = HD + 8;         // K tile row stride (bf16)
    constexpr int VLD = HD + 16;        // V tile row stride (bf16): rows an odd multiple of 8
                                        // banks apart, so the transposing reads are conflict-free
    constexpr int NKS = HD / 32;        // k-steps of the score product
    constexpr int NHT = HD / 16;        // 16-wide output tiles
    constexpr int CPR = HD / 8;         // 16-byte chunks per key row
    constexpr int NTH = 64 * NWA;
    constexpr int NCH = AM_KT * CPR;              // 16-byte chunks per tile, for K and for V
    constexpr int CPT = (NCH + NTH - 1) / NTH;    // per thread (threads past NCH load none)
    // one wave per block (decode items of one or two tiles): a single buffer, so that four
    // blocks share a CU; otherwise the next tile is staged while the current one is used
    constexpr int NB = NWA == 1 ? 1 : 2;
    __shared__ __align__(16) uint16_t Ks[NB][AM_KT * KLD];
    __shared__ __align__(16) uint16_t Vs[NB][AM_KT * VLD];
    const AttnItem it = dg.on ? dec_item(dg, blockIdx.x) : items[blockIdx.x];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qn = lane & 15, g = lane >> 4;
    const int r = wave * 16 + qn;                  // this lane's query row within the item
    const bool rv = r < it.nrows;
    const int qpos = !rv ? -1 : dg.on ? dg.pos0 + r : rows[it.row0 + r].pos;
    const int seq = it.seq;
    const uint16_t* Kg = kv + kv_base(D, seq, layer, 0, it.head);
    const uint16_t* Vg = kv + kv_base(D, seq, layer, 1, it.head);

    // queries (B operand of the score product), pre-scaled by log2(e)/sqrt(hd): the scores
    // come out in base-2 units, so each probability is one exp2 (the running max is
    // converted back to natural-log units where split partials are written)
    bf16x8_t qf[NKS];
    {
        const float scale = 1.4426950408889634f / sqrtf((float)HD);
        const float* qr = q + (int64_t)(it.row0 + (rv ? r : 0)) * D.d + it.head * HD;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            uint32_t p[4] = {0u, 0u, 0u, 0u};
            if (rv) {
                const float4 a = *(const float4*)(qr + 32 * ks + 8 * g);
                const float4 b = *(const float4*)(qr + 32 * ks + 8 * g + 4);
                p[0] = pack_bf2(a.x * scale, a.y * scale);
                p[1] = pack_bf2(a.z * scale, a.w * scale);
                p[2] = pack_bf2(b.x * scale, b.y * scale);
                p[3] = pack_bf2(b.z * scale, b.w * scale);
            }
            qf[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(p[0], p[1], p[2], p[3]));
        }
    }

    u32x4 kr[CPT], vr[CPT];
    auto gload = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + NTH * j;
            if (NCH % NTH != 0 && c >= NCH) break;
            const int key = min(t0 + c / CPR, it.hi - 1);   // rows past the range are masked
            const int col = (c % CPR) * 8;
            kr[j] = *(const u32x4*)(Kg + (int64_t)key * HD + col);
            vr[j] = *(const u32x4*)(Vg + (int64_t)key * HD + col);
        }
    };
    auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + NTH * j;
            if (NCH % NTH != 0 && c >= NCH) break;
            const int key = c / CPR, col = (c % CPR) * 8;
            *(u32x4*)&Ks[buf][key * KLD + col] = kr[j];
            *(u32x4*)&Vs[buf][key * VLD + col] = vr[j];
        }
    };

    f32x4_t o[NHT];
#pragma unroll
    for (int t = 0; t < NHT; ++t) o[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;
    // the wave's lowest query position (rows past nrows excluded): key tiles wholly at or
    // below it, and inside the item's range, need no mask
    int qmin = rv ? qpos : INT_MAX;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) qmin = min(qmin, __shfl_xor(qmin, off, 64));

    const int ntile = (it.hi - it.lo + AM_KT - 1) / AM_KT;
    gload(it.lo);
    lstore(0);
    __syncthreads();
    for (int tt = 0; tt < ntile; ++tt) {
        const int buf = NB == 1 ? 0 : tt & 1, t0 = it.lo + tt * AM_KT;
        if (tt + 1 < ntile) gload(t0 + AM_KT);
        // S^T for this tile: 4 key tiles of 16
        f32x4_t sc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            sc[mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const uint4 a = *(const uint4*)&Ks[buf][(16 * mt + qn) * KLD + 32 * ks + 8 * g];
                sc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qf[ks], sc[mt],
                                                                 0, 0, 0);
            }
        }
        // mask (causal and the item's key range; only on tiles that cross either bound) and
        // the running max of this lane's query
        const bool full = t0 + AM_KT <= it.hi && t0 + AM_KT - 1 <= qmin;   // wave-uniform
        float tmax = -INFINITY;
        if (full) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[mt][i]);
        } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = t0 + 16 * mt + 4 * g + i;
                    const bool ok = key < it.hi && key <= qpos;
                    sc[mt][i] = ok ? sc[mt][i] : -INFINITY;
                    tmax = fmaxf(tmax, sc[mt][i]);
                }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(m, tmax);
        const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
        float ps = 0.f;
        if (full) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(sc[mt][i] - mn);
                    sc[mt][i] = pv;
                    ps += pv;
                }
        } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = (sc[mt][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[mt][i] - mn);
                    sc[mt][i] = pv;
                    ps += pv;
                }
        }
        lsum = lsum * alpha + ps;
        m = mn;
#pragma unroll
        for (int t = 0; t < NHT; ++t) o[t] *= alpha;
        // O^T += V^T P^T over the tile's two 32-key steps
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 pb = make_uint4(pack_bf2(sc[2 * ks][0], sc[2 * ks][1]), pack_bf2(sc[2 * ks][2], sc[2 * ks][3]),
                                        pack_bf2(sc[2 * ks + 1][0], sc[2 * ks + 1][1]),
                                        pack_bf2(sc[2 * ks + 1][2], sc[2 * ks + 1][3]));
            const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pb);
            const uint16_t* vb = &Vs[buf][(32 * ks + 4 * g + (qn >> 2)) * VLD + 4 * (qn & 3)];
#pragma unroll
            for (int t = 0; t < NHT; ++t) {
                const uint2 lo = lds_read_tr16(vb + 16 * t);              // keys 32ks + 4g + 0..3
                const uint2 hi = lds_read_tr16(vb + 16 * VLD + 16 * t);   // keys 32ks + 16 + 4g + 0..3
                const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
                o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va), pf, o[t], 0, 0, 0);
            }
        }
        if (tt + 1 < ntile) {
            if constexpr (NB == 1) __syncthreads();   // the tile's reads are done before it is overwritten
            lstore(NB == 1 ? 0 : buf ^ 1);
        }
        __syncthreads();
    }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (rv && it.nsplit == 1) {
        const float inv = 1.0f / lsum;
        float* orow = out + (int64_t)(it.row0 + r) * D.d + it.head * HD;
#pragma unroll
        for (int t = 0; t < NHT; ++t)
            *(float4*)(orow + 16 * t + 4 * g) = make_float4(o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
    } else if (rv) {
        const int64_t slot = it.part + r;
        if (g == 0) {
            part_ml[2 * slot] = m * 0.6931471805599453f;   // back to natural-log units
            part_ml[2 * slot + 1] = lsum;
        }
        float* po = part_o + slot * HD;
#pragma unroll
        for (int t = 0; t < NHT; ++t) *(float4*)(po + 16 * t + 4 * g) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
    }
    stamp_end_lin(stamp, t_begin, STAMP_BLOCKS);
}

bool attn_mfma_ok(const LayerDims& D) { return D.kv_bf16 && (D.hd == 32 || D.hd == 64 || D.hd == 128); }

hipError_t launch_attn_mfma(const AttnItem* items, int n_items, const RowInfo* rows, const float* q, const void* kv,
                            int layer, const LayerDims& D, float* part_ml, float* part_o, float* out, hipStream_t st) {
    if (n_items <= 0) return hipSuccess;
    if (!attn_mfma_ok(D)) return hipErrorInvalidValue;
    constexpr int NWA = ATTN_MFMA_ROWS / 16;
    static_assert(NWA * 16 == ATTN_MFMA_ROWS && (NWA == 4 || NWA == 8), "64 or 128 rows per item");
    const uint16_t* k16 = (const uint16_t*)kv;
    const dim3 blk(64 * NWA);
    if (D.hd == 128)
        NV_LAUNCH(HIP_KERNEL_NAME(k_attn_mfma<128, NWA>), dim3(n_items), blk, 0, st, items, rows, q, k16, layer, D,
                  part_ml, part_o, out, t_stamp, DecGeom{});
    else if (D.hd == 64)
        NV_LAUNCH(HIP_KERNEL_NAME(k_attn_mfma<64, NWA>), dim3(n_items), blk, 0, st, items, rows, q, k16, layer, D,
                  part_ml, part_o, out, t_stamp, DecGeom{});
    else
        NV_LAUNCH(HIP_KERNEL_NAME(k_attn_mfma<32, NWA>), dim3(n_items), blk, 0, st, items, rows, q, k16, layer, D,
                  part_ml, part_o, out, t_stamp, DecGeom{});
    return hipGetLastError();
}

// The same kernel with one wave per block, for decode groups (items of up to 16 rows: the
// decode row blocks, with their key splits).  Its cost barely grows with the rows an item
// holds, where the vector-ALU decode kernel repeats its dot products per row.
hipError_t launch_attn_mfma16(const AttnItem* items, int n_items, const RowInfo* rows, const float* q,
                              const void* kv, int layer, const LayerDims& D, float* part_ml, float* part_o,
                              float* out, hipStream_t st, const DecGeom& dg) {
    if (n_items <= 0) return hipSuccess;
    if (!attn_mfma_ok(D)) return hipErrorInvalidValue;
    if (dg.on && (dg.nrows < 1 || dg.nrows > 16 || n_items != D.H * dg.nsplit)) return hipErrorInvalidValue;
    const uint16_t* k16 = (const uint16_t*)kv;
    if (t_ev_stop) snprintf(t_name, sizeof(t_name), "nv::k_attn_mfma<%d, 1>", D.hd);
    if (D.hd == 128)
        NV_LAUNCH(HIP_KERNEL_NAME(k_attn_mfma<128, 1>), dim3(n_items), dim3(64), 0, st, items, rows, q, k16, layer, D,
                  part_ml, part_o, out, t_stamp, dg);
    else if (D.hd == 64)
        NV_LAUNCH(HIP_KERNEL_NAME(k_attn_mfma<64, 1>), dim3(n_items), dim3(64), 0, st, items, rows, q, k16, layer, D,
                  part_ml, part_o, out, t_stamp, dg);
    else
        NV_LAUNCH(HIP_KERNEL_NAME(k_attn_mfma<32, 1>), dim3(n_items), dim3(64), 0, st, items, rows, q, k16, layer, D,
                  part_ml, part_o, out, t_stamp, dg);
    return hipGetLastError();
}

// Decode-sized groups (few (row, head) pairs, possibly many splits): one block of 512
// threads per pair.  The split maxima and the weights exp(m_s - M) are formed by all
// threads together (block reductions, weights kept in LDS); each value dim's weighted sum
// is then spread over 512 / hd thread subsets that take every (512 / hd)-th split, and the
// subsets are added in LDS.  The first splits' (max, sum) pairs and partial outputs are
// loaded before the reductions (indexes clamped to the last split, never summed), so the
// block waits on memory once for them.
constexpr int COMB_MAX = 4096;   // splits of one (row, head) whose weights LDS holds
constexpr int COMB_WAVE_MIN_PAIRS = 2048;   // (row, head) pairs from which one wave per pair is used
constexpr int COMB_PRE = 8;      // partial outputs per thread loaded ahead of the reductions

__global__ __launch_bounds__(512) void k_attn_combine_blk(const CombineInfo* ci, int R, LayerDims D,
                                                          const float* part_ml, const float* part_o, float* out,
                                                          unsigned long long* stamp, DecGeom dg) {
    const unsigned long long t_begin = stamp_begin(stamp);
    __shared__ float wsh[COMB_MAX];
    __shared__ float red[512];
    __shared__ float wred[8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = blockIdx.x / D.H, h = blockIdx.x - i * D.H;
    const CombineInfo c = dg.on ? dec_comb(dg, i) : ci[i];
    if (c.nsplit > 1) {
        const int ns = c.nsplit, hd = D.hd;
        const int64_t base = c.base + (int64_t)h * ns * c.nrows + c.off;   // split s adds s * nrows
        const int Q = 512 / hd, e = tid % hd, q = tid / hd;
        float pre[COMB_PRE];
#pragma unroll
        for (int j = 0; j < COMB_PRE; ++j)
            pre[j] = part_o[(base + (int64_t)min(q + j * Q, ns - 1) * c.nrows) * hd + e];
        const float2 ml0 = *(const float2*)(part_ml + 2 * (base + (int64_t)min(tid, ns - 1) * c.nrows));
        float mx = tid < ns ? ml0.x : -INFINITY;
        for (int sp = tid + 512; sp < ns; sp += 512) mx = fmaxf(mx, part_ml[2 * (base + (int64_t)sp * c.nrows)]);
        mx = wave_max(mx);
        if (lane == 0) wred[wave] = mx;
        __syncthreads();
        float M = wred[0];
#pragma unroll
        for (int w = 1; w < 8; ++w) M = fmaxf(M, wred[w]);
        __syncthreads();
        float ls = 0.f;
        if (tid < ns) {
            const float w = ml0.x == -INFINITY ? 0.f : expf(ml0.x - M);
            wsh[tid] = w;
            ls += w * ml0.y;
        }
        for (int sp = tid + 512; sp < ns; sp += 512) {
            const float2 ml = *(const float2*)(part_ml + 2 * (base + (int64_t)sp * c.nrows));
            const float w = ml.x == -INFINITY ? 0.f : expf(ml.x - M);
            wsh[sp] = w;
            ls += w * ml.y;
        }
        ls = wave_sum(ls);
        if (lane == 0) wred[wave] = ls;
        __syncthreads();
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) L += wred[w];
        float o = 0.f;
#pragma unroll
        for (int j = 0; j < COMB_PRE; ++j)
            if (q + j * Q < ns) o += wsh[q + j * Q] * pre[j];
#pragma unroll 4
        for (int sp = q + COMB_PRE * Q; sp < ns; sp += Q) o += wsh[sp] * part_o[(base + (int64_t)sp * c.nrows) * hd + e];
        red[tid] = o;
        __syncthreads();
        if (tid < hd) {
            float v = 0.f;
            for (int qq = 0; qq < Q; ++qq) v += red[qq * hd + tid];
            out[(int64_t)i * D.d + h * hd + tid] = v / L;
        }
    }
    stamp_end(stamp, t_begin);
}

// The softmax merge of one (row, head)'s split partials for this lane's two output dims
// e, e+1: the max M of the splits' maxima first, then the weights exp(max - M) applied to
// the sums and partial outputs, in split order.  Up to NS splits: every (max, sum) pair
// and partial output is loaded before any is used (indexes clamped to the last split,
// which the folds stop before), so the wave waits on memory once, not once per split.
template <int NS>
__device__ __forceinline__ float2 merge_splits_n(const float* part_ml, const float* part_o, int64_t base, int ns,
                                                 int nrows, int hd, int e) {
    float2 ml[NS], v[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int64_t slot = base + (int64_t)min(j, ns - 1) * nrows;
        ml[j] = *(const float2*)(part_ml + 2 * slot);
        v[j] = *(const float2*)(part_o + slot * hd + e);
    }
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < NS; ++j)
        if (j < ns) M = fmaxf(M, ml[j].x);
    float L = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j)
        if (j < ns) {
            const float w = ml[j].x == -INFINITY ? 0.f : expf(ml[j].x - M);
            L += w * ml[j].y;
            a0 += w * v[j].x;
            a1 += w * v[j].y;
        }
    return make_float2(a0 / L, a1 / L);
}

// The same merge for any number of splits, one split at a time.
__device__ __forceinline__ float2 merge_splits_any(const float* part_ml, const float* part_o, int64_t base, int ns,
                                                   int nrows, int hd, int e) {
    float M = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, part_ml[2 * (base + (int64_t)sp * nrows)]);
    float L = 0.f, a0 = 0.f, a1 = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
        const int64_t slot = base + (int64_t)sp * nrows;
        const float2 ml = *(const float2*)(part_ml + 2 * slot);
        const float w = ml.x == -INFINITY ? 0.f : expf(ml.x - M);
        L += w * ml.y;
        const float2 v = *(const float2*)(part_o + slot * hd + e);
        a0 += w * v.x;
        a1 += w * v.y;
    }
    return make_float2(a0 / L, a1 / L);
}

// Dispatch on the split count (uniform across the wave: one wave per (row, head)).
__device__ __forceinline__ float2 merge_splits(const float* part_ml, const float* part_o, int64_t base, int ns,
                                               int nrows, int hd, int e) {
    if (ns <= 2) return merge_splits_n<2>(part_ml, part_o, base, ns, nrows, hd, e);
    if (ns <= 4) return merge_splits_n<4>(part_ml, part_o, base, ns, nrows, hd, e);
    if (ns <= 8) return merge_splits_n<8>(part_ml, part_o, base, ns, nrows, hd, e);
    return merge_splits_any(part_ml, part_o, base, ns, nrows, hd, e);
}

// Merge the split partials of one (row, head), one wave each (four per block), each lane
// forming two output dims.  Rows whose key range was not split were written by the
// attention kernel and are skipped.
__global__ __launch_bounds__(256) void k_attn_combine(const CombineInfo* ci, int R, LayerDims D, const float* part_ml,
                                                      const float* part_o, float* out, unsigned long long* stamp) {
    const unsigned long long t_begin = stamp_begin(stamp);
    const int lane = threadIdx.x & 63;
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p < R * D.H) {
        const int i = p / D.H, h = p - i * D.H;
        const CombineInfo c = ci[i];
        const int e = 2 * lane;
        if (c.nsplit > 1 && e < D.hd) {
            const int64_t base = c.base + (int64_t)h * c.nsplit * c.nrows + c.off;   // split s adds s * nrows
            *(float2*)(out + (int64_t)i * D.d + h * D.hd + e) =
                merge_splits(part_ml, part_o, base, c.nsplit, c.nrows, D.hd, e);
        }
    }
    stamp_end(stamp, t_begin);
}

// As k_attn_combine, but every (row, head) is written as bf16 into the O product's rows
// (out_bf16 [R][d], rounded as k_rows_bf16 rounds): merged partials for split rows, the
// attention kernel's normalised fp32 output for the others.  The O product then needs no
// row pass of its own.
__global__ __launch_bounds__(256) void k_attn_combine_bf16(const CombineInfo* ci, int R, LayerDims D,
                                                           const float* part_ml, const float* part_o,
                                                           const float* attn_o, uint16_t* out_bf16) {
    const int lane = threadIdx.x & 63;
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= R * D.H) return;
    const int i = p / D.H, h = p - i * D.H;
    const CombineInfo c = ci[i];
    const int hd = D.hd, e = 2 * lane;
    if (e >= hd) return;
    const int64_t o = (int64_t)i * D.d + h * hd + e;
    float2 v;
    if (c.nsplit > 1) {
        const int64_t base = c.base + (int64_t)h * c.nsplit * c.nrows + c.off;   // split s adds s * nrows
        v = merge_splits(part_ml, part_o, base, c.nsplit, c.nrows, hd, e);
    } else {
        v = *(const float2*)(attn_o + o);
    }
    *(uint32_t*)(out_bf16 + o) = pack_bf2(v.x, v.y);
}

hipError_t launch_attn_combine_bf16(const CombineInfo* ci, int R, const LayerDims& D, const float* part_ml,
                                    const float* part_o, const float* attn_o, uint16_t* out_bf16, hipStream_t st) {
    if (R <= 0) return hipSuccess;
    if (D.hd % 2 || D.hd > 128) return hipErrorInvalidValue;
    NV_LAUNCH(k_attn_combine_bf16, dim3((R * D.H + 3) / 4), dim3(256), 0, st, ci, R, D, part_ml, part_o, attn_o,
              out_bf16);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnItem* items, int n_items, const RowInfo* rows, const float* q, const void* kv,
                       int layer, const LayerDims& D, float* part_ml, float* part_o, float* out, hipStream_t st) {
    if (n_items <= 0) return hipSuccess;
    const int tile = at_tile(D.hd);
    const size_t shm = ((size_t)tile * (D.hd + 1) + (size_t)tile * D.hd + (size_t)AT_MAX_ROWS * D.hd) * sizeof(float);
    NV_LAUNCH(k_attn, dim3(n_items), dim3(256), shm, st, items, rows, q, kv, layer, D, part_ml, part_o, out);
    return hipGetLastError();
}

hipError_t launch_attn_combine(const CombineInfo* ci, int R, const LayerDims& D, const float* part_ml,
                               const float* part_o, float* out, hipStream_t st, const DecGeom& dg) {
    if (R <= 0) return hipSuccess;
    if (dg.on && dg.nrows != R) return hipErrorInvalidValue;
    if (R * D.H >= COMB_WAVE_MIN_PAIRS && !dg.on) {
        if (t_ev_stop) snprintf(t_name, sizeof(t_name), "nv::k_attn_combine");
        NV_LAUNCH(k_attn_combine, dim3((R * D.H + 3) / 4), dim3(256), 0, st, ci, R, D, part_ml, part_o, out, t_stamp);
    } else {
        if (t_ev_stop) snprintf(t_name, sizeof(t_name), "nv::k_attn_combine_blk");
        NV_LAUNCH(k_attn_combine_blk, dim3(R * D.H), dim3(512), 0, st, ci, R, D, part_ml, part_o, out, t_stamp, dg);
    }
    return hipGetLastError();
}


// ------------------------------------------------------------------------------------------
// Decode attention: up to ATTN_DEC_ROWS consecutive positions of one sequence against the
// keys [lo, hi) of one head (one split of that row block's key range).  A key is read by
// hd/8 lanes, 16 bytes (8 dims) each, so one wave instruction covers 64/(hd/8) keys with
// fully used 16-byte loads of the K and V rows.  Each lane slot keeps an online-softmax
// state (max, sum, 8 output dims) per row over the keys it saw; slots, then the block's
// four waves, are merged.  With one split the output is written directly; otherwise the
// split's partial state is written and a separate combine pass (k_attn_combine) merges
// the splits: the kernel boundary makes the partials visible without a device-scope
// fence, which costs more than the whole kernel on this part.
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ void sm_merge(float& m, float& l, float* o, float m2, float l2, const float* o2, int n) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float a1 = expf(m - M), a2 = expf(m2 - M);
    l = a1 * l + a2 * l2;
    for (int e = 0; e < n; ++e) o[e] = a1 * o[e] + a2 * o2[e];
    m = M;
}

template <int HD, bool KVBF, int RM, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn_dec(const AttnItem* items, const RowInfo* rows, const float* q,
                                                      const void* kv, int layer, LayerDims D, float* part_ml,
                                                      float* part_o, float* out, unsigned long long* stamp,
                                                      DecGeom dg) {
    const unsigned long long t_begin = stamp_begin(stamp);
    constexpr int DPL = 8;
    constexpr int LPK = HD / DPL;       // lanes per key
    constexpr int KPI = 64 / LPK;       // keys per wave instruction
    // key groups per wave: a split holds at most NW * KPI * NIT keys
    constexpr int NIT = NW == ATTN_DEC_WIDE_WAVES ? ATTN_DEC_WIDE_ITERS : ATTN_DEC_ITERS;
    __shared__ float red[NW][RM][HD + 2];
    const AttnItem it = dg.on ? dec_item(dg, blockIdx.x) : items[blockIdx.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPK, dl = lane - g * LPK;
    const int nr = it.nrows;
    const int seq = it.seq;
    const int64_t kb = kv_base(D, seq, layer, 0, it.head) + dl * DPL;
    const int64_t vb = kv_base(D, seq, layer, 1, it.head) + dl * DPL;

    // the raw query first, then every key/value group of this wave; the query is scaled
    // only after the key loads are issued (scaling it earlier would make them wait for it),
    // so the first key groups can be used while later ones are still arriving
    // (unconditional: rows past nr read the last row and are masked when scaled)
    float4 qa[RM][2];
    int qpos[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        const int rr = it.row0 + min(r, nr - 1);
        const float* qp = q + (int64_t)rr * D.d + it.head * HD + dl * DPL;
        qa[r][0] = *(const float4*)qp;
        qa[r][1] = *(const float4*)(qp + 4);
        qpos[r] = dg.on ? dg.pos0 + rr : rows[rr].pos;
    }

    uint4 kr[NIT], vr[NIT];
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        // keys past the range load the last key (masked below): every load is unconditional,
        // so all are issued back to back and waited for in order
        const int key = min(it.lo + (i * NW + wave) * KPI + g, it.hi - 1);
        if constexpr (KVBF) {
            // read once per step: the cache of all layers outgrows the caches (D 0.979 ->
            // 0.971 ms per step with the hint, same-box A/B)
            kr[i] = stream_load16((const uint16_t*)kv + kb + (int64_t)key * HD);
            vr[i] = stream_load16((const uint16_t*)kv + vb + (int64_t)key * HD);
        } else {
            kr[i] = *(const uint4*)((const float*)kv + kb + (int64_t)key * HD);
            vr[i] = *(const uint4*)((const float*)kv + vb + (int64_t)key * HD);
        }
    }
    uint4 kr2[KVBF ? 1 : NIT], vr2[KVBF ? 1 : NIT];   // fp32 keys need a second 16-byte load
    if constexpr (!KVBF) {
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const int key = min(it.lo + (i * NW + wave) * KPI + g, it.hi - 1);
            kr2[i] = *(const uint4*)((const float*)kv + kb + (int64_t)key * HD + 4);
            vr2[i] = *(const uint4*)((const float*)kv + vb + (int64_t)key * HD + 4);
        }
    }

    __builtin_amdgcn_sched_barrier(0);
    const float scale = 1.0f / sqrtf((float)HD);
    float qv[RM][DPL];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        const float sr = r < nr ? scale : 0.f;
        qv[r][0] = qa[r][0].x * sr; qv[r][1] = qa[r][0].y * sr; qv[r][2] = qa[r][0].z * sr;
        qv[r][3] = qa[r][0].w * sr; qv[r][4] = qa[r][1].x * sr; qv[r][5] = qa[r][1].y * sr;
        qv[r][6] = qa[r][1].z * sr; qv[r][7] = qa[r][1].w * sr;
        if (r >= nr) qpos[r] = -1;
    }

    float m[RM], l[RM], o[RM][DPL];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[r][e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        const int key = it.lo + (i * NW + wave) * KPI + g;
        if (it.lo + (i * NW + wave) * KPI >= it.hi) break;     // wave-uniform
        const bool kin = key < it.hi;
        float kf[DPL], vf[DPL];
        if constexpr (KVBF) {
            const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
            const uint32_t vw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = bf_lo(kw[e]); kf[2 * e + 1] = bf_hi(kw[e]);
                vf[2 * e] = bf_lo(vw[e]); vf[2 * e + 1] = bf_hi(vw[e]);
            }
        } else {
            kf[0] = __uint_as_float(kr[i].x); kf[1] = __uint_as_float(kr[i].y);
            kf[2] = __uint_as_float(kr[i].z); kf[3] = __uint_as_float(kr[i].w);
            kf[4] = __uint_as_float(kr2[i].x); kf[5] = __uint_as_float(kr2[i].y);
            kf[6] = __uint_as_float(kr2[i].z); kf[7] = __uint_as_float(kr2[i].w);
            vf[0] = __uint_as_float(vr[i].x); vf[1] = __uint_as_float(vr[i].y);
            vf[2] = __uint_as_float(vr[i].z); vf[3] = __uint_as_float(vr[i].w);
            vf[4] = __uint_as_float(vr2[i].x); vf[5] = __uint_as_float(vr2[i].y);
            vf[6] = __uint_as_float(vr2[i].z); vf[7] = __uint_as_float(vr2[i].w);
        }
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            if (r < nr) {
                float sc = 0.f;
#pragma unroll
                for (int e = 0; e < DPL; ++e) sc = fmaf(qv[r][e], kf[e], sc);
                sc = group_sum<LPK>(sc);
                if (kin && key <= qpos[r]) {
                    const float mn = fmaxf(m[r], sc);
                    const float alpha = expf(m[r] - mn);
                    const float p = expf(sc - mn);
                    l[r] = l[r] * alpha + p;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) o[r][e] = fmaf(p, vf[e], o[r][e] * alpha);
                    m[r] = mn;
                }
            }
        }
    }
    // merge the key slots of the wave
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        if (r < nr) {
#pragma unroll
            for (int off = LPK; off < 64; off <<= 1) {
                float o2[DPL];
                const float m2 = __shfl_xor(m[r], off, 64), l2 = __shfl_xor(l[r], off, 64);
#pragma unroll
                for (int e = 0; e < DPL; ++e) o2[e] = __shfl_xor(o[r][e], off, 64);
                sm_merge(m[r], l[r], o[r], m2, l2, o2, DPL);
            }
            if (g == 0) {
                if (dl == 0) {
                    red[wave][r][0] = m[r];
                    red[wave][r][1] = l[r];
                }
#pragma unroll
                for (int e = 0; e < DPL; ++e) red[wave][r][2 + dl * DPL + e] = o[r][e];
            }
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nr * HD; idx += blockDim.x) {
        const int r = idx / HD, e = idx - r * HD;
        float M = -INFINITY;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, red[w][r][0]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
            for (int w = 0; w < NW; ++w) {
                const float a = expf(red[w][r][0] - M);
                L += a * red[w][r][1];
                O += a * red[w][r][2 + e];
            }
        }
        if (it.nsplit == 1) {
            out[(int64_t)(it.row0 + r) * D.d + it.head * HD + e] = O / L;
        } else {
            const int64_t slot = it.part + r;
            part_o[slot * HD + e] = O;
            if (e == 0) {
                part_ml[2 * slot] = M;
                part_ml[2 * slot + 1] = L;
            }
        }
    }
    stamp_end(stamp, t_begin);
}


hipError_t launch_attn_dec(const AttnItem* items, int n_items, int max_rows, const RowInfo* rows, const float* q,
                           const void* kv, int layer, const LayerDims& D, float* part_ml, float* part_o, float* out,
                           hipStream_t st, const DecGeom& dg, int wide) {
    if (n_items <= 0) return hipSuccess;
    if (dg.on && (dg.nrows < 1 || dg.nrows > ATTN_DEC_ROWS || dg.nrows > max_rows || n_items != D.H * dg.nsplit))
        return hipErrorInvalidValue;
    if (wide && (!D.kv_bf16 || max_rows > ATTN_DEC_WIDE_ROWS)) return hipErrorInvalidValue;
#define NV_DEC(HDV, BF, RMV, NWV)                                                                             \
    do {                                                                                                      \
        NV_LAUNCH(HIP_KERNEL_NAME(k_attn_dec<HDV, BF, RMV, NWV>), dim3(n_items), dim3(64 * NWV), 0, st, items, \
                  rows, q, kv, layer, D, part_ml, part_o, out, t_stamp, dg);                                  \
        if (t_ev_stop) snprintf(t_name, sizeof(t_name), "nv::k_attn_dec<%d, %s, %d, %d>", HDV,               \
                                BF ? "true" : "false", RMV, NWV);                                             \
    } while (0)
#define NV_DEC_R(HDV, BF)                                                                                     \
    do {                                                                                                     \
        if (max_rows <= 1) NV_DEC(HDV, BF, 1, 4);                                                            \
        else if (max_rows <= 2) NV_DEC(HDV, BF, 2, 4);                                                       \
        else if (max_rows <= 4) NV_DEC(HDV, BF, 4, 4);                                                       \
        else NV_DEC(HDV, BF, 8, 4);                                                                          \
    } while (0)
    if (wide) {
        if (D.hd == 128) {
            if (max_rows <= 1) NV_DEC(128, true, 1, ATTN_DEC_WIDE_WAVES); else NV_DEC(128, true, 2, ATTN_DEC_WIDE_WAVES);
        } else if (D.hd == 64) {
            if (max_rows <= 1) NV_DEC(64, true, 1, ATTN_DEC_WIDE_WAVES); else NV_DEC(64, true, 2, ATTN_DEC_WIDE_WAVES);
        } else {
            if (max_rows <= 1) NV_DEC(32, true, 1, ATTN_DEC_WIDE_WAVES); else NV_DEC(32, true, 2, ATTN_DEC_WIDE_WAVES);
        }
        return hipGetLastError();
    }
    if (D.hd == 128) {
        if (D.kv_bf16) NV_DEC_R(128, true); else NV_DEC_R(128, false);
    } else if (D.hd == 64) {
        if (D.kv_bf16) NV_DEC_R(64, true); else NV_DEC_R(64, false);
    } else {
        if (D.kv_bf16) NV_DEC_R(32, true); else NV_DEC_R(32, false);
    }
#undef NV_DEC_R
#undef NV_DEC
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Router gate at the end of a segment: w = sigmoid(g . h + b) in float64, stop iff u < w.
// ------------------------------------------------------------------------------------------

// The stop decision also goes to mapped host memory when host_flags is set: a plain
// vector store at system scope (fine-grained memory; nothing else needs ordering with it).
__device__ __forceinline__ void publish_stop(int* host_flags, int seq, int tag, int stop) {
    if (host_flags) __hip_atomic_store(host_flags + seq, tag * 2 + stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__global__ __launch_bounds__(256) void k_gate(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d,
                                              const float* gw, float bias, const float* uniforms, int ucol,
                                              double* w_out, int* stop_out, int* host_flags, int tag) {
    __shared__ double wsum[4];
    const int i = blockIdx.x;
    if (i >= n) return;
    const float* h = Hs + (int64_t)rows[i].hrow * d;
    double acc = 0.0;
    for (int k = threadIdx.x; k < d; k += blockDim.x) acc += (double)gw[k] * (double)h[k];
    // in-wave butterfly, then the four waves in a fixed order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double z = ((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) + (double)bias;
        double w;
        if (z >= 0.0) {
            w = 1.0 / (1.0 + exp(-z));
        } else {
            const double ez = exp(z);
            w = ez / (1.0 + ez);
        }
        const int seq = seqs[i];
        w_out[seq * 4 + ucol] = w;
        if (uniforms) {
            const int stop = ((double)uniforms[seq * 4 + ucol] < w) ? 1 : 0;
            stop_out[seq] = stop;
            publish_stop(host_flags, seq, tag, stop);
        }
    }
}

hipError_t launch_gate(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d, const float* gw, float bias,
                       const float* uniforms, int ucol, double* w_out, int* stop_out, hipStream_t st, int* host_flags,
                       int tag) {
    if (n <= 0) return hipSuccess;
    NV_LAUNCH(k_gate, dim3(n), dim3(256), 0, st, rows, seqs, n, Hs, d, gw, bias, uniforms, ucol, w_out,
                       stop_out, host_flags, tag);
    return hipGetLastError();
}

// Router MLP gate in two passes, all in float64.
//  k_router_hidden: one wave per (row, hidden unit j): hid[row][j] = silu(W1[j] . h + b1[j]);
//    lane l holds the float4 chunks 4l + 256t of h and of the W1 row (all in flight).
//  k_router_out: w = sigmoid(w2 . hid[row] + bias); stop iff u < w.
constexpr int GATE_MLP_MAX = 1024;
constexpr int GATE_MLP_KD = 8;       // float4 chunks per lane: d <= 2048

__global__ __launch_bounds__(256) void k_router_hidden(const RowInfo* rows, int n, const float* Hs, int d,
                                                       const float* w1, const float* b1, int rr, double* hid) {
    const int i = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (i >= n || j >= rr) return;
    const float* h = Hs + (int64_t)rows[i].hrow * d;
    const float* wr = w1 + (int64_t)j * d;
    float4 hv[GATE_MLP_KD], wv[GATE_MLP_KD];
#pragma unroll
    for (int t = 0; t < GATE_MLP_KD; ++t) {
        const int k = lane * 4 + 256 * t;
        hv[t] = k < d ? *(const float4*)(h + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        wv[t] = k < d ? *(const float4*)(wr + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    double acc = 0.0;
#pragma unroll
    for (int t = 0; t < GATE_MLP_KD; ++t) {
        acc += (double)wv[t].x * (double)hv[t].x + (double)wv[t].y * (double)hv[t].y;
        acc += (double)wv[t].z * (double)hv[t].z + (double)wv[t].w * (double)hv[t].w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) {
        const double x = acc + (double)b1[j];
        hid[(int64_t)i * rr + j] = x / (1.0 + exp(-x));
    }
}

__global__ __launch_bounds__(64) void k_router_out(const int* seqs, int n, const double* hid, const float* w2, int rr,
                                                   float bias, const float* uniforms, int ucol, double* w_out,
                                                   int* stop_out, int* host_flags, int tag) {
    const int i = blockIdx.x;
    if (i >= n) return;
    const int lane = threadIdx.x;
    double acc = 0.0;
    for (int j = lane; j < rr; j += 64) acc += (double)w2[j] * hid[(int64_t)i * rr + j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) {
        const double z = acc + (double)bias;
        double w;
        if (z >= 0.0) {
            w = 1.0 / (1.0 + exp(-z));
        } else {
            const double ez = exp(z);
            w = ez / (1.0 + ez);
        }
        const int seq = seqs[i];
        w_out[seq * 4 + ucol] = w;
        if (uniforms) {
            const int stop = ((double)uniforms[seq * 4 + ucol] < w) ? 1 : 0;
            stop_out[seq] = stop;
            publish_stop(host_flags, seq, tag, stop);
        }
    }
}

hipError_t launch_gate_mlp(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d, const float* w1,
                           const float* b1, const float* w2, int rr, float bias, const float* uniforms, int ucol,
                           double* hid, double* w_out, int* stop_out, hipStream_t st, int* host_flags, int tag) {
    if (n <= 0) return hipSuccess;
    if (rr < 1 || rr > GATE_MLP_MAX || d % 4 != 0 || d > 256 * GATE_MLP_KD) return hipErrorInvalidValue;
    NV_LAUNCH(k_router_hidden, dim3(n, (rr + 3) / 4), dim3(256), 0, st, rows, n, Hs, d, w1, b1, rr, hid);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    NV_LAUNCH(k_router_out, dim3(n), dim3(64), 0, st, seqs, n, hid, w2, rr, bias, uniforms, ucol, w_out, stop_out,
              host_flags, tag);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_copy_rows(const RowInfo* rows, int n, const float* Hs, int d, float* dst) {
    const int i = blockIdx.x;
    if (i >= n) return;
    const float* src = Hs + (int64_t)rows[i].hrow * d;
    for (int k = threadIdx.x; k < d; k += blockDim.x) dst[(int64_t)i * d + k] = src[k];
}

hipError_t launch_copy_rows(const RowInfo* rows, int n, const float* Hs, int d, float* dst, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    NV_LAUNCH(k_copy_rows, dim3(n), dim3(256), 0, st, rows, n, Hs, d, dst);
    return hipGetLastError();
}

// Log-probability of the target token under softmax(z) for each row: z[y] - max z -
// log sum exp(z - max z), exponentials in float32 summed in float64 (as the sampler).
// One row per block.  Each thread keeps its logits (k = t, t + 1024, ...) in registers
// when V <= 32768, so the row is read from memory once; the exponentials are summed in
// float64 in that fixed order either way.
constexpr int XE_PER = 32;
__global__ __launch_bounds__(1024) void k_xent(const float* logits, int64_t ld, int n, int V, const int* targets,
                                               double* out, int ostride, int ocol) {
    __shared__ float smax[16];
    __shared__ double ssum[16];
    const int i = blockIdx.x;
    if (i >= n) return;
    const float* z = logits + (int64_t)i * ld;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = blockDim.x >> 6;
    const bool regs = V <= XE_PER * (int)blockDim.x;
    const float zt = z[targets[i]];
    float zv[XE_PER];
    float mx = -INFINITY;
    if (regs) {
#pragma unroll
        for (int j = 0; j < XE_PER; ++j) {
            const int k = t + j * (int)blockDim.x;
            zv[j] = k < V ? z[k] : -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < XE_PER; ++j) mx = fmaxf(mx, zv[j]);
    } else {
        for (int k = t; k < V; k += blockDim.x) mx = fmaxf(mx, z[k]);
    }
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();
    mx = smax[0];
    for (int w = 1; w < nw; ++w) mx = fmaxf(mx, smax[w]);
    double acc = 0.0;
    if (regs) {
#pragma unroll
        for (int j = 0; j < XE_PER; ++j)
            if (t + j * (int)blockDim.x < V) acc += (double)expf(zv[j] - mx);
    } else {
        for (int k = t; k < V; k += blockDim.x) acc += (double)expf(z[k] - mx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) ssum[wave] = acc;
    __syncthreads();
    if (t == 0) {
        double tot = 0.0;
        for (int w = 0; w < nw; ++w) tot += ssum[w];
        out[(int64_t)i * ostride + ocol] = (double)zt - (double)mx - log(tot);
    }
}

// One wave per row: lane l folds groups l, l + 64, ... (the maximum first, then
// s_g exp(m_g - M) in float64), and the wave adds the lanes in a fixed tree order.
__global__ __launch_bounds__(256) void k_xent_merge(const float* part, const float* tgt, int n, int ngroups,
                                                    double* out, int ostride, int ocol) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= n) return;
    const float2* p = (const float2*)part + (int64_t)i * ngroups;
    float mx = -INFINITY;
    for (int gi = lane; gi < ngroups; gi += 64) mx = fmaxf(mx, p[gi].x);
    mx = wave_max(mx);
    double acc = 0.0;
    for (int gi = lane; gi < ngroups; gi += 64) {
        const float2 v = p[gi];
        acc += (double)v.y * exp((double)v.x - (double)mx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) out[(int64_t)i * ostride + ocol] = (double)tgt[i] - (double)mx - log(acc);
}

hipError_t launch_xent_merge(const float* part, const float* tgt, int n, int ngroups, double* out, int ostride,
                             int ocol, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (ngroups <= 0) return hipErrorInvalidValue;
    NV_LAUNCH(k_xent_merge, dim3((n + 3) / 4), dim3(256), 0, st, part, tgt, n, ngroups, out, ostride, ocol);
    return hipGetLastError();
}

hipError_t launch_xent(const float* logits, int64_t ld, int n, int V, const int* targets, double* out, int ostride,
                       int ocol, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    NV_LAUNCH(k_xent, dim3(n), dim3(1024), 0, st, logits, ld, n, V, targets, out, ostride, ocol);
    return hipGetLastError();
}

// Mixture objective per row (one block, fixed reduction order): the last exit's router
// output is 1; p_k = w_k prod_{j<k} (1 - w_j); nll = -log sum_k p_k pi_k(y), a log-sum-exp
// over the exits with p_k > 0; depth = sum_k p_k l_k / L.  sums = {mean nll, mean depth}.
__global__ __launch_bounds__(256) void k_loss_reduce(double* w, const double* lp, int n, ExitDepths dep, double* nll,
                                                     double* depth, double* sums) {
    __shared__ double sa[256], sb[256];
    const int t = threadIdx.x;
    double an = 0.0, ad = 0.0;
    for (int i = t; i < n; i += blockDim.x) {
        w[(int64_t)i * 4 + 3] = 1.0;
        double p[4], rest = 1.0;
        for (int k = 0; k < 4; ++k) {
            p[k] = w[(int64_t)i * 4 + k] * rest;
            rest *= 1.0 - w[(int64_t)i * 4 + k];
        }
        double mx = -INFINITY;
        for (int k = 0; k < 4; ++k)
            if (p[k] > 0.0) mx = fmax(mx, log(p[k]) + lp[(int64_t)i * 4 + k]);
        double se = 0.0, dp = 0.0;
        for (int k = 0; k < 4; ++k) {
            if (p[k] > 0.0) se += exp(log(p[k]) + lp[(int64_t)i * 4 + k] - mx);
            dp += p[k] * (double)dep.layer[k] / (double)dep.L;
        }
        const double v = -(mx + log(se));
        nll[i] = v;
        depth[i] = dp;
        an += v;
        ad += dp;
    }
    sa[t] = an;
    sb[t] = ad;
    __syncthreads();
    for (int o = blockDim.x / 2; o > 0; o >>= 1) {
        if (t < o) {
            sa[t] += sa[t + o];
            sb[t] += sb[t + o];
        }
        __syncthreads();
    }
    if (t == 0) {
        sums[0] = n > 0 ? sa[0] / n : 0.0;
        sums[1] = n > 0 ? sb[0] / n : 0.0;
    }
}

hipError_t launch_loss_reduce(double* w, const double* lp, int n, ExitDepths dep, double* nll, double* depth,
                              double* sums, hipStream_t st) {
    NV_LAUNCH(k_loss_reduce, dim3(1), dim3(256), 0, st, w, lp, n, dep, nll, depth, sums);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Inverse-CDF sampling of softmax(logits) in token-id order:
//   e_i = exp(z_i - max z) (float32 exp), Z = sum e_i in float64,
//   token = smallest i with u * Z < sum_{j<=i} e_j (float64 comparisons).
// 1024 threads; thread t owns a contiguous id range.  The range sums are prefixed by a
// fixed-order block scan (so prefix_{t+1} = prefix_t + S_t exactly), and the thread whose
// range holds u*Z walks it.
// ------------------------------------------------------------------------------------------

constexpr int SMP_THREADS = 1024;
constexpr int SMP_PER = 32;        // ids per thread held in registers (vocab <= 32768)

__global__ __launch_bounds__(SMP_THREADS) void k_sample(const float* logits, int64_t ld, const int* seqs, int n,
                                                        int V, const float* uniforms, int* tok_out) {
    __shared__ float smax[SMP_THREADS / 64];
    __shared__ double wsum[SMP_THREADS / 64];
    __shared__ int found;
    const int seq = seqs[blockIdx.x];
    const float* z = logits + (int64_t)seq * ld;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int b = t * SMP_PER;
    float zv[SMP_PER];
#pragma unroll
    for (int i = 0; i < SMP_PER; i += 4) {
        if (b + i + 3 < V) {
            const float4 v4 = *(const float4*)(z + b + i);
            zv[i] = v4.x; zv[i + 1] = v4.y; zv[i + 2] = v4.z; zv[i + 3] = v4.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) zv[i + j] = (b + i + j < V) ? z[b + i + j] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) mx = fmaxf(mx, zv[i]);
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    if (t == 0) found = 0x7fffffff;
    __syncthreads();
    float M = smax[0];
    for (int w = 1; w < SMP_THREADS / 64; ++w) M = fmaxf(M, smax[w]);
    float ev[SMP_PER];
    double S = 0.0;
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) {
        ev[i] = expf(zv[i] - M);          // 0 for padding (z = -inf)
        S += (double)ev[i];
    }
    // inclusive scan of S over the wave (fixed order), then over the waves
    double inc = S;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    double wpre = 0.0, Z = 0.0;
    for (int w = 0; w < SMP_THREADS / 64; ++w) {
        if (w < wave) wpre += wsum[w];
        Z += wsum[w];
    }
    double exc = __shfl_up(inc, 1, 64);       // inclusive sum of the previous lane
    if (lane == 0) exc = 0.0;
    const double hi = wpre + inc, lo = wpre + exc;   // lo_t == hi_{t-1}: same operands, same order
    const double target = (double)uniforms[seq * 4 + 3] * Z;
    if (b < V && lo <= target && target < hi) {
        double cum = lo;
        int tok = min(V, b + SMP_PER) - 1;
#pragma unroll
        for (int i = 0; i < SMP_PER; ++i) {
            cum += (double)ev[i];
            if (target < cum && b + i < V) {
                tok = b + i;
                break;
            }
        }
        atomicMin(&found, tok);
    }
    __syncthreads();
    if (t == 0) {
        int tok = found;
        if (tok == 0x7fffffff) {  // u*Z at or past the rounded total: last id with nonzero mass
            tok = V - 1;
            while (tok > 0 && expf(z[tok] - M) == 0.0f) --tok;
        }
        tok_out[seq] = tok;
    }
}

hipError_t launch_sample(const float* logits, int64_t ld, const int* seqs, int n, int V, const float* uniforms,
                         int* tok_out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    NV_LAUNCH(k_sample, dim3(n), dim3(SMP_THREADS), 0, st, logits, ld, seqs, n, V, uniforms, tok_out);
    return hipGetLastError();
}

template <bool WB, int CP, int C, int HD>
static hipError_t gv_attr() {
    return hipFuncSetAttribute((const void*)k_gemv<WB, CP, C, HD>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               160 * 1024);
}

template <bool WB, int CP, int HD>
static hipError_t gv_attr_all() {
    hipError_t e;
    if ((e = gv_attr<WB, CP, 1, HD>()) != hipSuccess) return e;
    if ((e = gv_attr<WB, CP, 2, HD>()) != hipSuccess) return e;
    if ((e = gv_attr<WB, CP, 3, HD>()) != hipSuccess) return e;
    if ((e = gv_attr<WB, CP, 4, HD>()) != hipSuccess) return e;
    return gv_attr<WB, CP, 8, HD>();
}

hipError_t init_kernel_attributes() {
    hipError_t e;
    if ((e = gv_attr_all<true, 4, 0>()) != hipSuccess) return e;
    if ((e = gv_attr_all<true, 4, 1>()) != hipSuccess) return e;
    if ((e = gv_attr_all<true, 2, 0>()) != hipSuccess) return e;
    if ((e = gv_attr_all<true, 2, 1>()) != hipSuccess) return e;
    if ((e = gv_attr_all<false, 4, 0>()) != hipSuccess) return e;
    if ((e = gv_attr_all<false, 4, 1>()) != hipSuccess) return e;
    if ((e = gv_attr_all<false, 2, 0>()) != hipSuccess) return e;
    return gv_attr_all<false, 2, 1>();
}

}  // namespace nv
