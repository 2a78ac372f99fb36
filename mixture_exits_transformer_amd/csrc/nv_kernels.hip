// HIP kernels of the N-vium decode step for gfx950 (CDNA4, wave64).
//
// Layer arithmetic follows the LLaMA-2 pre-norm block named in section 4 of the
// gist.science technical summary of N-vium; exits follow section 2, part
// "Architektur" (router w_k, stick-breaking p_k, per-exit distribution pi_k);
// causal chunks of deferred rows follow section 2, part "Inferenz: Piggybacking".
#include "nv_internal.h"

#include <math.h>

namespace nv {

// ------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float kv_load(const void* kv, int bf16, int64_t i) {
    if (bf16) return __uint_as_float(((uint32_t)((const uint16_t*)kv)[i]) << 16);
    return ((const float*)kv)[i];
}

__device__ __forceinline__ void kv_store(void* kv, int bf16, int64_t i, float v) {
    if (bf16)
        ((uint16_t*)kv)[i] = f2bf(v);
    else
        ((float*)kv)[i] = v;
}

// K (which = 0) or V (which = 1) of (seq, layer, head) at position 0.
__device__ __forceinline__ int64_t kv_base(const LayerDims& D, int seq, int layer, int which, int head) {
    return ((((int64_t)seq * D.L + layer) * 2 + which) * D.H + head) * (int64_t)D.max_ctx * D.hd;
}

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
    hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cs, max_ctx, hd,
                       (double)base);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// embedding gather: hidden row = E[token]
// ------------------------------------------------------------------------------------------

__global__ void k_embed(const int* tokens, const RowInfo* rows, int n, const void* E, int wbf16, float* Hs,
                        int d) {
    int r = blockIdx.x;
    if (r >= n) return;
    int64_t src = (int64_t)tokens[r] * d;
    float* dst = Hs + (int64_t)rows[r].hrow * d;
    for (int k = threadIdx.x; k < d; k += blockDim.x)
        dst[k] = wbf16 ? __uint_as_float(((uint32_t)((const uint16_t*)E)[src + k]) << 16)
                       : ((const float*)E)[src + k];
}

hipError_t launch_embed(const int* tokens, const RowInfo* rows, int n, const void* E, int wbf16, float* Hs, int d,
                        hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_embed, dim3(n), dim3(256), 0, st, tokens, rows, n, E, wbf16, Hs, d);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Skinny GEMM on the vector ALUs.  Each block owns GV_COLS consecutive output columns,
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

template <bool WBF>
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
                if (lane == 0) {
                    const int orow = a.o_rows ? a.o_rows[rt0 + r].hrow : rt0 + r;
                    float* o = a.out + (int64_t)orow * a.ldo;
                    if (a.epi == EPI_STORE) {
                        o[n0] = g;
                        o[n0 + 1] = u;
                    } else if (a.epi == EPI_RESID) {
                        o[n0] += g;
                        o[n0 + 1] += u;
                    } else {
                        o[n0 >> 1] = g / (1.0f + expf(-g)) * u;
                    }
                }
            }
        }
        __syncthreads();
    }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    if (a.R <= 0) return hipSuccess;
    const int rt = gv_row_tile(a.K);
    const size_t shm = ((size_t)rt * a.K + GV_RT_MAX) * sizeof(float);
    dim3 grid(a.N / GV_COLS);
    if (a.wbf16)
        hipLaunchKernelGGL(k_gemm_valu<true>, grid, dim3(256), shm, st, a);
    else
        hipLaunchKernelGGL(k_gemm_valu<false>, grid, dim3(256), shm, st, a);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// RoPE on q (in place) and k; k, v appended to the KV cache at the rows' positions.
// qkv row i = [q (d) | k (d) | v (d)], head h occupying [h*hd, (h+1)*hd) of each.
// ------------------------------------------------------------------------------------------

__global__ void k_rope_kv(float* qkv, const RowInfo* rows, int R, void* kv, int layer, LayerDims D,
                          const float* cs) {
    const int i = blockIdx.x;
    if (i >= R) return;
    const RowInfo ri = rows[i];
    float* q = qkv + (int64_t)i * 3 * D.d;
    const float* k = q + D.d;
    const float* v = k + D.d;
    const int half = D.hd / 2;
    const float* c = cs + (int64_t)ri.pos * half * 2;
    for (int idx = threadIdx.x; idx < D.H * half; idx += blockDim.x) {
        const int h = idx / half, j = idx - h * half;
        const float co = c[2 * j], si = c[2 * j + 1];
        const int e0 = h * D.hd + j, e1 = e0 + half;
        const float qa = q[e0], qb = q[e1];
        q[e0] = qa * co - qb * si;
        q[e1] = qb * co + qa * si;
        const float ka = k[e0], kb = k[e1];
        const int64_t kb0 = kv_base(D, ri.seq, layer, 0, h) + (int64_t)ri.pos * D.hd;
        const int64_t vb0 = kv_base(D, ri.seq, layer, 1, h) + (int64_t)ri.pos * D.hd;
        kv_store(kv, D.kv_bf16, kb0 + j, ka * co - kb * si);
        kv_store(kv, D.kv_bf16, kb0 + j + half, kb * co + ka * si);
        kv_store(kv, D.kv_bf16, vb0 + j, v[e0]);
        kv_store(kv, D.kv_bf16, vb0 + j + half, v[e1]);
    }
}

hipError_t launch_rope_kv(float* qkv, const RowInfo* rows, int R, void* kv, int layer, const LayerDims& D,
                          const float* cs, hipStream_t st) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rope_kv, dim3(R), dim3(256), 0, st, qkv, rows, R, kv, layer, D, cs);
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

__global__ __launch_bounds__(256) void k_attn(const AttnItem* items, const RowInfo* rows, const float* qkv,
                                              const void* kv, int layer, LayerDims D, float* part_ml,
                                              float* part_o) {
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
        Qs[idx] = qkv[(int64_t)(it.row0 + r) * 3 * D.d + it.head * hd + e] * scale;
    }
    const int seq = rows[it.row0].seq;
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
        const int64_t slot = it.part + r;
        if (lane == 0) {
            part_ml[2 * slot] = m[i];
            part_ml[2 * slot + 1] = l[i];
        }
        if (d0 < hd) part_o[slot * hd + d0] = o0[i];
        if (d1 < hd) part_o[slot * hd + d1] = o1[i];
    }
}

__global__ void k_attn_combine(const CombineInfo* ci, int R, LayerDims D, const float* part_ml,
                               const float* part_o, float* out) {
    const int i = blockIdx.x;
    if (i >= R) return;
    const CombineInfo c = ci[i];
    for (int idx = threadIdx.x; idx < D.H * D.hd; idx += blockDim.x) {
        const int h = idx / D.hd, e = idx - h * D.hd;
        float M = -INFINITY;
        for (int s = 0; s < c.nsplit; ++s) {
            const int64_t slot = c.base + (int64_t)(h * c.nsplit + s) * c.nrows + c.off;
            M = fmaxf(M, part_ml[2 * slot]);
        }
        float Ls = 0.f, acc = 0.f;
        for (int s = 0; s < c.nsplit; ++s) {
            const int64_t slot = c.base + (int64_t)(h * c.nsplit + s) * c.nrows + c.off;
            const float ms = part_ml[2 * slot];
            if (ms == -INFINITY) continue;
            const float w = expf(ms - M);
            Ls += w * part_ml[2 * slot + 1];
            acc += w * part_o[slot * D.hd + e];
        }
        out[(int64_t)i * D.d + idx] = acc / Ls;
    }
}

hipError_t launch_attn(const AttnItem* items, int n_items, const RowInfo* rows, const float* qkv, const void* kv,
                       int layer, const LayerDims& D, float* part_ml, float* part_o, hipStream_t st) {
    if (n_items <= 0) return hipSuccess;
    const int tile = at_tile(D.hd);
    const size_t shm = ((size_t)tile * (D.hd + 1) + (size_t)tile * D.hd + (size_t)AT_MAX_ROWS * D.hd) * sizeof(float);
    hipLaunchKernelGGL(k_attn, dim3(n_items), dim3(256), shm, st, items, rows, qkv, kv, layer, D, part_ml,
                       part_o);
    return hipGetLastError();
}

hipError_t launch_attn_combine(const CombineInfo* ci, int R, const LayerDims& D, const float* part_ml,
                               const float* part_o, float* out, hipStream_t st) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_attn_combine, dim3(R), dim3(256), 0, st, ci, R, D, part_ml, part_o, out);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Router gate at the end of a segment: w = sigmoid(g . h + b) in float64, stop iff u < w.
// ------------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_gate(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d,
                                              const float* gw, float bias, const float* uniforms, int ucol,
                                              double* w_out, int* stop_out) {
    __shared__ double red[256];
    const int i = blockIdx.x;
    if (i >= n) return;
    const float* h = Hs + (int64_t)rows[i].hrow * d;
    double acc = 0.0;
    for (int k = threadIdx.x; k < d; k += blockDim.x) acc += (double)gw[k] * (double)h[k];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double z = red[0] + (double)bias;
        double w;
        if (z >= 0.0) {
            w = 1.0 / (1.0 + exp(-z));
        } else {
            const double ez = exp(z);
            w = ez / (1.0 + ez);
        }
        const int seq = seqs[i];
        w_out[seq * 4 + ucol] = w;
        stop_out[seq] = ((double)uniforms[seq * 4 + ucol] < w) ? 1 : 0;
    }
}

hipError_t launch_gate(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d, const float* gw, float bias,
                       const float* uniforms, int ucol, double* w_out, int* stop_out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_gate, dim3(n), dim3(256), 0, st, rows, seqs, n, Hs, d, gw, bias, uniforms, ucol, w_out,
                       stop_out);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Inverse-CDF sampling of softmax(logits) in token-id order, in float64:
//   e_i = exp(z_i - max z), Z = sum e_i, token = smallest i with u * Z < sum_{j<=i} e_j.
// Thread t owns a contiguous id range; range sums are prefixed serially (so that the
// prefix of range t+1 is exactly prefix_t + S_t) and the range holding u*Z is scanned.
// ------------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_sample(const float* logits, int64_t ld, const int* seqs, int n, int V,
                                                const float* uniforms, int* tok_out) {
    __shared__ double sd[257];
    __shared__ float sf[256];
    __shared__ int found;
    const int seq = seqs[blockIdx.x];
    const float* z = logits + (int64_t)seq * ld;
    const int t = threadIdx.x;
    const int chunk = (V + 255) / 256;
    const int b = min(V, t * chunk), e = min(V, b + chunk);
    float mx = -INFINITY;
    for (int i = b; i < e; ++i) mx = fmaxf(mx, z[i]);
    sf[t] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s) sf[t] = fmaxf(sf[t], sf[t + s]);
        __syncthreads();
    }
    const double M = (double)sf[0];
    double S = 0.0;
    for (int i = b; i < e; ++i) S += exp((double)z[i] - M);
    sd[t + 1] = S;
    if (t == 0) found = 0x7fffffff;
    __syncthreads();
    if (t == 0) {
        sd[0] = 0.0;
        for (int i = 1; i <= 256; ++i) sd[i] += sd[i - 1];
    }
    __syncthreads();
    const double Z = sd[256];
    const double target = (double)uniforms[seq * 4 + 3] * Z;
    const double lo = sd[t], hi = sd[t + 1];
    if (b < e && lo <= target && target < hi) {
        double cum = lo;
        int tok = e - 1;
        for (int i = b; i < e; ++i) {
            cum += exp((double)z[i] - M);
            if (target < cum) {
                tok = i;
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
            while (tok > 0 && exp((double)z[tok] - M) == 0.0) --tok;
        }
        tok_out[seq] = tok;
    }
}

hipError_t launch_sample(const float* logits, int64_t ld, const int* seqs, int n, int V, const float* uniforms,
                         int* tok_out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_sample, dim3(n), dim3(256), 0, st, logits, ld, seqs, n, V, uniforms, tok_out);
    return hipGetLastError();
}

hipError_t init_kernel_attributes() { return hipSuccess; }

}  // namespace nv
