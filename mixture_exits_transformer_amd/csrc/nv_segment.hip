// Persistent segment kernel for gfx950: every layer of one N-vium segment for a single
// decode row (the current token of one sequence with no deferred rows at this segment)
// in one cooperative launch.
//
// The layer is the LLaMA-2 pre-norm block (section 4 of the gist.science technical
// summary of N-vium): RMSNorm, QKV with RoPE, causal attention over the KV cache,
// O projection + residual, RMSNorm, SwiGLU MLP + residual.  One launch per layer phase
// pays a dispatch ramp and a cold first-load latency of several microseconds for a few
// microseconds of streaming; here the next phases' weights are already in flight while
// a phase waits for its inputs.
//
// Roles of the 8 waves of a block (one block per CU, all blocks co-resident):
//  - waves 0..5 stream weights.  They keep their share of the weights of the next two
//    phases in registers, issued before they wait, and only ever wait on the block
//    barrier (an LDS-only fence, so their weight loads stay in flight across it) and on
//    their own loads.  They read inputs from LDS and write dot products to LDS.
//  - waves 6..7 are control waves.  They poll the tagged inputs of a phase (written by
//    other blocks), stage them into LDS, and after the dot products run the epilogues
//    (RoPE, KV append, residual adds, SwiGLU) and store the tagged outputs.
//
// Cross-block data are 64-bit words (epoch << 32 | fp32 bits) written and read with
// agent-scope atomic stores and loads: a consumer knows a value is the one of this phase
// when its tag equals the phase's epoch, so no grid barrier is needed.  Every poll gives
// up after a bounded time (flagging an error), so the kernel always finishes.
//
// Phases per layer and their per-block work (NB blocks, column ranges of NB-th parts):
//   QKV   columns [b*cq, (b+1)*cq) of the permuted QKV matrix; epilogue: q, k, v
//   ATT   split s of head h (b = h*S + s): keys [lo, hi) of the causal range 0..pos;
//         the block's partial softmax state goes to tpart; the last split to finish a
//         head merges the S partials into the head's attention output
//   O     columns [b*co, (b+1)*co) of W_o, residual on the same columns
//   GU    columns [b*cg, (b+1)*cg) of the interleaved gate/up matrix; SwiGLU
//   DOWN  columns [b*co, (b+1)*co) of W_d, residual; the next layer's input
#include "nv_internal.h"
#include "nv_device.h"

#include <math.h>

namespace nv {

namespace {

constexpr int PH_QKV = 1, PH_PART = 2, PH_ATT = 3, PH_X1 = 4, PH_ACT = 5, PH_X0 = 6;
constexpr int KC_D = SEG_DMAX / 512;      // 16-byte chunks per lane of a row of width d
constexpr int KC_F = SEG_FMAX / 512;      // ... of width F
constexpr int MQ = SEG_QCOLS / SEG_NS;    // QKV columns per streaming wave
constexpr int MG = SEG_GCOLS / SEG_NS;    // gate/up columns per streaming wave
constexpr int NR = 4;                     // key rounds (4 keys each) a wave prefetches
constexpr int NJ_D = SEG_DMAX / 128;      // tagged words per control lane, width d
constexpr int NJ_F = SEG_FMAX / 128;      // ... width F
constexpr int NJ_S = 4;                   // sampled words per control lane (<= 512 producers)

// The staged input row of a phase lives in two planes so that a lane's 16-byte chunk
// ch (8 values) is read as two conflict-free 16-byte LDS reads: values 8ch..8ch+3 at
// xlo[4ch], values 8ch+4..8ch+7 at xhi[4ch].
struct SegShared {
    float xlo[SEG_FMAX / 2], xhi[SEG_FMAX / 2];
    float dots[64];             // dot products of the block's columns
    float ss[2];                // sums of squares of the staged row, one per control wave
    float qs[SEG_HD], kn[SEG_HD], vn[SEG_HD];
    float wm[SEG_NS * 4], wl[SEG_NS * 4];   // softmax state per (wave, lane group)
    float wo[SEG_NS * 4][SEG_HD];
    float xres[SEG_OCOLS];      // layer input on the block's O / down columns
    float x1own[SEG_OCOLS];     // after the attention residual, same columns
    int bad;                    // a wait in this block gave up
};




// Block barrier that orders LDS only: global loads in flight stay in flight.
__device__ __forceinline__ void seg_bar() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


__device__ __forceinline__ void give_up(SegShared& sh, uint32_t* err) {
    sh.bad = 1;
    __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool timed_out(unsigned long long t_end) {
    return (unsigned long long)wall_clock64() > t_end;
}

// Control waves: put value v of row index i into the LDS planes.
__device__ __forceinline__ void plane_put(SegShared& sh, int i, float v) {
    const int ch = i >> 3, e = i & 7;
    (e < 4 ? sh.xlo : sh.xhi)[ch * 4 + (e & 3)] = v;
}

// Control waves: stage the n tagged words src[0..n) into the LDS planes once every tag
// equals ep, multiplied by g[i] when g is set; sh.ss[wc] gets this wave's sum of squares
// of the raw values.  Control wave wc takes words (2j + wc) * 64 + lane.  With
// stride > 0 the wave first polls only every stride-th word (one per producer block),
// which keeps 256 blocks from hammering the same few kilobytes.
template <int NJ>
__device__ void stage_tagged(const uint64_t* src, int n, uint32_t ep, int stride, const float* g, int wc, int lane,
                             unsigned long long spin, SegShared& sh, uint32_t* err) {
    if (sh.bad) return;
    const unsigned long long t_end = (unsigned long long)wall_clock64() + spin;
    const __amdgpu_buffer_rsrc_t r = coh_rsrc(src);
    float gv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int i = (2 * j + wc) * 64 + lane;
        gv[j] = (g && i < n) ? g[i] : 1.0f;
    }
    if (stride > 0) {
        const int ns = n / stride;
        for (;;) {
            bool ok = true;
#pragma unroll
            for (int j = 0; j < NJ_S; ++j) {
                const int k = (2 * j + wc) * 64 + lane;
                const uint64_t v = k < ns ? tload_b(r, k * stride * 8, 0) : tagv(ep, 0.f);
                ok = ok && (uint32_t)(v >> 32) == ep;
            }
            if (__all(ok)) break;
            if (timed_out(t_end)) {
                give_up(sh, err);
                return;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    // bulk load, then reloads of the words whose tag is not yet this phase's
    const int voff = (wc * 64 + lane) * 8;
    uint64_t v[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int i = (2 * j + wc) * 64 + lane;
        v[j] = i < n ? tload_b(r, voff, j * 1024) : tagv(ep, 0.f);
    }
    for (;;) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < NJ; ++j) ok = ok && (uint32_t)(v[j] >> 32) == ep;
        if (__all(ok)) break;
        if (timed_out(t_end)) {
            give_up(sh, err);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int i = (2 * j + wc) * 64 + lane;
            if (i < n && (uint32_t)(v[j] >> 32) != ep) v[j] = tload_b(r, voff, j * 1024);
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int i = (2 * j + wc) * 64 + lane;
        if (i < n) {
            const float x = __uint_as_float((uint32_t)v[j]);
            ss = fmaf(x, x, ss);
            plane_put(sh, i, x * gv[j]);
        }
    }
    ss = wave_total(ss);
    if (lane == 0) sh.ss[wc] = ss;
}

// Control waves: stage one head's SEG_HD tagged words into dst (lane: word wc*64 + lane).
__device__ void stage_head(const uint64_t* src, uint32_t ep, float* dst, int wc, int lane, unsigned long long spin,
                           SegShared& sh, uint32_t* err) {
    if (sh.bad) return;
    const unsigned long long t_end = (unsigned long long)wall_clock64() + spin;
    const __amdgpu_buffer_rsrc_t r = coh_rsrc(src);
    const int i = wc * 64 + lane;
    uint64_t v;
    for (;;) {
        v = tload_b(r, i * 8, 0);
        if (__all((uint32_t)(v >> 32) == ep)) break;
        if (timed_out(t_end)) {
            give_up(sh, err);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    dst[i] = __uint_as_float((uint32_t)v);
}

// Control waves: the same as stage_tagged from plain fp32 memory written before this launch.
template <int NJ>
__device__ void stage_plain(const float* src, int n, const float* g, int wc, int lane, SegShared& sh) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int i = (2 * j + wc) * 64 + lane;
        if (i < n) {
            const float x = src[i];
            ss = fmaf(x, x, ss);
            plane_put(sh, i, g ? x * g[i] : x);
        }
    }
    ss = wave_total(ss);
    if (lane == 0) sh.ss[wc] = ss;
}

// Streaming waves: issue this wave's weight chunks of the block's columns
// [col0, col0 + ncols) of the [N][K] bf16 matrix W.  Column c of the block goes to wave
// c % SEG_NS (slot c / SEG_NS); lane `lane` holds 16-byte chunk j * 64 + lane of K.
// Every slot issues a load (slots past the columns or past K reload column col0, chunk
// 0, and are never used): with no branches around the loads the compiler can count
// them and wait for exactly the ones a phase uses, leaving later phases' loads in flight.
template <int MC, int KC>
__device__ __forceinline__ void w_issue(uint4 (&w)[MC][KC], const uint16_t* W, int K, int col0, int ncols, int wave,
                                        int lane) {
    const int nch = K >> 3;
#pragma unroll
    for (int i = 0; i < MC; ++i) {
        const int c = wave + SEG_NS * i;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int ch = j * 64 + lane;
            const bool ok = c < ncols && ch < nch;
            const int64_t off = ok ? (int64_t)(col0 + c) * K + (int64_t)ch * 8 : (int64_t)col0 * K;
            w[i][j] = *(const uint4*)(W + off);
        }
    }
}

// Streaming waves: dot products of this wave's columns with the staged row (times
// `scale`), written to sh.dots[local column].
template <int MC, int KC>
__device__ __forceinline__ void w_dot(const uint4 (&w)[MC][KC], SegShared& sh, int K, float scale, int ncols, int wave,
                                      int lane) {
    float acc[MC];
#pragma unroll
    for (int i = 0; i < MC; ++i) acc[i] = 0.f;
    const int nch = K >> 3;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const int ch = j * 64 + lane;
        if (ch < nch) {
            const float4 lo = *(const float4*)(sh.xlo + ch * 4), hi = *(const float4*)(sh.xhi + ch * 4);
            const float x[8] = {lo.x * scale, lo.y * scale, lo.z * scale, lo.w * scale,
                                hi.x * scale, hi.y * scale, hi.z * scale, hi.w * scale};
#pragma unroll
            for (int i = 0; i < MC; ++i) {
                const uint32_t u[4] = {w[i][j].x, w[i][j].y, w[i][j].z, w[i][j].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[i] = fmaf(bf_lo(u[e]), x[2 * e], acc[i]);
                    acc[i] = fmaf(bf_hi(u[e]), x[2 * e + 1], acc[i]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MC; ++i) {
        const float tot = wave_total(acc[i]);
        const int c = wave + SEG_NS * i;
        if (lane == 0 && c < ncols) sh.dots[c] = tot;
    }
}

// The block's attention work item.
struct AttItem {
    bool on;        // the block owns a split
    int h, s;       // head, split
    int lo, hi;     // keys [lo, hi)
    int old_hi;     // keys below this come from the cache (the current position does not)
    bool has_new;   // the split holds the current position
};

__device__ __forceinline__ AttItem att_item(const SegArgs& a) {
    AttItem t;
    const int b = blockIdx.x;
    t.on = b < a.D.H * a.S;
    t.h = t.on ? b / a.S : 0;
    t.s = t.on ? b % a.S : 0;
    const int ctx = a.pos + 1;
    const int per = (ctx + a.S - 1) / a.S;
    t.lo = min(t.s * per, ctx);
    t.hi = min(ctx, t.lo + per);
    t.old_hi = min(t.hi, a.pos);
    t.has_new = t.on && t.lo <= a.pos && a.pos < t.hi;
    return t;
}

// Key slot of (wave, round i, lane): 16 lanes per key, 4 keys per round.
__device__ __forceinline__ int key_of(int base, int wave, int i, int lane) {
    return base + 4 * (wave + SEG_NS * i) + (lane >> 4);
}

// Issue the K and V pieces of round i (i < NR) of this wave's keys from `base`.  Slots
// without a key (past old_hi, blocks without a split, want = false) reload key 0 of the
// head and are never used; every slot loads, so the loads can be counted (see w_issue).
__device__ __forceinline__ void kv_issue(uint4 (&kp)[NR], uint4 (&vp)[NR], const SegArgs& a, int layer,
                                         const AttItem& t, int base, bool want, int wave, int lane) {
    const uint16_t* K = (const uint16_t*)a.kv + kv_base(a.D, a.seq, layer, 0, t.h);
    const uint16_t* V = (const uint16_t*)a.kv + kv_base(a.D, a.seq, layer, 1, t.h);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int kk = key_of(base, wave, i, lane);
        const bool ok = want && t.on && kk < t.old_hi;
        const int64_t o = (int64_t)(ok ? kk : 0) * SEG_HD + (lane & 15) * 8;
        kp[i] = *(const uint4*)(K + o);
        vp[i] = *(const uint4*)(V + o);
    }
}

// Online-softmax update of one lane group (16 lanes, 8 dims each) with one key.
__device__ __forceinline__ void att_update(float& m, float& l, float (&o)[8], float sc, const float (&v)[8],
                                           bool valid) {
    if (valid) {
        const float mn = fmaxf(m, sc);
        const float c = expf(m - mn), p = expf(sc - mn);
        l = l * c + p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = o[e] * c + p * v[e];
        m = mn;
    }
}

__device__ __forceinline__ void att_rounds(const uint4 (&kp)[NR], const uint4 (&vp)[NR], const float (&q)[8], float scale,
                                           int base, int old_hi, int wave, int lane, float& m, float& l,
                                           float (&o)[8]) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const uint32_t ku[4] = {kp[i].x, kp[i].y, kp[i].z, kp[i].w};
        const uint32_t vu[4] = {vp[i].x, vp[i].y, vp[i].z, vp[i].w};
        float sc = 0.f, v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sc = fmaf(q[2 * e], bf_lo(ku[e]), sc);
            sc = fmaf(q[2 * e + 1], bf_hi(ku[e]), sc);
            v[2 * e] = bf_lo(vu[e]);
            v[2 * e + 1] = bf_hi(vu[e]);
        }
        sc = group_sum<16>(sc) * scale;
        att_update(m, l, o, sc, v, key_of(base, wave, i, lane) < old_hi);
    }
}

// Streaming waves, attention phase: the wave's keys of the block's split; the softmax
// state (max, sum, output) of each lane group goes to slot wave * 4 + group of sh.wm /
// sh.wl / sh.wo.
__device__ void att_stream(const SegArgs& a, SegShared& sh, const AttItem& t, int layer, const uint4 (&kp)[NR],
                           const uint4 (&vp)[NR], int wave, int lane) {
    const float scale = 1.0f / sqrtf((float)SEG_HD);
    float q[8], o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        q[e] = sh.qs[(lane & 15) * 8 + e];
        o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    att_rounds(kp, vp, q, scale, t.lo, t.old_hi, wave, lane, m, l, o);
    // keys beyond the prefetched rounds (long contexts), loaded here
    constexpr int STEP = 4 * SEG_NS * NR;
    for (int base = t.lo + STEP; base < t.old_hi; base += STEP) {
        uint4 k2[NR], v2[NR];
        kv_issue(k2, v2, a, layer, t, base, true, wave, lane);
        att_rounds(k2, v2, q, scale, base, t.old_hi, wave, lane, m, l, o);
    }
    if (t.has_new && wave == 0) {   // the current position, from the tagged copies in LDS
        float sc = 0.f, v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sc = fmaf(q[e], sh.kn[(lane & 15) * 8 + e], sc);
            v[e] = sh.vn[(lane & 15) * 8 + e];
        }
        sc = group_sum<16>(sc) * scale;
        att_update(m, l, o, sc, v, lane < 16);
    }
    const int slot = wave * 4 + (lane >> 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) sh.wo[slot][(lane & 15) * 8 + e] = o[e];
    if ((lane & 15) == 0) {
        sh.wm[slot] = m;
        sh.wl[slot] = l;
    }
}

__device__ void seg_streamer(const SegArgs& a, SegShared& sh, int wave, int lane) {
    const int b = blockIdx.x, NB = gridDim.x;
    const int d = a.D.d, F = a.D.F;
    const int cq = 3 * d / NB, co = d / NB, cg = 2 * F / NB;
    const AttItem t = att_item(a);
    uint4 wq[MQ][KC_D], kp[NR], vp[NR], wo[1][KC_D], wgu[MG][KC_D], wd[1][KC_F];
    w_issue<MQ, KC_D>(wq, a.lw[0].wqkv, d, b * cq, cq, wave, lane);
    kv_issue(kp, vp, a, a.l0, t, t.lo, true, wave, lane);
    for (int li = 0; li < a.nl; ++li) {
        const int l = a.l0 + li;
        const SegLayerW& W = a.lw[li];
        // QKV
        seg_bar();
        float inv = 1.0f / sqrtf((sh.ss[0] + sh.ss[1]) / (float)d + a.eps);
        w_dot<MQ, KC_D>(wq, sh, d, inv, cq, wave, lane);
        seg_bar();
        w_issue<1, KC_D>(wo, W.wo, d, b * co, co, wave, lane);
        // attention
        seg_bar();
        if (t.on) att_stream(a, sh, t, l, kp, vp, wave, lane);
        seg_bar();
        w_issue<MG, KC_D>(wgu, W.wgu, d, b * cg, cg, wave, lane);
        // O projection
        seg_bar();
        w_dot<1, KC_D>(wo, sh, d, 1.0f, co, wave, lane);
        seg_bar();
        w_issue<1, KC_F>(wd, W.wd, F, b * co, co, wave, lane);
        // gate / up
        seg_bar();
        inv = 1.0f / sqrtf((sh.ss[0] + sh.ss[1]) / (float)d + a.eps);
        w_dot<MG, KC_D>(wgu, sh, d, inv, cg, wave, lane);
        seg_bar();
        // (after the last layer: ncols 0 loads column 0 again, never used)
        const bool more = li + 1 < a.nl;
        w_issue<MQ, KC_D>(wq, a.lw[more ? li + 1 : li].wqkv, d, b * cq, more ? cq : 0, wave, lane);
        // down
        seg_bar();
        w_dot<1, KC_F>(wd, sh, F, 1.0f, co, wave, lane);
        seg_bar();
        kv_issue(kp, vp, a, more ? l + 1 : l, t, t.lo, more, wave, lane);
    }
}

__device__ void seg_control(const SegArgs& a, SegShared& sh, int wc, int lane) {
    const int b = blockIdx.x, NB = gridDim.x;
    const LayerDims& D = a.D;
    const int d = D.d, F = D.F, hd = SEG_HD, half = SEG_HD / 2;
    const int cq = 3 * d / NB, co = d / NB, cg = 2 * F / NB;
    const AttItem t = att_item(a);
    const unsigned long long spin = a.spin_ticks;
    const int dd = wc * 64 + lane;   // head dimension this lane handles in the attention merges
    for (int li = 0; li < a.nl; ++li) {
        const int l = a.l0 + li;
        const SegLayerW& W = a.lw[li];
        const uint32_t ep = a.epoch + (uint32_t)(SEG_PHASES * li);
        // ---- QKV: stage the layer input times the attention norm weight
        if (li == 0) {
            stage_plain<NJ_D>(a.Hs + a.hrow * d, d, W.attn_norm, wc, lane, sh);
            if (wc == 0 && lane < co) sh.xres[lane] = a.Hs[a.hrow * d + b * co + lane];
        } else {
            stage_tagged<NJ_D>(a.tx0, d, ep - SEG_PHASES + PH_X0, co, W.attn_norm, wc, lane, spin, sh, a.err);
        }
        seg_bar();
        seg_bar();
        // epilogue: column pair (2t, 2t+1) of the block = rotation partners
        for (int tp = wc * 64 + lane; tp < cq / 2; tp += 128) {
            const float v0 = sh.dots[2 * tp], v1 = sh.dots[2 * tp + 1];
            const int p = (b * cq) / 2 + tp;
            const int part = p / (d / 2);
            const int pp = p - part * (d / 2);
            const int h = pp / half, j = pp - h * half;
            if (part == 2) {
                const uint16_t b0 = f2bf(v0), b1 = f2bf(v1);
                uint16_t* vc = (uint16_t*)a.kv + kv_base(D, a.seq, l, 1, h) + (int64_t)a.pos * hd;
                vc[j] = b0;
                vc[j + half] = b1;
                tstore(a.tv + h * hd + j, ep + PH_QKV, __uint_as_float((uint32_t)b0 << 16));
                tstore(a.tv + h * hd + j + half, ep + PH_QKV, __uint_as_float((uint32_t)b1 << 16));
            } else {
                const float c = a.rope[((int64_t)a.pos * half + j) * 2], s = a.rope[((int64_t)a.pos * half + j) * 2 + 1];
                const float r0 = v0 * c - v1 * s, r1 = v1 * c + v0 * s;
                if (part == 0) {
                    tstore(a.tq + h * hd + j, ep + PH_QKV, r0);
                    tstore(a.tq + h * hd + j + half, ep + PH_QKV, r1);
                } else {
                    const uint16_t b0 = f2bf(r0), b1 = f2bf(r1);
                    uint16_t* kc = (uint16_t*)a.kv + kv_base(D, a.seq, l, 0, h) + (int64_t)a.pos * hd;
                    kc[j] = b0;
                    kc[j + half] = b1;
                    tstore(a.tk + h * hd + j, ep + PH_QKV, __uint_as_float((uint32_t)b0 << 16));
                    tstore(a.tk + h * hd + j + half, ep + PH_QKV, __uint_as_float((uint32_t)b1 << 16));
                }
            }
        }
        // ---- attention: stage q (and the current key / value when this split holds them)
        if (t.on) {
            stage_head(a.tq + t.h * hd, ep + PH_QKV, sh.qs, wc, lane, spin, sh, a.err);
            if (t.has_new) {
                stage_head(a.tk + t.h * hd, ep + PH_QKV, sh.kn, wc, lane, spin, sh, a.err);
                stage_head(a.tv + t.h * hd, ep + PH_QKV, sh.vn, wc, lane, spin, sh, a.err);
            }
        }
        seg_bar();
        seg_bar();
        if (t.on) {
            // the block's partial state over its keys (lane: head dimension dd), merged over
            // the 4 lane groups of each streaming wave
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < SEG_NS * 4; ++w) M = fmaxf(M, sh.wm[w]);
            float L = 0.f, O = 0.f;
#pragma unroll
            for (int w = 0; w < SEG_NS * 4; ++w) {
                const float mw = sh.wm[w];
                const float c = mw == -INFINITY ? 0.f : expf(mw - M);
                L = fmaf(c, sh.wl[w], L);
                O = fmaf(c, sh.wo[w][dd], O);
            }
            uint64_t* pt = a.tpart + ((int64_t)t.h * SEG_SMAX + t.s) * (2 + hd);
            tstore(pt + 2 + dd, ep + PH_PART, O);
            if (lane == 0) {
                tstore(pt, ep + PH_PART, M);
                tstore(pt + 1, ep + PH_PART, L);
            }
            if (t.s == 0 && !sh.bad) {
                // split 0 of each head merges the head's S partials (dimension dd)
                const uint64_t* ph = a.tpart + (int64_t)t.h * SEG_SMAX * (2 + hd);
                const uint32_t e2 = ep + PH_PART;
                const unsigned long long t_end = (unsigned long long)wall_clock64() + spin;
                const __amdgpu_buffer_rsrc_t r = coh_rsrc(ph);
                constexpr int SPLIT_BYTES = (2 + SEG_HD) * 8;
                uint64_t ml[2], ov[SEG_SMAX];
                for (;;) {
                    ml[0] = lane < a.S ? tload_b(r, lane * SPLIT_BYTES, 0) : tagv(e2, -INFINITY);
                    ml[1] = lane < a.S ? tload_b(r, lane * SPLIT_BYTES, 8) : tagv(e2, 0.f);
#pragma unroll
                    for (int s = 0; s < SEG_SMAX; ++s)
                        ov[s] = s < a.S ? tload_b(r, (2 + dd) * 8, s * SPLIT_BYTES) : tagv(e2, 0.f);
                    bool ok = (uint32_t)(ml[0] >> 32) == e2 && (uint32_t)(ml[1] >> 32) == e2;
#pragma unroll
                    for (int s = 0; s < SEG_SMAX; ++s) ok = ok && (uint32_t)(ov[s] >> 32) == e2;
                    if (__all(ok)) break;
                    if (timed_out(t_end)) {
                        give_up(sh, a.err);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                // lane s < S holds split s's (max, sum); split s weighs exp(m_s - Mt)
                const float ms = __uint_as_float((uint32_t)ml[0]), ls = __uint_as_float((uint32_t)ml[1]);
                const float Mt = wave_max(lane < a.S ? ms : -INFINITY);
                const float cs = (lane < a.S && ms != -INFINITY) ? expf(ms - Mt) : 0.f;
                const float Lt = wave_total(cs * ls);
                float Ot = 0.f;
#pragma unroll
                for (int s = 0; s < SEG_SMAX; ++s) Ot = fmaf(__shfl(cs, s, 64), __uint_as_float((uint32_t)ov[s]), Ot);
                tstore(a.tatt + t.h * hd + dd, ep + PH_ATT, Ot / Lt);
            }
        }
        // ---- O projection: stage the attention output (no norm)
        stage_tagged<NJ_D>(a.tatt, d, ep + PH_ATT, 64, nullptr, wc, lane, spin, sh, a.err);
        seg_bar();
        seg_bar();
        if (wc == 0 && lane < co) {
            const float x1 = sh.xres[lane] + sh.dots[lane];
            tstore(a.tx1 + b * co + lane, ep + PH_X1, x1);
            sh.x1own[lane] = x1;
        }
        // ---- gate / up: stage x1 times the MLP norm weight
        stage_tagged<NJ_D>(a.tx1, d, ep + PH_X1, co, W.mlp_norm, wc, lane, spin, sh, a.err);
        seg_bar();
        seg_bar();
        for (int tp = wc * 64 + lane; tp < cg / 2; tp += 128) {
            const float g = sh.dots[2 * tp], u = sh.dots[2 * tp + 1];
            tstore(a.tact + b * (cg / 2) + tp, ep + PH_ACT, g / (1.0f + expf(-g)) * u);
        }
        // ---- down: stage the SwiGLU output
        stage_tagged<NJ_F>(a.tact, F, ep + PH_ACT, cg / 2, nullptr, wc, lane, spin, sh, a.err);
        seg_bar();
        seg_bar();
        if (wc == 0 && lane < co) {
            const float x0 = sh.x1own[lane] + sh.dots[lane];
            tstore(a.tx0 + b * co + lane, ep + PH_X0, x0);
            sh.xres[lane] = x0;
            if (li + 1 == a.nl) a.Hs[a.hrow * d + b * co + lane] = x0;
        }
    }
}

__global__ __launch_bounds__(SEG_THREADS, 1) void k_segment(SegArgs a) {
    __shared__ SegShared sh;
    const unsigned long long t0 = stamp_begin(a.stamp);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (threadIdx.x == 0) sh.bad = 0;
    __syncthreads();
    if (wave < SEG_NS)
        seg_streamer(a, sh, wave, lane);
    else
        seg_control(a, sh, wave - SEG_NS, lane);
    stamp_end(a.stamp, t0);
}

}  // namespace

int segment_blocks(const LayerDims& D, int n_cu) {
    if (D.kv_bf16 != 1 || D.hd != SEG_HD || D.d % 256 != 0 || D.d > SEG_DMAX || D.F % 256 != 0 || D.F > SEG_FMAX)
        return 0;
    for (int nb = n_cu; nb >= 1; --nb) {
        if (D.d % nb || (D.d / nb) % 2 || D.d / nb > SEG_OCOLS) continue;
        if ((3 * D.d) % nb || (3 * D.d / nb) % 2 || 3 * D.d / nb > SEG_QCOLS) continue;
        if ((2 * D.F) % nb || (2 * D.F / nb) % 2 || 2 * D.F / nb > SEG_GCOLS) continue;
        if (D.H > nb) continue;
        return nb;
    }
    return 0;
}

hipError_t launch_segment(const SegArgs& a, int blocks, hipStream_t st) {
    if (blocks < 1 || blocks > STAMP_BLOCKS || a.S < 1 || a.S > SEG_SMAX || a.D.H * a.S > blocks || a.nl < 1 ||
        a.nl > SEG_LMAX ||
        a.pos < 0 || a.pos >= a.D.max_ctx || segment_blocks(a.D, blocks) != blocks)
        return hipErrorInvalidValue;
    SegArgs b = a;
    b.stamp = current_launch_stamp();
    hipEvent_t e0 = nullptr, e1 = nullptr;
    current_launch_events(&e0, &e1);
    if (e0) {
        hipError_t e = hipEventRecord(e0, st);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&b};
    note_launch_blocks(blocks);
    hipError_t e = hipLaunchCooperativeKernel((const void*)k_segment, dim3(blocks), dim3(SEG_THREADS), args, 0, st);
    if (e != hipSuccess) return e;
    if (e1) e = hipEventRecord(e1, st);
    return e;
}

}  // namespace nv
