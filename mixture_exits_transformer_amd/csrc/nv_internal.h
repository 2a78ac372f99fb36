// Internal declarations shared by the kernels and the host runtime of libnvium.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nv {

struct RowInfo;
struct CombineInfo;

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3 };

struct LayerDims {
    int L, d, H, hd, F, V, max_ctx, kv_bf16;
};

// out[i][n] (+)= sum_k A'[i][k] * W[n][k], where A' is row i of A, RMSNormed when
// norm_w is set.  Rows of A and of out are addressed through optional index lists
// so that hidden states of several sequences can be used in place.
struct GemmArgs {
    const float* A;       // fp32 rows
    int64_t lda;
    const struct RowInfo* a_rows;  // row i of A is A + a_rows[i].hrow * lda (identity if null)
    const float* norm_w;  // RMSNorm weight (length K) or null
    float eps;
    const void* W;        // [N][K], fp32 or bf16 (wbf16)
    int N, K, R;
    int wbf16;
    int epi;              // EPI_STORE: out = acc; EPI_RESID: out += acc;
                          // EPI_SWIGLU: columns (2j, 2j+1) = (gate_j, up_j), out[j] = silu(g) * u
                          // EPI_QKV: columns (2p, 2p+1) are rotation partners (see below):
                          //   q -> RoPE -> q_out[row]; k -> RoPE -> KV cache; v -> KV cache
    float* out;
    int64_t ldo;
    const struct RowInfo* o_rows;  // row i of out is out + o_rows[i].hrow * ldo (identity if null)
    int head;             // 1: an exit head (separate kernel symbol, so profiles tell them apart)
    float* rms_ws;        // [R] scratch for per-row inverse RMS (matrix-core path with norm_w)
    int mfma_min_rows;    // use the matrix-core path when R >= this (0: never)
    // EPI_QKV only.  Weight row 2p + i (i = 0, 1) of the fused QKV matrix is original
    // row part*d + h*hd + j + i*hd/2, where p = part*(d/2) + h*(hd/2) + j, part 0/1/2 = q/k/v.
    float* q_out;         // [R][d]
    void* kv;
    const float* rope;    // [max_ctx][hd/2] (cos, sin)
    int layer;
    LayerDims D;
    // Timing only: when set, block b stores its start and end (device wall-clock ticks) at
    // stamp[2b] and stamp[2b + 1] (vector-ALU and matrix-core decode kernels).
    unsigned long long* stamp;
    // Single-row attention output merged on the fly (vector-ALU path, R == 1): when set,
    // the activation row is the merge of the split partials described by comb[0]
    // (rows whose key range was not split are read from A).
    const struct CombineInfo* comb;
    const float* part_ml;
    const float* part_o;
};

// One row of a chunk: position `pos` of sequence `seq`; hrow = seq * max_ctx + pos
// indexes the hidden-state array.
struct RowInfo {
    int hrow, seq, pos, pad;
};

// Attention work item: rows row0..row0+nrows-1 of the compact row list (consecutive
// positions of one sequence) against keys/values at positions [lo, hi) of head `head`.
// Partial results go to slots part + r (r < nrows).
struct AttnItem {
    int row0, nrows, head, lo, hi, part;
    int split, nsplit;    // split index and count over the key range of (row block, head)
    int pad[4];
};

// Where the split partials of compact row i live: slot(h, s) =
// base + (h * nsplit + s) * nrows + off.
struct CombineInfo {
    int base, off, nsplit, nrows;
};

// Launch wrappers (nv_kernels.hip).
hipError_t launch_rope_table(float* cs, int max_ctx, int hd, float base, hipStream_t st);
hipError_t launch_embed(const int* tokens, const RowInfo* rows, int n, const void* E, int wbf16,
                        float* Hs, int d, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
// Decode-sized row blocks (<= ATTN_DEC_ROWS rows): each item is one split of one
// (row block, head); split partials are merged by launch_attn_combine.
constexpr int ATTN_DEC_ROWS = 8;
constexpr int ATTN_DEC_ITERS = 4;
constexpr int ATTN_COMB_MAX = 4096;      // splits of one (row, head) the combine pass holds   // key groups per wave: a split covers <= 16 * (512 / head_dim) keys
hipError_t launch_attn_dec(const AttnItem* items, int n_items, int max_rows, const RowInfo* rows, const float* q,
                           const void* kv, int layer, const LayerDims& D, float* part_ml, float* part_o,
                           float* out, hipStream_t st);
hipError_t launch_attn(const AttnItem* items, int n_items, const RowInfo* rows, const float* q,
                       const void* kv, int layer, const LayerDims& D, float* part_ml,
                       float* part_o, float* out, hipStream_t st);
hipError_t launch_attn_combine(const CombineInfo* ci, int R, const LayerDims& D,
                               const float* part_ml, const float* part_o, float* out,
                               hipStream_t st);
hipError_t launch_gate(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d,
                       const float* gw, float bias, const float* uniforms, int ucol,
                       double* w_out, int* stop_out, hipStream_t st);
hipError_t launch_sample(const float* logits, int64_t ld, const int* seqs, int n, int V,
                         const float* uniforms, int* tok_out, hipStream_t st);
hipError_t init_kernel_attributes();
// Timing: the next launch stamps `start` at its start; every launch stamps `stop` at its
// end, until cleared with (nullptr, nullptr).
void set_launch_events(hipEvent_t start, hipEvent_t stop);
const char* last_launch_name();   // symbol of the last kernel issued while timing
// Timing: block-stamp buffer the next stamped kernels write (nullptr: none).
void set_launch_stamp(unsigned long long* stamps);
constexpr int STAMP_BLOCKS = 8192;  // largest grid the timing stamps cover
hipError_t launch_stamp_reduce(unsigned long long* stamps, int n, unsigned long long* rec, hipStream_t st);

}  // namespace nv
