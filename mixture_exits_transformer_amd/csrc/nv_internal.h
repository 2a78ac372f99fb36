// Internal declarations shared by the kernels and the host runtime of libnvium.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nv {

struct RowInfo;

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };

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
    float* out;
    int64_t ldo;
    const struct RowInfo* o_rows;  // row i of out is out + o_rows[i].hrow * ldo (identity if null)
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
    int row0, nrows, head, lo, hi, part, pad0, pad1;
};

// Where the split partials of compact row i live: slot(h, s) =
// base + (h * nsplit + s) * nrows + off.
struct CombineInfo {
    int base, off, nsplit, nrows;
};

struct LayerDims {
    int L, d, H, hd, F, V, max_ctx, kv_bf16;
};

// Launch wrappers (nv_kernels.hip).
hipError_t launch_rope_table(float* cs, int max_ctx, int hd, float base, hipStream_t st);
hipError_t launch_embed(const int* tokens, const RowInfo* rows, int n, const void* E, int wbf16,
                        float* Hs, int d, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
hipError_t launch_rope_kv(float* qkv, const RowInfo* rows, int R, void* kv, int layer,
                          const LayerDims& D, const float* cs, hipStream_t st);
hipError_t launch_attn(const AttnItem* items, int n_items, const RowInfo* rows, const float* qkv,
                       const void* kv, int layer, const LayerDims& D, float* part_ml,
                       float* part_o, hipStream_t st);
hipError_t launch_attn_combine(const CombineInfo* ci, int R, const LayerDims& D,
                               const float* part_ml, const float* part_o, float* out,
                               hipStream_t st);
hipError_t launch_gate(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d,
                       const float* gw, float bias, const float* uniforms, int ucol,
                       double* w_out, int* stop_out, hipStream_t st);
hipError_t launch_sample(const float* logits, int64_t ld, const int* seqs, int n, int V,
                         const float* uniforms, int* tok_out, hipStream_t st);
hipError_t init_kernel_attributes();

}  // namespace nv
