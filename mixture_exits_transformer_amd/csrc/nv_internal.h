// Internal declarations shared by the kernels and the host runtime of libnvium.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nv {

struct RowInfo;

// Where the split partials of compact row i live: slot(h, s) =
// base + (h * nsplit + s) * nrows + off.
struct CombineInfo {
    int base, off, nsplit, nrows;
};

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3, EPI_SILU = 4 };

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
    int epi;              // EPI_STORE: out = acc; EPI_RESID: out += acc; EPI_SILU: out = silu(acc);
                          // EPI_SWIGLU: columns (2j, 2j+1) = (gate_j, up_j), out[j] = silu(g) * u
                          // EPI_QKV: columns (2p, 2p+1) are rotation partners (see below):
                          //   q -> RoPE -> q_out[row]; k -> RoPE -> KV cache; v -> KV cache
    float* out;
    int64_t ldo;
    const struct RowInfo* o_rows;  // row i of out is out + o_rows[i].hrow * ldo (identity if null)
    int head;             // 1: an exit head (separate kernel symbol, so profiles tell them apart)
    float* rms_ws;        // [R] scratch for per-row inverse RMS (matrix-core path with norm_w)
    uint16_t* abf;        // [R][K] bf16 scratch: the rows, normalised and rounded once (long chunks), or null
    int abf_ready;        // abf already holds this product's rows (launch_rows_bf16 ran, or the
                          // producing epilogue wrote them)
    uint16_t* out_bf16;   // EPI_SWIGLU only, or null: silu(g) * u goes here as bf16 [R][ldo],
                          // rounded as launch_rows_bf16 would round it, instead of to out
    int mfma_min_rows;    // use the matrix-core path when R >= this (0: never)
    // Rows of one contiguous chunk (vector-ALU decode kernel only): when `contig` is set, row r
    // is position pos0 + r of sequence seq0, its row of A is a_row0 + r (when a_rows is set;
    // else r) and its row of out is o_row0 + r (when o_rows is set; else r).  The kernel then
    // computes every address without loading the row tables, issues all its weight loads
    // before any wait, and fetches the epilogue's inputs (RoPE table entries, residual
    // values) right after them.
    int contig, a_row0, o_row0, seq0, pos0;
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
    int comb_ns;          // with contig and comb_ns > 0: comb[0] = {0, 0, comb_ns, 1}, by value
    // Exit heads of the mixture objective on the long-chunk path (k_gemm_bf16 only): when
    // xent_part is set, the logits are not stored.  Each block writes, per row and per
    // 64-column group g, (max, sum of exp(z - max)) at xent_part[2 (row * N/64 + g)], and
    // the block holding a row's target column writes that logit to xent_tgt[row];
    // launch_xent_merge then forms the log-probabilities.
    float* xent_part;     // [R][N/64][2]
    float* xent_tgt;      // [R]
    const int* xent_targets;   // [R] target token ids in [0, N)
    // Exit head with the softmax partials (head == 2, one row, vector-ALU decode GEMV): block b
    // also writes the (max, sum of exp(z - max)) of its KS_CPB logits to xd_part[2b], [2b+1];
    // launch_exit_draw then draws the token from them without re-reading every logit.
    float* xd_part;       // [N / 8][2]
    // Decode-sized row groups on the matrix cores with K split across blocks (non-head
    // products, sk_min_rows <= R <= sk_max_rows, K a multiple of SK_KC): each K slice's
    // fp32 partial tile goes to sk_ws ([K/SK_KC][R][N], then the per-slice sums of squares
    // [K/SK_KC][R] for RMSNorm), and a second kernel adds the slices in order and applies
    // the epilogue.  sk_cap is sk_ws's size in floats; sk_min_rows 0 turns the path off.
    float* sk_ws;
    int64_t sk_cap;
    int sk_min_rows, sk_max_rows;
    int sk_ntb;           // 16-column tiles per block: bits 0-3 with RMSNorm, bits 4-7 without (1 or 2)
};

// K slice of one block of the split-K decode product (k_gemm_sk).
constexpr int SK_KC = 512;
constexpr int SK_MAX_ROWS = 64;

// The exit draw: one block of XD_THREADS threads merges the head product's per-block
// partials; a thread holds at most XD_PER of them (N / 8 <= XD_PER * XD_THREADS).
constexpr int XD_THREADS = 512;
constexpr int XD_PER = 16;
// token[0] = inverse-CDF draw with u from softmax(logits[0..V)), V = 8 * nb, from the
// partials `part` [nb][2] the head product wrote beside the logits.
hipError_t launch_exit_draw(const float* part, int nb, const float* logits, float u, int* token, hipStream_t st);

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
    int seq;              // the rows' sequence (spares the kernels a dependent row-table load)
    int pad[3];
};


// A decode group of one contiguous chunk of at most ATTN_DEC_ROWS rows (one row block):
// everything its attention items, split-combine records and row table would hold, passed by
// value so that no kernel starts with a dependent table load.  Block b of the attention
// launch is split s = b % nsplit of head b / nsplit over keys [s * per, min(ctx, (s+1) * per)),
// ctx = pos0 + nrows; its partial state for row r goes to slot (b * nrows + r).
struct DecGeom {
    int on;          // 0: read the uploaded tables instead
    int seq, pos0, nrows, nsplit, per;
};

__host__ __device__ inline AttnItem dec_item(const DecGeom& g, int b) {
    AttnItem it{};
    const int h = b / g.nsplit, s = b - h * g.nsplit;
    const int ctx = g.pos0 + g.nrows;
    it.row0 = 0;
    it.nrows = g.nrows;
    it.head = h;
    it.lo = s * g.per;
    it.hi = ctx < it.lo + g.per ? ctx : it.lo + g.per;
    it.part = b * g.nrows;
    it.split = s;
    it.nsplit = g.nsplit;
    it.seq = g.seq;
    return it;
}

__host__ __device__ inline CombineInfo dec_comb(const DecGeom& g, int row) {
    return CombineInfo{0, row, g.nsplit, g.nrows};
}

// Launch wrappers (nv_kernels.hip).
hipError_t launch_rope_table(float* cs, int max_ctx, int hd, float base, hipStream_t st);
// Hs row rows[i].hrow = embedding of tokens[i] (by_seq: of tokens[rows[i].seq]).
hipError_t launch_embed(const int* tokens, const RowInfo* rows, int n, const void* E, int wbf16,
                        float* Hs, int d, hipStream_t st, int by_seq = 0);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
// Long chunks on bf16 weights take the bf16-row path: k_rows_bf16 writes the rows of A
// (normalised when norm_w is set) to abf, then k_gemm_bf16 runs on them.  With
// launch_rows_bf16 first and abf_ready set, launch_gemm runs only the product.
bool gemm_uses_bf16_rows(const GemmArgs& a);
// K slices of the split-K decode product when `a` takes it, else 0.
int sk_slices(const GemmArgs& a);
hipError_t launch_rows_bf16(const GemmArgs& a, hipStream_t st);
// Decode-sized row blocks (<= ATTN_DEC_ROWS rows): each item is one split of one
// (row block, head); split partials are merged by launch_attn_combine.
constexpr int ATTN_DEC_ROWS = 8;
// Decode groups whose row blocks reach this many rows run on the matrix-core attention
// (one wave per item); one- to three-row blocks stay on the vector-ALU decode kernel.
// At an 8K context a 4- to 8-row block costs 24-41 us per layer there, about 30 on the
// matrix cores; at one row the vector kernel is as fast.
constexpr int ATTN_DEC_MFMA_ROWS = 4;
static_assert(ATTN_DEC_ROWS <= 16, "a decode row block fits one 16-row wave of the matrix-core attention");
// key groups per wave: a split covers at most 4 waves x (512 / head_dim) keys x 8 groups
// (128 keys at head_dim 128; 8 groups measured better than 4 at batch 1, 16 and an 8K
// context: fewer, longer splits with more loads in flight per wave)
constexpr int ATTN_DEC_ITERS = 8;
constexpr int ATTN_COMB_MAX = 4096;      // splits of one (row, head) the combine pass holds
// Long contexts (row blocks of at most ATTN_DEC_WIDE_ROWS rows, some context past
// ATTN_DEC_WIDE_MIN_KEYS keys, bf16 K/V): blocks of ATTN_DEC_WIDE_WAVES waves, a split covering
// up to 16 x ATTN_DEC_WIDE_ITERS x (64 / (head_dim / 8)) keys (576 at head_dim 128), one block
// per CU on about 3/4 of the CUs.  An 8K context then takes 15-16 splits per head at 12 heads
// instead of 65, so the one-row O product merges them as it loads (no combine launch), in two
// batches of 8 (512-key splits made 17 past 8192 keys, and a third batch)
constexpr int ATTN_DEC_WIDE_WAVES = 16;
constexpr int ATTN_DEC_WIDE_ITERS = 9;
constexpr int ATTN_DEC_WIDE_ROWS = 2;
constexpr int ATTN_DEC_WIDE_MIN_KEYS = 4096;
// wide: use the ATTN_DEC_WIDE_WAVES-wave blocks (bf16 K/V, max_rows <= ATTN_DEC_WIDE_ROWS)
hipError_t launch_attn_dec(const AttnItem* items, int n_items, int max_rows, const RowInfo* rows, const float* q,
                           const void* kv, int layer, const LayerDims& D, float* part_ml, float* part_o,
                           float* out, hipStream_t st, const DecGeom& dg = DecGeom{}, int wide = 0);
// Matrix-core variant of launch_attn for a bf16 KV cache and head_dim 32, 64 or 128:
// items of up to 64 rows, key ranges starting at multiples of 64.
bool attn_mfma_ok(const LayerDims& D);
// Rows per item of the matrix-core chunk attention: one wave per 16 rows (4 or 8 waves).
constexpr int ATTN_MFMA_ROWS = 128;
hipError_t launch_attn_mfma(const AttnItem* items, int n_items, const RowInfo* rows, const float* q, const void* kv,
                            int layer, const LayerDims& D, float* part_ml, float* part_o, float* out, hipStream_t st);
// Decode groups on the matrix cores: one wave per item (at most 16 rows), used for groups
// whose row blocks reach ATTN_DEC_MFMA_ROWS rows.
hipError_t launch_attn_mfma16(const AttnItem* items, int n_items, const RowInfo* rows, const float* q,
                              const void* kv, int layer, const LayerDims& D, float* part_ml, float* part_o,
                              float* out, hipStream_t st, const DecGeom& dg = DecGeom{});
hipError_t launch_attn(const AttnItem* items, int n_items, const RowInfo* rows, const float* q,
                       const void* kv, int layer, const LayerDims& D, float* part_ml,
                       float* part_o, float* out, hipStream_t st);
hipError_t launch_attn_combine(const CombineInfo* ci, int R, const LayerDims& D,
                               const float* part_ml, const float* part_o, float* out,
                               hipStream_t st, const DecGeom& dg = DecGeom{});
// The combine for a product on bf16 rows: every (row, head) of the attention output goes
// to out_bf16 [R][d] as bf16 (split rows merged, the others converted from out).
hipError_t launch_attn_combine_bf16(const CombineInfo* ci, int R, const LayerDims& D, const float* part_ml,
                                    const float* part_o, const float* attn_o, uint16_t* out_bf16, hipStream_t st);
// Gates write w_out[seqs[i] * 4 + ucol]; with uniforms null they take no stop decision.
// With host_flags set (device address of mapped, coherent host memory), each decision is
// also stored there as host_flags[seq] = tag * 2 + stop, so the host can wait for it
// without a copy or a stream synchronisation.
hipError_t launch_gate(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d,
                       const float* gw, float bias, const float* uniforms, int ucol,
                       double* w_out, int* stop_out, hipStream_t st, int* host_flags = nullptr, int tag = 0);
hipError_t launch_sample(const float* logits, int64_t ld, const int* seqs, int n, int V,
                         const float* uniforms, int* tok_out, hipStream_t st);
// Router MLP gate: w = sigmoid(w2 . silu(W1 h + b1) + bias) in float64 (W1 [rr][d]);
// hid: [n][rr] float64 scratch for the hidden units.
hipError_t launch_gate_mlp(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d, const float* w1,
                           const float* b1, const float* w2, int rr, float bias, const float* uniforms, int ucol,
                           double* hid, double* w_out, int* stop_out, hipStream_t st, int* host_flags = nullptr,
                           int tag = 0);
// dst row i = Hs row rows[i].hrow (d floats each).
hipError_t launch_copy_rows(const RowInfo* rows, int n, const float* Hs, int d, float* dst, hipStream_t st);
// out[i * ostride + ocol] = log softmax(logits row i)[targets[i]] (float64).
// Log-probability of each row's target from the per-group partials of a fused head
// product (GemmArgs::xent_part): out[i * ostride + ocol] = z_y - M - log sum_g s_g e^(m_g - M).
hipError_t launch_xent_merge(const float* part, const float* tgt, int n, int ngroups, double* out, int ostride,
                             int ocol, hipStream_t st);
hipError_t launch_xent(const float* logits, int64_t ld, int n, int V, const int* targets, double* out, int ostride,
                       int ocol, hipStream_t st);
// Exit layers l_k and the layer count L, for the expected depth sum_k p_k l_k / L.
struct ExitDepths {
    int layer[4];
    int L;
};
// Rows i < n of w and lp are [n][4] (router outputs, log pi_k of the target); writes
// w[i][3] = 1, the per-row mixture NLL and expected depth, and their means to sums[0..1].
hipError_t launch_loss_reduce(double* w, const double* lp, int n, ExitDepths dep, double* nll, double* depth,
                              double* sums, hipStream_t st);
hipError_t init_kernel_attributes();
// Timing: the next launch stamps `start` at its start; every launch stamps `stop` at its
// end, until cleared with (nullptr, nullptr).
void set_launch_events(hipEvent_t start, hipEvent_t stop);
const char* last_launch_name();   // symbol of the last kernel issued while timing
int take_launch_blocks();          // most blocks of a launch since the last call (then 0)
void note_launch_blocks(int n);    // a launch issued outside the wrappers' macro had n blocks
// Timing: block-stamp buffer the next stamped kernels write (nullptr: none).
void set_launch_stamp(unsigned long long* stamps);
constexpr int STAMP_BLOCKS = 65536;  // largest grid the timing stamps cover
unsigned long long* current_launch_stamp();
void current_launch_events(hipEvent_t* start, hipEvent_t* stop);

// ------------------------------------------------------------------------------------------
// Persistent segment kernel (nv_segment.hip): every layer of one segment for a single
// decode row in one cooperative launch.  Blocks exchange activations through buffers of
// tagged values (high 32 bits: epoch of the write, low 32 bits: the fp32 value) that
// consumers poll; see nv_segment.hip for the roles of the waves.
// ------------------------------------------------------------------------------------------
constexpr int SEG_THREADS = 512;    // 6 streaming waves + 2 control waves
constexpr int SEG_NS = 6;           // streaming waves per block
constexpr int SEG_DMAX = 1536;      // largest model width
constexpr int SEG_FMAX = 4096;      // largest MLP width
constexpr int SEG_HD = 128;         // head dimension
constexpr int SEG_SMAX = 32;        // most key splits per head
constexpr int SEG_QCOLS = 18;       // most QKV columns per block (3 per streaming wave)
constexpr int SEG_OCOLS = 6;        // most O / down columns per block (1 per streaming wave)
constexpr int SEG_GCOLS = 36;       // most gate/up columns per block (6 per streaming wave)
constexpr int SEG_PHASES = 8;       // epoch stride per layer
constexpr int SEG_LMAX = 16;        // most layers per segment

struct SegLayerW {
    const float* attn_norm;
    const uint16_t* wqkv;   // [3d][d], RoPE partners in adjacent rows (see GemmArgs)
    const uint16_t* wo;     // [d][d]
    const float* mlp_norm;
    const uint16_t* wgu;    // [2F][d], rows 2j / 2j+1 = gate j / up j
    const uint16_t* wd;     // [d][F]
};

struct SegArgs {
    SegLayerW lw[SEG_LMAX]; // weights of layers l0 .. l0 + nl - 1 (kernel arguments are read
                            // through the scalar cache, away from the vector loads in flight)
    int l0, nl;
    LayerDims D;
    float eps;
    float* Hs;              // hidden-state rows; row `hrow` is read at l0 and written after the last layer
    int64_t hrow;
    int seq, pos;           // the row: position `pos` of sequence `seq`
    void* kv;               // bf16 KV cache
    const float* rope;      // [max_ctx][hd/2] (cos, sin)
    uint64_t* tx0;          // [d]  layer input (written by the down projection)
    uint64_t* tq;           // [d]  rotated query
    uint64_t* tk;           // [d]  rotated key of `pos`, bf16-rounded
    uint64_t* tv;           // [d]  value of `pos`, bf16-rounded
    uint64_t* tpart;        // [H][SEG_SMAX][2 + hd] split partials (max, sum, output); split 0
                            // of each head merges them
    uint64_t* tatt;         // [d]  attention output
    uint64_t* tx1;          // [d]  after the attention residual
    uint64_t* tact;         // [F]  SwiGLU output
    uint32_t* err;          // set to 1 when a wait gave up
    uint32_t epoch;         // tags of this launch: epoch + SEG_PHASES * (l - l0) + phase
    int S;                  // key splits per head
    unsigned long long spin_ticks;   // a wait gives up after this many wall-clock ticks
    unsigned long long* stamp;       // timing stamps (or null)
};

// Grid size for the model's shape (0: the shape does not fit the kernel).
int segment_blocks(const LayerDims& D, int n_cu);
hipError_t launch_segment(const SegArgs& a, int blocks, hipStream_t st);
hipError_t launch_stamp_reduce(unsigned long long* stamps, int n, unsigned long long* rec, hipStream_t st);

}  // namespace nv
