// Host runtime of libnvium: the C ABI declared in include/nvium.h.
//
// Scheduling follows section 2, part "Inferenz: Piggybacking" of the gist.science
// technical summary of N-vium: a token that exits at node k leaves its layers above
// that exit pending; when a later token of the same sequence reaches those depths the
// pending hidden states are concatenated with the current one and run as one causal
// chunk.  Per sequence the runtime keeps one frontier per segment (every position below
// frontier[s] has completed segment s) and one hidden-state row per position (the output
// of the last segment that position completed), so the chunk of segment s at position p
// is the contiguous range [frontier[s], p] and runs in place.
#include "nv_internal.h"
#include "nvium.h"

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

using namespace nv;

namespace {

constexpr int kMaxExits = 4;
constexpr int kAttnRowsPerItem = 32;
constexpr int kDecodeRows = 64;          // launch groups up to this many rows use decode attention
constexpr int kAttnBlocksTarget = 512;   // decode attention: aim for about this many blocks
constexpr size_t kAlign = 256;

struct LayerPtrs {
    float* attn_norm;
    void* wqkv;   // [3d][d]: rows of W_q, then W_k, then W_v
    void* wo;     // [d][d]
    float* mlp_norm;
    void* wgu;    // [2F][d]: row 2j = W_gate row j, row 2j+1 = W_up row j
    void* wd;     // [d][F]
};

struct ExitPtrs {
    float* gate_w;          // linear router: [d]
    float* router_w1;       // router MLP: [rr][d], [rr], [rr]
    float* router_b1;
    float* router_w2;
    float* norm;            // RMSNorm before the head (the shared final norm in the shared form)
    void* head;             // [V][d] (the shared head in the shared form)
    void* adapter_down;     // shared form, exits 1..3: [r][d]
    void* adapter_up;       // [d][r]
    float bias;
};

struct SeqHost {
    bool live = false;
    int n = 0;                 // positions consumed
    int f[kMaxExits] = {0, 0, 0, 0};
    int pending = 0;
    int last_exit = 0;
};

struct Chunk {
    int seq, pos0, nrows;
};

constexpr size_t kEventPairs = 8192;
constexpr int kRing = 4;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sizes of everything the model keeps in device memory.
struct Plan {
    size_t es = 0, kes = 0;
    size_t embed = 0, layer_w = 0, exit_w = 0, shared_head = 0;
    size_t hidden = 0, kv = 0, rope = 0;
    int R_max = 0, part_cap = 0, items_cap = 0;
    size_t qbuf = 0, attn_o = 0, mlp = 0, part_ml = 0, part_o = 0, rms = 0, abf = 0;
    size_t tables = 0, small = 0, logits = 0, router_hid = 0;
    size_t seg = 0;     // persistent segment kernel: tagged exchange buffers, counters, layer table
    size_t xd = 0;      // exit draw: the head product's per-block softmax partials
    int64_t sk_floats = 0;   // split-K decode products: slice partials and sums of squares
    int loss_ch = 0;    // mixture objective: rows per head pass
    size_t loss = 0;    // its logits, per-row router outputs / log-probabilities / losses, row tables
    size_t total = 0;
};

struct FileHeader {
    nv_config c;
};

bool read_header(const char* path, nv_config* c, std::string* err) {
    int fd = ::open(path, O_RDONLY);
    if (fd < 0) {
        *err = std::string("cannot open weights file: ") + path;
        return false;
    }
    unsigned char h[256];
    ssize_t got = ::pread(fd, h, sizeof(h), 0);
    ::close(fd);
    if (got != (ssize_t)sizeof(h) || std::memcmp(h, "NVIUMW01", 8) != 0) {
        *err = "weights file header missing or wrong magic";
        return false;
    }
    int32_t iv[9];
    std::memcpy(iv, h + 8, sizeof(iv));
    if (iv[0] != 256) {
        *err = "unsupported weights header size";
        return false;
    }
    c->n_layers = iv[1];
    c->d_model = iv[2];
    c->n_heads = iv[3];
    c->head_dim = iv[4];
    c->ffn = iv[5];
    c->vocab = iv[6];
    c->n_exits = iv[7];
    c->wdtype = iv[8];
    std::memcpy(&c->norm_eps, h + 44, 4);
    std::memcpy(&c->rope_base, h + 48, 4);
    std::memcpy(c->exit_layer, h + 52, 16);
    std::memcpy(c->gate_bias, h + 68, 16);
    int32_t forms[4];
    std::memcpy(forms, h + 84, 16);
    c->head_form = forms[0];
    c->adapter_dim = forms[1];
    c->router_form = forms[2];
    c->router_dim = forms[3];
    const int L = c->n_layers, d = c->d_model;
    bool ok = L > 0 && d > 0 && c->n_heads > 0 && c->head_dim > 0 && c->n_heads * c->head_dim == d &&
              c->ffn > 0 && c->vocab > 0 && c->n_exits == kMaxExits && (c->wdtype == 0 || c->wdtype == 1) &&
              L % kMaxExits == 0 && (c->head_dim == 32 || c->head_dim == 64 || c->head_dim == 128) &&
              d % 8 == 0 && c->ffn % 8 == 0 && c->vocab % 8 == 0 && c->vocab <= 32768;
    for (int k = 0; ok && k < kMaxExits; ++k) ok = c->exit_layer[k] == (k + 1) * (L / kMaxExits);
    ok = ok && (c->head_form == 0 || (c->head_form == 1 && c->adapter_dim > 0 && c->adapter_dim % 8 == 0 &&
                                     c->adapter_dim <= 4096));
    ok = ok && (c->head_form == 1 || c->adapter_dim == 0) && c->adapter_dim <= c->ffn;
    ok = ok && (c->router_form == 0 || (c->router_form == 1 && c->router_dim > 0 && c->router_dim <= 1024));
    ok = ok && (c->router_form == 1 || c->router_dim == 0);
    if (!ok) {
        *err = "weights header describes an unsupported shape";
        return false;
    }
    return true;
}

Plan make_plan(const nv_config& c, int max_batch, int max_ctx) {
    Plan p;
    const size_t L = c.n_layers, d = c.d_model, F = c.ffn, V = c.vocab, H = c.n_heads, hd = c.head_dim;
    p.es = c.wdtype == 1 ? 2 : 4;
    p.kes = p.es;
    p.embed = align_up(V * d * p.es);
    p.layer_w = align_up(d * 4) * 2 + align_up(3 * d * d * p.es) + align_up(d * d * p.es) +
                align_up(2 * F * d * p.es) + align_up(d * F * p.es);
    // per exit: router, then the own norm + head or the adapter; the shared norm + head once
    const size_t rr = c.router_dim, r = c.adapter_dim;
    const size_t router_w = c.router_form == 1 ? align_up(rr * d * 4) + 2 * align_up(rr * 4) : align_up(d * 4);
    const size_t head_w = c.head_form == 1 ? 2 * align_up(r * d * p.es) : align_up(d * 4) + align_up(V * d * p.es);
    p.exit_w = router_w + head_w;
    p.shared_head = c.head_form == 1 ? align_up(d * 4) + align_up(V * d * p.es) : 0;
    p.hidden = align_up((size_t)max_batch * max_ctx * d * 4);
    p.kv = align_up((size_t)max_batch * L * 2 * H * max_ctx * hd * p.kes);
    p.rope = align_up((size_t)max_ctx * hd * 4);
    size_t rmax = std::max<size_t>(64, std::min<size_t>((size_t)max_batch * max_ctx, 4096));
    p.R_max = (int)rmax;
    p.part_cap = (int)(rmax * H * 4);
    p.items_cap = p.part_cap;
    p.qbuf = align_up(rmax * d * 4);

    p.attn_o = align_up(rmax * d * 4);
    p.mlp = align_up(rmax * F * 4);
    p.part_ml = align_up((size_t)p.part_cap * 2 * 4);
    p.part_o = align_up((size_t)p.part_cap * hd * 4);
    p.rms = align_up(rmax * 4);
    p.abf = align_up(rmax * std::max(d, F) * 2);
    p.tables = align_up(rmax * sizeof(RowInfo) * 2 + rmax * sizeof(CombineInfo) +
                        (size_t)p.items_cap * sizeof(AttnItem) + rmax * 4);
    // uniforms, router outputs, stop flags, tokens in/out, head lists
    p.small = align_up((size_t)max_batch * (16 + 4 + sizeof(RowInfo))) +
              2 * align_up((size_t)max_batch * (4 + 2 * sizeof(RowInfo))) + align_up((size_t)max_batch * 32) +
              2 * align_up((size_t)max_batch * 4);
    p.logits = align_up((size_t)max_batch * V * 4);
    p.seg = 6 * align_up((size_t)d * 8) + align_up((size_t)F * 8) +
            align_up((size_t)c.n_heads * SEG_SMAX * (2 + hd) * 8) + align_up(4);
    p.router_hid = align_up((size_t)max_batch * (c.router_dim > 0 ? c.router_dim : 1) * 8);
    p.xd = align_up((size_t)(V / 8) * 2 * 4);
    // the largest (K / SK_KC) x N over the layer products and the exit heads, for
    // SK_MAX_ROWS rows
    {
        const int64_t kd = (int64_t)d / SK_KC, kf = (int64_t)F / SK_KC;
        const int64_t kn = std::max({kd * 3 * (int64_t)d, kd * 2 * (int64_t)F, kf * (int64_t)d, kd * (int64_t)V});
        p.sk_floats = kn > 0 ? (int64_t)SK_MAX_ROWS * (kn + std::max(kd, kf)) : 0;
    }
    // rows per head pass of the mixture objective: every pass re-reads the head weights, so
    // a pass takes as many rows as a 256 MiB logits workspace holds (at least 256, at most
    // the row capacity); NVIUM_LOSS_ROWS sets it instead (tests of ragged passes)
    size_t lch = std::max<size_t>(256, (size_t(256) << 20) / ((size_t)V * 4));
    if (const char* e = std::getenv("NVIUM_LOSS_ROWS")) {
        const long v = std::atol(e);
        if (v > 0) lch = (size_t)v;
    }
    p.loss_ch = (int)std::min<size_t>(lch, rmax);
    p.loss = align_up((size_t)p.loss_ch * V * 4) + 4 * align_up((size_t)max_ctx * 32) + align_up(64) +
             2 * align_up((size_t)max_ctx * 4) + align_up((size_t)max_ctx * sizeof(RowInfo)) +
             align_up((size_t)p.loss_ch * (c.router_dim > 0 ? c.router_dim : 1) * 8) +
             align_up((size_t)p.loss_ch * ((V + 63) / 64) * 8) + align_up((size_t)p.loss_ch * 4);
    p.total = p.abf + p.loss + p.router_hid + p.embed + L * p.layer_w + kMaxExits * p.exit_w + p.shared_head +
              p.hidden + p.kv + p.rope + p.qbuf + p.attn_o +
              p.mlp + p.part_ml + p.part_o + p.rms + p.tables + p.small + p.logits + p.seg + p.xd +
              align_up((size_t)p.sk_floats * 4) + kAlign;
    return p;
}

}  // namespace

struct nv_model {
    nv_config cfg{};
    int L = 0, d = 0, H = 0, hd = 0, F = 0, V = 0, seg = 0;
    bool bf16 = false;
    int max_batch = 0, max_ctx = 0;
    Plan plan;
    hipStream_t st = nullptr;
    char* arena = nullptr;
    size_t arena_off = 0;
    bool own_arena = false;
    bool dead = false;

    void* embed = nullptr;
    std::vector<LayerPtrs> layers;
    ExitPtrs exits[kMaxExits]{};
    float* Hs = nullptr;
    void* kv = nullptr;
    float* rope = nullptr;
    float* qbuf = nullptr;     // [R_max][d] rotated queries

    float* attn_o = nullptr;
    float* mlp = nullptr;
    float* part_ml = nullptr;
    float* part_o = nullptr;
    float* rms_ws = nullptr;   // [R_max] per-row inverse RMS for the matrix-core GEMM
    uint16_t* abf = nullptr;   // [R_max][max(d, F)] bf16 rows for the long-chunk GEMM
    double* router_hid = nullptr;   // [max_batch][router_dim] router MLP hidden units
    // mixture objective over one sequence of up to max_ctx tokens (rows = positions)
    float* loss_logits = nullptr;   // [loss_ch][V]
    double *loss_w = nullptr, *loss_lp = nullptr;       // [max_ctx][4]
    double *loss_nll = nullptr, *loss_depth = nullptr;  // [max_ctx] (allocated [max_ctx][4])
    double* loss_sums = nullptr;    // [2] means
    int *loss_tgt = nullptr, *loss_ids = nullptr;       // [max_ctx] target tokens, row ids 0..n-1
    RowInfo* loss_rows = nullptr;   // [max_ctx]
    double* loss_hid = nullptr;     // [loss_ch][router_dim]
    float* loss_xpart = nullptr;    // [loss_ch][V/64][2] fused cross-entropy partials
    float* loss_xtgt = nullptr;     // [loss_ch] target logits
    // chunks of at least this many rows use the matrix cores; up to 8 rows the vector-ALU
    // decode GEMV (LDS-free reductions, every weight load in flight before any wait) beats
    // the 16-row matrix-core tiles, which leave half their rows empty at 5-8 rows
    // (batch-1 decode: 0.417 -> 0.411 ms per segment-token against a threshold of 5)
    int mfma_min_rows = 9;
    // row groups of sk_min_rows..sk_max_rows rows take the split-K matrix-core product when
    // K is a multiple of SK_KC (0: never).  Batch-16 decode (1.5B, 16 x 32 tokens): 1.766 ms
    // per segment-step with none, 1.617 for 9-32 rows, 1.560 for 5-32, 1.526 for 5-64; batch
    // 1 at prompt 512 and 8192 within 2 %, the same or better
    int sk_min_rows = 5, sk_max_rows = SK_MAX_ROWS;
    int sk_ntb = 2 | (1 << 4);   // 16-column tiles per block with / without RMSNorm
    // greedy scheduling: weight of the longest wait (ticks) in a segment's score.  Workload C
    // (16 sequences, 1.5B): 0 -> 4632 tokens/s, 0.5 -> 4836, 2 -> 4839, 4 -> 5093, 8 -> 5216,
    // 16 and more -> 5288-5294 (the lock-step schedule; lock-step itself 5291-5298)
    double sched_age = 16.0;
    float* sk_ws = nullptr;
    int64_t sk_cap = 0;
    int n_cu = 256;               // compute units of the device (decode attention grid sizing)
    char* d_tables = nullptr;
    // Small per-step blocks; each has a pinned host mirror of the same layout so that it
    // goes up in one copy.  step: [uniforms MB*4 f32][pending tokens MB i32][current rows MB]
    // list (gate, head): [sequence ids MB i32][current rows MB][output rows MB]
    char* d_stepblk = nullptr;
    char* d_gatelist = nullptr;
    char* d_headlist = nullptr;
    float* xd_part = nullptr;        // exit draw: the head product's per-block (max, sum exp)
    double* d_w = nullptr;
    int* d_stop = nullptr;
    int* d_tok_out = nullptr;
    float* logits = nullptr;

    // persistent segment kernel (single decode rows); seg_nb == 0: not used
    int seg_nb = 0;
    uint64_t *seg_x0 = nullptr, *seg_q = nullptr, *seg_k = nullptr, *seg_v = nullptr, *seg_part = nullptr,
             *seg_att = nullptr, *seg_x1 = nullptr, *seg_act = nullptr;
    uint32_t* seg_err = nullptr;   // set by the kernel when a wait gave up
    uint32_t seg_epoch = 8;        // next launch's first tag
    bool seg_ran = false;          // launched since the error word was last checked
    unsigned long long seg_spin = 0;
    char* seg_base = nullptr;

    char* h_stage = nullptr;   // pinned; mirrors the device table region
    size_t h_stage_bytes = 0;
    bool stage_busy = false;   // an async copy from h_stage may still be pending
    // h_headlist has two halves used in turn; a half is busy from its upload until the
    // next stream synchronisation (a step can launch two head passes with no sync between)
    bool hl_busy[2] = {false, false};
    int hl_next = 0;
    char* h_stepblk = nullptr;
    char* h_gatelist = nullptr;
    char* h_headlist = nullptr;
    char* h_out = nullptr;     // pinned: stop flags, tokens, router outputs coming back
    int* h_ring = nullptr;     // pinned [kRing][max_batch]: sampled tokens coming back (nv_generate)
    // mapped, coherent [max_batch]: gate decisions stored by the gate kernels as tag * 2 + stop
    int* h_flags = nullptr;
    int* d_flags = nullptr;    // device address of h_flags
    int gate_tag = 0;          // tag of the last gate launch
    bool sb_busy = false;      // an async copy from h_stepblk may still be pending

    size_t stepblk_bytes() const { return (size_t)max_batch * (16 + 4 + sizeof(RowInfo)); }
    size_t list_bytes() const { return (size_t)max_batch * (4 + 2 * sizeof(RowInfo)); }
    static float* unif(char* b) { return (float*)b; }
    int* tok_in(char* b) const { return (int*)(b + (size_t)max_batch * 16); }
    RowInfo* cur_rows(char* b) const { return (RowInfo*)(b + (size_t)max_batch * 20); }
    static int* lseqs(char* b) { return (int*)b; }
    RowInfo* lrows(char* b) const { return (RowInfo*)(b + (size_t)max_batch * 4); }
    RowInfo* lorows(char* b) const { return (RowInfo*)(b + (size_t)max_batch * (4 + sizeof(RowInfo))); }

    std::vector<SeqHost> seqs;
    std::vector<double> last_w;   // [max_batch][4]
    std::string err;

    // optional per-class kernel timing with HIP events on the work stream
    bool timing = false;
    bool timing_stamps = false;   // also stamp every block (adds a fold kernel after each launch)
    std::vector<hipEvent_t> ev;   // pairs
    std::vector<int> ev_kind;
    std::vector<double> ev_bytes;
    std::vector<std::string> ev_name;
    unsigned long long* d_stamps = nullptr;   // [kEventPairs][2] device wall-clock spans
    unsigned long long* d_blkstamps = nullptr;  // [STAMP_BLOCKS][2] per-block stamps of one launch
    std::vector<int> ev_stamped;
    double wall_khz = 0.0;
    struct KStat {
        std::string name;
        int kind;
        double ms, bytes;      // ms: launch to completion (HIP events around each launch)
        int64_t n;
        double span_ms = 0.0;  // first block start to last block end (device stamps), if stamped
        int64_t n_span = 0;
    };
    std::vector<KStat> kstats;
    size_t ev_used = 0;
    double t_ms[NV_TIME_CLASSES] = {0}, t_bytes[NV_TIME_CLASSES] = {0};
    int64_t t_n[NV_TIME_CLASSES] = {0};

    LayerDims dims() const {
        LayerDims D;
        D.L = L;
        D.d = d;
        D.H = H;
        D.hd = hd;
        D.F = F;
        D.V = V;
        D.max_ctx = max_ctx;
        D.kv_bf16 = bf16 ? 1 : 0;
        return D;
    }

    char* take(size_t n) {
        char* p = arena + arena_off;
        arena_off += align_up(n);
        return p;
    }
};

namespace {

nv_status fail(nv_model* m, nv_status s, const std::string& msg) {
    if (m) m->err = msg;
    return s;
}

#define NV_HIP(m, expr)                                                                           \
    do {                                                                                          \
        hipError_t e_ = (expr);                                                                   \
        if (e_ != hipSuccess) {                                                                   \
            (m)->dead = true;                                                                     \
            return fail((m), NV_EDEVICE, std::string(#expr) + ": " + hipGetErrorString(e_));      \
        }                                                                                         \
    } while (0)

// Read `n` bytes at `off` of the weights file into host memory.
bool pread_all(int fd, void* dst, size_t n, size_t off) {
    char* p = (char*)dst;
    while (n > 0) {
        ssize_t r = ::pread(fd, p, n, (off_t)off);
        if (r <= 0) return false;
        p += r;
        n -= (size_t)r;
        off += (size_t)r;
    }
    return true;
}

// Accumulate the durations of recorded event pairs (the stream must be idle).
nv_status resolve_timing(nv_model* m) {
    std::vector<unsigned long long> st(2 * m->ev_used);
    if (m->ev_used) {
        NV_HIP(m, hipMemcpy(st.data(), m->d_stamps, st.size() * 8, hipMemcpyDeviceToHost));
    }
    for (size_t i = 0; i < m->ev_used; ++i) {
        float ms = 0.f;
        NV_HIP(m, hipEventElapsedTime(&ms, m->ev[2 * i], m->ev[2 * i + 1]));
        // stamped kernels also report first block start to last block end on the device clock
        const bool spanned = m->ev_stamped[i] && st[2 * i + 1] > st[2 * i];
        const double span = spanned ? (double)(st[2 * i + 1] - st[2 * i]) / m->wall_khz : 0.0;
        const int k = m->ev_kind[i];
        m->t_ms[k] += ms;
        m->t_bytes[k] += m->ev_bytes[i];
        m->t_n[k] += 1;
        auto it = std::find_if(m->kstats.begin(), m->kstats.end(),
                               [&](const nv_model::KStat& ks) { return ks.name == m->ev_name[i] && ks.kind == k; });
        if (it == m->kstats.end()) {
            m->kstats.push_back({m->ev_name[i], k, 0.0, 0.0, 0, 0.0, 0});
            it = m->kstats.end() - 1;
        }
        it->ms += ms;
        it->bytes += m->ev_bytes[i];
        it->n += 1;
        if (spanned) {
            it->span_ms += span;
            it->n_span += 1;
        }
    }
    m->ev_used = 0;
    // reset the spans: start = max, end = 0
    std::vector<unsigned long long> init(2 * kEventPairs);
    for (size_t i = 0; i < kEventPairs; ++i) {
        init[2 * i] = ~0ull;
        init[2 * i + 1] = 0ull;
    }
    NV_HIP(m, hipMemcpy(m->d_stamps, init.data(), init.size() * 8, hipMemcpyHostToDevice));
    return NV_OK;
}

// Issue one launch; with timing on, bracket it with events and note its algorithmic bytes.
template <class F>
nv_status timed(nv_model* m, int kind, double bytes, F&& launch, const char* name = nullptr) {
    if (!m->timing) {
        NV_HIP(m, launch());
        return NV_OK;
    }
    if (m->ev_used == kEventPairs) {
        NV_HIP(m, hipStreamSynchronize(m->st));
        nv_status s = resolve_timing(m);
        if (s != NV_OK) return s;
    }
    const size_t i = m->ev_used++;
    // kernels that support stamps use them; others leave (max, 0)
    m->ev_stamped[i] = m->timing_stamps ? 1 : 0;
    if (m->timing_stamps) set_launch_stamp(m->d_blkstamps);
    (void)take_launch_blocks();
    set_launch_events(m->ev[2 * i], m->ev[2 * i + 1]);
    const hipError_t le = launch();
    set_launch_events(nullptr, nullptr);
    set_launch_stamp(nullptr);
    NV_HIP(m, le);
    // fold (and reset) only the stamp entries this launch's blocks wrote
    const int nb = std::min(STAMP_BLOCKS, std::max(1, take_launch_blocks()));
    if (m->timing_stamps) NV_HIP(m, launch_stamp_reduce(m->d_blkstamps, nb, m->d_stamps + 2 * i, m->st));
    m->ev_kind[i] = kind;
    m->ev_bytes[i] = bytes;
    m->ev_name[i] = name ? name : last_launch_name();
    return NV_OK;
}

double gemm_bytes(const nv_model* m, const GemmArgs& g) {
    const double es = m->plan.es;
    const double nout = g.epi == EPI_SWIGLU ? g.N / 2 : g.N;
    const double out_rw = g.epi == EPI_RESID ? 2.0 : 1.0;
    const double in_es = gemm_uses_bf16_rows(g) ? 2.0 : 4.0;   // the product reads bf16 rows
    const double out_es = g.out_bf16 ? 2.0 : 4.0;
    if (g.xent_part)   // fused cross-entropy: per-row group partials and the target logit
        return (double)g.N * g.K * es + (double)g.R * g.K * in_es + (double)g.R * ((g.N / 64) * 8.0 + 8.0);
    return (double)g.N * g.K * es + (double)g.R * g.K * in_es + (double)g.R * nout * out_es * out_rw;
}

#define NV_TRY(expr)                      \
    do {                                  \
        nv_status s_ = (expr);            \
        if (s_ != NV_OK) return s_;       \
    } while (0)

// One product, timed; on the long-chunk path the bf16 row pass is timed as its own launch.
nv_status run_gemm(nv_model* m, int kind, GemmArgs g) {
    if (gemm_uses_bf16_rows(g) && !g.abf_ready) {
        NV_TRY(timed(m, kind, (double)g.R * g.K * 6, [&] { return launch_rows_bf16(g, m->st); }, "nv::k_rows_bf16"));
        g.abf_ready = 1;
    }
    return timed(m, kind, gemm_bytes(m, g), [&] { return launch_gemm(g, m->st); });
}

// The work stream was synchronised: every async copy from a pinned staging buffer is done.
void stream_synced(nv_model* m) {
    m->stage_busy = false;
    m->sb_busy = false;
    m->hl_busy[0] = m->hl_busy[1] = false;
}

nv_status stage_sync(nv_model* m) {
    if (m->stage_busy) {
        NV_HIP(m, hipStreamSynchronize(m->st));
        stream_synced(m);
    }
    return NV_OK;
}

// Build and upload the tables for one launch group of causal chunks at one segment:
// compact rows, attention items and combine info.  Layout in the device table region:
// [rows R][comb R][items n_items], R being this group's rows.
struct Tables {
    RowInfo* rows;
    CombineInfo* comb;
    AttnItem* items;
    int R, n_items;
    int hrow0;         // hidden-state row of the first row
    bool contig;       // one chunk: row r is position pos0 + r of sequence seq0, hidden row hrow0 + r
    int seq0, pos0;
    DecGeom dg;        // one chunk of at most ATTN_DEC_ROWS rows: the attention plan by value
    bool on_device;    // the tables were uploaded (some kernel of this group reads them)
    bool dec;          // decode-sized group: attention combines its splits in-kernel
    int max_rows;      // most rows in one decode-attention row block
    bool wide = false; // decode attention on ATTN_DEC_WIDE_WAVES-wave blocks (long contexts)
    bool any_split;    // some row's key range was split (the combine pass is needed)
    int max_split;     // most splits of one row's key range
    double kv_bytes;   // keys and values the attention items read
};

// Whether every block product of an R-row group runs on the vector-ALU decode GEMV (the one
// kernel that needs no row table for a contiguous chunk): the shape limits of that path in
// launch_gemm, for the four block products.
bool gemv_only(const nv_model* m, int R) {
    if (R < 1 || R > 8) return false;
    if (m->bf16 && m->mfma_min_rows > 0 && R >= m->mfma_min_rows) return false;
    // the split-K matrix-core product reads the row tables
    if (m->bf16 && m->sk_ws && m->mfma_min_rows > 0 && m->sk_min_rows > 0 && R >= m->sk_min_rows &&
        R <= m->sk_max_rows)
        return false;
    const int epc = m->bf16 ? 8 : 4;
    for (int K : {m->d, m->F})
        if (K % epc || K % 4 || (K / epc + 63) / 64 > 8) return false;
    for (int N : {3 * m->d, m->d, 2 * m->F})
        if (N % 8) return false;
    return true;
}

// Whether a one-row exit head runs on the vector-ALU decode GEMV (the kernel that can write
// the per-block softmax partials of the exit draw).
bool head_gemv_ok(const nv_model* m) {
    const int epc = m->bf16 ? 8 : 4;
    return m->d % epc == 0 && m->d % 4 == 0 && (m->d / epc + 63) / 64 <= 8 && m->V % 8 == 0 &&
           (!m->bf16 || m->mfma_min_rows == 0 || m->mfma_min_rows > 1);
}

int c_max_ctx(const std::vector<Chunk>& chunks) {
    int mx = 0;
    for (const Chunk& c : chunks) mx = std::max(mx, c.pos0 + c.nrows);
    return mx;
}

nv_status upload_tables(nv_model* m, const std::vector<Chunk>& chunks, Tables* t) {
    nv_status s = stage_sync(m);
    if (s != NV_OK) return s;
    const Plan& P = m->plan;
    int R = 0;
    for (const Chunk& c : chunks) R += c.nrows;
    if (R > P.R_max) return fail(m, NV_ECAPACITY, "internal: launch group exceeds workspace rows");
    // compact layout for this group: [rows R][comb R][items], so a decode step copies a
    // few KB rather than the worst case
    const size_t comb_off = sizeof(RowInfo) * (size_t)R, items_off = comb_off + sizeof(CombineInfo) * (size_t)R;
    RowInfo* hrows = (RowInfo*)m->h_stage;
    CombineInfo* hcomb = (CombineInfo*)(m->h_stage + comb_off);
    AttnItem* hitems = (AttnItem*)(m->h_stage + items_off);
    // rows
    int r = 0;
    for (const Chunk& c : chunks)
        for (int i = 0; i < c.nrows; ++i, ++r) {
            hrows[r].seq = c.seq;
            hrows[r].pos = c.pos0 + i;
            hrows[r].hrow = c.seq * m->max_ctx + c.pos0 + i;
            hrows[r].pad = 0;
        }
    int n_items = 0;
    const bool dec = R <= kDecodeRows;
    if (dec) {
        // decode-sized group: row blocks of ATTN_DEC_ROWS rows; each block's key range is cut
        // into nsplit pieces (at least 64 keys each, about 512 blocks in all) whose partial
        // softmax states the combine pass merges
        int nrb = 0, mx_nr = 0, mx_ctx = 0;
        for (const Chunk& c : chunks) {
            nrb += (c.nrows + ATTN_DEC_ROWS - 1) / ATTN_DEC_ROWS;
            mx_nr = std::max(mx_nr, std::min(ATTN_DEC_ROWS, c.nrows));
            mx_ctx = std::max(mx_ctx, c.pos0 + c.nrows);
        }
        // long contexts on bf16 K/V: blocks of ATTN_DEC_WIDE_WAVES waves with long splits, at
        // most one block per CU (so the splits of a row stay few enough for the O product to
        // merge them as it loads)
        t->wide = m->bf16 && mx_nr <= ATTN_DEC_WIDE_ROWS && mx_ctx > ATTN_DEC_WIDE_MIN_KEYS;
        const int nw = t->wide ? ATTN_DEC_WIDE_WAVES : 4;
        // (wide: about 3/4 of the CUs; the attention takes as long on 192 blocks as on 252 at
        // an 8K context, and the O product merges fewer splits: D -1.4 % per step)
        const int want = t->wide ? std::max(1, (m->n_cu * 3 / 4) / (m->H * nrb))
                                 : std::max(1, (kAttnBlocksTarget + m->H * nrb - 1) / (m->H * nrb));
        // keys per split: at most what one block's waves hold in flight
        const int max_keys = nw * (t->wide ? ATTN_DEC_WIDE_ITERS : ATTN_DEC_ITERS) * (64 / (m->hd / 8));
        int slot = 0, row0 = 0, rbi = 0;
        t->max_rows = 0;
        t->dg = DecGeom{};
        for (const Chunk& c : chunks) {
            for (int rb = 0; rb < c.nrows; rb += ATTN_DEC_ROWS, ++rbi) {
                const int nr = std::min(ATTN_DEC_ROWS, c.nrows - rb);
                t->max_rows = std::max(t->max_rows, nr);
                const int ctx = c.pos0 + rb + nr;
                const int ns0 = std::max((ctx + max_keys - 1) / max_keys, std::min(want, (ctx + 63) / 64));
                const int per = (ctx + ns0 - 1) / ns0;
                // with per rounded up, fewer splits may cover the range: drop the empty ones
                // (at 8K keys and 128 splits, per = 65 leaves the last split past ctx)
                const int ns = (ctx + per - 1) / per;
                if (ns > ATTN_COMB_MAX) return fail(m, NV_ECAPACITY, "internal: too many attention splits");
                if (nrb == 1) t->dg = DecGeom{1, c.seq, c.pos0, nr, ns, per};   // the same plan, by value
                for (int h = 0; h < m->H; ++h)
                    for (int s2 = 0; s2 < ns; ++s2) {
                        AttnItem& it = hitems[n_items++];
                        it.row0 = row0 + rb;
                        it.nrows = nr;
                        it.head = h;
                        it.lo = s2 * per;
                        it.hi = std::min(ctx, (s2 + 1) * per);
                        it.part = slot + (h * ns + s2) * nr;
                        it.split = s2;
                        it.nsplit = ns;
                        it.seq = c.seq;
                        it.pad[0] = it.pad[1] = it.pad[2] = 0;
                    }
                for (int i = 0; i < nr; ++i) {
                    CombineInfo& ci = hcomb[row0 + rb + i];
                    ci.base = slot;
                    ci.off = i;
                    ci.nsplit = ns;
                    ci.nrows = nr;
                }
                slot += m->H * ns * nr;
            }
            row0 += c.nrows;
        }
        if (slot > P.part_cap || n_items > P.items_cap)
            return fail(m, NV_ECAPACITY, "internal: attention partials exceed the workspace");
    } else {
        // long chunks: row blocks of 32 rows (64 on the matrix cores) sharing LDS key tiles;
        // the key range is split into pieces of split_len keys (doubling until the partial
        // slots fit), combined by a separate pass
        const int rpi = attn_mfma_ok(m->dims()) ? ATTN_MFMA_ROWS : kAttnRowsPerItem;
        int split_len = 512;
        for (;;) {
            long slots = 0, items = 0;
            for (const Chunk& c : chunks)
                for (int rb = 0; rb < c.nrows; rb += rpi) {
                    int nr = std::min(rpi, c.nrows - rb);
                    int ctx = c.pos0 + rb + nr;
                    int ns = (ctx + split_len - 1) / split_len;
                    slots += (long)m->H * ns * nr;
                    items += (long)m->H * ns;
                }
            if (slots <= P.part_cap && items <= P.items_cap &&
                (c_max_ctx(chunks) + split_len - 1) / split_len <= ATTN_COMB_MAX)
                break;
            split_len *= 2;
        }
        int slot = 0, row0 = 0;
        for (const Chunk& c : chunks) {
            for (int rb = 0; rb < c.nrows; rb += rpi) {
                int nr = std::min(rpi, c.nrows - rb);
                int ctx = c.pos0 + rb + nr;
                int ns = (ctx + split_len - 1) / split_len;
                for (int h = 0; h < m->H; ++h)
                    for (int s2 = 0; s2 < ns; ++s2) {
                        AttnItem& it = hitems[n_items++];
                        it.row0 = row0 + rb;
                        it.nrows = nr;
                        it.head = h;
                        it.lo = s2 * split_len;
                        it.hi = std::min(ctx, (s2 + 1) * split_len);
                        it.part = slot + (h * ns + s2) * nr;
                        it.split = s2;
                        it.nsplit = ns;
                        it.seq = c.seq;
                        it.pad[0] = it.pad[1] = it.pad[2] = 0;
                    }
                for (int i = 0; i < nr; ++i) {
                    CombineInfo& ci = hcomb[row0 + rb + i];
                    ci.base = slot;
                    ci.off = i;
                    ci.nsplit = ns;
                    ci.nrows = nr;
                }
                slot += m->H * ns * nr;
            }
            row0 += c.nrows;
        }
    }
    t->dec = dec;
    t->hrow0 = R > 0 ? hrows[0].hrow : 0;
    t->seq0 = R > 0 ? hrows[0].seq : 0;
    t->pos0 = R > 0 ? hrows[0].pos : 0;
    t->any_split = false;
    t->max_split = 1;
    for (int i = 0; i < n_items; ++i) {
        t->any_split |= hitems[i].nsplit > 1;
        t->max_split = std::max(t->max_split, hitems[i].nsplit);
    }
    t->contig = chunks.size() == 1;
    if (!t->contig) t->dg = DecGeom{};
    // a one-chunk decode group whose products all take the vector-ALU decode GEMV reads no
    // table: rows, attention items and split records are all passed by value
    t->on_device = !(t->dg.on && gemv_only(m, R));
    if (t->on_device) {
        const size_t bytes = items_off + sizeof(AttnItem) * (size_t)n_items;
        NV_HIP(m, hipMemcpyAsync(m->d_tables, m->h_stage, bytes, hipMemcpyHostToDevice, m->st));
        m->stage_busy = true;
    }
    t->rows = (RowInfo*)m->d_tables;
    t->comb = (CombineInfo*)(m->d_tables + comb_off);
    t->items = (AttnItem*)(m->d_tables + items_off);
    t->R = R;
    t->n_items = n_items;
    double kvb = 0;
    for (int i = 0; i < n_items; ++i) kvb += (double)(hitems[i].hi - hitems[i].lo);
    t->kv_bytes = kvb * 2.0 * m->hd * m->plan.kes;
    return NV_OK;
}

// A single decode row whose key range has at most 32 splits: the O projection merges the
// attention splits as it loads its activations (one launch less per layer).
bool fuse_merge(const nv_model* m, const Tables& t) { return t.dec && t.R == 1 && m->bf16 && t.max_split <= 32; }

// Run the layers of segment s (0-based) over the rows of the uploaded tables.
nv_status run_segment(nv_model* m, int s, const Tables& t) {
    const LayerDims D = m->dims();
    const int d = m->d;
    for (int l = s * m->seg; l < (s + 1) * m->seg; ++l) {
        const LayerPtrs& W = m->layers[l];
        GemmArgs g{};
        g.eps = m->cfg.norm_eps;
        g.wbf16 = m->bf16 ? 1 : 0;
        g.R = t.R;
        g.rms_ws = m->rms_ws;
        g.abf = m->abf;
        g.mfma_min_rows = m->mfma_min_rows;
        g.sk_ws = m->sk_ws;
        g.sk_cap = m->sk_cap;
        g.sk_min_rows = m->sk_min_rows;
        g.sk_max_rows = m->sk_max_rows;
        g.sk_ntb = m->sk_ntb;
        g.contig = t.contig ? 1 : 0;
        g.a_row0 = g.o_row0 = t.hrow0;
        g.seq0 = t.seq0;
        g.pos0 = t.pos0;
        // q, k, v = RMSNorm(x) W_qkv^T
        g.A = m->Hs;
        g.lda = d;
        g.a_rows = t.rows;
        g.norm_w = W.attn_norm;
        g.W = W.wqkv;
        g.N = 3 * d;
        g.K = d;
        g.epi = EPI_QKV;
        g.out = nullptr;
        g.ldo = 0;
        g.o_rows = nullptr;
        g.q_out = m->qbuf;
        g.kv = m->kv;
        g.rope = m->rope;
        g.layer = l;
        g.D = D;
        NV_TRY(run_gemm(m, NV_TIME_BLOCK_GEMM, g));
        // long chunks whose O product runs on bf16 rows: the combine pass writes those rows
        GemmArgs go = g;
        go.A = m->attn_o;
        go.lda = d;
        go.a_rows = nullptr;
        go.norm_w = nullptr;
        go.W = W.wo;
        go.N = d;
        go.K = d;
        go.epi = EPI_RESID;
        const bool o_bf16 = !t.dec && gemm_uses_bf16_rows(go);
        auto combine = [&] {
            if (o_bf16)
                return timed(m, NV_TIME_ATTENTION, (double)t.R * d * 6, [&] {
                    return launch_attn_combine_bf16(t.comb, t.R, D, m->part_ml, m->part_o, m->attn_o, m->abf, m->st);
                }, "nv::k_attn_combine_bf16");
            return timed(m, NV_TIME_ATTENTION, (double)t.R * d * 4, [&] {
                return launch_attn_combine(t.comb, t.R, D, m->part_ml, m->part_o, m->attn_o, m->st);
            });
        };
        if (t.dec) {
            if (t.max_rows >= ATTN_DEC_MFMA_ROWS && attn_mfma_ok(D))
                NV_TRY(timed(m, NV_TIME_ATTENTION, t.kv_bytes + (double)t.R * d * 8, [&] {
                    return launch_attn_mfma16(t.items, t.n_items, t.rows, m->qbuf, m->kv, l, D, m->part_ml,
                                              m->part_o, m->attn_o, m->st, t.dg);
                }));
            else
                NV_TRY(timed(m, NV_TIME_ATTENTION, t.kv_bytes + (double)t.R * d * 8, [&] {
                    return launch_attn_dec(t.items, t.n_items, t.max_rows, t.rows, m->qbuf, m->kv, l, D, m->part_ml,
                                           m->part_o, m->attn_o, m->st, t.dg, t.wide ? 1 : 0);
                }));
            // one row: the O projection merges the splits itself (no combine pass)
            if (t.any_split && !fuse_merge(m, t))
                NV_TRY(timed(m, NV_TIME_ATTENTION, (double)t.R * d * 4, [&] {
                    return launch_attn_combine(t.comb, t.R, D, m->part_ml, m->part_o, m->attn_o, m->st, t.dg);
                }));
        } else if (attn_mfma_ok(D)) {
            NV_TRY(timed(m, NV_TIME_ATTENTION, t.kv_bytes, [&] {
                return launch_attn_mfma(t.items, t.n_items, t.rows, m->qbuf, m->kv, l, D, m->part_ml, m->part_o,
                                        m->attn_o, m->st);
            }, "nv::k_attn_mfma"));
            NV_TRY(combine());
        } else {
            NV_TRY(timed(m, NV_TIME_ATTENTION, t.kv_bytes, [&] {
                return launch_attn(t.items, t.n_items, t.rows, m->qbuf, m->kv, l, D, m->part_ml, m->part_o, m->attn_o,
                                   m->st);
            }, "nv::k_attn"));
            NV_TRY(combine());
        }
        // x += o W_o^T
        g.epi = EPI_RESID;
        g.A = m->attn_o;
        g.lda = d;
        g.a_rows = nullptr;
        g.norm_w = nullptr;
        g.W = W.wo;
        if (fuse_merge(m, t)) {
            g.comb = t.comb;
            g.comb_ns = t.dg.on ? t.dg.nsplit : 0;
            g.part_ml = m->part_ml;
            g.part_o = m->part_o;
            g.D = D;
        }
        g.N = d;
        g.K = d;
        g.epi = EPI_RESID;
        g.out = m->Hs;
        g.ldo = d;
        g.o_rows = t.rows;
        g.abf_ready = o_bf16 ? 1 : 0;
        NV_TRY(run_gemm(m, NV_TIME_BLOCK_GEMM, g));
        g.abf_ready = 0;
        g.comb = nullptr;
        // u = silu(RMSNorm(x) W_g^T) * (RMSNorm(x) W_u^T)
        g.A = m->Hs;
        g.lda = d;
        g.a_rows = t.rows;
        g.norm_w = W.mlp_norm;
        g.W = W.wgu;
        g.N = 2 * m->F;
        g.K = d;
        g.epi = EPI_SWIGLU;
        g.out = m->mlp;
        g.ldo = m->F;
        g.o_rows = nullptr;
        // x += u W_d^T
        GemmArgs gd = g;
        gd.A = m->mlp;
        gd.lda = m->F;
        gd.a_rows = nullptr;
        gd.norm_w = nullptr;
        gd.W = W.wd;
        gd.N = d;
        gd.K = m->F;
        gd.epi = EPI_RESID;
        gd.out = m->Hs;
        gd.ldo = d;
        gd.o_rows = t.rows;
        if (gemm_uses_bf16_rows(g) && gemm_uses_bf16_rows(gd)) {
            // both products on bf16 rows: the SwiGLU epilogue writes u as the down
            // product's bf16 rows (in the mlp buffer, which holds [R][F] fp32)
            g.out_bf16 = (uint16_t*)m->mlp;
            gd.abf = (uint16_t*)m->mlp;
            gd.abf_ready = 1;
        }
        NV_TRY(run_gemm(m, NV_TIME_BLOCK_GEMM, g));
        NV_TRY(run_gemm(m, NV_TIME_BLOCK_GEMM, gd));
    }
    return NV_OK;
}

// ------------------------------------------------------------------------------------------
// Persistent segment kernel: one launch per segment for a single decode row.
// ------------------------------------------------------------------------------------------

// Zero the tagged exchange buffers and counters and restart the tags (the stream orders it
// before the next launch).
nv_status seg_reset(nv_model* m) {
    const size_t tagged = (size_t)((char*)m->seg_err - m->seg_base) + align_up(4);
    NV_HIP(m, hipMemsetAsync(m->seg_base, 0, tagged, m->st));
    m->seg_epoch = 8;
    return NV_OK;
}

nv_status seg_setup(nv_model* m) {
    m->seg_nb = 0;
    if (!m->bf16) return NV_OK;
    // opt-in for now (NVIUM_SEGMENT=1): on the 1.5B shape it is not yet faster than the
    // per-phase kernels
    const char* e = std::getenv("NVIUM_SEGMENT");
    if (!e || std::string(e) != "1") return NV_OK;
    int dev = 0, ncu = 0, coop = 0, khz = 0;
    NV_HIP(m, hipGetDevice(&dev));
    NV_HIP(m, hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    NV_HIP(m, hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
    NV_HIP(m, hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
    const int nb = coop ? segment_blocks(m->dims(), ncu) : 0;
    if (nb <= 0) return NV_OK;
    char* p = m->seg_base;
    auto carve = [&](size_t n) {
        char* r = p;
        p += align_up(n);
        return r;
    };
    const size_t d = m->d;
    m->seg_x0 = (uint64_t*)carve(d * 8);
    m->seg_q = (uint64_t*)carve(d * 8);
    m->seg_k = (uint64_t*)carve(d * 8);
    m->seg_v = (uint64_t*)carve(d * 8);
    m->seg_att = (uint64_t*)carve(d * 8);
    m->seg_x1 = (uint64_t*)carve(d * 8);
    m->seg_act = (uint64_t*)carve((size_t)m->F * 8);
    m->seg_part = (uint64_t*)carve((size_t)m->H * SEG_SMAX * (2 + m->hd) * 8);
    m->seg_err = (uint32_t*)carve(4);
    if ((size_t)(p - m->seg_base) > m->plan.seg) return fail(m, NV_ECAPACITY, "internal: segment buffers exceed the plan");
    if (m->seg > SEG_LMAX) return NV_OK;
    NV_TRY(seg_reset(m));
    // a wait gives up after half a second of device time
    m->seg_spin = (unsigned long long)(khz > 0 ? khz : 100000) * 500ull;
    m->seg_nb = nb;
    return NV_OK;
}

// After the stream is idle: a wait that gave up inside the segment kernel leaves the
// handle unusable.
nv_status seg_check(nv_model* m, const uint32_t* h_err) {
    if (m->seg_ran && *h_err) {
        m->dead = true;
        return fail(m, NV_EDEVICE, "segment kernel: a cross-block wait gave up (blocks not co-resident?)");
    }
    m->seg_ran = false;
    return NV_OK;
}

// Wait for the stream; then report a wait that gave up in a segment launch since the
// last check.
nv_status sync_and_check(nv_model* m) {
    uint32_t* h_err = (uint32_t*)(m->h_out + (size_t)m->max_batch * 48);
    if (m->seg_ran) NV_HIP(m, hipMemcpyAsync(h_err, m->seg_err, 4, hipMemcpyDeviceToHost, m->st));
    NV_HIP(m, hipStreamSynchronize(m->st));
    stream_synced(m);
    return seg_check(m, h_err);
}

// Key splits per head for a context of ctx keys: about 64 keys per split, as many as
// the grid holds.
int seg_splits(const nv_model* m, int ctx) {
    const int cap = std::min(SEG_SMAX, m->seg_nb / m->H);
    return std::max(1, std::min(cap, (ctx + 63) / 64));
}

nv_status run_segment_persistent(nv_model* m, int s, const Chunk& c) {
    if (m->seg_epoch > 0xF0000000u) NV_TRY(seg_reset(m));
    SegArgs a{};
    for (int i = 0; i < m->seg; ++i) {
        const LayerPtrs& W = m->layers[s * m->seg + i];
        a.lw[i] = SegLayerW{W.attn_norm, (const uint16_t*)W.wqkv, (const uint16_t*)W.wo, W.mlp_norm,
                            (const uint16_t*)W.wgu, (const uint16_t*)W.wd};
    }
    a.l0 = s * m->seg;
    a.nl = m->seg;
    a.D = m->dims();
    a.eps = m->cfg.norm_eps;
    a.Hs = m->Hs;
    a.hrow = (int64_t)c.seq * m->max_ctx + c.pos0;
    a.seq = c.seq;
    a.pos = c.pos0;
    a.kv = m->kv;
    a.rope = m->rope;
    a.tx0 = m->seg_x0;
    a.tq = m->seg_q;
    a.tk = m->seg_k;
    a.tv = m->seg_v;
    a.tpart = m->seg_part;
    a.tatt = m->seg_att;
    a.tx1 = m->seg_x1;
    a.tact = m->seg_act;
    a.err = m->seg_err;
    a.epoch = m->seg_epoch;
    a.S = seg_splits(m, c.pos0 + 1);
    a.spin_ticks = m->seg_spin;
    const double d = m->d, F = m->F, es = m->plan.es;
    const double layer_bytes = (4 * d * d + 3 * d * F) * es + 2 * d * 4;
    const double bytes = a.nl * (layer_bytes + (double)c.pos0 * 2 * d * es + 2 * d * es) + 2 * d * 4;
    NV_TRY(timed(m, NV_TIME_BLOCK_GEMM, bytes, [&] { return launch_segment(a, m->seg_nb, m->st); }, "nv::k_segment"));
    m->seg_epoch += (uint32_t)(SEG_PHASES * (a.nl + 1));
    m->seg_ran = true;
    return NV_OK;
}

// Run segment s over a list of chunks, splitting into launch groups that fit the
// workspace.  Pieces of one sequence go in ascending position order and in separate
// groups, so each piece sees the KV of the pieces before it.
nv_status run_chunks(nv_model* m, int s, const std::vector<Chunk>& chunks) {
    const int cap = m->plan.R_max;
    std::vector<Chunk> pieces;
    for (const Chunk& c : chunks)
        for (int o = 0; o < c.nrows; o += cap) pieces.push_back({c.seq, c.pos0 + o, std::min(cap, c.nrows - o)});
    std::vector<bool> done(pieces.size(), false);
    size_t left = pieces.size();
    while (left > 0) {
        std::vector<Chunk> group;
        std::vector<int> seqs_in;
        int rows = 0;
        for (size_t i = 0; i < pieces.size(); ++i) {
            if (done[i]) continue;
            const Chunk& p = pieces[i];
            bool seq_taken = std::find(seqs_in.begin(), seqs_in.end(), p.seq) != seqs_in.end();
            if (seq_taken) continue;
            seqs_in.push_back(p.seq);   // later pieces of this sequence wait for the next group
            if (rows + p.nrows > cap) continue;
            group.push_back(p);
            rows += p.nrows;
            done[i] = true;
            --left;
        }
        if (m->seg_nb > 0 && group.size() == 1 && group[0].nrows == 1) {
            nv_status st = run_segment_persistent(m, s, group[0]);
            if (st != NV_OK) return st;
            continue;
        }
        Tables t;
        nv_status st = upload_tables(m, group, &t);
        if (st != NV_OK) return st;
        st = run_segment(m, s, t);
        if (st != NV_OK) return st;
    }
    return NV_OK;
}

nv_status check_seq(nv_model* m, int seq) {
    if (!m) return NV_EINVAL;
    if (m->dead) return fail(m, NV_EDEVICE, "model handle unusable after a device error");
    if (seq < 0 || seq >= m->max_batch) return fail(m, NV_EINVAL, "sequence index out of range");
    return NV_OK;
}

}  // namespace

// ==========================================================================================
// C ABI
// ==========================================================================================

extern "C" {

size_t nv_mem_required(const char* weights_path, int32_t max_batch, int32_t max_ctx) {
    if (!weights_path || max_batch < 1 || max_ctx < 1) return 0;
    nv_config c;
    std::string err;
    if (!read_header(weights_path, &c, &err)) return 0;
    return make_plan(c, max_batch, max_ctx).total;
}

const char* nv_last_error(const nv_model* m) { return m ? m->err.c_str() : "null model handle"; }

nv_status nv_get_config(const nv_model* m, nv_config* out) {
    if (!m || !out) return NV_EINVAL;
    *out = m->cfg;
    return NV_OK;
}

void nv_free(nv_model* m) {
    if (!m) return;
    if (m->st) (void)hipStreamSynchronize(m->st);
    if (m->own_arena && m->arena) (void)hipFree(m->arena);
    if (m->h_stage) (void)hipHostFree(m->h_stage);
    for (hipEvent_t e : m->ev) (void)hipEventDestroy(e);
    if (m->d_stamps) (void)hipFree(m->d_stamps);
    if (m->d_blkstamps) (void)hipFree(m->d_blkstamps);
    if (m->h_stepblk) (void)hipHostFree(m->h_stepblk);
    if (m->h_gatelist) (void)hipHostFree(m->h_gatelist);
    if (m->h_headlist) (void)hipHostFree(m->h_headlist);
    if (m->h_out) (void)hipHostFree(m->h_out);
    if (m->h_ring) (void)hipHostFree(m->h_ring);
    if (m->h_flags) (void)hipHostFree(m->h_flags);
    delete m;
}

nv_status nv_load(const char* path, int32_t max_batch, int32_t max_ctx, void* device_arena, size_t arena_bytes,
                  void* hip_stream, nv_model** out) {
    if (!path || !out || max_batch < 1 || max_ctx < 1) return NV_EINVAL;
    *out = nullptr;
    nv_model* m = new nv_model();
    std::string err;
    if (!read_header(path, &m->cfg, &err)) {
        m->err = err;
        *out = m;
        return NV_EIO;
    }
    *out = m;
    const nv_config& c = m->cfg;
    m->L = c.n_layers;
    m->d = c.d_model;
    m->H = c.n_heads;
    m->hd = c.head_dim;
    m->F = c.ffn;
    m->V = c.vocab;
    m->seg = c.n_layers / kMaxExits;
    m->bf16 = c.wdtype == 1;
    m->max_batch = max_batch;
    m->max_ctx = max_ctx;
    m->plan = make_plan(c, max_batch, max_ctx);
    const Plan& P = m->plan;
    if (c.head_form == 1 && max_batch > P.R_max)
        return fail(m, NV_ECAPACITY, "shared head: max_batch exceeds the row workspace");
    m->st = (hipStream_t)hip_stream;

    // check the file length before touching the device
    struct stat sb;
    size_t need = 256;
    {
        const size_t d = m->d, F = m->F, V = m->V, es = P.es;
        size_t off = 256;
        auto adv = [&](size_t n) { off = align_up(off) + n; };
        adv(V * d * es);
        for (int l = 0; l < m->L; ++l) {
            adv(d * 4);
            adv(d * d * es);
            adv(d * d * es);
            adv(d * d * es);
            adv(d * d * es);
            adv(d * 4);
            adv(F * d * es);
            adv(F * d * es);
            adv(d * F * es);
        }
        const size_t rr = c.router_dim, r = c.adapter_dim;
        for (int k = 0; k < kMaxExits; ++k) {
            if (c.router_form == 1) {
                adv(rr * d * 4);
                adv(rr * 4);
                adv(rr * 4);
            } else {
                adv(d * 4);
            }
            if (c.head_form == 1) {
                if (k < kMaxExits - 1) {
                    adv(r * d * es);
                    adv(d * r * es);
                }
            } else {
                adv(d * 4);
                adv(V * d * es);
            }
        }
        if (c.head_form == 1) {
            adv(d * 4);
            adv(V * d * es);
        }
        need = off;
    }
    if (::stat(path, &sb) != 0 || (size_t)sb.st_size < need) return fail(m, NV_EIO, "weights file truncated");

    if (device_arena) {
        if (arena_bytes < P.total) return fail(m, NV_ECAPACITY, "device arena smaller than nv_mem_required()");
        m->arena = (char*)device_arena;
    } else {
        NV_HIP(m, hipMalloc((void**)&m->arena, P.total));
        m->own_arena = true;
    }
    m->arena = (char*)align_up((size_t)m->arena);
    NV_HIP(m, init_kernel_attributes());
    {
        int dev = 0, ncu = 0;
        NV_HIP(m, hipGetDevice(&dev));
        NV_HIP(m, hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
        if (ncu > 0) m->n_cu = ncu;
    }

    // carve the arena
    m->embed = m->take(P.embed);
    m->layers.resize(m->L);
    for (int l = 0; l < m->L; ++l) {
        LayerPtrs& W = m->layers[l];
        W.attn_norm = (float*)m->take((size_t)m->d * 4);
        W.mlp_norm = (float*)m->take((size_t)m->d * 4);
        W.wqkv = m->take(3 * (size_t)m->d * m->d * P.es);
        W.wo = m->take((size_t)m->d * m->d * P.es);
        W.wgu = m->take(2 * (size_t)m->F * m->d * P.es);
        W.wd = m->take((size_t)m->d * m->F * P.es);
    }
    const size_t rr = c.router_dim, ra = c.adapter_dim;
    for (int k = 0; k < kMaxExits; ++k) {
        ExitPtrs& X = m->exits[k];
        X = ExitPtrs{};
        if (c.router_form == 1) {
            X.router_w1 = (float*)m->take(rr * m->d * 4);
            X.router_b1 = (float*)m->take(rr * 4);
            X.router_w2 = (float*)m->take(rr * 4);
        } else {
            X.gate_w = (float*)m->take((size_t)m->d * 4);
        }
        if (c.head_form == 1) {
            X.adapter_down = m->take(ra * m->d * P.es);
            X.adapter_up = m->take(ra * m->d * P.es);
        } else {
            X.norm = (float*)m->take((size_t)m->d * 4);
            X.head = m->take((size_t)m->V * m->d * P.es);
        }
        X.bias = c.gate_bias[k];
    }
    if (c.head_form == 1) {
        float* fnorm = (float*)m->take((size_t)m->d * 4);
        void* head = m->take((size_t)m->V * m->d * P.es);
        for (int k = 0; k < kMaxExits; ++k) {
            m->exits[k].norm = fnorm;
            m->exits[k].head = head;
        }
    }
    m->Hs = (float*)m->take(P.hidden);
    m->kv = m->take(P.kv);
    m->rope = (float*)m->take(P.rope);
    m->qbuf = (float*)m->take(P.qbuf);

    m->attn_o = (float*)m->take(P.attn_o);
    m->mlp = (float*)m->take(P.mlp);
    m->part_ml = (float*)m->take(P.part_ml);
    m->part_o = (float*)m->take(P.part_o);
    m->rms_ws = (float*)m->take(P.rms);
    m->abf = (uint16_t*)m->take(P.abf);
    if (const char* e = std::getenv("NVIUM_MFMA_MIN_ROWS")) m->mfma_min_rows = std::atoi(e);
    if (P.sk_floats > 0) {
        m->sk_ws = (float*)m->take(align_up((size_t)P.sk_floats * 4));
        m->sk_cap = P.sk_floats;
    }
    if (const char* e = std::getenv("NVIUM_SK_MIN_ROWS")) m->sk_min_rows = std::atoi(e);
    if (const char* e = std::getenv("NVIUM_SK_MAX_ROWS")) m->sk_max_rows = std::atoi(e);
    if (const char* e = std::getenv("NVIUM_SCHED_AGE")) m->sched_age = std::atof(e);
    if (const char* e = std::getenv("NVIUM_SK_NTB")) {   // "<with RMSNorm>,<without>"
        int a = 0, b = 0;
        if (std::sscanf(e, "%d,%d", &a, &b) == 2) m->sk_ntb = (a & 15) | ((b & 15) << 4);
    }
    m->d_tables = m->take(P.tables);
    m->d_stepblk = m->take(m->stepblk_bytes());
    m->d_gatelist = m->take(m->list_bytes());
    m->d_headlist = m->take(m->list_bytes());
    m->d_w = (double*)m->take((size_t)max_batch * 32);
    m->d_stop = (int*)m->take((size_t)max_batch * 4);
    m->d_tok_out = (int*)m->take((size_t)max_batch * 4);
    m->logits = (float*)m->take(P.logits);
    m->router_hid = (double*)m->take(P.router_hid);
    m->loss_logits = (float*)m->take((size_t)P.loss_ch * m->V * 4);
    m->loss_w = (double*)m->take((size_t)max_ctx * 32);
    m->loss_lp = (double*)m->take((size_t)max_ctx * 32);
    m->loss_nll = (double*)m->take((size_t)max_ctx * 32);
    m->loss_depth = (double*)m->take((size_t)max_ctx * 32);
    m->loss_sums = (double*)m->take(64);
    m->loss_tgt = (int*)m->take((size_t)max_ctx * 4);
    m->loss_ids = (int*)m->take((size_t)max_ctx * 4);
    m->loss_rows = (RowInfo*)m->take((size_t)max_ctx * sizeof(RowInfo));
    m->loss_hid = (double*)m->take((size_t)P.loss_ch * (m->cfg.router_dim > 0 ? m->cfg.router_dim : 1) * 8);
    m->loss_xpart = (float*)m->take((size_t)P.loss_ch * ((m->V + 63) / 64) * 8);
    m->loss_xtgt = (float*)m->take((size_t)P.loss_ch * 4);
    m->seg_base = m->take(P.seg);
    m->xd_part = (float*)m->take(P.xd);
    if (m->arena_off > P.total) return fail(m, NV_ECAPACITY, "internal: arena plan too small");

    m->h_stage_bytes = P.tables;
    NV_HIP(m, hipHostMalloc((void**)&m->h_stage, m->h_stage_bytes, hipHostMallocDefault));
    NV_HIP(m, hipHostMalloc((void**)&m->h_stepblk, m->stepblk_bytes(), hipHostMallocDefault));
    NV_HIP(m, hipHostMalloc((void**)&m->h_gatelist, m->list_bytes(), hipHostMallocDefault));
    NV_HIP(m, hipHostMalloc((void**)&m->h_headlist, 2 * m->list_bytes(), hipHostMallocDefault));
    NV_HIP(m, hipHostMalloc((void**)&m->h_out, (size_t)max_batch * 48 + 16, hipHostMallocDefault));
    NV_HIP(m, hipHostMalloc((void**)&m->h_ring, (size_t)kRing * max_batch * 4, hipHostMallocDefault));
    NV_HIP(m, hipHostMalloc((void**)&m->h_flags, (size_t)max_batch * 4, hipHostMallocMapped | hipHostMallocCoherent));
    for (int i = 0; i < max_batch; ++i) m->h_flags[i] = -1;
    NV_HIP(m, hipHostGetDevicePointer((void**)&m->d_flags, m->h_flags, 0));

    // weights: file tensors -> pinned bounce buffer -> device (repacking W_gate/W_up rows)
    int fd = ::open(path, O_RDONLY);
    if (fd < 0) return fail(m, NV_EIO, "cannot open weights file");
    const size_t d = m->d, F = m->F, V = m->V, es = P.es;
    const size_t bounce_bytes = 64ull << 20;
    char* bounce = nullptr;
    if (hipHostMalloc((void**)&bounce, bounce_bytes, hipHostMallocDefault) != hipSuccess) {
        ::close(fd);
        m->dead = true;
        return fail(m, NV_EDEVICE, "hipHostMalloc failed for the load buffer");
    }
    size_t off = 256;
    bool io_ok = true;
    hipError_t herr = hipSuccess;
    auto copy_tensor = [&](void* dst, size_t nbytes) {
        off = align_up(off);
        size_t done = 0;
        while (io_ok && herr == hipSuccess && done < nbytes) {
            size_t n = std::min(bounce_bytes, nbytes - done);
            if (!pread_all(fd, bounce, n, off + done)) {
                io_ok = false;
                break;
            }
            herr = hipMemcpy((char*)dst + done, bounce, n, hipMemcpyHostToDevice);
            done += n;
        }
        off += nbytes;
    };
    // W_gate rows go to even rows of wgu, W_up rows to odd rows.
    auto copy_interleaved = [&](void* dst, size_t rows, size_t row_bytes, int parity) {
        off = align_up(off);
        const size_t rows_per = bounce_bytes / row_bytes;
        size_t done = 0;
        while (io_ok && herr == hipSuccess && done < rows) {
            size_t n = std::min(rows_per, rows - done);
            if (!pread_all(fd, bounce, n * row_bytes, off + done * row_bytes)) {
                io_ok = false;
                break;
            }
            herr = hipMemcpy2D((char*)dst + (2 * done + parity) * row_bytes, 2 * row_bytes, bounce, row_bytes,
                               row_bytes, n, hipMemcpyHostToDevice);
            done += n;
        }
        off += rows * row_bytes;
    };
    // W_q, W_k, W_v are adjacent in the file; device row 2p + i of the fused matrix is
    // original row part*d + h*hd + j + i*hd/2 (p = part*d/2 + h*hd/2 + j), so RoPE partners
    // land in adjacent output columns of the QKV product
    std::vector<char> qkv_file(3 * d * d * es), qkv_dev(3 * d * d * es);
    auto copy_qkv = [&](void* dst) {
        off = align_up(off);
        for (int part = 0; part < 3 && io_ok; ++part) {
            off = align_up(off);
            if (!pread_all(fd, qkv_file.data() + part * d * d * es, d * d * es, off)) io_ok = false;
            off += d * d * es;
        }
        if (!io_ok || herr != hipSuccess) return;
        const size_t half = m->hd / 2, row = d * es;
        for (size_t pr = 0; pr < 3 * d / 2; ++pr) {
            const size_t part = pr / (d / 2), pp = pr % (d / 2), h = pp / half, j = pp % half;
            const size_t src0 = part * d + h * m->hd + j;
            std::memcpy(qkv_dev.data() + (2 * pr) * row, qkv_file.data() + src0 * row, row);
            std::memcpy(qkv_dev.data() + (2 * pr + 1) * row, qkv_file.data() + (src0 + half) * row, row);
        }
        herr = hipMemcpy(dst, qkv_dev.data(), qkv_dev.size(), hipMemcpyHostToDevice);
    };
    copy_tensor(m->embed, V * d * es);
    for (int l = 0; l < m->L && io_ok && herr == hipSuccess; ++l) {
        LayerPtrs& W = m->layers[l];
        copy_tensor(W.attn_norm, d * 4);
        copy_qkv(W.wqkv);
        copy_tensor(W.wo, d * d * es);
        copy_tensor(W.mlp_norm, d * 4);
        copy_interleaved(W.wgu, F, d * es, 0);
        copy_interleaved(W.wgu, F, d * es, 1);
        copy_tensor(W.wd, d * F * es);
    }
    for (int k = 0; k < kMaxExits && io_ok && herr == hipSuccess; ++k) {
        const ExitPtrs& X = m->exits[k];
        if (c.router_form == 1) {
            copy_tensor(X.router_w1, (size_t)c.router_dim * d * 4);
            copy_tensor(X.router_b1, (size_t)c.router_dim * 4);
            copy_tensor(X.router_w2, (size_t)c.router_dim * 4);
        } else {
            copy_tensor(X.gate_w, d * 4);
        }
        if (c.head_form == 1) {
            if (k < kMaxExits - 1) {
                copy_tensor(X.adapter_down, (size_t)c.adapter_dim * d * es);
                copy_tensor(X.adapter_up, (size_t)c.adapter_dim * d * es);
            }
        } else {
            copy_tensor(X.norm, d * 4);
            copy_tensor(X.head, V * d * es);
        }
    }
    if (c.head_form == 1 && io_ok && herr == hipSuccess) {
        copy_tensor(m->exits[0].norm, d * 4);
        copy_tensor(m->exits[0].head, V * d * es);
    }
    ::close(fd);
    (void)hipHostFree(bounce);
    if (!io_ok) return fail(m, NV_EIO, "weights file read failed");
    NV_HIP(m, herr);
    NV_HIP(m, launch_rope_table(m->rope, max_ctx, m->hd, c.rope_base, m->st));
    NV_TRY(seg_setup(m));

    NV_HIP(m, hipStreamSynchronize(m->st));
    m->seqs.assign(max_batch, SeqHost());
    m->last_w.assign((size_t)max_batch * 4, NAN);
    return NV_OK;
}

nv_status nv_prefill(nv_model* m, int32_t seq, const int32_t* tokens, int32_t n) {
    nv_status s = check_seq(m, seq);
    if (s != NV_OK) return s;
    if (!tokens || n < 1) return fail(m, NV_EINVAL, "prefill needs at least one token");
    if (n > m->max_ctx) return fail(m, NV_ECAPACITY, "prompt longer than max_ctx");
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->V) return fail(m, NV_EINVAL, "token id out of range");
    SeqHost& S = m->seqs[seq];
    S = SeqHost();
    S.live = true;
    S.pending = tokens[n - 1];
    const int np = n - 1;
    // embed positions 0..np-1 in pieces
    const int cap = m->plan.R_max;
    for (int o = 0; o < np; o += cap) {
        const int k = std::min(cap, np - o);
        if ((s = stage_sync(m)) != NV_OK) return s;
        RowInfo* hr = (RowInfo*)m->h_stage;
        int* ht = (int*)(m->h_stage + sizeof(RowInfo) * k);
        for (int i = 0; i < k; ++i) {
            hr[i] = RowInfo{seq * m->max_ctx + o + i, seq, o + i, 0};
            ht[i] = tokens[o + i];
        }
        NV_HIP(m, hipMemcpyAsync(m->d_tables, m->h_stage, (sizeof(RowInfo) + 4) * k, hipMemcpyHostToDevice, m->st));
        m->stage_busy = true;
        NV_HIP(m, launch_embed((const int*)(m->d_tables + sizeof(RowInfo) * k), (const RowInfo*)m->d_tables, k,
                               m->embed, m->bf16, m->Hs, m->d, m->st));
    }
    if (np > 0) {
        std::vector<Chunk> ch{{seq, 0, np}};
        for (int sg = 0; sg < kMaxExits; ++sg)
            if ((s = run_chunks(m, sg, ch)) != NV_OK) return s;
    }
    NV_TRY(sync_and_check(m));
    S.n = np;
    for (int k = 0; k < kMaxExits; ++k) S.f[k] = np;
    for (int k = 0; k < 4; ++k) m->last_w[(size_t)seq * 4 + k] = NAN;
    return NV_OK;
}

// Logits and the inverse-CDF draw for sequences `seqs` (exit exit_of[i], 1-based) at their
// current positions; logits go to row `seq` of the logits buffer.
//   own heads:   the exit's RMSNorm and LM head on the hidden row (seqs share one exit);
//   shared head: hidden rows are gathered (seqs ordered by exit), exits 1..3 add their
//                adapter U silu(D h), then one pass of the final RMSNorm and LM head.
// u4: host copy of each listed sequence's token uniform, indexed by sequence (one stopping
// sequence takes the fused head product + draw), or null.
static nv_status run_heads(nv_model* m, const std::vector<int>& seqs, const std::vector<int>& exit_of,
                           const float* d_unif, const float* u4 = nullptr) {
    if (m->hl_busy[m->hl_next]) {
        NV_HIP(m, hipStreamSynchronize(m->st));
        stream_synced(m);
    }
    char* hl = m->h_headlist + (size_t)m->hl_next * m->list_bytes();
    m->hl_busy[m->hl_next] = true;
    m->hl_next ^= 1;
    const int ns = (int)seqs.size();
    for (int j = 0; j < ns; ++j) {
        const int i = seqs[j];
        nv_model::lseqs(hl)[j] = i;
        m->lrows(hl)[j] = RowInfo{i * m->max_ctx + m->seqs[i].n, i, m->seqs[i].n, 0};
        m->lorows(hl)[j] = RowInfo{i, i, 0, 0};
    }
    NV_HIP(m, hipMemcpyAsync(m->d_headlist, hl, m->list_bytes(), hipMemcpyHostToDevice, m->st));
    const int ex0 = exit_of[seqs[0]] - 1;
    GemmArgs g{};
    g.eps = m->cfg.norm_eps;
    g.wbf16 = m->bf16 ? 1 : 0;
    g.rms_ws = m->rms_ws;
    g.abf = m->abf;
    g.mfma_min_rows = m->mfma_min_rows;
    g.sk_ws = m->sk_ws;
    g.sk_cap = m->sk_cap;
    g.sk_min_rows = m->sk_min_rows;
    g.sk_max_rows = m->sk_max_rows;
    g.sk_ntb = m->sk_ntb;
    if (m->cfg.head_form == 1) {
        float* X = m->attn_o;   // [ns][d] gathered rows, then adapter outputs
        float* S = m->mlp;      // [ns][r] adapter hidden units
        const int d = m->d, r = m->cfg.adapter_dim;
        NV_TRY(timed(m, NV_TIME_EXIT_HEAD, (double)ns * d * 8, [&] {
            return launch_copy_rows(m->lrows(m->d_headlist), ns, m->Hs, d, X, m->st);
        }, "nv::k_copy_rows"));
        for (int j0 = 0; j0 < ns;) {
            const int k = exit_of[seqs[j0]] - 1;
            int j1 = j0;
            while (j1 < ns && exit_of[seqs[j1]] - 1 == k) ++j1;
            if (k < kMaxExits - 1) {
                GemmArgs a = g;
                a.A = X + (int64_t)j0 * d;
                a.lda = d;
                a.W = m->exits[k].adapter_down;
                a.N = r;
                a.K = d;
                a.R = j1 - j0;
                a.epi = EPI_SILU;
                a.out = S + (int64_t)j0 * r;
                a.ldo = r;
                NV_TRY(run_gemm(m, NV_TIME_EXIT_HEAD, a));
                GemmArgs b = g;
                b.A = S + (int64_t)j0 * r;
                b.lda = r;
                b.W = m->exits[k].adapter_up;
                b.N = d;
                b.K = r;
                b.R = j1 - j0;
                b.epi = EPI_RESID;
                b.out = X + (int64_t)j0 * d;
                b.ldo = d;
                NV_TRY(run_gemm(m, NV_TIME_EXIT_HEAD, b));
            }
            j0 = j1;
        }
        g.A = X;
        g.lda = d;
        g.a_rows = nullptr;
    } else {
        g.A = m->Hs;
        g.lda = m->d;
        g.a_rows = m->lrows(m->d_headlist);
        g.a_row0 = m->lrows(hl)[0].hrow;
    }
    // one stopping sequence: its logits row (the sequence index) is known here
    g.contig = ns == 1 ? 1 : 0;
    g.o_row0 = seqs[0];
    g.norm_w = m->exits[ex0].norm;
    g.W = m->exits[ex0].head;
    g.N = m->V;
    g.K = m->d;
    g.R = ns;
    g.epi = EPI_STORE;
    g.out = m->logits;
    g.ldo = m->V;
    g.o_rows = m->lorows(m->d_headlist);
    g.head = 1;
    if (ns == 1 && u4 && m->V % 8 == 0 && m->V / 8 <= XD_PER * XD_THREADS && head_gemv_ok(m)) {
        // one stopping sequence: the head product also writes its per-block softmax partials,
        // and one block draws the token from them
        g.head = 2;
        g.xd_part = m->xd_part;
        NV_TRY(run_gemm(m, NV_TIME_EXIT_HEAD, g));
        const float* lg = m->logits + (int64_t)seqs[0] * m->V;
        return timed(m, NV_TIME_OTHER, (double)(m->V / 8) * 8 + 32, [&] {
            return launch_exit_draw(m->xd_part, m->V / 8, lg, u4[seqs[0]], m->d_tok_out + seqs[0], m->st);
        }, "nv::k_exit_draw");
    }
    NV_TRY(run_gemm(m, NV_TIME_EXIT_HEAD, g));
    NV_TRY(timed(m, NV_TIME_OTHER, (double)ns * m->V * 4, [&] {
        return launch_sample(m->logits, m->V, nv_model::lseqs(m->d_headlist), ns, m->V, d_unif, m->d_tok_out,
                             m->st);
    }, "nv::k_sample"));
    return NV_OK;
}

// Wait until the gate kernels have published the decisions of `run` with this tag in
// mapped host memory.  The stream is polled now and then, so that a failed launch or a
// device fault is reported instead of waited on.
static nv_status wait_gate_flags(nv_model* m, const std::vector<int>& run, int tag) {
    const volatile int* f = m->h_flags;
    auto all_in = [&] {
        for (int i : run)
            if ((f[i] >> 1) != tag) return false;
        return true;
    };
    for (unsigned it = 1;; ++it) {
        if (all_in()) return NV_OK;
        if ((it & 255) == 0) {
            const hipError_t e = hipStreamQuery(m->st);
            if (e == hipSuccess) {
                if (all_in()) return NV_OK;
                m->dead = true;
                return fail(m, NV_EDEVICE, "gate decision missing after the stream drained");
            }
            if (e != hipErrorNotReady) NV_HIP(m, e);
        }
    }
}

// Router gate sg on the current rows of sequences `run`: the walk's decision (u_sg < w_sg)
// comes back to the host, which then launches the next segment or the head.  Every
// launch before the gate has completed when the decisions arrive (stream order), so the
// pinned staging buffers are free again.  `run` splits into the sequences that stop here
// and the rest.
static nv_status run_gates(nv_model* m, int sg, const std::vector<int>& run, const float* d_unif,
                           std::vector<int>* stopping, std::vector<int>* rest) {
    char* gl = m->h_gatelist;
    const int na = (int)run.size();
    for (int j = 0; j < na; ++j) {
        const int i = run[j];
        nv_model::lseqs(gl)[j] = i;
        m->lrows(gl)[j] = RowInfo{i * m->max_ctx + m->seqs[i].n, i, m->seqs[i].n, 0};
    }
    NV_HIP(m, hipMemcpyAsync(m->d_gatelist, gl, m->list_bytes(), hipMemcpyHostToDevice, m->st));
    m->gate_tag = m->gate_tag >= (1 << 29) ? 1 : m->gate_tag + 1;
    const int tag = m->gate_tag;
    if (m->cfg.router_form == 1) {
        const ExitPtrs& X = m->exits[sg];
        NV_TRY(timed(m, NV_TIME_OTHER, (double)na * m->d * 8 + (double)m->cfg.router_dim * m->d * 4, [&] {
            return launch_gate_mlp(m->lrows(m->d_gatelist), nv_model::lseqs(m->d_gatelist), na, m->Hs, m->d,
                                   X.router_w1, X.router_b1, X.router_w2, m->cfg.router_dim, X.bias, d_unif, sg,
                                   m->router_hid, m->d_w, m->d_stop, m->st, m->d_flags, tag);
        }, "nv::k_router_hidden + nv::k_router_out"));
    } else {
        NV_TRY(timed(m, NV_TIME_OTHER, (double)na * m->d * 8, [&] {
            return launch_gate(m->lrows(m->d_gatelist), nv_model::lseqs(m->d_gatelist), na, m->Hs, m->d,
                               m->exits[sg].gate_w, m->exits[sg].bias, d_unif, sg, m->d_w, m->d_stop, m->st,
                               m->d_flags, tag);
        }, "nv::k_gate"));
    }
    NV_TRY(wait_gate_flags(m, run, tag));
    stream_synced(m);
    for (int i : run) ((m->h_flags[i] & 1) ? *stopping : *rest).push_back(i);
    return NV_OK;
}

static nv_status step_impl(nv_model* m, const float* u, const int32_t* forced, int32_t* tok_out, int32_t* exit_out) {
    if (!m) return NV_EINVAL;
    if (m->dead) return fail(m, NV_EDEVICE, "model handle unusable after a device error");
    if (!u || !tok_out || !exit_out) return fail(m, NV_EINVAL, "null pointer");
    int n = 0;
    while (n < m->max_batch && m->seqs[n].live) ++n;
    if (n == 0) return fail(m, NV_ESTATE, "no prefilled sequence");
    for (int i = n; i < m->max_batch; ++i)
        if (m->seqs[i].live) return fail(m, NV_ESTATE, "prefilled sequences are not numbered 0..n-1");
    for (int i = 0; i < n * 4; ++i)
        if (!(u[i] >= 0.0f && u[i] < 1.0f)) return fail(m, NV_EINVAL, "uniform outside [0,1) or NaN");
    if (forced)
        for (int i = 0; i < n; ++i)
            if (forced[i] < 0 || forced[i] >= m->V) return fail(m, NV_EINVAL, "forced token out of range");
    for (int i = 0; i < n; ++i)
        if (m->seqs[i].n + 1 > m->max_ctx) return fail(m, NV_ECAPACITY, "sequence reached max_ctx");

    nv_status s = stage_sync(m);
    if (s != NV_OK) return s;
    // uniforms, pending tokens and current-position rows in one upload
    char* hb = m->h_stepblk;
    std::memcpy(nv_model::unif(hb), u, (size_t)n * 16);
    for (int i = 0; i < n; ++i) {
        m->tok_in(hb)[i] = m->seqs[i].pending;
        m->cur_rows(hb)[i] = RowInfo{i * m->max_ctx + m->seqs[i].n, i, m->seqs[i].n, 0};
    }
    NV_HIP(m, hipMemcpyAsync(m->d_stepblk, hb, m->stepblk_bytes(), hipMemcpyHostToDevice, m->st));
    const float* d_unif = nv_model::unif(m->d_stepblk);
    NV_TRY(timed(m, NV_TIME_OTHER, (double)n * m->d * (m->plan.es + 4), [&] {
        return launch_embed(m->tok_in(m->d_stepblk), m->cur_rows(m->d_stepblk), n, m->embed, m->bf16, m->Hs, m->d,
                            m->st);
    }, "nv::k_embed"));

    std::vector<int> active(n), exit_of(n, kMaxExits);
    for (int i = 0; i < n; ++i) active[i] = i;
    for (int i = 0; i < n * 4; ++i) m->last_w[i] = NAN;
    std::vector<float> u4(n);
    for (int i = 0; i < n; ++i) u4[i] = u[i * 4 + 3];
    int* htok_out = (int*)(m->h_out + (size_t)m->max_batch * 4);
    double* hw = (double*)(m->h_out + (size_t)m->max_batch * 8);
    std::vector<int> stopped;   // shared head: the step's stopping sequences, in exit order
    for (int sg = 0; sg < kMaxExits && !active.empty(); ++sg) {
        std::vector<Chunk> ch;
        for (int i : active) {
            const SeqHost& S = m->seqs[i];
            ch.push_back({i, S.f[sg], S.n - S.f[sg] + 1});
        }
        if ((s = run_chunks(m, sg, ch)) != NV_OK) return s;
        std::vector<int> stopping;
        if (sg < kMaxExits - 1) {
            std::vector<int> rest;
            NV_TRY(run_gates(m, sg, active, d_unif, &stopping, &rest));
            active.swap(rest);
        } else {
            stopping = active;
            active.clear();
        }
        for (int i : stopping) exit_of[i] = sg + 1;
        if (m->cfg.head_form == 1) {
            // shared head: every stopping sequence of this step goes through one head pass
            for (int i : stopping) stopped.push_back(i);
        } else if (!stopping.empty()) {
            NV_TRY(run_heads(m, stopping, exit_of, d_unif, u4.data()));
        }
    }
    if (!stopped.empty()) NV_TRY(run_heads(m, stopped, exit_of, d_unif, u4.data()));
    NV_HIP(m, hipMemcpyAsync(htok_out, m->d_tok_out, (size_t)n * 4, hipMemcpyDeviceToHost, m->st));
    NV_HIP(m, hipMemcpyAsync(hw, m->d_w, (size_t)n * 32, hipMemcpyDeviceToHost, m->st));
    NV_TRY(sync_and_check(m));
    if (m->timing) NV_TRY(resolve_timing(m));
    for (int i = 0; i < n; ++i)
        if (htok_out[i] < 0 || htok_out[i] >= m->V) {
            m->dead = true;
            return fail(m, NV_EDEVICE, "exit draw: the head product's blocks did not all report");
        }
    for (int i = 0; i < n; ++i) {
        SeqHost& S = m->seqs[i];
        const int e = exit_of[i];
        for (int k = 0; k < e && k < kMaxExits - 1; ++k) m->last_w[(size_t)i * 4 + k] = hw[i * 4 + k];
        if (e == kMaxExits) m->last_w[(size_t)i * 4 + 3] = 1.0;
        for (int k = 0; k < e; ++k) S.f[k] = S.n + 1;
        S.n += 1;
        S.last_exit = e;
        tok_out[i] = htok_out[i];
        exit_out[i] = e;
        S.pending = forced ? forced[i] : htok_out[i];
    }
    return NV_OK;
}

nv_status nv_step(nv_model* m, const float* uniforms, int32_t* tokens_out, int32_t* exits_out) {
    return step_impl(m, uniforms, nullptr, tokens_out, exits_out);
}

nv_status nv_step_forced(nv_model* m, const float* uniforms, const int32_t* next_inputs, int32_t* tokens_out,
                         int32_t* exits_out) {
    if (!next_inputs) return m ? fail(m, NV_EINVAL, "null next_inputs") : NV_EINVAL;
    return step_impl(m, uniforms, next_inputs, tokens_out, exits_out);
}

// Decoding with sequences advancing through the segments independently.  Each tick runs
// one segment over the sequences whose current token waits there (with their deferred
// rows), then that segment's gate; the sequences that stop get their head and draw, and
// their next token enters segment 1.  The policy picks the tick's segment.  Each
// sequence's computation is the one nv_step performs for it, so its tokens and exits
// depend only on its own uniforms.
nv_status nv_generate(nv_model* m, const int32_t* seqs, int32_t n_seq, int32_t n_tokens, const float* uniforms,
                      int32_t policy, int32_t* tokens_out, int32_t* exits_out) {
    if (!m) return NV_EINVAL;
    if (m->dead) return fail(m, NV_EDEVICE, "model handle unusable after a device error");
    if (!seqs || !uniforms || !tokens_out || !exits_out) return fail(m, NV_EINVAL, "null pointer");
    if (n_seq < 1 || n_seq > m->max_batch) return fail(m, NV_EINVAL, "n_seq outside 1..max_batch");
    if (n_tokens < 0) return fail(m, NV_EINVAL, "negative n_tokens");
    if (policy != NV_SCHED_LOCKSTEP && policy != NV_SCHED_GREEDY) return fail(m, NV_EINVAL, "unknown policy");
    std::vector<int> idx_of(m->max_batch, -1);
    for (int i = 0; i < n_seq; ++i) {
        const int q = seqs[i];
        if (q < 0 || q >= m->max_batch) return fail(m, NV_EINVAL, "sequence index out of range");
        if (idx_of[q] >= 0) return fail(m, NV_EINVAL, "sequence listed twice");
        idx_of[q] = i;
        if (!m->seqs[q].live) return fail(m, NV_ESTATE, "sequence not prefilled");
        if (m->seqs[q].n + (int64_t)n_tokens > m->max_ctx) return fail(m, NV_ECAPACITY, "sequence would pass max_ctx");
    }
    const int T = n_tokens;
    for (size_t i = 0; i < (size_t)n_seq * T * 4; ++i)
        if (!(uniforms[i] >= 0.0f && uniforms[i] < 1.0f)) return fail(m, NV_EINVAL, "uniform outside [0,1) or NaN");
    if (T == 0) return NV_OK;
    NV_HIP(m, hipStreamSynchronize(m->st));
    stream_synced(m);

    struct Gen {
        int slot, t, q, age;   // token index, segment its current token waits at, ticks waited
        bool fresh;            // current token not embedded yet
    };
    std::vector<Gen> g(n_seq);
    char* hb = m->h_stepblk;
    for (int i = 0; i < n_seq; ++i) {
        g[i] = Gen{seqs[i], 0, 0, 0, true};
        m->tok_in(hb)[seqs[i]] = m->seqs[seqs[i]].pending;
    }
    // the embedding reads sequence s's input token at d_tok_out[s], where its draws land
    NV_HIP(m, hipMemcpyAsync(m->d_tok_out, m->tok_in(hb), (size_t)m->max_batch * 4, hipMemcpyHostToDevice, m->st));
    m->sb_busy = true;
    const float* d_unif = nv_model::unif(m->d_stepblk);

    // drawn tokens come back through a ring of pinned buffers; an entry is read after
    // the next stream synchronisation
    struct RingEntry {
        std::vector<std::pair<int, int>> items;   // (slot, token index)
        bool pending = false;
    };
    RingEntry ring[kRing];
    int ring_next = 0;
    auto drain = [&]() {
        for (int e = 0; e < kRing; ++e) {
            if (!ring[e].pending) continue;
            const int* hv = m->h_ring + (size_t)e * m->max_batch;
            for (const auto& it : ring[e].items) tokens_out[(size_t)idx_of[it.first] * T + it.second] = hv[it.first];
            ring[e].items.clear();
            ring[e].pending = false;
        }
    };
    auto full_sync = [&]() -> nv_status {
        NV_HIP(m, hipStreamSynchronize(m->st));
        stream_synced(m);
        drain();
        return NV_OK;
    };

    std::vector<int> exit_of(m->max_batch, kMaxExits);
    std::vector<float> u4(m->max_batch, 0.f);
    int remaining = n_seq;
    while (remaining > 0) {
        int cnt[kMaxExits] = {0, 0, 0, 0}, oldest[kMaxExits] = {0, 0, 0, 0};
        for (const Gen& x : g)
            if (x.t < T) {
                ++cnt[x.q];
                oldest[x.q] = std::max(oldest[x.q], x.age);
            }
        int sg = 0;
        if (policy == NV_SCHED_LOCKSTEP) {
            // finish the round's deeper segments before the next tokens start
            for (int k = 1; k < kMaxExits; ++k)
                if (cnt[k]) {
                    sg = k;
                    break;
                }
        } else {
            // the segment with the most waiting sequences, plus sched_age times the
            // longest wait there in ticks; ties go to the deeper segment
            double best = -1.0;
            for (int k = 0; k < kMaxExits; ++k)
                if (cnt[k]) {
                    const double sc = cnt[k] + m->sched_age * oldest[k];
                    if (sc >= best) {
                        best = sc;
                        sg = k;
                    }
                }
        }
        std::vector<int> run;
        for (const Gen& x : g)
            if (x.t < T && x.q == sg) run.push_back(x.slot);
        if (sg == 0) {
            // new tokens: their uniforms and embeddings
            int nf = 0;
            for (const Gen& x : g)
                if (x.t < T && x.q == 0 && x.fresh) ++nf;
            if (nf > 0) {
                if (m->sb_busy) NV_TRY(full_sync());
                int j = 0;
                for (Gen& x : g) {
                    if (!(x.t < T && x.q == 0 && x.fresh)) continue;
                    const SeqHost& S = m->seqs[x.slot];
                    const float* u = uniforms + ((size_t)idx_of[x.slot] * T + x.t) * 4;
                    for (int c = 0; c < 4; ++c) nv_model::unif(hb)[x.slot * 4 + c] = u[c];
                    m->cur_rows(hb)[j++] = RowInfo{x.slot * m->max_ctx + S.n, x.slot, S.n, 0};
                    x.fresh = false;
                }
                NV_HIP(m, hipMemcpyAsync(m->d_stepblk, hb, m->stepblk_bytes(), hipMemcpyHostToDevice, m->st));
                m->sb_busy = true;
                NV_TRY(timed(m, NV_TIME_OTHER, (double)nf * m->d * (m->plan.es + 4), [&] {
                    return launch_embed(m->d_tok_out, m->cur_rows(m->d_stepblk), nf, m->embed, m->bf16, m->Hs, m->d,
                                        m->st, 1);
                }, "nv::k_embed"));
            }
        }
        std::vector<Chunk> ch;
        for (int slot : run) {
            const SeqHost& S = m->seqs[slot];
            ch.push_back({slot, S.f[sg], S.n - S.f[sg] + 1});
        }
        nv_status s = run_chunks(m, sg, ch);
        if (s != NV_OK) return s;
        std::vector<int> stopping, rest;
        if (sg < kMaxExits - 1) {
            NV_TRY(run_gates(m, sg, run, d_unif, &stopping, &rest));
            drain();
        } else {
            stopping = run;
        }
        for (Gen& x : g)
            if (x.t < T) ++x.age;
        for (int slot : rest) g[idx_of[slot]].q = sg + 1;
        if (stopping.empty()) continue;
        for (int slot : stopping) {
            exit_of[slot] = sg + 1;
            // the token uniform on the host, for the head product with the fused draw
            u4[slot] = uniforms[((size_t)idx_of[slot] * T + g[idx_of[slot]].t) * 4 + 3];
        }
        NV_TRY(run_heads(m, stopping, exit_of, d_unif, u4.data()));
        if (ring[ring_next].pending) NV_TRY(full_sync());
        NV_HIP(m, hipMemcpyAsync(m->h_ring + (size_t)ring_next * m->max_batch, m->d_tok_out,
                                 (size_t)m->max_batch * 4, hipMemcpyDeviceToHost, m->st));
        RingEntry& E = ring[ring_next];
        E.pending = true;
        ring_next = (ring_next + 1) % kRing;
        for (int slot : stopping) {
            Gen& x = g[idx_of[slot]];
            SeqHost& S = m->seqs[slot];
            const int e = sg + 1;
            E.items.push_back({slot, x.t});
            exits_out[(size_t)idx_of[slot] * T + x.t] = e;
            for (int k = 0; k < e; ++k) S.f[k] = S.n + 1;
            S.n += 1;
            S.last_exit = e;
            x.t += 1;
            x.q = 0;
            x.age = 0;
            x.fresh = true;
            if (x.t == T) --remaining;
        }
    }
    NV_TRY(sync_and_check(m));
    drain();
    if (m->timing) NV_TRY(resolve_timing(m));
    for (int i = 0; i < n_seq; ++i) {
        SeqHost& S = m->seqs[seqs[i]];
        S.pending = tokens_out[(size_t)i * T + T - 1];
        for (int k = 0; k < 4; ++k) m->last_w[(size_t)seqs[i] * 4 + k] = NAN;
    }
    return NV_OK;
}

// Mixture objective, rows o..o+k-1 of the loss pass after segment sg: the exit's router
// output for each row, its logits (own head, or adapter + shared head) into the loss logits
// workspace and log pi_k of each row's target token.
static nv_status loss_exit(nv_model* m, int sg, int o, int k) {
    const ExitPtrs& X = m->exits[sg];
    const RowInfo* rows = m->loss_rows + o;
    if (sg < kMaxExits - 1) {
        if (m->cfg.router_form == 1) {
            NV_TRY(timed(m, NV_TIME_OTHER, (double)k * m->d * 8 + (double)m->cfg.router_dim * m->d * 4, [&] {
                return launch_gate_mlp(rows, m->loss_ids + o, k, m->Hs, m->d, X.router_w1, X.router_b1, X.router_w2,
                                       m->cfg.router_dim, X.bias, nullptr, sg, m->loss_hid, m->loss_w, nullptr,
                                       m->st);
            }, "nv::k_router_hidden + nv::k_router_out"));
        } else {
            NV_TRY(timed(m, NV_TIME_OTHER, (double)k * m->d * 8, [&] {
                return launch_gate(rows, m->loss_ids + o, k, m->Hs, m->d, X.gate_w, X.bias, nullptr, sg, m->loss_w,
                                   nullptr, m->st);
            }, "nv::k_gate"));
        }
    }
    GemmArgs g{};
    g.eps = m->cfg.norm_eps;
    g.wbf16 = m->bf16 ? 1 : 0;
    g.rms_ws = m->rms_ws;
    g.abf = m->abf;
    g.mfma_min_rows = m->mfma_min_rows;
    const int d = m->d;
    if (m->cfg.head_form == 1) {
        float* A = m->attn_o;   // [k][d] gathered rows, then adapter outputs
        NV_TRY(timed(m, NV_TIME_EXIT_HEAD, (double)k * d * 8, [&] {
            return launch_copy_rows(rows, k, m->Hs, d, A, m->st);
        }, "nv::k_copy_rows"));
        if (sg < kMaxExits - 1) {
            const int r = m->cfg.adapter_dim;
            GemmArgs a = g;
            a.A = A;
            a.lda = d;
            a.W = X.adapter_down;
            a.N = r;
            a.K = d;
            a.R = k;
            a.epi = EPI_SILU;
            a.out = m->mlp;
            a.ldo = r;
            NV_TRY(run_gemm(m, NV_TIME_EXIT_HEAD, a));
            GemmArgs b = g;
            b.A = m->mlp;
            b.lda = r;
            b.W = X.adapter_up;
            b.N = d;
            b.K = r;
            b.R = k;
            b.epi = EPI_RESID;
            b.out = A;
            b.ldo = d;
            NV_TRY(run_gemm(m, NV_TIME_EXIT_HEAD, b));
        }
        g.A = A;
        g.lda = d;
    } else {
        g.A = m->Hs;
        g.lda = d;
        g.a_rows = rows;
    }
    g.norm_w = X.norm;
    g.W = X.head;
    g.N = m->V;
    g.K = d;
    g.R = k;
    g.epi = EPI_STORE;
    g.out = m->loss_logits;
    g.ldo = m->V;
    g.head = 1;
    // on the long-chunk path the head product reduces its logits to per-row partials in
    // its epilogue (the logits never reach memory); elsewhere they are stored and k_xent
    // reads them back
    if (gemm_uses_bf16_rows(g)) {
        g.out = nullptr;
        g.xent_part = m->loss_xpart;
        g.xent_tgt = m->loss_xtgt;
        g.xent_targets = m->loss_tgt + o;
        NV_TRY(run_gemm(m, NV_TIME_EXIT_HEAD, g));
        NV_TRY(timed(m, NV_TIME_OTHER, (double)k * (m->V / 64) * 8, [&] {
            return launch_xent_merge(m->loss_xpart, m->loss_xtgt, k, m->V / 64, m->loss_lp + (int64_t)o * 4, 4, sg,
                                     m->st);
        }, "nv::k_xent_merge"));
        return NV_OK;
    }
    NV_TRY(run_gemm(m, NV_TIME_EXIT_HEAD, g));
    NV_TRY(timed(m, NV_TIME_OTHER, (double)k * m->V * 4, [&] {
        return launch_xent(m->loss_logits, m->V, k, m->V, m->loss_tgt + o, m->loss_lp + (int64_t)o * 4, 4, sg, m->st);
    }, "nv::k_xent"));
    return NV_OK;
}

nv_status nv_mixture_loss(nv_model* m, int32_t seq, const int32_t* tokens, int32_t n, double beta, double* out,
                          double* per_pos) {
    nv_status s = check_seq(m, seq);
    if (s != NV_OK) return s;
    if (!tokens || !out || n < 2) return fail(m, NV_EINVAL, "the mixture objective needs out and at least two tokens");
    if (n > m->max_ctx) return fail(m, NV_ECAPACITY, "token sequence longer than max_ctx");
    if (!std::isfinite(beta)) return fail(m, NV_EINVAL, "beta is not finite");
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->V) return fail(m, NV_EINVAL, "token id out of range");
    const int np = n - 1;
    // row tables for the whole pass: rows, row ids, target tokens
    if ((s = stage_sync(m)) != NV_OK) return s;
    std::vector<RowInfo> hr(np);
    std::vector<int> ids(np), tgt(np);
    for (int i = 0; i < np; ++i) {
        hr[i] = RowInfo{seq * m->max_ctx + i, seq, i, 0};
        ids[i] = i;
        tgt[i] = tokens[i + 1];
    }
    NV_HIP(m, hipMemcpyAsync(m->loss_rows, hr.data(), sizeof(RowInfo) * np, hipMemcpyHostToDevice, m->st));
    NV_HIP(m, hipMemcpyAsync(m->loss_ids, ids.data(), 4 * (size_t)np, hipMemcpyHostToDevice, m->st));
    NV_HIP(m, hipMemcpyAsync(m->loss_tgt, tgt.data(), 4 * (size_t)np, hipMemcpyHostToDevice, m->st));
    NV_HIP(m, hipStreamSynchronize(m->st));
    stream_synced(m);
    // the prefill of the first n-1 tokens, with every exit's router and head after its segment
    SeqHost& S = m->seqs[seq];
    S = SeqHost();
    S.live = true;
    S.pending = tokens[n - 1];
    const int cap = m->plan.R_max;
    for (int o = 0; o < np; o += cap) {
        const int k = std::min(cap, np - o);
        if ((s = stage_sync(m)) != NV_OK) return s;
        int* ht = (int*)m->h_stage;
        for (int i = 0; i < k; ++i) ht[i] = tokens[o + i];
        NV_HIP(m, hipMemcpyAsync(m->d_tables, m->h_stage, 4 * (size_t)k, hipMemcpyHostToDevice, m->st));
        m->stage_busy = true;
        NV_TRY(timed(m, NV_TIME_OTHER, (double)k * m->d * (m->plan.es + 4), [&] {
            return launch_embed((const int*)m->d_tables, m->loss_rows + o, k, m->embed, m->bf16, m->Hs, m->d, m->st);
        }, "nv::k_embed"));
    }
    const std::vector<Chunk> ch{{seq, 0, np}};
    for (int sg = 0; sg < kMaxExits; ++sg) {
        if ((s = run_chunks(m, sg, ch)) != NV_OK) return s;
        for (int o = 0; o < np; o += m->plan.loss_ch)
            NV_TRY(loss_exit(m, sg, o, std::min(m->plan.loss_ch, np - o)));
    }
    ExitDepths dep{};
    for (int k = 0; k < kMaxExits; ++k) dep.layer[k] = m->cfg.exit_layer[k];
    dep.L = m->L;
    NV_TRY(timed(m, NV_TIME_OTHER, (double)np * 80, [&] {
        return launch_loss_reduce(m->loss_w, m->loss_lp, np, dep, m->loss_nll, m->loss_depth, m->loss_sums, m->st);
    }, "nv::k_loss_reduce"));
    double sums[2];
    NV_HIP(m, hipMemcpyAsync(sums, m->loss_sums, 16, hipMemcpyDeviceToHost, m->st));
    std::vector<double> pw, plp, pn, pd;
    if (per_pos) {
        pw.resize((size_t)np * 4);
        plp.resize((size_t)np * 4);
        pn.resize(np);
        pd.resize(np);
        NV_HIP(m, hipMemcpyAsync(pw.data(), m->loss_w, (size_t)np * 32, hipMemcpyDeviceToHost, m->st));
        NV_HIP(m, hipMemcpyAsync(plp.data(), m->loss_lp, (size_t)np * 32, hipMemcpyDeviceToHost, m->st));
        NV_HIP(m, hipMemcpyAsync(pn.data(), m->loss_nll, (size_t)np * 8, hipMemcpyDeviceToHost, m->st));
        NV_HIP(m, hipMemcpyAsync(pd.data(), m->loss_depth, (size_t)np * 8, hipMemcpyDeviceToHost, m->st));
    }
    NV_TRY(sync_and_check(m));
    if (m->timing) NV_TRY(resolve_timing(m));
    S.n = np;
    for (int k = 0; k < kMaxExits; ++k) S.f[k] = np;
    for (int k = 0; k < 4; ++k) m->last_w[(size_t)seq * 4 + k] = NAN;
    out[0] = sums[0];
    out[1] = sums[1];
    out[2] = sums[0] + beta * sums[1];
    if (per_pos)
        for (int i = 0; i < np; ++i) {
            double* r = per_pos + (size_t)i * 10;
            for (int k = 0; k < 4; ++k) {
                r[k] = pw[(size_t)i * 4 + k];
                r[4 + k] = plp[(size_t)i * 4 + k];
            }
            r[8] = pn[i];
            r[9] = pd[i];
        }
    return NV_OK;
}

nv_status nv_flush(nv_model* m, int32_t seq) {
    if (!m) return NV_EINVAL;
    if (m->dead) return fail(m, NV_EDEVICE, "model handle unusable after a device error");
    if (seq < -1 || seq >= m->max_batch) return fail(m, NV_EINVAL, "sequence index out of range");
    std::vector<int> targets;
    for (int i = 0; i < m->max_batch; ++i)
        if (m->seqs[i].live && (seq == -1 || seq == i)) targets.push_back(i);
    nv_status s;
    for (int sg = 1; sg < kMaxExits; ++sg) {
        std::vector<Chunk> ch;
        for (int i : targets) {
            const SeqHost& S = m->seqs[i];
            if (S.n > S.f[sg]) ch.push_back({i, S.f[sg], S.n - S.f[sg]});
        }
        if (!ch.empty() && (s = run_chunks(m, sg, ch)) != NV_OK) return s;
        for (int i : targets) m->seqs[i].f[sg] = m->seqs[i].n;
    }
    return sync_and_check(m);
}

nv_status nv_debug_frontiers(nv_model* m, int32_t seq, int32_t* n_consumed, int32_t frontier[4]) {
    nv_status s = check_seq(m, seq);
    if (s != NV_OK) return s;
    if (!n_consumed || !frontier) return fail(m, NV_EINVAL, "null pointer");
    *n_consumed = m->seqs[seq].n;
    for (int k = 0; k < kMaxExits; ++k) frontier[k] = m->seqs[seq].f[k];
    return NV_OK;
}

nv_status nv_debug_logits(nv_model* m, int32_t seq, float* out) {
    nv_status s = check_seq(m, seq);
    if (s != NV_OK) return s;
    if (!out) return fail(m, NV_EINVAL, "null pointer");
    NV_HIP(m, hipMemcpy(out, m->logits + (size_t)seq * m->V, (size_t)m->V * 4, hipMemcpyDeviceToHost));
    return NV_OK;
}

nv_status nv_debug_gates(nv_model* m, int32_t seq, double* out) {
    nv_status s = check_seq(m, seq);
    if (s != NV_OK) return s;
    if (!out) return fail(m, NV_EINVAL, "null pointer");
    for (int k = 0; k < 4; ++k) out[k] = m->last_w[(size_t)seq * 4 + k];
    return NV_OK;
}

nv_status nv_debug_kv(nv_model* m, int32_t seq, int32_t layer, int32_t pos0, int32_t n, float* k_out,
                      float* v_out) {
    nv_status s = check_seq(m, seq);
    if (s != NV_OK) return s;
    if (!k_out || !v_out || layer < 0 || layer >= m->L || pos0 < 0 || n < 0 || pos0 + n > m->max_ctx)
        return fail(m, NV_EINVAL, "bad kv range");
    NV_HIP(m, hipStreamSynchronize(m->st));
    const size_t kes = m->plan.kes;
    std::vector<char> buf((size_t)n * m->hd * kes);
    for (int which = 0; which < 2; ++which)
        for (int h = 0; h < m->H; ++h) {
            const size_t base = ((((size_t)seq * m->L + layer) * 2 + which) * m->H + h) * (size_t)m->max_ctx * m->hd;
            NV_HIP(m, hipMemcpy(buf.data(), (char*)m->kv + (base + (size_t)pos0 * m->hd) * kes, buf.size(),
                                hipMemcpyDeviceToHost));
            float* dst = which ? v_out : k_out;
            for (int p = 0; p < n; ++p)
                for (int e = 0; e < m->hd; ++e) {
                    float v;
                    const size_t i = (size_t)p * m->hd + e;
                    if (kes == 2) {
                        uint32_t b = ((uint32_t)((uint16_t*)buf.data())[i]) << 16;
                        std::memcpy(&v, &b, 4);
                    } else {
                        v = ((float*)buf.data())[i];
                    }
                    dst[((size_t)p * m->H + h) * m->hd + e] = v;
                }
        }
    return NV_OK;
}

nv_status nv_debug_hidden(nv_model* m, int32_t seq, int32_t pos0, int32_t n, float* out) {
    nv_status s = check_seq(m, seq);
    if (s != NV_OK) return s;
    if (!out || pos0 < 0 || n < 0 || pos0 + n > m->max_ctx) return fail(m, NV_EINVAL, "bad hidden range");
    NV_HIP(m, hipStreamSynchronize(m->st));
    NV_HIP(m, hipMemcpy(out, m->Hs + ((size_t)seq * m->max_ctx + pos0) * m->d, (size_t)n * m->d * 4,
                        hipMemcpyDeviceToHost));
    return NV_OK;
}

nv_status nv_timing_enable(nv_model* m, int32_t on) {
    if (!m) return NV_EINVAL;
    if (on < 0 || on > 2) return fail(m, NV_EINVAL, "timing mode must be 0, 1 or 2");
    if (m->dead) return fail(m, NV_EDEVICE, "model handle unusable after a device error");
    NV_HIP(m, hipStreamSynchronize(m->st));
    if (on && m->ev.empty()) {
        m->ev.resize(2 * kEventPairs);
        m->ev_kind.resize(kEventPairs);
        m->ev_bytes.resize(kEventPairs);
        m->ev_name.resize(kEventPairs);
        m->ev_stamped.assign(kEventPairs, 0);
        NV_HIP(m, hipMalloc((void**)&m->d_stamps, kEventPairs * 16));
        NV_HIP(m, hipMalloc((void**)&m->d_blkstamps, (size_t)STAMP_BLOCKS * 16));
        std::vector<unsigned long long> blk(2 * STAMP_BLOCKS);
        for (int b = 0; b < STAMP_BLOCKS; ++b) {
            blk[2 * b] = ~0ull;
            blk[2 * b + 1] = 0ull;
        }
        NV_HIP(m, hipMemcpy(m->d_blkstamps, blk.data(), blk.size() * 8, hipMemcpyHostToDevice));
        int khz = 0;
        NV_HIP(m, hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, 0));
        m->wall_khz = khz > 0 ? (double)khz : 1e5;
        for (auto& e : m->ev) NV_HIP(m, hipEventCreate(&e));
    }
    m->ev_used = 0;
    m->kstats.clear();
    if (on) NV_TRY(resolve_timing(m));   // also resets the device spans
    for (int k = 0; k < NV_TIME_CLASSES; ++k) {
        m->t_ms[k] = m->t_bytes[k] = 0;
        m->t_n[k] = 0;
    }
    m->timing = on != 0;
    m->timing_stamps = on == 2;
    return NV_OK;
}

nv_status nv_timing_read(nv_model* m, double* ms, double* bytes, int64_t* launches) {
    if (!m || !ms || !bytes || !launches) return m ? fail(m, NV_EINVAL, "null pointer") : NV_EINVAL;
    NV_HIP(m, hipStreamSynchronize(m->st));
    NV_TRY(resolve_timing(m));
    for (int k = 0; k < NV_TIME_CLASSES; ++k) {
        ms[k] = m->t_ms[k];
        bytes[k] = m->t_bytes[k];
        launches[k] = m->t_n[k];
    }
    return NV_OK;
}

nv_status nv_timing_kernels(nv_model* m, char* out, size_t cap) {
    if (!m || !out || cap == 0) return m ? fail(m, NV_EINVAL, "null pointer") : NV_EINVAL;
    NV_HIP(m, hipStreamSynchronize(m->st));
    NV_TRY(resolve_timing(m));
    std::string txt;
    char line[512];
    for (const auto& ks : m->kstats) {
        snprintf(line, sizeof(line), "%d\t%lld\t%.6f\t%.0f\t%.6f\t%s\n", ks.kind, (long long)ks.n, ks.ms, ks.bytes,
                 ks.n_span == ks.n ? ks.span_ms : -1.0, ks.name.c_str());
        txt += line;
    }
    if (txt.size() + 1 > cap) return fail(m, NV_ECAPACITY, "timing report buffer too small");
    std::memcpy(out, txt.c_str(), txt.size() + 1);
    return NV_OK;
}

}  // extern "C"
