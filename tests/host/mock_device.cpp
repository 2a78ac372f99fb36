// Host stand-ins for the HIP runtime calls and the kernel launch wrappers that libnvium's host
// runtime (nv_runtime.cpp) uses, so that the runtime builds and runs on a machine without a
// GPU under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Device memory is host memory and every launch completes on the calling thread.  No
// stand-in computes the model.  Each one checks the plan the runtime hands the kernel it
// replaces, and writes placeholder outputs that make the decode walk deterministic.
//
// Checks, for every launch:
//   - row tables: row (seq, pos) lives at hidden row seq * max_ctx + pos, pos < max_ctx;
//   - per hidden row, the block products run in model order: QKV, O, gate/up, down of layer 0,
//     then of layer 1, ...; a router gate k (or an exit head) reads a row that has passed
//     exactly the layers up to exit k;
//   - attention: every key an item reads has its K/V written at that layer (the KV
//     completeness the deferred layers must restore); the splits of one (row block, head)
//     tile [0, last row's position + 1) without gaps, overlaps or empty pieces; no two
//     items write the same partial slot;
//   - split merges (the combine pass and the O product that merges on load) read only
//     slots the last attention launch wrote.
// Placeholder outputs: gate w = 1/2 and stop iff u_k < 1/2; a draw gives token
// floor(u_4 * V); loss terms are fixed finite values.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "nv_internal.h"

// ------------------------------------------------------------------------------------------
// Checks
// ------------------------------------------------------------------------------------------

[[noreturn]] static void violated(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::fprintf(stderr, "mock device: plan check failed: ");
    std::vfprintf(stderr, fmt, ap);
    std::fprintf(stderr, "\n");
    va_end(ap);
    std::fflush(stderr);
    std::abort();
}

#define CHECK(cond, ...)                     \
    do {                                     \
        if (!(cond)) violated(__VA_ARGS__); \
    } while (0)

namespace {

struct RowState {
    int layer = 0;   // layers completed
    int phase = 0;   // products of the current layer done: 0 none, 1 QKV, 2 O, 3 gate/up
};

struct MockState {
    int max_ctx = 0, hd = 0;
    nv::LayerDims D{};
    bool have_dims = false;
    std::unordered_map<int, RowState> rows;      // hidden row -> state
    std::unordered_map<int, int> embedded;       // hidden row -> token embedded there
    std::map<std::pair<int, int>, std::vector<unsigned char>> kv;   // (layer, seq) -> written per position
    std::set<int> slots;                         // partial slots of the last attention launch
    long long launches = 0;
    std::map<void*, size_t> allocs;              // live device allocations
    unsigned long long* stamp = nullptr;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
};

MockState g_mock;

int seg_len() { return g_mock.D.L / 4; }

void check_row(const nv::RowInfo& r, const char* what) {
    CHECK(g_mock.max_ctx > 0, "%s: launch before the model's RoPE table", what);
    CHECK(r.seq >= 0 && r.pos >= 0 && r.pos < g_mock.max_ctx, "%s: row (seq %d, pos %d) outside max_ctx %d", what,
          r.seq, r.pos, g_mock.max_ctx);
    CHECK(r.hrow == r.seq * g_mock.max_ctx + r.pos, "%s: hidden row %d is not seq %d * max_ctx + pos %d", what, r.hrow,
          r.seq, r.pos);
}

nv::RowInfo row_of(int hrow) { return nv::RowInfo{hrow, hrow / g_mock.max_ctx, hrow % g_mock.max_ctx, 0}; }

std::vector<unsigned char>& kv_of(int layer, int seq) {
    auto& v = g_mock.kv[{layer, seq}];
    if (v.empty()) v.assign((size_t)g_mock.max_ctx, 0);
    return v;
}

// The row a product reads from A (hidden rows only), or -1.
int a_hidden_row(const nv::GemmArgs& a, int r) {
    if (!a.a_rows) return -1;
    if (a.contig) return a.a_row0 + r;
    check_row(a.a_rows[r], "product input rows");
    return a.a_rows[r].hrow;
}

int o_hidden_row(const nv::GemmArgs& a, int r) {
    if (!a.o_rows) return -1;
    if (a.contig) return a.o_row0 + r;
    check_row(a.o_rows[r], "product output rows");
    return a.o_rows[r].hrow;
}

void check_exit_row(int hrow, int exit_k, const char* what) {
    const RowState& s = g_mock.rows[hrow];
    CHECK(s.phase == 0 && s.layer == (exit_k + 1) * seg_len(),
          "%s: row (seq %d, pos %d) has passed %d layers (phase %d), exit %d reads layer %d", what, hrow / g_mock.max_ctx,
          hrow % g_mock.max_ctx, s.layer, s.phase, exit_k + 1, (exit_k + 1) * seg_len());
}

void check_at_some_exit(int hrow, const char* what) {
    const RowState& s = g_mock.rows[hrow];
    CHECK(s.phase == 0 && s.layer >= seg_len() && s.layer % seg_len() == 0,
          "%s: row (seq %d, pos %d) is not at an exit (%d layers, phase %d)", what, hrow / g_mock.max_ctx,
          hrow % g_mock.max_ctx, s.layer, s.phase);
}

// Split merge of compact row `row`: every slot of every head must come from the last
// attention launch.
void check_merge(const nv::CombineInfo& c, int row, const char* what) {
    CHECK(c.nsplit >= 1 && c.nrows >= 1 && c.off >= 0 && c.off < c.nrows, "%s: bad record for row %d", what, row);
    if (c.nsplit == 1) return;   // the attention wrote that row's output itself
    for (int h = 0; h < g_mock.D.H; ++h)
        for (int s = 0; s < c.nsplit; ++s) {
            const int slot = c.base + (h * c.nsplit + s) * c.nrows + c.off;
            CHECK(g_mock.slots.count(slot), "%s: row %d head %d split %d reads slot %d, which no item wrote", what, row,
                  h, s, slot);
        }
}

// Attention launch over `n` items (or the by-value decode plan): rows, key coverage, KV
// completeness, slot ownership.
void check_attention(const nv::AttnItem* items, int n, const nv::RowInfo* rows, int layer, const nv::LayerDims& D,
                     const nv::DecGeom& dg, const char* what) {
    g_mock.slots.clear();
    CHECK(layer >= 0 && layer < D.L, "%s: layer %d", what, layer);
    struct Block {
        int seq = -1, ctx = 0, nrows = 0;
        std::map<int, std::pair<int, int>> splits;   // split index -> [lo, hi)
        int nsplit = 0;
    };
    std::map<std::pair<int, int>, Block> blocks;   // (row0, head)
    for (int b = 0; b < n; ++b) {
        const nv::AttnItem it = dg.on ? nv::dec_item(dg, b) : items[b];
        CHECK(it.head >= 0 && it.head < D.H, "%s: item %d head %d", what, b, it.head);
        CHECK(it.nrows >= 1 && it.row0 >= 0, "%s: item %d rows", what, b);
        CHECK(it.lo >= 0 && it.lo < it.hi, "%s: item %d has an empty key range [%d, %d)", what, b, it.lo, it.hi);
        CHECK(it.nsplit >= 1 && it.split >= 0 && it.split < it.nsplit, "%s: item %d split %d of %d", what, b, it.split,
              it.nsplit);
        // the item's rows: consecutive positions of its sequence, QKV of this layer done
        int last_pos = -1;
        for (int r = 0; r < it.nrows; ++r) {
            nv::RowInfo row;
            if (dg.on) {
                row = nv::RowInfo{dg.seq * g_mock.max_ctx + dg.pos0 + r, dg.seq, dg.pos0 + r, 0};
            } else {
                row = rows[it.row0 + r];
            }
            check_row(row, what);
            CHECK(row.seq == it.seq, "%s: item %d row %d belongs to seq %d, item says %d", what, b, r, row.seq, it.seq);
            CHECK(r == 0 || row.pos == last_pos + 1, "%s: item %d rows are not consecutive", what, b);
            last_pos = row.pos;
            const RowState& s = g_mock.rows[row.hrow];
            CHECK(s.layer == layer && s.phase == 1, "%s: row (seq %d, pos %d) at layer %d phase %d, attention of layer %d",
                  what, row.seq, row.pos, s.layer, s.phase, layer);
        }
        CHECK(it.hi <= last_pos + 1, "%s: item %d reads key %d past its last row's position %d", what, b, it.hi - 1,
              last_pos);
        // every key read has its K/V at this layer
        const auto& w = kv_of(layer, it.seq);
        for (int k = it.lo; k < it.hi; ++k)
            CHECK(w[k], "%s: layer %d seq %d key %d read before its K/V was written", what, layer, it.seq, k);
        Block& bl = blocks[{it.row0, it.head}];
        if (bl.seq < 0) {
            bl.seq = it.seq;
            bl.ctx = last_pos + 1;
            bl.nrows = it.nrows;
            bl.nsplit = it.nsplit;
        }
        CHECK(bl.seq == it.seq && bl.nrows == it.nrows && bl.nsplit == it.nsplit,
              "%s: items of one row block disagree on seq, rows or split count", what);
        CHECK(!bl.splits.count(it.split), "%s: split %d of row block %d head %d listed twice", what, it.split, it.row0,
              it.head);
        bl.splits[it.split] = {it.lo, it.hi};
        if (it.nsplit > 1)
            for (int r = 0; r < it.nrows; ++r)
                CHECK(g_mock.slots.insert(it.part + r).second, "%s: partial slot %d written by two items", what,
                      it.part + r);
    }
    for (const auto& kvb : blocks) {
        const Block& bl = kvb.second;
        CHECK((int)bl.splits.size() == bl.nsplit, "%s: row block %d head %d has %zu of %d splits", what, kvb.first.first,
              kvb.first.second, bl.splits.size(), bl.nsplit);
        int at = 0;
        for (const auto& sp : bl.splits) {
            CHECK(sp.second.first == at, "%s: row block %d head %d: split %d starts at %d, expected %d", what,
                  kvb.first.first, kvb.first.second, sp.first, sp.second.first, at);
            at = sp.second.second;
        }
        CHECK(at == bl.ctx, "%s: row block %d head %d covers keys [0, %d) of %d", what, kvb.first.first,
              kvb.first.second, at, bl.ctx);
    }
    ++g_mock.launches;
}

}  // namespace

// Queries for the driver.
extern "C" int mock_embedded_token(int hrow) {
    auto it = g_mock.embedded.find(hrow);
    return it == g_mock.embedded.end() ? -1 : it->second;
}
extern "C" int mock_row_layers(int hrow) { return g_mock.rows[hrow].layer; }
extern "C" int mock_kv_written(int layer, int seq, int pos) { return kv_of(layer, seq)[pos]; }
extern "C" long long mock_launches() { return g_mock.launches; }
extern "C" long long mock_live_allocations() { return (long long)g_mock.allocs.size(); }

// ------------------------------------------------------------------------------------------
// HIP runtime calls
// ------------------------------------------------------------------------------------------

extern "C" {

hipError_t hipMalloc(void** ptr, size_t size) {
    if (!ptr) return hipErrorInvalidValue;
    *ptr = std::calloc(1, size ? size : 1);
    if (!*ptr) return hipErrorOutOfMemory;
    g_mock.allocs[*ptr] = size;
    return hipSuccess;
}

hipError_t hipFree(void* ptr) {
    if (!ptr) return hipSuccess;
    CHECK(g_mock.allocs.erase(ptr) == 1, "hipFree of %p, which hipMalloc did not return", ptr);
    std::free(ptr);
    return hipSuccess;
}

hipError_t hipHostMalloc(void** ptr, size_t size, unsigned int) { return hipMalloc(ptr, size); }
hipError_t hipHostFree(void* ptr) { return hipFree(ptr); }

hipError_t hipHostGetDevicePointer(void** devPtr, void* hstPtr, unsigned int) {
    *devPtr = hstPtr;
    return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
    if (n) std::memmove(dst, src, n);
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
    if (n) std::memmove(dst, src, n);
    return hipSuccess;
}

hipError_t hipMemcpy2D(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                       hipMemcpyKind) {
    for (size_t r = 0; r < height; ++r) std::memcpy((char*)dst + r * dpitch, (const char*)src + r * spitch, width);
    return hipSuccess;
}

hipError_t hipMemsetAsync(void* dst, int value, size_t n, hipStream_t) {
    std::memset(dst, value, n);
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamQuery(hipStream_t) { return hipSuccess; }

hipError_t hipEventCreate(hipEvent_t* event) {
    *event = reinterpret_cast<hipEvent_t>(new int(0));
    return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t event) {
    delete reinterpret_cast<int*>(event);
    return hipSuccess;
}

hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
    *ms = 0.001f;
    return hipSuccess;
}

hipError_t hipGetDevice(int* id) {
    *id = 0;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* pi, hipDeviceAttribute_t attr, int) {
    switch (attr) {
        case hipDeviceAttributeMultiprocessorCount: *pi = 256; break;
        case hipDeviceAttributeCooperativeLaunch: *pi = 1; break;
        case hipDeviceAttributeWallClockRate: *pi = 100000; break;
        default: *pi = 0;
    }
    return hipSuccess;
}

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "mock device error"; }

}  // extern "C"

// ------------------------------------------------------------------------------------------
// Kernel launch wrappers
// ------------------------------------------------------------------------------------------

namespace nv {

// The shape rules the host runtime branches on, as the kernels state them.
int sk_slices(const GemmArgs& a) {
    if (!a.wbf16 || a.head > 1 || a.comb || !a.sk_ws || a.mfma_min_rows <= 0 || a.sk_min_rows <= 0 || a.R < a.sk_min_rows ||
        a.R > a.sk_max_rows || a.R > SK_MAX_ROWS || a.K % SK_KC || a.N % 32 || a.out_bf16 || a.abf_ready || a.xent_part ||
        a.xd_part || a.epi < EPI_STORE || a.epi > EPI_SILU)
        return 0;
    const int ntb = a.norm_w ? (a.sk_ntb & 15) : ((a.sk_ntb >> 4) & 15);
    if ((ntb != 1 && ntb != 2) || a.N % (16 * ntb)) return 0;
    const int nks = a.K / SK_KC;
    return (int64_t)nks * a.R * (a.N + 1) > a.sk_cap ? 0 : nks;
}

bool gemm_uses_bf16_rows(const GemmArgs& a) {
    return a.wbf16 && a.abf && a.mfma_min_rows > 0 && a.R >= 33 && a.N % 64 == 0 && a.K % 64 == 0 && !a.comb &&
           !sk_slices(a);
}

bool attn_mfma_ok(const LayerDims& D) { return D.kv_bf16 && (D.hd == 32 || D.hd == 64 || D.hd == 128); }

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

hipError_t init_kernel_attributes() { return hipSuccess; }

void set_launch_events(hipEvent_t start, hipEvent_t stop) {
    g_mock.ev0 = start;
    g_mock.ev1 = stop;
}
void current_launch_events(hipEvent_t* start, hipEvent_t* stop) {
    *start = g_mock.ev0;
    *stop = g_mock.ev1;
}
const char* last_launch_name() { return "mock kernel"; }
int take_launch_blocks() { return 1; }
void note_launch_blocks(int) {}
void set_launch_stamp(unsigned long long* stamps) { g_mock.stamp = stamps; }
unsigned long long* current_launch_stamp() { return g_mock.stamp; }

hipError_t launch_stamp_reduce(unsigned long long* stamps, int n, unsigned long long* rec, hipStream_t) {
    CHECK(stamps && n > 0 && rec, "stamp fold arguments");
    rec[0] = 1000;
    rec[1] = 1100;
    return hipSuccess;
}

hipError_t launch_rope_table(float* cs, int max_ctx, int hd, float base, hipStream_t) {
    CHECK(cs && max_ctx > 0 && hd > 0 && hd % 2 == 0 && base > 0.f, "RoPE table arguments");
    // a model load: start from a clean device
    g_mock.max_ctx = max_ctx;
    g_mock.hd = hd;
    g_mock.have_dims = false;
    g_mock.rows.clear();
    g_mock.embedded.clear();
    g_mock.kv.clear();
    g_mock.slots.clear();
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_embed(const int* tokens, const RowInfo* rows, int n, const void* E, int, float* Hs, int d,
                        hipStream_t, int by_seq) {
    CHECK(tokens && rows && E && Hs && n > 0 && d > 0, "embedding arguments");
    for (int i = 0; i < n; ++i) {
        check_row(rows[i], "embedding");
        const int tok = by_seq ? tokens[rows[i].seq] : tokens[i];
        CHECK(tok >= 0, "embedding: token %d", tok);
        const int h = rows[i].hrow;
        g_mock.embedded[h] = tok;
        g_mock.rows[h] = RowState{};
        // a new token at this position: its keys and values are to be written again
        for (auto& kvp : g_mock.kv)
            if (kvp.first.second == rows[i].seq) kvp.second[rows[i].pos] = 0;
        std::memset(Hs + (size_t)h * d, 0, sizeof(float) * d);
    }
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_rows_bf16(const GemmArgs& a, hipStream_t) {
    CHECK(gemm_uses_bf16_rows(a) && a.A && a.abf, "bf16 row pass on a product that does not take it");
    return hipSuccess;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t) {
    CHECK(a.A && a.W && a.N > 0 && a.K > 0 && a.R >= 1, "product arguments (N %d, K %d, R %d)", a.N, a.K, a.R);
    if (a.epi == EPI_QKV) {
        CHECK(a.q_out && a.kv && a.rope && a.a_rows, "QKV product arguments");
        if (!g_mock.have_dims) {
            g_mock.D = a.D;
            g_mock.have_dims = true;
            CHECK(a.D.max_ctx == g_mock.max_ctx && a.D.hd == g_mock.hd && a.D.L % 4 == 0, "model dimensions");
        }
        CHECK(a.N == 3 * a.D.d && a.K == a.D.d, "QKV shape");
        if (a.contig) CHECK(a.a_row0 == a.seq0 * g_mock.max_ctx + a.pos0, "contiguous chunk: first row mismatch");
        for (int r = 0; r < a.R; ++r) {
            const int h = a_hidden_row(a, r);
            const RowInfo row = row_of(h);
            if (a.contig) CHECK(row.seq == a.seq0 && row.pos == a.pos0 + r, "contiguous chunk: row %d", r);
            RowState& s = g_mock.rows[h];
            CHECK(s.layer == a.layer && s.phase == 0, "QKV of layer %d on row (seq %d, pos %d) at layer %d phase %d",
                  a.layer, row.seq, row.pos, s.layer, s.phase);
            s.phase = 1;
            kv_of(a.layer, row.seq)[row.pos] = 1;
        }
    } else if (a.head) {
        CHECK(a.epi == EPI_STORE && a.N == (g_mock.have_dims ? g_mock.D.V : a.N), "exit head shape");
        for (int r = 0; r < a.R; ++r) {
            const int h = a_hidden_row(a, r);
            if (h >= 0) check_at_some_exit(h, "exit head");
        }
        if (a.o_rows && !a.contig)
            for (int r = 0; r < a.R; ++r) CHECK(a.o_rows[r].hrow == a.o_rows[r].seq, "head output rows: logits row");
        if (a.head == 2) CHECK(a.R == 1 && a.xd_part && a.N % 8 == 0, "head with draw partials");
        // logits: whatever the draw reads must be finite
        if (a.out && !a.xent_part) {
            for (int r = 0; r < a.R; ++r) {
                const int orow = !a.o_rows ? r : a.contig ? a.o_row0 + r : a.o_rows[r].hrow;
                std::memset(a.out + (size_t)orow * a.ldo, 0, sizeof(float) * a.N);
            }
        }
    } else if (a.epi == EPI_RESID && a.o_rows) {
        // O projection (phase 1 -> 2) or down projection (phase 3 -> next layer)
        if (a.comb) {
            CHECK(a.R == 1, "split merge on load needs one row");
            const CombineInfo c = a.contig && a.comb_ns > 0 ? CombineInfo{0, 0, a.comb_ns, 1} : a.comb[0];
            check_merge(c, 0, "O product merging splits");
        }
        if (a.contig) CHECK(a.o_row0 == a.seq0 * g_mock.max_ctx + a.pos0, "contiguous chunk: first output row");
        for (int r = 0; r < a.R; ++r) {
            const int h = o_hidden_row(a, r);
            const RowInfo row = row_of(h);
            RowState& s = g_mock.rows[h];
            CHECK(s.layer == a.layer, "residual product of layer %d on row (seq %d, pos %d) at layer %d", a.layer,
                  row.seq, row.pos, s.layer);
            if (s.phase == 1) {
                CHECK(a.K == g_mock.D.d, "O product K");
                s.phase = 2;
            } else {
                CHECK(s.phase == 3 && a.K == g_mock.D.F, "down product on row (seq %d, pos %d) at phase %d", row.seq,
                      row.pos, s.phase);
                s.layer += 1;
                s.phase = 0;
            }
        }
    } else if (a.epi == EPI_SWIGLU && a.a_rows) {
        CHECK(a.N == 2 * g_mock.D.F && a.K == g_mock.D.d, "gate/up shape");
        for (int r = 0; r < a.R; ++r) {
            const int h = a_hidden_row(a, r);
            const RowInfo row = row_of(h);
            RowState& s = g_mock.rows[h];
            CHECK(s.layer == a.layer && s.phase == 2, "gate/up of layer %d on row (seq %d, pos %d) at layer %d phase %d",
                  a.layer, row.seq, row.pos, s.layer, s.phase);
            s.phase = 3;
        }
    }
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_attn_dec(const AttnItem* items, int n_items, int max_rows, const RowInfo* rows, const float* q,
                           const void* kv, int layer, const LayerDims& D, float* part_ml, float* part_o, float* out,
                           hipStream_t, const DecGeom& dg, int wide) {
    if (n_items <= 0) return hipSuccess;
    CHECK(q && kv && part_ml && part_o && out && max_rows >= 1 && max_rows <= ATTN_DEC_ROWS, "decode attention args");
    CHECK(!wide || (D.kv_bf16 && max_rows <= ATTN_DEC_WIDE_ROWS), "wide decode attention on a group it does not take");
    // a split holds at most the keys the block's waves load at once
    const int max_keys = (wide ? ATTN_DEC_WIDE_WAVES * ATTN_DEC_WIDE_ITERS : 4 * ATTN_DEC_ITERS) * (64 / (D.hd / 8));
    for (int b = 0; b < n_items; ++b) {
        const AttnItem it = dg.on ? dec_item(dg, b) : items[b];
        CHECK(it.hi - it.lo <= max_keys, "decode attention: item %d covers %d keys, a block holds %d", b, it.hi - it.lo,
              max_keys);
    }
    if (dg.on)
        CHECK(dg.nrows >= 1 && dg.nrows <= max_rows && n_items == D.H * dg.nsplit, "decode attention plan by value");
    else
        CHECK(items && rows, "decode attention tables");
    check_attention(items, n_items, rows, layer, D, dg, "decode attention");
    return hipSuccess;
}

hipError_t launch_attn_mfma16(const AttnItem* items, int n_items, const RowInfo* rows, const float* q, const void* kv,
                              int layer, const LayerDims& D, float* part_ml, float* part_o, float* out, hipStream_t,
                              const DecGeom& dg) {
    if (n_items <= 0) return hipSuccess;
    CHECK(attn_mfma_ok(D) && q && kv && part_ml && part_o && out, "matrix-core decode attention args");
    check_attention(items, n_items, rows, layer, D, dg, "matrix-core decode attention");
    return hipSuccess;
}

hipError_t launch_attn_mfma(const AttnItem* items, int n_items, const RowInfo* rows, const float* q, const void* kv,
                            int layer, const LayerDims& D, float* part_ml, float* part_o, float* out, hipStream_t) {
    if (n_items <= 0) return hipSuccess;
    CHECK(attn_mfma_ok(D) && items && rows && q && kv, "matrix-core chunk attention args");
    for (int i = 0; i < n_items; ++i)
        CHECK(items[i].nrows <= ATTN_MFMA_ROWS && items[i].lo % 64 == 0, "matrix-core item %d shape", i);
    check_attention(items, n_items, rows, layer, D, DecGeom{}, "matrix-core chunk attention");
    return hipSuccess;
}

hipError_t launch_attn(const AttnItem* items, int n_items, const RowInfo* rows, const float* q, const void* kv,
                       int layer, const LayerDims& D, float* part_ml, float* part_o, float* out, hipStream_t) {
    if (n_items <= 0) return hipSuccess;
    CHECK(items && rows && q && kv && part_ml && part_o && out, "chunk attention args");
    check_attention(items, n_items, rows, layer, D, DecGeom{}, "chunk attention");
    return hipSuccess;
}

hipError_t launch_attn_combine(const CombineInfo* ci, int R, const LayerDims& D, const float* part_ml,
                               const float* part_o, float* out, hipStream_t, const DecGeom& dg) {
    CHECK(part_ml && part_o && out && R >= 1 && D.H == g_mock.D.H, "combine arguments");
    for (int i = 0; i < R; ++i) check_merge(dg.on ? dec_comb(dg, i) : ci[i], i, "combine");
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_attn_combine_bf16(const CombineInfo* ci, int R, const LayerDims& D, const float* part_ml,
                                    const float* part_o, const float* attn_o, uint16_t* out_bf16, hipStream_t) {
    CHECK(ci && part_ml && part_o && attn_o && out_bf16 && R >= 1 && D.H == g_mock.D.H, "bf16 combine arguments");
    for (int i = 0; i < R; ++i) check_merge(ci[i], i, "bf16 combine");
    ++g_mock.launches;
    return hipSuccess;
}

static void gate_common(const RowInfo* rows, const int* seqs, int n, const float* uniforms, int ucol, double* w_out,
                        int* stop_out, int* host_flags, int tag, const char* what) {
    CHECK(rows && seqs && w_out && ucol >= 0 && ucol < 3, "%s arguments", what);
    for (int i = 0; i < n; ++i) {
        check_row(rows[i], what);
        check_exit_row(rows[i].hrow, ucol, what);
        const int seq = seqs[i];
        w_out[seq * 4 + ucol] = 0.5;
        if (uniforms) {
            CHECK(stop_out, "%s: stop output", what);
            const int stop = uniforms[seq * 4 + ucol] < 0.5f ? 1 : 0;
            stop_out[seq] = stop;
            if (host_flags) host_flags[seq] = tag * 2 + stop;
        }
    }
    ++g_mock.launches;
}

hipError_t launch_gate(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d, const float* gw, float,
                       const float* uniforms, int ucol, double* w_out, int* stop_out, hipStream_t, int* host_flags,
                       int tag) {
    if (n <= 0) return hipSuccess;
    CHECK(Hs && gw && d > 0, "gate arguments");
    gate_common(rows, seqs, n, uniforms, ucol, w_out, stop_out, host_flags, tag, "router gate");
    return hipSuccess;
}

hipError_t launch_gate_mlp(const RowInfo* rows, const int* seqs, int n, const float* Hs, int d, const float* w1,
                           const float* b1, const float* w2, int rr, float, const float* uniforms, int ucol,
                           double* hid, double* w_out, int* stop_out, hipStream_t, int* host_flags, int tag) {
    if (n <= 0) return hipSuccess;
    CHECK(Hs && w1 && b1 && w2 && hid && rr >= 1 && d > 0, "router MLP arguments");
    gate_common(rows, seqs, n, uniforms, ucol, w_out, stop_out, host_flags, tag, "router MLP");
    return hipSuccess;
}

hipError_t launch_sample(const float* logits, int64_t ld, const int* seqs, int n, int V, const float* uniforms,
                         int* tok_out, hipStream_t) {
    CHECK(logits && seqs && uniforms && tok_out && n >= 1 && V >= 1 && ld >= V, "sampler arguments");
    for (int i = 0; i < n; ++i) {
        const int seq = seqs[i];
        const float u = uniforms[seq * 4 + 3];
        CHECK(u >= 0.f && u < 1.f, "sampler: uniform %g", (double)u);
        tok_out[seq] = std::min(V - 1, (int)std::floor((double)u * V));
    }
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_exit_draw(const float* part, int nb, const float* logits, float u, int* token, hipStream_t) {
    CHECK(part && logits && token && nb >= 1 && nb <= XD_PER * XD_THREADS && u >= 0.f && u < 1.f, "exit draw args");
    const int V = 8 * nb;
    token[0] = std::min(V - 1, (int)std::floor((double)u * V));
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_copy_rows(const RowInfo* rows, int n, const float* Hs, int d, float* dst, hipStream_t) {
    CHECK(rows && Hs && dst && d > 0, "row gather arguments");
    for (int i = 0; i < n; ++i) {
        check_row(rows[i], "row gather");
        check_at_some_exit(rows[i].hrow, "row gather for the shared head");
    }
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_xent(const float* logits, int64_t ld, int n, int V, const int* targets, double* out, int ostride,
                       int ocol, hipStream_t) {
    CHECK(logits && targets && out && ld >= V && ostride >= 4 && ocol >= 0 && ocol < 4, "cross-entropy arguments");
    for (int i = 0; i < n; ++i) {
        CHECK(targets[i] >= 0 && targets[i] < V, "cross-entropy target %d", targets[i]);
        out[(size_t)i * ostride + ocol] = -1.0;
    }
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_xent_merge(const float* part, const float* tgt, int n, int ngroups, double* out, int ostride,
                             int ocol, hipStream_t) {
    CHECK(part && tgt && out && ngroups >= 1 && ostride >= 4 && ocol >= 0 && ocol < 4, "cross-entropy merge arguments");
    for (int i = 0; i < n; ++i) out[(size_t)i * ostride + ocol] = -1.0;
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_loss_reduce(double* w, const double* lp, int n, ExitDepths dep, double* nll, double* depth,
                              double* sums, hipStream_t) {
    CHECK(w && lp && nll && depth && sums && n >= 1 && dep.L > 0, "loss reduction arguments");
    for (int i = 0; i < n; ++i) {
        w[(size_t)i * 4 + 3] = 1.0;
        nll[i] = 1.0;
        depth[i] = 0.5;
    }
    sums[0] = 1.0;
    sums[1] = 0.5;
    ++g_mock.launches;
    return hipSuccess;
}

hipError_t launch_segment(const SegArgs& a, int blocks, hipStream_t) {
    CHECK(blocks >= 1 && a.nl >= 1 && a.nl <= SEG_LMAX && a.S >= 1 && a.S <= SEG_SMAX && a.err && a.tpart,
          "segment kernel arguments");
    const RowInfo row = row_of((int)a.hrow);
    CHECK(row.seq == a.seq && row.pos == a.pos, "segment kernel row");
    RowState& s = g_mock.rows[(int)a.hrow];
    CHECK(s.layer == a.l0 && s.phase == 0, "segment kernel from layer %d on a row at layer %d", a.l0, s.layer);
    for (int l = a.l0; l < a.l0 + a.nl; ++l) {
        auto& w = kv_of(l, a.seq);
        for (int k = 0; k < a.pos; ++k)
            CHECK(w[k], "segment kernel: layer %d seq %d key %d read before its K/V was written", l, a.seq, k);
        w[a.pos] = 1;
    }
    s.layer += a.nl;
    ++g_mock.launches;
    return hipSuccess;
}

}  // namespace nv
