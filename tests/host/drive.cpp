// Drives libnvium's C ABI on the host-only build (nv_runtime.cpp over mock_device.cpp),
// so that the runtime's planning and bookkeeping run under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU.  The mock device checks the plan of every
// launch; this driver checks what the C ABI reports against the deterministic walk the
// mock defines (exit = first k < 3 with u_k < 1/2, else 4; token = floor(u_4 * V)):
// tokens, exits, the token fed back at the next position, the per-segment frontiers,
// the layers each row has passed, and that flushing completes every layer's K/V.
//
//   drive <weights file> <max_batch> <max_ctx> <prompt lengths, comma separated>
//
// Exit status 0 and the last line "host runtime checks passed" on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "nvium.h"

extern "C" int mock_embedded_token(int hrow);
extern "C" int mock_row_layers(int hrow);
extern "C" int mock_kv_written(int layer, int seq, int pos);
extern "C" long long mock_launches();
extern "C" long long mock_live_allocations();

#define EXPECT(cond, ...)                                                   \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "drive: %s:%d: ", __FILE__, __LINE__);     \
            std::fprintf(stderr, __VA_ARGS__);                              \
            std::fprintf(stderr, "\n");                                     \
            std::exit(1);                                                   \
        }                                                                   \
    } while (0)

#define OK(m, call)                                                                                   \
    do {                                                                                              \
        const nv_status s_ = (call);                                                                  \
        EXPECT(s_ == NV_OK, "%s -> %d (%s)", #call, (int)s_, (m) ? nv_last_error(m) : "no handle");   \
    } while (0)

namespace {

struct Rng {   // splitmix64
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    float uni() { return (float)((next() >> 40) * (1.0 / 16777216.0)); }   // [0, 1) on the float grid
    int below(int n) { return (int)(next() % (uint64_t)n); }
};

struct Host {
    nv_model* m = nullptr;
    nv_config c{};
    int B = 0, ctx = 0, seg = 0;
    std::vector<int> n, pending, f;   // per sequence: positions consumed, next input, frontiers [B][4]
    std::vector<bool> live;
};

int expect_exit(const float* u) {
    for (int k = 0; k < 3; ++k)
        if (u[k] < 0.5f) return k + 1;
    return 4;
}

int expect_token(const Host& H, float u4) { return std::min(H.c.vocab - 1, (int)std::floor((double)u4 * H.c.vocab)); }

void check_frontiers(Host& H, int seq) {
    int32_t nc = -1, fr[4];
    OK(H.m, nv_debug_frontiers(H.m, seq, &nc, fr));
    EXPECT(nc == H.n[seq], "seq %d consumed %d, expected %d", seq, nc, H.n[seq]);
    for (int k = 0; k < 4; ++k)
        EXPECT(fr[k] == H.f[seq * 4 + k], "seq %d frontier %d is %d, expected %d", seq, k, fr[k], H.f[seq * 4 + k]);
}

void prefill(Host& H, Rng& rng, int seq, int len) {
    std::vector<int32_t> toks(len);
    for (int& t : toks) t = rng.below(H.c.vocab);
    OK(H.m, nv_prefill(H.m, seq, toks.data(), len));
    H.live[seq] = true;
    H.n[seq] = len - 1;
    H.pending[seq] = toks[len - 1];
    for (int k = 0; k < 4; ++k) H.f[seq * 4 + k] = len - 1;
    check_frontiers(H, seq);
    for (int p = 0; p < len - 1; ++p) {
        const int hrow = seq * H.ctx + p;
        EXPECT(mock_embedded_token(hrow) == toks[p], "prefill: row %d embedded %d, prompt has %d", p,
               mock_embedded_token(hrow), toks[p]);
        EXPECT(mock_row_layers(hrow) == H.c.n_layers, "prefill: row %d passed %d layers", p, mock_row_layers(hrow));
        for (int l = 0; l < H.c.n_layers; ++l) EXPECT(mock_kv_written(l, seq, p), "prefill: K/V of layer %d pos %d", l, p);
    }
}

// Bookkeeping after sequence `seq` consumed its token at position n with exit e.
void advance(Host& H, int seq, int e, int next_input) {
    const int hrow = seq * H.ctx + H.n[seq];
    EXPECT(mock_row_layers(hrow) == e * H.seg, "seq %d pos %d exited at %d after %d layers", seq, H.n[seq], e,
           mock_row_layers(hrow));
    for (int k = 0; k < e; ++k) H.f[seq * 4 + k] = H.n[seq] + 1;
    H.n[seq] += 1;
    H.pending[seq] = next_input;
}

void steps(Host& H, Rng& rng, int count, bool forced) {
    int nb = 0;
    while (nb < H.B && H.live[nb]) ++nb;
    std::vector<float> u(nb * 4);
    std::vector<int32_t> tok(nb), ex(nb), nxt(nb);
    for (int t = 0; t < count; ++t) {
        for (float& x : u) x = rng.uni();
        for (int i = 0; i < nb; ++i) nxt[i] = rng.below(H.c.vocab);
        const bool fz = forced && (t % 2 == 1);
        if (fz)
            OK(H.m, nv_step_forced(H.m, u.data(), nxt.data(), tok.data(), ex.data()));
        else
            OK(H.m, nv_step(H.m, u.data(), tok.data(), ex.data()));
        for (int i = 0; i < nb; ++i) {
            const int hrow = i * H.ctx + H.n[i];
            EXPECT(mock_embedded_token(hrow) == H.pending[i], "step: seq %d pos %d embedded %d, expected %d", i, H.n[i],
                   mock_embedded_token(hrow), H.pending[i]);
            EXPECT(ex[i] == expect_exit(&u[i * 4]), "step: seq %d exit %d, expected %d", i, ex[i],
                   expect_exit(&u[i * 4]));
            EXPECT(tok[i] == expect_token(H, u[i * 4 + 3]), "step: seq %d token %d, expected %d", i, tok[i],
                   expect_token(H, u[i * 4 + 3]));
            advance(H, i, ex[i], fz ? nxt[i] : tok[i]);
            check_frontiers(H, i);
        }
    }
}

void flush_all(Host& H, int seq) {
    OK(H.m, nv_flush(H.m, seq));
    for (int i = 0; i < H.B; ++i) {
        if (!H.live[i] || (seq >= 0 && seq != i)) continue;
        for (int k = 0; k < 4; ++k) H.f[i * 4 + k] = H.n[i];
        check_frontiers(H, i);
        for (int p = 0; p < H.n[i]; ++p) {
            EXPECT(mock_row_layers(i * H.ctx + p) == H.c.n_layers, "flush: seq %d pos %d passed %d layers", i, p,
                   mock_row_layers(i * H.ctx + p));
            for (int l = 0; l < H.c.n_layers; ++l)
                EXPECT(mock_kv_written(l, i, p), "flush: seq %d layer %d pos %d K/V missing", i, l, p);
        }
    }
}

void generate(Host& H, Rng& rng, const std::vector<int>& seqs, int T, int policy) {
    const int ns = (int)seqs.size();
    std::vector<float> u((size_t)ns * T * 4);
    for (float& x : u) x = rng.uni();
    std::vector<int32_t> tok((size_t)ns * T, -1), ex((size_t)ns * T, -1);
    std::vector<int32_t> sq(seqs.begin(), seqs.end());
    const std::vector<int> n0 = H.n;
    OK(H.m, nv_generate(H.m, sq.data(), ns, T, u.data(), policy, tok.data(), ex.data()));
    for (int i = 0; i < ns; ++i) {
        const int s = seqs[i];
        for (int t = 0; t < T; ++t) {
            const float* ut = &u[((size_t)i * T + t) * 4];
            const int hrow = s * H.ctx + n0[s] + t;
            EXPECT(mock_embedded_token(hrow) == H.pending[s], "generate: seq %d token %d embedded %d, expected %d", s, t,
                   mock_embedded_token(hrow), H.pending[s]);
            EXPECT(ex[(size_t)i * T + t] == expect_exit(ut), "generate: seq %d token %d exit %d, expected %d", s, t,
                   ex[(size_t)i * T + t], expect_exit(ut));
            EXPECT(tok[(size_t)i * T + t] == expect_token(H, ut[3]), "generate: seq %d token %d drew %d, expected %d", s,
                   t, tok[(size_t)i * T + t], expect_token(H, ut[3]));
            // the frontiers after token t; a later deferred chunk may already have moved the
            // row's layers on, so only its lower bound holds here
            const int e = ex[(size_t)i * T + t];
            EXPECT(mock_row_layers(hrow) >= e * H.seg, "generate: seq %d pos %d passed %d layers, exit %d", s,
                   n0[s] + t, mock_row_layers(hrow), e);
            for (int k = 0; k < e; ++k) H.f[s * 4 + k] = H.n[s] + 1;
            H.n[s] += 1;
            H.pending[s] = tok[(size_t)i * T + t];
        }
        check_frontiers(H, s);
    }
}

void errors(Host& H) {
    int nb = 0;
    while (nb < H.B && H.live[nb]) ++nb;
    std::vector<float> u(nb * 4, 0.25f);
    std::vector<int32_t> tok(nb), ex(nb);
    u[0] = 1.0f;
    EXPECT(nv_step(H.m, u.data(), tok.data(), ex.data()) == NV_EINVAL, "uniform 1.0 accepted");
    u[0] = NAN;
    EXPECT(nv_step(H.m, u.data(), tok.data(), ex.data()) == NV_EINVAL, "NaN uniform accepted");
    int32_t two[2] = {0, 0};
    std::vector<float> ug(2 * 4, 0.5f);
    if (H.B > 1 && H.live[0]) {
        std::vector<int32_t> t2(2), e2(2);
        EXPECT(nv_generate(H.m, two, 2, 1, ug.data(), NV_SCHED_GREEDY, t2.data(), e2.data()) == NV_EINVAL,
               "sequence listed twice accepted");
    }
    std::vector<int32_t> big(H.ctx + 1, 1);
    EXPECT(nv_prefill(H.m, 0, big.data(), H.ctx + 1) == NV_ECAPACITY, "prompt past max_ctx accepted");
    big[0] = H.c.vocab;
    EXPECT(nv_prefill(H.m, 0, big.data(), 4) == NV_EINVAL, "token id out of range accepted");
    EXPECT(nv_prefill(H.m, H.B, big.data(), 1) == NV_EINVAL, "sequence index out of range accepted");
    EXPECT(nv_flush(H.m, H.B) == NV_EINVAL, "flush of an out-of-range sequence accepted");
    EXPECT(nv_timing_enable(H.m, 3) == NV_EINVAL, "timing mode 3 accepted");
    int32_t one = 0;
    std::vector<float> ul((size_t)(H.ctx + 1) * 4, 0.75f);
    std::vector<int32_t> tl(H.ctx + 1), el(H.ctx + 1);
    EXPECT(nv_generate(H.m, &one, 1, H.ctx + 1, ul.data(), NV_SCHED_GREEDY, tl.data(), el.data()) == NV_ECAPACITY,
           "generation past max_ctx accepted");
    EXPECT(nv_generate(H.m, &one, 1, 1, ul.data(), 7, tl.data(), el.data()) == NV_EINVAL, "unknown policy accepted");
}

void timing(Host& H, Rng& rng) {
    for (int mode : {1, 2}) {
        OK(H.m, nv_timing_enable(H.m, mode));
        steps(H, rng, 2, false);
        double ms[NV_TIME_CLASSES], by[NV_TIME_CLASSES];
        int64_t nl[NV_TIME_CLASSES];
        OK(H.m, nv_timing_read(H.m, ms, by, nl));
        int64_t total = 0;
        for (int k = 0; k < NV_TIME_CLASSES; ++k) total += nl[k];
        EXPECT(total > 0 && nl[NV_TIME_BLOCK_GEMM] > 0, "timing: no launches counted");
        std::vector<char> txt(1 << 16);
        OK(H.m, nv_timing_kernels(H.m, txt.data(), txt.size()));
        EXPECT(std::strchr(txt.data(), '\t') != nullptr, "timing: empty kernel table");
        char tiny[4];
        EXPECT(nv_timing_kernels(H.m, tiny, sizeof(tiny)) == NV_ECAPACITY, "timing: small buffer accepted");
    }
    OK(H.m, nv_timing_enable(H.m, 0));
}

void debug_reads(Host& H) {
    std::vector<float> lg(H.c.vocab), kk((size_t)4 * H.c.d_model), vv((size_t)4 * H.c.d_model), hh((size_t)4 * H.c.d_model);
    double w[4];
    OK(H.m, nv_debug_logits(H.m, 0, lg.data()));
    OK(H.m, nv_debug_gates(H.m, 0, w));
    const int p0 = H.n[0] >= 4 ? H.n[0] - 4 : 0;
    const int cnt = H.n[0] >= 4 ? 4 : H.n[0];
    if (cnt > 0) {
        OK(H.m, nv_debug_kv(H.m, 0, H.c.n_layers - 1, p0, cnt, kk.data(), vv.data()));
        OK(H.m, nv_debug_hidden(H.m, 0, p0, cnt, hh.data()));
    }
    EXPECT(nv_debug_kv(H.m, 0, H.c.n_layers, 0, 1, kk.data(), vv.data()) == NV_EINVAL, "layer out of range accepted");
}

void loss(Host& H, Rng& rng, int seq, int n) {
    std::vector<int32_t> toks(n);
    for (int& t : toks) t = rng.below(H.c.vocab);
    double out[3];
    std::vector<double> per((size_t)(n - 1) * 10);
    OK(H.m, nv_mixture_loss(H.m, seq, toks.data(), n, 0.5, out, per.data()));
    EXPECT(std::isfinite(out[0]) && std::isfinite(out[1]) && std::isfinite(out[2]), "loss not finite");
    for (int i = 0; i < n - 1; ++i) EXPECT(per[(size_t)i * 10 + 3] == 1.0, "loss: last router output of row %d", i);
    H.live[seq] = true;
    H.n[seq] = n - 1;
    H.pending[seq] = toks[n - 1];
    for (int k = 0; k < 4; ++k) H.f[seq * 4 + k] = n - 1;
    check_frontiers(H, seq);
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 5) {
        std::fprintf(stderr, "usage: drive <weights> <max_batch> <max_ctx> <prompt lengths>\n");
        return 2;
    }
    const char* path = argv[1];
    Host H;
    H.B = std::atoi(argv[2]);
    H.ctx = std::atoi(argv[3]);
    std::vector<int> lens;
    for (const char* p = argv[4]; *p;) {
        lens.push_back(std::atoi(p));
        while (*p && *p != ',') ++p;
        if (*p == ',') ++p;
    }
    EXPECT((int)lens.size() == H.B, "one prompt length per sequence");
    Rng rng{12345};

    EXPECT(nv_mem_required(path, H.B, H.ctx) > 0, "nv_mem_required");
    // caller arena first: nv_free must leave it alone
    for (int use_arena = 1; use_arena >= 0; --use_arena) {
        void* arena = nullptr;
        const size_t bytes = nv_mem_required(path, H.B, H.ctx);
        if (use_arena) EXPECT(hipMalloc(&arena, bytes) == hipSuccess, "arena");
        const long long live0 = mock_live_allocations();
        OK(H.m, nv_load(path, H.B, H.ctx, arena, use_arena ? bytes : 0, nullptr, &H.m));
        OK(H.m, nv_get_config(H.m, &H.c));
        EXPECT(H.c.n_layers % 4 == 0 && H.c.exit_layer[3] == H.c.n_layers, "config");
        H.seg = H.c.n_layers / 4;
        H.n.assign(H.B, 0);
        H.pending.assign(H.B, 0);
        H.f.assign((size_t)H.B * 4, 0);
        H.live.assign(H.B, false);
        for (int i = 0; i < H.B; ++i) prefill(H, rng, i, lens[i]);
        steps(H, rng, 6, false);
        steps(H, rng, 4, true);
        flush_all(H, 0);
        steps(H, rng, 3, false);
        flush_all(H, -1);
        steps(H, rng, 2, false);
        std::vector<int> sub;
        for (int i = H.B - 1; i >= 0; i -= 2) sub.push_back(i);
        generate(H, rng, sub, 5, NV_SCHED_GREEDY);
        std::vector<int> all;
        for (int i = 0; i < H.B; ++i) all.push_back(i);
        generate(H, rng, all, 4, NV_SCHED_LOCKSTEP);
        steps(H, rng, 2, false);
        timing(H, rng);
        debug_reads(H);
        errors(H);
        loss(H, rng, 0, std::min(H.ctx, std::max(3, lens[0])));
        steps(H, rng, 2, false);
        flush_all(H, -1);
        nv_free(H.m);
        H.m = nullptr;
        EXPECT(mock_live_allocations() == live0 - (use_arena ? 0 : 0), "nv_free left %lld device/pinned allocations",
               mock_live_allocations() - live0);
        if (use_arena) EXPECT(hipFree(arena) == hipSuccess, "arena free");
        std::printf("%s arena: ok (%lld launches so far)\n", use_arena ? "caller" : "own", mock_launches());
    }
    std::printf("host runtime checks passed\n");
    return 0;
}
