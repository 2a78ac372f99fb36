// Stand-alone exit draw on caller buffers: one exit's RMSNorm + LM head applied to one hidden
// row, and the token drawn from softmax(logits) by inverse CDF in token-id order (the
// gist.science technical summary of N-vium, section 3: the exit's distribution is sampled
// exactly; section 2, part "Architektur": each exit ends in its own head).  The same kernels
// nv_step runs for one stopping sequence: the one-row head product with its per-block
// softmax partials, then the one-block draw.
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>

#include "nv_internal.h"
#include "nvium.h"

// The scratch of nv_exit_draw_static, for callers that cannot allocate: the head product's
// per-block softmax partials for up to 65536 ids (64 KiB).  Each GPU the library runs on
// holds its own copy until the process ends.  Host code never passes the array's name as
// an address (on the host it only stands in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device.  Every call writes each partial it later reads, so
// nothing has to start at zero; calls that overlap on one GPU race on it.
constexpr int XD_STATIC_FLOATS = nv::XD_PER * nv::XD_THREADS * 2;
static __device__ __align__(256) float scratch[XD_STATIC_FLOATS];

namespace {

using namespace nv;

// Shapes the two kernels take: the vector-ALU decode GEMV (K split over at most 8 waves of
// 16-byte chunks, 8 columns per block) and the draw's reach (V / 8 partials).
bool exit_shape_ok(int32_t wdtype, int32_t d, int32_t V) {
    const int epc = wdtype == 1 ? 8 : 4;
    return (wdtype == 0 || wdtype == 1) && d > 0 && V > 0 && d % epc == 0 && d % 4 == 0 &&
           (d / epc + 63) / 64 <= 8 && V % 8 == 0 && V / 8 <= XD_PER * XD_THREADS;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (its address looked up on the first call there).
hipError_t scratch_on_device(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = (float*)p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t nv_exit_draw_workspace(int32_t vocab) {
    if (vocab <= 0 || vocab % 8 != 0 || vocab / 8 > XD_PER * XD_THREADS) return 0;
    return (size_t)(vocab / 8) * 2 * sizeof(float);
}

nv_status nv_exit_draw(const float* h, const float* norm_w, const void* head_w, int32_t wdtype, int32_t d,
                       int32_t vocab, float eps, float u, float* logits, int32_t* token, void* workspace,
                       size_t workspace_bytes, void* hip_stream) {
    if (!h || !norm_w || !head_w || !logits || !token || !workspace) return NV_EINVAL;
    if (!exit_shape_ok(wdtype, d, vocab) || !(u >= 0.0f && u < 1.0f) || !(eps > 0.0f)) return NV_EINVAL;
    if (workspace_bytes < nv_exit_draw_workspace(vocab)) return NV_ECAPACITY;
    hipStream_t st = (hipStream_t)hip_stream;
    GemmArgs g{};
    g.A = h;
    g.lda = d;
    g.norm_w = norm_w;
    g.eps = eps;
    g.W = head_w;
    g.N = vocab;
    g.K = d;
    g.R = 1;
    g.wbf16 = wdtype == 1 ? 1 : 0;
    g.epi = EPI_STORE;
    g.out = logits;
    g.ldo = vocab;
    g.head = 2;
    g.xd_part = (float*)workspace;
    if (launch_gemm(g, st) != hipSuccess) return NV_EDEVICE;
    if (launch_exit_draw((const float*)workspace, vocab / 8, logits, u, (int*)token, st) != hipSuccess)
        return NV_EDEVICE;
    return NV_OK;
}

nv_status nv_exit_draw_static(const float* h, const float* norm_w, const void* head_w, int32_t wdtype, int32_t d,
                              int32_t vocab, float eps, float u, float* logits, int32_t* token, void* hip_stream) {
    if (!h || !norm_w || !head_w || !logits || !token) return NV_EINVAL;
    if (!exit_shape_ok(wdtype, d, vocab) || !(u >= 0.0f && u < 1.0f) || !(eps > 0.0f)) return NV_EINVAL;
    if (nv_exit_draw_workspace(vocab) > sizeof(float) * XD_STATIC_FLOATS) return NV_ECAPACITY;
    float* ws = nullptr;
    if (scratch_on_device(&ws) != hipSuccess) return NV_EDEVICE;
    return nv_exit_draw(h, norm_w, head_w, wdtype, d, vocab, eps, u, logits, token, ws, sizeof(float) * XD_STATIC_FLOATS,
                        hip_stream);
}

}  // extern "C"
