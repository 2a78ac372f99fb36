// Device helpers shared by the kernels of libnvium.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nv_internal.h"

namespace nv {

// ------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// float -> bf16 bits, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one instruction
// for a pair).
typedef __bf16 nv_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float nv_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((nv_f32x2_t){lo, hi}, nv_bf16x2_t));
}
__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)cvt_bf2(f, 0.0f); }

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

// Cross-lane adds with DPP (no LDS traffic).  quad_perm [1,0,3,2] and [2,3,0,1] pair lanes
// within a quad; row_half_mirror / row_mirror pair lane i with 7-i / 15-i of its 8 / 16.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of G lanes (G = 4, 8 or 16); every lane of a group gets the sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    if constexpr (G >= 8) v += dpp_f<0x141>(v);
    if constexpr (G >= 16) v += dpp_f<0x140>(v);
    return v;
}

// Sum over all 64 lanes, every lane gets it: DPP within rows of 16, then the four row sums
// read as scalars (no LDS round trips).
__device__ __forceinline__ float wave_total(float v) {
    v = group_sum<16>(v);
    const int iv = __float_as_int(v);
    return (__int_as_float(__builtin_amdgcn_readlane(iv, 0)) + __int_as_float(__builtin_amdgcn_readlane(iv, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(iv, 32)) + __int_as_float(__builtin_amdgcn_readlane(iv, 48)));
}

// Sum N values per lane (N a power of two, 4 <= N <= 64) over the 64 lanes of a wave with
// gfx950's half swaps and DPP, without LDS traffic.  v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second, v_permlane16_swap the odd
// 16-lane rows of the first with the even rows of the second (layout checked on the
// device), so one swap and one add give each half (row) the pairwise sums of half of the
// values.  Afterwards slot j < N/4 of every lane of row r (lanes 16r..16r+15) holds the sum
// of value index r * N/4 + j.
template <int N>
__device__ __forceinline__ void wave_rowsum_transpose(float (&v)[N]) {
    static_assert((N & (N - 1)) == 0 && N >= 4 && N <= 64, "N must be a power of two in [4, 64]");
    constexpr int H = N / 2, Q = N / 4;
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + H]), false, false);
        v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + Q]), false, false);
        v[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
#pragma unroll
    for (int i = 0; i < Q; ++i) v[i] = group_sum<16>(v[i]);
}

// Tagged words for exchanges between the blocks of one launch: the high 32 bits carry the
// epoch of the write, the low 32 bits an fp32 value, so a reader knows a word is the one
// it waits for without any fence.  Written with agent-scope stores, read with loads that
// skip the caches a writer on another XCD cannot have updated.
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint64_t tagv(uint32_t ep, float v) { return ((uint64_t)ep << 32) | __float_as_uint(v); }

__device__ __forceinline__ void tstore(uint64_t* p, uint32_t ep, float v) {
    __hip_atomic_store(p, tagv(ep, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ uint64_t tload_b(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 16);
    return ((uint64_t)v.y << 32) | v.x;
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

// Kernel-span stamps for timing mode: each block stores its start and end (device
// wall clock) at stamp[2 * block], stamp[2 * block + 1]; k_stamp_reduce folds them.
__device__ __forceinline__ unsigned long long stamp_begin(const unsigned long long* stamp) {
    return stamp ? (unsigned long long)wall_clock64() : 0ull;
}

__device__ __forceinline__ void stamp_end(unsigned long long* stamp, unsigned long long t0) {
    if (stamp) {
        __syncthreads();
        if (threadIdx.x == 0) {
            stamp[2 * blockIdx.x] = t0;
            stamp[2 * blockIdx.x + 1] = (unsigned long long)wall_clock64();
        }
    }
}

// As stamp_end for a grid of any shape: block (x, y) stores at its linear index, if that
// index is below `cap`.
__device__ __forceinline__ void stamp_end_lin(unsigned long long* stamp, unsigned long long t0, int cap) {
    if (stamp) {
        __syncthreads();
        const int b = blockIdx.y * gridDim.x + blockIdx.x;
        if (threadIdx.x == 0 && b < cap) {
            stamp[2 * b] = t0;
            stamp[2 * b + 1] = (unsigned long long)wall_clock64();
        }
    }
}

// Sum N values per lane over the 64 lanes of a wave.  Transposed reduction: each step
// halves the values a lane keeps (exchanging the other half with the partner lane), so
// after log2(N) steps lane L holds one value and a final butterfly finishes the sum.
// Returns the sum of value index (L >> (6 - log2 N)) in lane L (all lanes of a group).
template <int N>
__device__ __forceinline__ float wave_transpose_sum(float (&v)[N], int lane) {
    static_assert((N & (N - 1)) == 0 && N <= 64, "N must be a power of two <= 64");
    constexpr int LOG = (N == 1) ? 0 : (N == 2) ? 1 : (N == 4) ? 2 : (N == 8) ? 3 : (N == 16) ? 4 : (N == 32) ? 5 : 6;
    int n = N;
#pragma unroll
    for (int st = 0; st < LOG; ++st) {
        const int m = 32 >> st;
        const bool upper = (lane & m) != 0;
        n >>= 1;
        const int um = upper ? -1 : 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            if (i < n) {
                // select by masks on the values (a conditional operator here becomes an
                // indexed access over the whole array)
                const int lo = __float_as_int(v[i]), hi = __float_as_int(v[i + n]);
                const float send = __int_as_float((lo & um) | (hi & ~um));
                const float keep = __int_as_float((hi & um) | (lo & ~um));
                v[i] = keep + __shfl_xor(send, m, 64);
            }
        }
    }
    float r = v[0];
#pragma unroll
    for (int m = 32 >> LOG; m > 0; m >>= 1) r += __shfl_xor(r, m, 64);
    return r;
}

}  // namespace nv
