// Internal helpers shared by the HIP kernels and the host layer of libmdt.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mdt.h"

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Record a formatted error for mdt_last_error() and return `st`.
mdt_status mdt_fail(mdt_status st, const char* fmt, ...);
// After a kernel launch: map a HIP launch error to MDT_ERR_HIP (with its message).
mdt_status mdt_launched(const char* kernel);
// Start/stop events for the next launch when a profiling attachment is active on this
// thread (both null otherwise); names the launch for mdt_profile_kernel().
void mdt_profile_slot(const char* kernel, hipEvent_t* start, hipEvent_t* stop);

// Launch through hipExtLaunchKernelGGL so that an attached profiler gets the kernel's own
// start and stop timestamps.
#define MDT_LAUNCH(name, kernel, grid, block, lds, stream, ...)                              \
    do {                                                                                    \
        hipEvent_t mdt_e0_, mdt_e1_;                                                        \
        mdt_profile_slot(name, &mdt_e0_, &mdt_e1_);                                         \
        hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, mdt_e0_, mdt_e1_, 0, __VA_ARGS__); \
    } while (0)
// Number of compute units of the current device (cached per device).
int mdt_num_cus();
// Validate the host-side scalars and pointers of a device tree.
mdt_status mdt_check_tree(const mdt_tree_dev* t);

#define MDT_REQUIRE(cond, st, ...)                         \
    do {                                                   \
        if (!(cond)) return mdt_fail((st), __VA_ARGS__);   \
    } while (0)

inline bool mdt_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// device side
// ---------------------------------------------------------------------------

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round a float to bf16, nearest, ties to even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;  // NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// Round a double to bf16 directly (one rounding), nearest, ties to even.
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    uint64_t lsb = (u >> 45) & 1ull;
    u = (u + ((1ull << 44) - 1ull) + lsb) & ~((1ull << 45) - 1ull);
    // the result has at most 8 significant bits: float conversion is exact
    return f32_to_bf16((float)__longlong_as_double((long long)u));
}

// Storage-type traits: load/store one element as float.
template <typename ST> struct Elt;
template <> struct Elt<float> {
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
    static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
    static __device__ __forceinline__ void st64(float* p, double v) { *p = (float)v; }
};
template <> struct Elt<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
    static __device__ __forceinline__ void st64(bf16_t* p, double v) { *p = f64_to_bf16(v); }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// Cross-lane steps without LDS.  v_permlane32_swap(x, x) gives every lane the pair
// (x[l mod 32], x[32 + l mod 32]), v_permlane16_swap(x, x) the pair (x[row 2k], x[row 2k+1])
// of its 16-lane rows; combining the pair in that order leaves the same value in both
// partner lanes.
__device__ __forceinline__ float2 swap32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 swap16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max / sum over the lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float xor_max_16_32(float x) {
    float2 p = swap32(x);
    p = swap16(fmaxf(p.x, p.y));
    return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float xor_sum_16_32(float x) {
    float2 p = swap32(x);
    p = swap16(p.x + p.y);
    return p.x + p.y;
}
// Sum over the wave, every lane getting the same value: DPP within each row of 16 (lane
// pairs, quad pairs, mirrored halves, mirrored rows), then the two swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
    x = dpp_plus<0xb1>(x);   // quad_perm [1,0,3,2]
    x = dpp_plus<0x4e>(x);   // quad_perm [2,3,0,1]
    x = dpp_plus<0x141>(x);  // row_half_mirror
    x = dpp_plus<0x140>(x);  // row_mirror
    return xor_sum_16_32(x);
}

// (value desc, index asc) total order used by every top-k / argmax decision.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// XCD-aware tile order for a grid of Mb x Nb workgroups that share weight blocks across the
// Mb row blocks.  The dispatcher deals workgroups round-robin over the 8 XCDs (linear id g
// goes to XCD g % 8), and each XCD has its own L2.  The linear ids are remapped so that
// all Mb workgroups of one weight block land on the same XCD, one after another: XCD x
// takes weight blocks x, x + 8, ... (of the first Nb - Nb % 8), each with its Mb row
// blocks; the remaining blocks keep the plain order.
#ifndef MDT_NUM_XCD
#define MDT_NUM_XCD 8
#endif
__device__ __forceinline__ void xcd_tile(int g, int Mb, int Nb, int& m, int& n) {
    const int nfull = Nb - Nb % MDT_NUM_XCD;
    if (g < Mb * nfull) {
        const int xcd = g % MDT_NUM_XCD, slot = g / MDT_NUM_XCD;
        m = slot % Mb;
        n = (slot / Mb) * MDT_NUM_XCD + xcd;
    } else {
        const int r = g - Mb * nfull;
        m = r % Mb;
        n = nfull + r / Mb;
    }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        float ov = __shfl_xor(v, off, 64);
        int oi = __shfl_xor(i, off, 64);
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// One DPP step of a (value desc, index asc) reduction: combine with the lane that the
// data-parallel-primitive control CTRL selects; lanes outside ROW_MASK keep their pair.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_argmax_step(float& v, int& i) {
    const int vb = __builtin_bit_cast(int, v);
    const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(vb, vb, CTRL, ROW_MASK, 0xf, false));
    const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xf, false);
    if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Best (value, index) of the wave, returned uniformly to all lanes.  Swaps within
// quads, then row half-mirror and mirror give every lane its 16-lane row's best;
// row broadcasts 15 and 31 carry rows 0-2 into row 3; lane 63 is read out.
__device__ __forceinline__ void wave_argmax_dpp(float& v, int& i) {
    dpp_argmax_step<0xB1, 0xf>(v, i);   // quad_perm [1,0,3,2]
    dpp_argmax_step<0x4E, 0xf>(v, i);   // quad_perm [2,3,0,1]
    dpp_argmax_step<0x141, 0xf>(v, i);  // row_half_mirror
    dpp_argmax_step<0x140, 0xf>(v, i);  // row_mirror
    dpp_argmax_step<0x142, 0xa>(v, i);  // row_bcast:15 into rows 1 and 3
    dpp_argmax_step<0x143, 0xc>(v, i);  // row_bcast:31 into rows 2 and 3
    v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    i = __builtin_amdgcn_readlane(i, 63);
}
