// Device helpers for the gfx950 paged-attention kernels: element types,
// 16-byte vector widening, round-to-nearest-even narrowing and wavefront
// (64-lane) reductions built on DPP row permutes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;

// Storage element types.  `bits` is the raw container in memory.
struct F32 {
    using bits = uint32_t;
};
struct F16 {
    using bits = uint16_t;
};
struct BF16 {
    using bits = uint16_t;
};

template <class T>
constexpr int kVec = 16 / sizeof(typename T::bits);  // elements per 16-byte load

__device__ __forceinline__ float u32_as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Widen one 32-bit word holding packed elements into floats (exact).
template <class T>
__device__ __forceinline__ void widen_word(uint32_t w, float* f);

template <>
__device__ __forceinline__ void widen_word<F32>(uint32_t w, float* f) {
    f[0] = u32_as_f32(w);
}
template <>
__device__ __forceinline__ void widen_word<F16>(uint32_t w, float* f) {
    half2_t h = __builtin_bit_cast(half2_t, w);
    f[0] = static_cast<float>(h[0]);
    f[1] = static_cast<float>(h[1]);
}
template <>
__device__ __forceinline__ void widen_word<BF16>(uint32_t w, float* f) {
    f[0] = u32_as_f32(w << 16);
    f[1] = u32_as_f32(w & 0xFFFF0000u);
}

// Widen a 16-byte chunk (kVec<T> elements) into floats.
template <class T>
__device__ __forceinline__ void widen16(const uint4& r, float* f) {
    constexpr int per = kVec<T> / 4;  // elements per 32-bit word
    widen_word<T>(r.x, f + 0 * per);
    widen_word<T>(r.y, f + 1 * per);
    widen_word<T>(r.z, f + 2 * per);
    widen_word<T>(r.w, f + 3 * per);
}

// Round a float to the storage type, nearest-even.
template <class T>
__device__ __forceinline__ typename T::bits narrow(float x);

template <>
__device__ __forceinline__ uint32_t narrow<F32>(float x) {
    return f32_as_u32(x);
}
template <>
__device__ __forceinline__ uint16_t narrow<F16>(float x) {
    // v_cvt_f16_f32 rounds to nearest even in the default rounding mode.
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
template <>
__device__ __forceinline__ uint16_t narrow<BF16>(float x) {
    uint32_t u = f32_as_u32(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN stays a quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load.  NT = 1 marks it non-temporal (streamed data that is
// read once), which lets the memory system skip keeping it in the caches.
template <int NT = 0>
__device__ __forceinline__ uint4 load16(const void* p) {
    u32x4 v;
    if constexpr (NT)
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else
        v = *reinterpret_cast<const u32x4*>(p);
    return uint4{v.x, v.y, v.z, v.w};
}

// 2^x with the hardware v_exp_f32 (no denormal-range fix-up: callers only
// take it of non-positive arguments whose tiny results may flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Wavefront reductions.
//
// Lanes are grouped into rows of LPR consecutive lanes (a power of two).  The
// steps below exchange values between lanes at distance 1, 2, 4, 8, 16, 32.
// Steps 1 and 2 are true XOR exchanges (DPP quad_perm).  Steps 4 and 8 use
// the DPP row_half_mirror / row_mirror permutes, which pair lane i with lane
// 7-i (resp. 15-i); once every aligned group of 4 (resp. 8) lanes already
// holds one common value, that pairing delivers the other group's value just
// like an XOR would, so the all-reduce result is the same.  Steps 16 and 32
// cross DPP rows and go through ds_bpermute.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

struct OpAdd {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// All-reduce over lane distances FROM, 2*FROM, ..., UPTO/2 (FROM, UPTO powers
// of two, 1 <= FROM, UPTO <= 64) for values that are UNIFORM within aligned
// groups of FROM lanes on entry (a row's score, its running sum, the wave
// maximum).  Afterwards every lane holds the reduction over its aligned group
// of UPTO lanes.  The mirror permutes are only valid under that uniformity.
template <int FROM, int UPTO, class Op>
__device__ __forceinline__ float group_reduce(float x, Op op) {
    if constexpr (FROM <= 1 && UPTO > 1) x = op(x, dpp<kDppXor1>(x));
    if constexpr (FROM <= 2 && UPTO > 2) x = op(x, dpp<kDppXor2>(x));
    if constexpr (FROM <= 4 && UPTO > 4) x = op(x, dpp<kDppHalfMirror>(x));
    if constexpr (FROM <= 8 && UPTO > 8) x = op(x, dpp<kDppMirror>(x));
    if constexpr (FROM <= 16 && UPTO > 16) x = op(x, __shfl_xor(x, 16));
    if constexpr (FROM <= 32 && UPTO > 32) x = op(x, __shfl_xor(x, 32));
    return x;
}

// Sum over lanes at XOR distances FROM, 2*FROM, ..., 32 with no uniformity
// assumption: lane i ends with the sum over all lanes j with j % FROM == i % FROM.
// Used once per workgroup to fold the rows' per-channel accumulators.
template <int FROM>
__device__ __forceinline__ float xor_sum_from(float x) {
    if constexpr (FROM <= 1) x += dpp<kDppXor1>(x);
    if constexpr (FROM <= 2) x += dpp<kDppXor2>(x);
    if constexpr (FROM <= 4) x += __shfl_xor(x, 4);
    if constexpr (FROM <= 8) x += __shfl_xor(x, 8);
    if constexpr (FROM <= 16) x += __shfl_xor(x, 16);
    if constexpr (FROM <= 32) x += __shfl_xor(x, 32);
    return x;
}

}  // namespace pa
