// Shared device helpers for the gfx950 kernels: bf16 unpacking, the fused scale-clamp-cast
// into both FP8 encodings, wave reductions and host-side argument checks.
//
// FP8 encodings (ai-radar.it "FP8 su GPU AMD ...", section "La correttezza del formato viene
// prima del tuning": e4m3fnuz, largest value 240, no NaN/Inf code; latestnews.news "AMD Boosts
// PyTorch FP8 Training on Instinct GPUs", third paragraph: the FNUZ encoding has only finite
// codes and one unsigned zero).  OCP e4m3fn (largest 448) is the encoding gfx950's conversion
// and matrix instructions use natively.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8_quant_grouped.h"

namespace fp8q {

constexpr float kEps = 1e-12f;        // floor of the absmax in the scale
constexpr float kFmaxFnuz = 240.0f;
constexpr float kFmaxFn = 448.0f;

template <int FMT>
struct Fmt;
template <>
struct Fmt<FP8Q_E4M3FNUZ> {
    static constexpr float fmax = kFmaxFnuz;
    // The cast multiplies by 2*s: a fnuz code's value is half the e4m3fn value of the same
    // byte (all codes but 0x80 and +-0x7F), so encoding 2*y in e4m3fn gives the fnuz byte of y.
    // Doubling is exact, so RN32(x * 2s) == 2 * RN32(x * s) wherever the result can encode to a
    // nonzero byte.
    static constexpr float mult = 2.0f;
};
template <>
struct Fmt<FP8Q_E4M3FN> {
    static constexpr float fmax = kFmaxFn;
    static constexpr float mult = 1.0f;
};

// 16-byte load with the non-temporal hint (data read exactly once).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 8- and 16-byte stores with the non-temporal hint (output written once and not read back by
// the same kernel).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_nt8(void* p, uint32_t a, uint32_t b) {
    __builtin_nontemporal_store(u32x2_t{a, b}, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}
// Outputs larger than this go out with streaming stores: they cannot stay in the 256 MB
// last-level cache for their consumer anyway (measured on the quantizers' outputs).
constexpr double kStreamBytes = 128.0 * 1024 * 1024;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Packed max of two 16-bit magnitudes per dword (|bf16| order equals the order of its 15
// magnitude bits for finite values).
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    ushort2_t x = __builtin_bit_cast(ushort2_t, a);
    ushort2_t y = __builtin_bit_cast(ushort2_t, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}
__device__ __forceinline__ uint32_t mag2(uint32_t w) { return w & 0x7FFF7FFFu; }
// Largest magnitude held in a packed pair, as bf16 bits.
__device__ __forceinline__ uint32_t hmax16(uint32_t w) {
    uint32_t lo = w & 0xFFFFu, hi = w >> 16;
    return lo > hi ? lo : hi;
}

// Scale from an absmax: s = FMAX / max(amax, 1e-12f), IEEE division rounded to nearest (HIP's
// default single-precision division is correctly rounded; the build never enables fast-math).
template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax) {
    return Fmt<FMT>::fmax / fmaxf(amax, kEps);
}

// Encode four values that are already multiplied by (mult * s); returns the bytes packed
// little-endian (a in byte 0).  e4m3fn: clamp to +-448 then the hardware RNE conversion
// (v_cvt_pk_fp8_f32, OCP e4m3fn on gfx950).  e4m3fnuz: the same conversion of the doubled
// value, with |2y| > 464 (|y| > 232, past the 224/240 midpoint) mapped to the 240 code and the
// e4m3fn negative zero 0x80 (the fnuz NaN) mapped to 0x00.
template <int FMT>
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d) {
    const float m = FMT == FP8Q_E4M3FN ? kFmaxFn : 448.0f;
    float ca = __builtin_amdgcn_fmed3f(a, -m, m);
    float cb = __builtin_amdgcn_fmed3f(b, -m, m);
    float cc = __builtin_amdgcn_fmed3f(c, -m, m);
    float cd = __builtin_amdgcn_fmed3f(d, -m, m);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, w, true);
    uint32_t u = (uint32_t)w;
    if (FMT == FP8Q_E4M3FNUZ) {
        uint32_t big = (fabsf(a) > 464.0f ? 0x01u : 0u) | (fabsf(b) > 464.0f ? 0x0100u : 0u) |
                       (fabsf(c) > 464.0f ? 0x010000u : 0u) | (fabsf(d) > 464.0f ? 0x01000000u : 0u);
        u |= big;
        uint32_t z = u ^ 0x80808080u;                          // bytes equal to 0x80 -> 0x00
        uint32_t nz = ((z & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | z;  // bit 7 set in nonzero bytes
        u &= ~(~nz & 0x80808080u);                            // clear the sign of 0x80 bytes
    }
    return u;
}

// Wave-wide maximum of an unsigned value (64 lanes).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// Group of a row: the first g with offsets[g] > r, clamped to [0, G-1] so that any offsets
// content keeps indices in range.
__device__ __forceinline__ int group_of_row(const int32_t* __restrict__ offsets, int G, int64_t r) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)offsets[mid] > r) hi = mid; else lo = mid + 1;
    }
    return lo;
}
// Start row of group g (0 for g == 0), as stored.
__device__ __forceinline__ int64_t group_start(const int32_t* __restrict__ offsets, int g) {
    return g == 0 ? 0 : (int64_t)offsets[g - 1];
}

}  // namespace fp8q

// ------------------------------------------------------------------------------------ host
#define FP8Q_CHECK_LAUNCH()                                     \
    do {                                                        \
        if (hipGetLastError() != hipSuccess) return FP8Q_ERR_HIP; \
    } while (0)

static inline bool fp8q_fmt_ok(int fmt) { return fmt == FP8Q_E4M3FNUZ || fmt == FP8Q_E4M3FN; }
static inline bool fp8q_aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
