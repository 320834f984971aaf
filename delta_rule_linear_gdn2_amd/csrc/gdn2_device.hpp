// Device-side helpers shared by the gfx950 kernels of the GDN-2 library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

// bf16 values are carried as raw 16-bit patterns.
using bf16raw = uint16_t;

// Per token and key channel, the chunk kernels clamp log2(alpha) to
// [kLog2AlphaFloor, 0] (alpha to [2^-15, 1]); the bound on the decay per token
// keeps the decay factors of a chunk representable (see the chunk kernels).
constexpr float kLog2AlphaFloor = -15.0f;

__device__ __forceinline__ float bf16_to_f32(bf16raw x) { return __uint_as_float(uint32_t(x) << 16); }

// Round to nearest even (gfx950's bf16 conversion instruction, which rounds
// as the mode register says: nearest even by default); NaN stays NaN.
__device__ __forceinline__ bf16raw f32_to_bf16(float f) { return __builtin_bit_cast(bf16raw, static_cast<__bf16>(f)); }

// Two values packed as one 32-bit word, the first in the low half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float load_as_f32(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_as_f32(const bf16raw* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void store_from_f32(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void store_from_f32(bf16raw* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }

__device__ __forceinline__ float log2_decay(float alpha)
{
    return fminf(fmaxf(__log2f(alpha), kLog2AlphaFloor), 0.0f);
}

// Token range [bos, eos) and batch row of sequence n.  Packed offsets are
// clamped to [0, T] so a malformed array cannot cause out-of-bounds access.
__device__ __forceinline__ void sequence_bounds(const int32_t* cu_seqlens, int32_t n, int32_t T,
                                                int64_t& bos, int64_t& eos, int64_t& brow)
{
    if (cu_seqlens) {
        int64_t a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        bos = a;
        eos = b;
        brow = 0;
    } else {
        bos = 0;
        eos = T;
        brow = n;
    }
}

}  // namespace gdn2
