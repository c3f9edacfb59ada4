// gdn_device.hpp -- device-side helpers shared by the gfx950 kernels of libgdn.
//
// bf16 is carried as raw uint16_t bit patterns in memory and as __bf16 vectors only where
// an MFMA consumes it.  Widening uses the bf16 definition (the upper 16 bits of an IEEE
// binary32 word); narrowing goes through the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32, round to nearest even).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Element loads/stores for the two storage types.
template <typename T> struct Elem;

template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p) { return *p; }
    static __device__ __forceinline__ void store(float *p, float x) { *p = x; }
};

template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t *p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void store(uint16_t *p, float x) {
        *(__bf16 *)p = (__bf16)x;
    }
};

// Four consecutive elements as floats.
__device__ __forceinline__ f32x4 load4(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ f32x4 load4(const uint16_t *p) {
    u32x2 w = *(const u32x2 *)p;
    f32x4 r;
    r[0] = __uint_as_float(w[0] << 16);
    r[1] = __uint_as_float(w[0] & 0xffff0000u);
    r[2] = __uint_as_float(w[1] << 16);
    r[3] = __uint_as_float(w[1] & 0xffff0000u);
    return r;
}
__device__ __forceinline__ void store4(float *p, f32x4 x) { *(f32x4 *)p = x; }
__device__ __forceinline__ void store4(uint16_t *p, f32x4 x) {
    *(bf16x4 *)p = __builtin_convertvector(x, bf16x4);
}

__device__ __forceinline__ float wave_xor(float x, int m) { return __shfl_xor(x, m, kWave); }

// x summed over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane rows), in every lane: the
// gfx950 row swaps pair rows 0-1 and 2-3, then the two halves (VALU, no LDS round trip).  The
// same sum, bit for bit, as adding the xor-16 and then the xor-32 partner.
__device__ __forceinline__ float row_sum4(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace gdn
