// gdn_split_bf16.hpp -- products of 16 x 16 fp32 blocks on bf16 MFMAs with each operand
// split into a bf16 high part and a bf16 remainder, shared by the chunk-record kernels of the
// prefill and of the backward (both invert the unit lower triangular I + diag(beta) L).
#pragma once

#include "gdn_device.hpp"

namespace gdn {

// C += A B for 16 x 16 fp32 blocks with hi/lo bf16 splitting (relative error about 2^-16):
// A_hi B_hi + A_lo B_hi + A_hi B_lo on three v_mfma_f32_16x16x16_bf16.  A arrives in the row
// layout (lane (ln, lg) holds A[ln][4lg + s]) and B in the accumulator layout (lane holds
// B[4lg + s][ln]), which are the operand layouts of that instruction.  A value that enters
// several products is split once (Sp).
struct Sp {
    bf16x4 hi, lo;
};
// Pairs go through one two-lane conversion each, and the rounded high parts come back to
// fp32 by shifting the bf16 bits into place (exact), so a split takes twelve instructions.
__device__ __forceinline__ Sp split4(f32x4 x)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const uint32_t h01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2));
    const uint32_t h23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2));
    const f32x4 hf = {__builtin_bit_cast(float, h01 << 16), __builtin_bit_cast(float, h01 & 0xffff0000u),
                      __builtin_bit_cast(float, h23 << 16), __builtin_bit_cast(float, h23 & 0xffff0000u)};
    const f32x4 r = x - hf;
    const uint32_t l01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r[0], r[1]}, bf16x2));
    const uint32_t l23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r[2], r[3]}, bf16x2));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    return Sp{__builtin_bit_cast(bf16x4, u32x2{h01, h23}), __builtin_bit_cast(bf16x4, u32x2{l01, l23})};
}
__device__ __forceinline__ void mm3(f32x4 &c, const Sp &a, const Sp &b)
{
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s ah = __builtin_bit_cast(v4s, a.hi), al = __builtin_bit_cast(v4s, a.lo);
    const v4s bh = __builtin_bit_cast(v4s, b.hi), bl = __builtin_bit_cast(v4s, b.lo);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mm3r(const Sp &a, const Sp &b)
{
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    mm3(c, a, b);
    return c;
}

}  // namespace gdn
