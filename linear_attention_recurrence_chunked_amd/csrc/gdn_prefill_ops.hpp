// gdn_prefill_ops.hpp -- device helpers of the bf16 chunk kernels (gdn_prefill_split.hip,
// gdn_prefill_wide.hip): the internal token / state-row order, MFMA operand packing, split
// bf16 products (gdn_split_bf16.hpp), the transposing LDS read and the K/Q tile swizzle.
#pragma once

#include "gdn_prefill_common.hpp"
#include "gdn_split_bf16.hpp"

namespace gdn {

// 16 bytes of a key row (the entry points accept only 16-byte aligned q, k and v, and rows
// of 64 or 128 bf16 keep every 8-element granule aligned).
__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *(const u32x4 *)p; }

__device__ __forceinline__ long long first_row(const PrefillArgs &a, int n)
{
    if (a.cu) return a.cu[n];
    return (a.total_T / a.num_seqs) * n;
}

__device__ __forceinline__ long long first_slot(const PrefillArgs &a, int n)
{
    return (first_row(a, n) >> 6) + n;
}

// Internal row order of the state (over d_k) and of the chunk's tokens in the K and T' tiles
// that the scan reads.  Within every aligned block of 32, internal position 16h + 4g + r
// holds original index 8g + 4h + r.  The accumulator layout gives lane group g the internal
// rows 4g .. 4g+3 of two consecutive 16-row blocks, which are then the original indices
// 8g .. 8g+7: exactly the eight contraction indices that a plain 16-byte fragment load of
// the other operand gives the same lanes.  The permutation moves whole groups of four rows,
// so every tile stays a set of whole rows (copied granule for granule).
__device__ __forceinline__ int split_orig(int i)
{
    return (i & ~31) | (((i >> 2) & 3) << 3) | (((i >> 4) & 1) << 2) | (i & 3);
}
__device__ __forceinline__ int split_pos(int o)
{
    return (o & ~31) | (((o >> 2) & 1) << 4) | (((o >> 3) & 3) << 2) | (o & 3);
}

// Two accumulator blocks (rows 4g..4g+3 of blocks 2kb and 2kb+1) as one bf16 operand.
__device__ __forceinline__ bf16x8 pack8s(f32x4 a, f32x4 b)
{
    const bf16x4 l = __builtin_convertvector(a, bf16x4);
    const bf16x4 h = __builtin_convertvector(b, bf16x4);
    return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
}

__device__ __forceinline__ f32x4 exp2x4(f32x4 x)
{
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_exp2f(x[i]);
    return r;
}

// Four bf16 values by the gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each
// group of 16 lanes, lane j receives element (j % 4) of the 8-byte rows addressed by lanes
// j / 4, j / 4 + 4, j / 4 + 8 and j / 4 + 12, in that order.
__device__ __forceinline__ bf16x4 ldtr(const unsigned char *p)
{
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)p);
    return __builtin_bit_cast(bf16x4, r);
}

// Swizzle of the K and Q tiles of the pipelined scan.  The gfx950 LDS has 64 four-byte banks
// (256 bytes per cycle).  The bank-conflict counters, read over single-wave probes of many
// address patterns, fit this model: a 16-byte read (ds_read_b128) serves two groups of eight
// lanes per cycle, lanes 8a .. 8a+7 with lanes
// 8(a^3) .. 8(a^3)+7, and it takes an extra cycle unless each group stays within one
// 128-byte half of the banks on distinct 16-byte slots and the two groups use different
// halves; the transposing read (ds_read_b64_tr_b16) serves 32 lanes per cycle, eight bytes
// each.  For 256-byte rows, logical granule g of row r is stored at slot pi(g) ^ (r & 7),
// pi(g) = (g & 1) << 3 | g >> 1 (the half is the granule's parity):
//   - a fragment load reads granule g of 16 consecutive rows (lane group ln / 8 = 0 or 1,
//     lg = granule offset); each group of eight rows meets eight distinct slots of the
//     half g & 1, and the paired group (granule g ^ 1) the other half: no conflicts;
//   - a transposing read of K^T meets rows 4a .. 4a+3 of one eight-row block at four
//     consecutive granules (two per half) and reads the same eight bytes of each, so every
//     slot serves exactly two of the 32 lanes of a cycle, the least that this shape allows.
// 128-byte rows keep the XOR key of swz_key.
template <int DK>
__device__ __forceinline__ int kq_slot(int row, int g)
{
    if constexpr (DK * 2 >= 256) {
        return (((g & 1) << 3) | ((g >> 1) & 7)) ^ (row & 7);
    } else {
        return g ^ swz_key<uint16_t, DK>(row);
    }
}
// the logical granule that slot p of row `row` holds (inverse of kq_slot)
template <int DK>
__device__ __forceinline__ int kq_logical(int row, int p)
{
    if constexpr (DK * 2 >= 256) {
        const int x = p ^ (row & 7);
        return ((x & 7) << 1) | (x >> 3);
    } else {
        return p ^ swz_key<uint16_t, DK>(row);
    }
}
template <int DK>
__device__ __forceinline__ int swz_kq(int row, int col)
{
    const int b = col * 2;
    return row * (DK * 2) + (kq_slot<DK>(row, b >> 4) << 4) + (b & 15);
}
template <int DK>
__device__ __forceinline__ bf16x8 ldfrag_kq(const unsigned char *base, int row, int k0)
{
    return *(const bf16x8 *)(base + swz_kq<DK>(row, k0));
}

}  // namespace gdn
