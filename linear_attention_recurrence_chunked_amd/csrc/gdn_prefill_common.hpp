// gdn_prefill_common.hpp -- definitions shared by the chunked prefill kernels of libgdn.
//
// MFMA operand wrappers, the XOR-swizzled LDS addressing, the segment table entry and the
// argument block of the prefill kernels.  See gdn_prefill.hip for the method.
#pragma once

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

constexpr int kThreads = 256;
constexpr float kLog2AlphaFloor = -126.0f;   // log2 alpha clamp: keeps alpha = 0 finite

// Drain after a chain of v_mfma_f32_16x16x4_f32 whose result is read by anything but the
// next MFMA's accumulator input.  The compiler separates the chain's last MFMA from a VALU
// read of its result by 11 wait states (an s_nop 9 in the AMD assembly it emits for gfx950),
// the CDNA3 ISA's required count for reading the result of an 8-pass XDL instruction.  On
// gfx950 reads at that distance returned stale accumulator values for this instruction (the
// fp32-input prefill then failed its parity tests) and correct ones once 32 wait states
// separated them, so the drain issues four s_nop 7 (32 wait states, more than the 19 that
// table requires even for a 16-pass instruction).
__device__ __forceinline__ void mfma_f32_drain()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------------------
// MFMA wrappers.  A "K-block" is 32 values of the contraction index.  Each lane holds 8 of
// them for one row of A and the same 8 for one column of B: lane (r = lane % 16,
// g = lane / 16) takes elements k0 + 8g .. k0 + 8g + 7 of row (m0 + r) of A, stored row
// major with the contraction index contiguous, and likewise of row (n0 + r) of B^T.  A and B
// use the same assignment, so the pairing of contraction indices is exact whatever order the
// hardware sums them in.  The accumulator layout of every 16x16 MFMA is: lane holds column
// (lane % 16), rows 4 (lane / 16) + 0..3.
// ---------------------------------------------------------------------------------------
template <typename OP> struct Mma;

template <> struct Mma<uint16_t> {
    typedef bf16x8 frag;
    static __device__ __forceinline__ frag load(const uint16_t *p) {
        return *(const bf16x8 *)p;
    }
    static __device__ __forceinline__ void mma(f32x4 &c, const frag &a, const frag &b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ void put4(uint16_t *p, f32x4 x) {
        *(bf16x4 *)p = __builtin_convertvector(x, bf16x4);
    }
    static __device__ __forceinline__ f32x4 get4(const uint16_t *p) { return load4(p); }
    static __device__ __forceinline__ frag from_f32(f32x4 lo, f32x4 hi) {
        const bf16x4 l = __builtin_convertvector(lo, bf16x4);
        const bf16x4 h = __builtin_convertvector(hi, bf16x4);
        return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
    }
};

template <> struct Mma<float> {
    struct frag { f32x4 lo, hi; };
    static __device__ __forceinline__ frag load(const float *p) {
        frag f;
        f.lo = *(const f32x4 *)p;
        f.hi = *(const f32x4 *)(p + 4);
        return f;
    }
    static __device__ __forceinline__ void mma(f32x4 &c, const frag &a, const frag &b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
        mfma_f32_drain();
    }
    static __device__ __forceinline__ void put4(float *p, f32x4 x) { *(f32x4 *)p = x; }
    static __device__ __forceinline__ f32x4 get4(const float *p) { return *(const f32x4 *)p; }
    static __device__ __forceinline__ frag from_f32(f32x4 lo, f32x4 hi) {
        frag f;
        f.lo = lo;
        f.hi = hi;
        return f;
    }
};

// Four consecutive elements of the storage type held in registers.
template <typename T> struct Quad;
template <> struct Quad<uint16_t> {
    u32x2 w;
    static __device__ __forceinline__ Quad load(const uint16_t *p) { Quad q; q.w = *(const u32x2 *)p; return q; }
    static __device__ __forceinline__ Quad zero() { Quad q; q.w[0] = 0; q.w[1] = 0; return q; }
    __device__ __forceinline__ void store(uint16_t *p) const { *(u32x2 *)p = w; }
    __device__ __forceinline__ void mask(unsigned m) { w[0] &= m; w[1] &= m; }
    // column j of a 4x4 block given as four row quads
    static __device__ __forceinline__ Quad column(const Quad *r, int j) {
        Quad o;
        const int word = j >> 1;
        if (j & 1) {
            o.w[0] = (r[0].w[word] >> 16) | (r[1].w[word] & 0xffff0000u);
            o.w[1] = (r[2].w[word] >> 16) | (r[3].w[word] & 0xffff0000u);
        } else {
            o.w[0] = (r[0].w[word] & 0xffffu) | (r[1].w[word] << 16);
            o.w[1] = (r[2].w[word] & 0xffffu) | (r[3].w[word] << 16);
        }
        return o;
    }
};
template <> struct Quad<float> {
    f32x4 w;
    static __device__ __forceinline__ Quad load(const float *p) { Quad q; q.w = *(const f32x4 *)p; return q; }
    static __device__ __forceinline__ Quad zero() { Quad q; q.w = f32x4{0.f, 0.f, 0.f, 0.f}; return q; }
    __device__ __forceinline__ void store(float *p) const { *(f32x4 *)p = w; }
    __device__ __forceinline__ void mask(unsigned m) {
        w = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, w) & m);
    }
    static __device__ __forceinline__ Quad column(const Quad *r, int j) {
        Quad o;
        o.w[0] = r[0].w[j];
        o.w[1] = r[1].w[j];
        o.w[2] = r[2].w[j];
        o.w[3] = r[3].w[j];
        return o;
    }
};

// ---------------------------------------------------------------------------------------
// LDS layout.  Operand tiles are stored unpadded with the 16-byte granules of each row
// XOR-swizzled by a key of the row (swz_key), so that a fragment load (eight consecutive
// elements of 16 consecutive rows), a quad store from the accumulator layout (four
// consecutive elements of 16 rows) and the transposing quad stores of the input tiles all
// spread over distinct banks.  Regions are reused by liveness within a chunk:
//   U1: K and Q, row major (phases a-b)   |  R^T, U^T, scaled U^T (phases c-f)
//   U2: V^T (phases a-b)                  |  the four diagonal blocks of X (phases c-d)
// ---------------------------------------------------------------------------------------
// Swizzle key of a row: rows of 16 or more granules (256 bytes) take a 4-bit key, so that the
// 16 rows of a fragment load land on 16 different granule positions; narrower rows a 3-bit
// key (odd and even rows already fall in different halves of a 256-byte bank window).
template <typename OP, int W>
__device__ __forceinline__ int swz_key(int row)
{
    if constexpr (W * (int)sizeof(OP) >= 256) return (row ^ (row >> 4)) & 15;
    else return (row ^ (row >> 3)) & 7;
}

template <typename OP, int W>
__device__ __forceinline__ int swz(int row, int col)
{
    constexpr int E = (int)sizeof(OP);
    const int b = col * E;
    return row * (W * E) + (((b >> 4) ^ swz_key<OP, W>(row)) << 4) + (b & 15);
}

template <int DK, int DVT, typename OP>
struct Lds {
    static constexpr int E = sizeof(OP);
    static constexpr int al(int x) { return (x + 255) & ~255; }
    static constexpr int mx(int a, int b) { return a > b ? a : b; }
    static constexpr int szRow = kChunk * DK * E;     // [64][DK]
    static constexpr int szTr = DVT * kChunk * E;     // [DVT][64]
    static constexpr int LDA = kChunk + 4;            // padded fp32 rows of the solve
    static constexpr int LDX = 20;                    // padded rows of a diagonal X block
    static constexpr int oK = 0, oQ = szRow;
    static constexpr int oRt = 0, oUt = szTr, oUs = 2 * szTr;
    static constexpr int U1 = al(mx(2 * szRow, 3 * szTr));
    static constexpr int oVt = U1, oX = U1;
    static constexpr int U2 = al(mx(szTr, 4 * 16 * LDX * 4));
    static constexpr int oKt = U1 + U2;
    static constexpr int oA = al(oKt + DK * kChunk * E);
    static constexpr int oP = al(oA + kChunk * LDA * 4);
    static constexpr int oT = al(oP + kChunk * kChunk * E);
    static constexpr int oSt = al(oT + kChunk * kChunk * E);
    static constexpr int oG = al(oSt + DVT * DK * E);
    static constexpr int oB = oG + kChunk * 4;
    static constexpr int total = oB + kChunk * 4;
};

// What one workgroup does, decoded from its block index and (when sequences are split into
// segments) from the segment table.
struct Job {
    int n;            // sequence
    int h;            // head
    int col0;         // first column of the tile in the (augmented) state
    long long tok0;   // first packed row of the segment
    int len;          // tokens in the segment
    int seg;          // segment index within the sequence
    int nseg;         // segments of the sequence
    int entry;        // table entry (segment id) or -1 without a table
};

// Segment table entry (int32 x 4): sequence, first row (low 31 bits suffice for the
// supported sizes is NOT assumed: rows are stored as two int32 halves), length, segment id.
struct SegEntry {
    int32_t n;
    int32_t len;
    int32_t seg;
    int32_t nseg;
    int64_t tok0;
};

enum Mode { kModeScan = 0, kModeAug = 1 };

struct PrefillArgs {
    const void *q, *k, *v;
    const float *alpha, *beta;
    const float *s0;
    const int32_t *cu;
    int num_seqs;
    long long total_T;
    int H, dv;
    void *y;
    float *s_final;
    const SegEntry *table;     // null: one job per sequence
    const int32_t *n_entries;  // device count of valid table entries
    float *segB;               // [entries, H, DK, DV]  segment end states / start states
    float *segM;               // [entries, H, DK, DK]  segment transition matrices
    int ntiles;                // column tiles per (unit, head)
    long long units;           // sequences or table capacity
    void *prep;                // chunk records of the two-launch path, or null
    const float *gate_A;       // non-null: alpha, beta hold the gate pre-activations a, b and
    const float *gate_b_alpha; // the record kernel forms log2 alpha and beta from them
    // output gate applied as y leaves the one-launch scan (null og_z: plain y):
    // y <- sigmoid(z) y / sqrt(mean(y^2) + og_eps) (1 + og_w), per row of d_v values
    const void *og_z;
    const float *og_w;
    float og_eps;
};

// Arguments of the one-launch bf16 scan (gdn_prefill_wide.hip).
struct WideArgs {
    PrefillArgs a;
    int32_t *counter;      // job counter (segmented plans; zeroed before the launch) or null
    int32_t *flags;        // [entries, H]: column waves that published the end state
    float *seg_state;      // [entries, H, DK, DV] end states of segments
    int32_t *error;        // set when a wait gives up (never expected)
    int wmax;              // longest warm-up window, chunks
};
hipError_t launch_wide_scan(const WideArgs &w, long long jobs, hipStream_t stream);

__device__ __forceinline__ void seq_bounds(const PrefillArgs &a, int n, long long &t0, int &len) {
    if (a.cu) {
        const long long b0 = a.cu[n], b1 = a.cu[n + 1];
        t0 = b0;
        len = (int)(b1 - b0);
    } else {
        const long long per = a.total_T / a.num_seqs;
        t0 = per * n;
        len = (int)per;
    }
}

// DPP move within a wave; lanes without a source (or outside row_mask) read 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f32(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWMASK, 0xf,
                                                      false));
}

template <typename OP, int W>
__device__ __forceinline__ typename Mma<OP>::frag ldfrag(const unsigned char *base, int row,
                                                        int k0)
{
    if constexpr (sizeof(OP) == 2) {
        return *(const bf16x8 *)(base + swz<OP, W>(row, k0));
    } else {
        typename Mma<OP>::frag f;
        f.lo = *(const f32x4 *)(base + swz<OP, W>(row, k0));
        f.hi = *(const f32x4 *)(base + swz<OP, W>(row, k0 + 4));
        return f;
    }
}


// Two-launch bf16 path (gdn_prefill_split.hip): chunk records, then the state scan with
// 16, 32 or 64 state columns per workgroup; d_k in {64, 128}.
template <int DK>
hipError_t launch_chunk_prep(const PrefillArgs &args, long long nslots, hipStream_t stream);
template <int DK, int DVT, int MODE>
hipError_t launch_scan_split(const PrefillArgs &args, long long units, int ntiles,
                             hipStream_t stream);

}  // namespace gdn
