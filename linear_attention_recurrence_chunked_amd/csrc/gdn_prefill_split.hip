// gdn_prefill_split.hip -- chunked prefill for bf16 inputs in two launches (gfx950).
//
// The chunk algebra is the one of gdn_prefill.hip (the WY / UT form of the reading notes'
// transition-matrix recurrence, Gated DeltaNet, section 2.1).  Everything that does not
// depend on the state is computed once per (chunk, head) by a chunk-parallel launch, so the
// sequential part of the method only carries the state products:
//
//   chunk_prep_kernel (one workgroup per (chunk slot, head), all independent):
//     g   = within-chunk inclusive prefix of log2 alpha,  gamma = 2^g
//     A   = diag(beta) strictlower(K K^T (.) Gamma),  Gamma_ti = gamma_t / gamma_i
//     T'  = (I + A)^{-1} diag(beta)            (blocked inversion, see below)
//     P   = lower_incl(Q K^T (.) Gamma)
//   and writes T', P and g to the workspace (16640 bytes per record).
//
//   scan_split_kernel (one workgroup per (sequence or segment, head, column tile)):
//     two loader waves stream K, Q, V and the record of chunk c+1 into a second LDS stage
//     while the scan waves apply chunk c to the state held in MFMA accumulator registers:
//     R = V - diag(gamma) K S,  U = T' R,  Y^T = S^T Q^T diag(gamma) + U^T P^T,
//     S = gamma_C S + K^T diag(gamma_C / gamma) U.   One barrier per chunk.
//
// Chunk slots: chunk c of sequence n (first row t0_n) has slot floor(t0_n / 64) + n + c.
// Slots of different chunks differ, and all are below floor(total_T / 64) + num_seqs.
#include <type_traits>

#include "gdn_prefill_common.hpp"

namespace gdn {

// Record of one (slot, head): T' [64][64] bf16 (rows in the internal token order defined
// below) and P [64][64] bf16, both in the XOR-swizzled byte layout of a 64-wide LDS tile (so
// both launches copy them granule for granule), then g [64] fp32.
constexpr int kRecT = 0;
constexpr int kRecP = kChunk * kChunk * 2;
constexpr int kRecG = 2 * kChunk * kChunk * 2;
static_assert(kRecG + kChunk * 4 == kPrepRecordBytes, "record layout");
constexpr int kRecGranules = kPrepRecordBytes / 16;

// 16 bytes from global memory that is only guaranteed 8-byte aligned.
__device__ __forceinline__ u32x4 ld16(const uint16_t *p)
{
    const u32x2 lo = *(const u32x2 *)p;
    const u32x2 hi = *(const u32x2 *)(p + 4);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

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

// C += A B for 16 x 16 fp32 blocks on v_mfma_f32_16x16x32_bf16 with hi/lo bf16 splitting
// (relative error about 2^-16).  A arrives in the row layout (lane (ln, lg) holds
// A[ln][4lg + s]) and B in the accumulator layout (lane holds B[4lg + s][ln]); the 32-wide K
// of the instruction carries (A_hi | A_lo) x (B_hi | B_hi), then (A_hi | 0) x (B_lo | 0).
__device__ __forceinline__ void mm16s(f32x4 &c, f32x4 arow, f32x4 bcol)
{
    const bf16x4 ah = __builtin_convertvector(arow, bf16x4);
    const bf16x4 al = __builtin_convertvector(arow - __builtin_convertvector(ah, f32x4), bf16x4);
    const bf16x4 bh = __builtin_convertvector(bcol, bf16x4);
    const bf16x4 bl = __builtin_convertvector(bcol - __builtin_convertvector(bh, f32x4), bf16x4);
    const __bf16 z = (__bf16)0.f;
    const bf16x8 a1 = {ah[0], ah[1], ah[2], ah[3], al[0], al[1], al[2], al[3]};
    const bf16x8 b1 = {bh[0], bh[1], bh[2], bh[3], bh[0], bh[1], bh[2], bh[3]};
    const bf16x8 a2 = {ah[0], ah[1], ah[2], ah[3], z, z, z, z};
    const bf16x8 b2 = {bl[0], bl[1], bl[2], bl[3], z, z, z, z};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, b2, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mm16sr(f32x4 arow, f32x4 bcol)
{
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    mm16s(c, arow, bcol);
    return c;
}

// =========================================================================================
// Launch 1: per (chunk slot, head) record T', P, g.  Four waves; wave w owns block row /
// column w of the 4 x 4 grid of 16 x 16 blocks.
// =========================================================================================
template <int DK>
struct LdsPrep {
    static constexpr int szRow = kChunk * DK * 2;
    static constexpr int LDA = kChunk + 4;          // padded fp32 rows of A
    static constexpr int LDX = 20;                  // padded rows of a diagonal X block
    static constexpr int oT = kRecT, oP = kRecP, oG = kRecG;
    static constexpr int oBeta = kPrepRecordBytes;
    static constexpr int oK = oBeta + 256;          // K, Q rows (phases 1-2) ...
    static constexpr int oQ = oK + szRow;
    static constexpr int oA = oK;                   // ... then A and the X blocks (phase 3)
    static constexpr int oX = oA + kChunk * LDA * 4;
    static constexpr int total = oK + (2 * szRow > kChunk * LDA * 4 + 4 * 16 * LDX * 4
                                           ? 2 * szRow
                                           : kChunk * LDA * 4 + 4 * 16 * LDX * 4);
};

template <int DK>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrefillArgs a, long long nslots)
{
    using L = LdsPrep<DK>;
    using OP = uint16_t;
    using M = Mma<OP>;
    constexpr int KBD = DK / 32;
    constexpr int GR = DK / 8;                       // 16-byte granules per row
    constexpr int NG = kChunk * GR / 256;            // row granules per thread
    __shared__ __align__(16) unsigned char smem[L::total];
    float *const sG = (float *)(smem + L::oG);
    float *const sBeta = (float *)(smem + L::oBeta);
    float *const sA = (float *)(smem + L::oA);
    float *const sX = (float *)(smem + L::oX);
    unsigned char *const bK = smem + L::oK;
    unsigned char *const bQ = smem + L::oQ;
    unsigned char *const bP = smem + L::oP;
    unsigned char *const bT = smem + L::oT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int H = a.H;
    const long long slot = (long long)blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    if (slot >= nslots) return;
    // sequence of the slot: the last n with first_slot(n) <= slot
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first_slot(a, mid) <= slot) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    long long st0;
    int slen;
    seq_bounds(a, n, st0, slen);
    const long long c = slot - ((st0 >> 6) + n);
    if (c < 0 || c * kChunk >= slen) return;          // unused slot
    const long long t0 = st0 + c * kChunk;
    const int nv = (int)((slen - c * kChunk) < kChunk ? (slen - c * kChunk) : kChunk);

    // ---- phase 1: K, Q rows (zero beyond the chunk's last row), g, beta ----
    {
        const OP *gk = (const OP *)a.k;
        const OP *gq = (const OP *)a.q;
        u32x4 rk[NG], rq[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int idx = tid + 256 * j;
            const int row = idx / GR, gc = idx % GR;
            const int tc = row < nv ? row : nv - 1;
            const long long off = ((t0 + tc) * H + h) * (long long)DK + 8 * gc;
            rk[j] = ld16(gk + off);
            rq[j] = ld16(gq + off);
        }
        float pa = 0.f;
        if (wave < 2) {
            const int tc = lane < nv ? lane : nv - 1;
            pa = (wave == 0 ? a.alpha : a.beta)[(t0 + tc) * H + h];
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int idx = tid + 256 * j;
            const int row = idx / GR, gc = idx % GR;
            const u32x4 z = {0u, 0u, 0u, 0u};
            *(u32x4 *)(bK + swz<OP, DK>(row, 8 * gc)) = row < nv ? rk[j] : z;
            *(u32x4 *)(bQ + swz<OP, DK>(row, 8 * gc)) = row < nv ? rq[j] : z;
        }
        if (wave == 0) {
            float x = lane < nv ? fmaxf(__builtin_amdgcn_logf(pa), kLog2AlphaFloor) : 0.f;
            x += dpp_f32<0x111, 0xf>(x);
            x += dpp_f32<0x112, 0xf>(x);
            x += dpp_f32<0x114, 0xf>(x);
            x += dpp_f32<0x118, 0xf>(x);
            x += dpp_f32<0x142, 0xa>(x);
            x += dpp_f32<0x143, 0xc>(x);
            sG[lane] = x;
        } else if (wave == 1) {
            sBeta[lane] = lane < nv ? pa : 0.f;
        }
    }
    __syncthreads();

    // ---- phase 2: Gram tiles; wave w takes the diagonal pair (w, w) and the off-diagonal
    // pairs {(1,0),(3,0)}, {(2,0),(3,1)}, {(2,1)}, {(3,2)} (t-block, i-block) ----
    const int d0 = wave * 16;
    const int np = wave < 2 ? 3 : 2;
    const int tb0 = wave == 0 ? 1 : (wave == 1 ? 2 : (wave == 2 ? 2 : 3));
    const int ib0 = wave == 0 ? 0 : (wave == 1 ? 0 : (wave == 2 ? 1 : 2));
    const int ib1 = wave == 0 ? 0 : 1;
    const int tbs[3] = {wave, tb0, 3};
    const int ibs[3] = {wave, ib0, ib1};
    f32x4 accG[3], accP[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        accG[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        accP[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            if (p < np) {
                const auto ai = ldfrag<OP, DK>(bK, ibs[p] * 16 + ln, kb * 32 + 8 * lg);
                const auto bt = ldfrag<OP, DK>(bK, tbs[p] * 16 + ln, kb * 32 + 8 * lg);
                const auto bq = ldfrag<OP, DK>(bQ, tbs[p] * 16 + ln, kb * 32 + 8 * lg);
                M::mma(accG[p], ai, bt);
                M::mma(accP[p], ai, bq);
            }
        }
    }
    // accG[p][r] = k_i . k_t, accP[p][r] = k_i . q_t for i = ib*16 + 4lg + r, t = tb*16 + ln.
    // Masked values: A^T block (row i, column t) and P (row t, column i).
    auto masked = [&](int tb, int ib, f32x4 g_, f32x4 p_, f32x4 &av) {
        const int t = tb * 16 + ln;
        const float gt = sG[t];
        const float bt_ = sBeta[t];
        const f32x4 gi = *(const f32x4 *)(sG + ib * 16 + 4 * lg);
        f32x4 pv4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ib * 16 + 4 * lg + r;
            const float dec = (i <= t) ? __builtin_amdgcn_exp2f(gt - gi[r]) : 0.f;
            av[r] = (i < t) ? bt_ * g_[r] * dec : 0.f;
            pv4[r] = p_[r] * dec;
        }
        M::put4((OP *)(bP + swz<OP, kChunk>(t, ib * 16 + 4 * lg)), pv4);
    };
    f32x4 nT, a1, a2;
    masked(wave, wave, accG[0], accP[0], nT);
    masked(tb0, ib0, accG[1], accP[1], a1);
    if (np == 3) masked(3, ib1, accG[2], accP[2], a2);
    // N (accumulator layout of the strictly lower diagonal block, row i, column t)
    f32x4 nC;
    {
        const int t = d0 + ln;
        const float gt = sG[t];
        const f32x4 gi = *(const f32x4 *)(sG + d0 + 4 * lg);
        const f32x4 bi = *(const f32x4 *)(sBeta + d0 + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = d0 + 4 * lg + r;
            nC[r] = (t < i) ? bi[r] * accG[0][r] * __builtin_amdgcn_exp2f(gi[r] - gt) : 0.f;
        }
    }
    // zero blocks above the diagonal of T' and P: wave w clears blocks (w, j), j > w
#pragma unroll
    for (int j = 1; j < 4; ++j) {
        if (j > wave) {
            M::put4((OP *)(bP + swz<OP, kChunk>(d0 + ln, 16 * j + 4 * lg)),
                    f32x4{0.f, 0.f, 0.f, 0.f});
            M::put4((OP *)(bT + swz<OP, kChunk>(split_pos(d0 + ln), 16 * j + 4 * lg)),
                    f32x4{0.f, 0.f, 0.f, 0.f});
        }
    }
    // (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since N^16 = 0.  C = the
    // accumulator layout of a block, T = of its transpose (which is the row layout of it).
    f32x4 eye;
#pragma unroll
    for (int r = 0; r < 4; ++r) eye[r] = (4 * lg + r == ln) ? 1.f : 0.f;
    const f32x4 n2C = mm16sr(nT, nC), n2T = mm16sr(nC, nT);
    const f32x4 m1C = mm16sr(nT, n2C), m1T = mm16sr(n2C, nT);
    const f32x4 n4C = mm16sr(n2T, n2C), n4T = mm16sr(n2C, n2T);
    const f32x4 p1C = eye - nC + n2C - m1C, p1T = eye - nT + n2T - m1T;
    const f32x4 n8C = mm16sr(n4T, n4C);
    f32x4 p2C = p1C, p2T = p1T;
    mm16s(p2C, p1T, n4C);
    mm16s(p2T, n4C, p1T);
    f32x4 xC = p2C, xT = p2T;
    mm16s(xC, p2T, n8C);
    mm16s(xT, n8C, p2T);
    __syncthreads();   // K and Q are dead: their space now holds A and the X blocks

    // ---- phase 3 (stores): A blocks, X_ww in the row layout, T' diagonal block ----
    *(f32x4 *)(sA + (tb0 * 16 + ln) * L::LDA + ib0 * 16 + 4 * lg) = a1;
    if (np == 3) *(f32x4 *)(sA + (3 * 16 + ln) * L::LDA + ib1 * 16 + 4 * lg) = a2;
    *(f32x4 *)(sX + (d0 + ln) * L::LDX + 4 * lg) = xT;
    {
        const f32x4 bcol = *(const f32x4 *)(sBeta + d0 + 4 * lg);
        M::put4((OP *)(bT + swz<OP, kChunk>(split_pos(d0 + ln), d0 + 4 * lg)), xT * bcol);
    }
    __syncthreads();

    // ---- phase 4: off-diagonal blocks of X down block column j = wave:
    // X_ij = -X_ii sum_{m=j}^{i-1} A_im X_mj, stored as T'_ij = X_ij diag(beta_j) ----
    {
        const int j = wave;
        const float bcol = sBeta[16 * j + ln];
        auto arow = [&](int i, int m) {
            return *(const f32x4 *)(sA + (16 * i + ln) * L::LDA + 16 * m + 4 * lg);
        };
        auto xrow = [&](int i) { return *(const f32x4 *)(sX + (16 * i + ln) * L::LDX + 4 * lg); };
        auto put_t = [&](int i, f32x4 z) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Elem<OP>::store((OP *)(bT + swz<OP, kChunk>(split_pos(16 * i + 4 * lg + r), 16 * j + ln)),
                                z[r] * bcol);
        };
        if (j <= 2) {
            const f32x4 xjj = xC;
            f32x4 acc1 = mm16sr(arow(j + 1, j), xjj);
            f32x4 acc2 = {0.f, 0.f, 0.f, 0.f}, acc3 = {0.f, 0.f, 0.f, 0.f};
            if (j + 2 <= 3) acc2 = mm16sr(arow(j + 2, j), xjj);
            if (j + 3 <= 3) acc3 = mm16sr(arow(j + 3, j), xjj);
            const f32x4 x1 = -mm16sr(xrow(j + 1), acc1);            // X_{j+1,j}
            put_t(j + 1, x1);
            if (j + 2 <= 3) {
                mm16s(acc2, arow(j + 2, j + 1), x1);
                if (j + 3 <= 3) mm16s(acc3, arow(j + 3, j + 1), x1);
                const f32x4 x2 = -mm16sr(xrow(j + 2), acc2);        // X_{j+2,j}
                put_t(j + 2, x2);
                if (j + 3 <= 3) {
                    mm16s(acc3, arow(j + 3, j + 2), x2);
                    const f32x4 x3 = -mm16sr(xrow(j + 3), acc3);    // X_{j+3,j}
                    put_t(j + 3, x3);
                }
            }
        }
    }
    __syncthreads();

    // ---- phase 5: the record, granule for granule ----
    u32x4 *dst = (u32x4 *)((unsigned char *)a.prep + (slot * H + h) * (long long)kPrepRecordBytes);
    for (int i = tid; i < kRecGranules; i += 256) dst[i] = *(const u32x4 *)(smem + 16 * i);
}

// =========================================================================================
// Launch 2: the state scan.  Waves 0-1 load, waves 2 .. 2 + DVT/16 - 1 scan.
// =========================================================================================
// Loader waves per workgroup: enough in-flight loads per CU to cover the memory latency.
template <int DVT> constexpr int loaders_for() { return 2; }

// Both stages of an array sit next to each other, so that the stage of a chunk is an
// immediate offset of the LDS instructions (the chunk loop is unrolled by two).
template <int DK, int DVT>
struct LdsSplit {
    static constexpr int szRow = kChunk * DK * 2;       // [64][DK] bf16
    static constexpr int szV = DVT * kChunk * 2;        // [DVT][64] bf16
    static constexpr int sK = 0;                        // K rows (d_k permuted)
    static constexpr int sQ = 2 * szRow;                // Q rows (d_k permuted)
    static constexpr int sKt = 4 * szRow;               // K^T [DK][64] (tokens permuted)
    static constexpr int sRec = 6 * szRow;              // T', P, g (the record)
    static constexpr int sV = sRec + 2 * kPrepRecordBytes;   // V^T tile [DVT][64]
    static constexpr int total = sV + 2 * szV;
    static constexpr int stK = szRow, stKt = szRow, stRec = kPrepRecordBytes, stV = szV;
};

template <int DK, int DVT, int MODE>
__global__ __launch_bounds__(64 * (DVT / 16 + loaders_for<DVT>())) void scan_split_kernel(PrefillArgs a)
{
    using L = LdsSplit<DK, DVT>;
    using OP = uint16_t;
    using M = Mma<OP>;
    using Q4 = Quad<OP>;
    constexpr int MBK = DK / 16;           // 16-row blocks of the state
    constexpr int KBD = DK / 32;           // K-blocks over the key dimension
    constexpr int kLoaders = loaders_for<DVT>();
    constexpr int KG = DK / 8;             // 16-byte granules per key row
    constexpr int VG = DVT / 8;            // 16-byte granules per value-tile row
    constexpr int KB8 = (16 * KG) / 64;    // 4-row x 8-column blocks of K per lane of wave 1
    constexpr int NVB = 16 * VG;           // 4-row x 8-column blocks of the V tile
    constexpr int VB8 = (NVB + 63) / 64;   // ... per lane of wave 1
    constexpr int QI = (kChunk * KG) / 64; // 1 KiB copies of Q rows (wave 0)
    constexpr int RI = kRecG / 1024;       // 1 KiB copies of T' and P (wave 0)
    constexpr bool kY = (MODE == kModeScan);
    static_assert(kLoaders == 2 && (16 * KG) % 64 == 0, "loader split");

    __shared__ __align__(16) unsigned char smem[L::total];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const bool loader = wave < kLoaders;
    const int sw = wave - kLoaders;        // scan wave index (scan waves only)

    // ---- job ----
    const int xcd = blockIdx.x & 7;
    const int rest = blockIdx.x >> 3;
    const int tile = rest % a.ntiles;
    const long long uh = (long long)(rest / a.ntiles) * 8 + xcd;
    if (uh >= a.units * a.H) return;
    Job job;
    job.h = (int)(uh % a.H);
    const long long unit = uh / a.H;
    job.col0 = tile * DVT;
    if (a.table) {
        if (unit >= (long long)*a.n_entries) return;
        const SegEntry e = a.table[unit];
        job.n = e.n;
        job.tok0 = e.tok0;
        job.len = e.len;
        job.seg = e.seg;
        job.nseg = e.nseg;
        job.entry = (int)unit;
    } else {
        job.n = (int)unit;
        seq_bounds(a, job.n, job.tok0, job.len);
        job.seg = 0;
        job.nseg = 1;
        job.entry = -1;
    }
    const bool mpart = (MODE == kModeAug) && job.col0 >= a.dv;
    if (MODE == kModeAug) {
        if (job.seg == job.nseg - 1) return;
        if (mpart && job.seg == 0) return;
    }
    const int H = a.H;
    const int DV = a.dv;
    const int nchunks = (job.len + kChunk - 1) / kChunk;
    // slot of the job's first chunk (segments start on chunk boundaries of their sequence)
    const long long srow0 = first_row(a, job.n);
    const long long slot0 = (srow0 >> 6) + job.n + (job.tok0 - srow0) / kChunk;
    auto nvalid_of = [&](int c) {
        const int r = job.len - c * kChunk;
        return r < kChunk ? r : kChunk;
    };

    // ================================================================ loader waves
    if (loader) {
        // Wave 0 copies Q rows and the record of a chunk global -> LDS with the direct-to-LDS
        // loads (16 bytes per lane; lane l lands at the wave's LDS pointer + 16 l).  It makes
        // no other LDS access, so nothing waits on these copies before the chunk's barrier:
        // the copies of chunk c+1 are issued at the start of iteration c, into the stage that
        // iteration c-1 finished reading.  Wave 1 moves K and the V tile through registers
        // (4-row x 8-column blocks, loaded one chunk ahead), because they are also stored
        // transposed.  Global addresses are a per-chunk base plus 32-bit byte offsets.
        typedef __attribute__((address_space(3))) void lds_void;
        const unsigned rsK = (unsigned)(H * DK) * 2, rsV = (unsigned)(H * DV) * 2;  // bytes
        auto bytes = [](const void *p, unsigned off) {
            return (const void *)((const unsigned char *)p + off);
        };
        auto row_base = [&](const void *t, long long t0, int D) {
            return (const unsigned char *)t + ((t0 * H + job.h) * (long long)D) * 2;
        };
        const std::integral_constant<int, 0> st0{};
        const std::integral_constant<int, 1> st1{};
        if (wave == 0) {
            auto copy = [&](auto stc, int c) {
                constexpr int ST = decltype(stc)::value;
                const long long t0 = job.tok0 + (long long)c * kChunk;
                const int last = nvalid_of(c) - 1;
                if (kY) {
                    const unsigned char *cq = row_base(a.q, t0, DK);
#pragma unroll
                    for (int j = 0; j < QI; ++j) {
                        // physical granule P of the swizzled tile <- logical granule pg ^ s(r)
                        const int P = 64 * j + lane;
                        const int r = P / KG, pg = P % KG;
                        const int rc = r < last ? r : last;
                        const unsigned off = (unsigned)rc * rsK + 16 * (pg ^ swz_key<OP, DK>(r));
                        __builtin_amdgcn_global_load_lds(
                            (const void *)(cq + off),
                            (lds_void *)(smem + L::sQ + ST * L::stK + 1024 * j), 16, 0, 0);
                    }
                }
                const unsigned char *rec = (const unsigned char *)a.prep +
                                           ((slot0 + c) * H + job.h) * (long long)kPrepRecordBytes;
#pragma unroll
                for (int j = 0; j < RI; ++j)
                    __builtin_amdgcn_global_load_lds(
                        (const void *)(rec + 16 * (64 * j + lane)),
                        (lds_void *)(smem + L::sRec + ST * L::stRec + 1024 * j), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(
                    (const void *)(rec + kRecG + 4 * lane),
                    (lds_void *)(smem + L::sRec + ST * L::stRec + kRecG), 4, 0, 0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            };
            if (nchunks > 0) {
                copy(st0, 0);
                __syncthreads();
            }
            for (int c = 0; c < nchunks; c += 2) {
                if (c + 1 < nchunks) copy(st1, c + 1);
                __syncthreads();
                if (c + 1 < nchunks) {
                    if (c + 2 < nchunks) copy(st0, c + 2);
                    __syncthreads();
                }
            }
            return;
        }
        const int ltid = lane;              // wave 1
        unsigned gK[KB8][4], gV[VB8][4];
#pragma unroll
        for (int j = 0; j < KB8; ++j) {
            const int b = ltid + 64 * j;
            const int dg = b / 16, tq = b % 16;
#pragma unroll
            for (int i = 0; i < 4; ++i) gK[j][i] = (unsigned)(4 * tq + i) * rsK + 16 * dg;
        }
#pragma unroll
        for (int j = 0; j < VB8; ++j) {
            const int b = (ltid + 64 * j) % NVB;
            const int dg = b / 16, tq = b % 16;
#pragma unroll
            for (int i = 0; i < 4; ++i) gV[j][i] = (unsigned)(4 * tq + i) * rsV + 16 * dg;
        }
        // Block b = lane + 64 j covers token rows 4 tq .. 4 tq + 3 (tq = b % 16, the fastest,
        // so that the transposed quad stores of 16 lanes fill whole rows of K^T and V^T) and
        // columns 8 dg .. 8 dg + 7 (dg = b / 16).
        // LDS byte offsets of this lane's stores (within a stage)
        unsigned lKr[KB8][4], lKt[KB8][8], lVt[VB8][8];
#pragma unroll
        for (int j = 0; j < KB8; ++j) {
            const int b = ltid + 64 * j;
            const int dg = b / 16, tq = b % 16;
            const int pr = split_pos(4 * tq);
#pragma unroll
            for (int i = 0; i < 4; ++i) lKr[j][i] = (unsigned)(L::sK + swz<OP, DK>(pr + i, 8 * dg));
#pragma unroll
            for (int e = 0; e < 8; ++e)
                lKt[j][e] = (unsigned)(L::sKt + swz<OP, kChunk>(split_pos(8 * dg + e), 4 * tq));
        }
#pragma unroll
        for (int j = 0; j < VB8; ++j) {
            const int b = (ltid + 64 * j) % NVB;
            const int dg = b / 16, tq = b % 16;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                lVt[j][e] = (unsigned)(L::sV + swz<OP, kChunk>(8 * dg + e, 4 * tq));
        }
        u32x4 pk[KB8][4], pv[VB8][4];
        auto vblock = [&](int j) { return ltid + 64 * j < NVB; };
        // register loads of K and V of chunk c
        auto load = [&](int c) {
            const long long t0 = job.tok0 + (long long)c * kChunk;
            const int last = nvalid_of(c) - 1;
            const unsigned char *ck = row_base(a.k, t0, DK);
            const unsigned char *cv = row_base(a.v, t0, DV) + job.col0 * 2;
            if (last == kChunk - 1) {
#pragma unroll
                for (int j = 0; j < KB8; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pk[j][i] = *(const u32x4 *)bytes(ck, gK[j][i]);
                if (!mpart) {
#pragma unroll
                    for (int j = 0; j < VB8; ++j)
                        if (vblock(j)) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                pv[j][i] = *(const u32x4 *)bytes(cv, gV[j][i]);
                        }
                }
            } else {
                // the job's last chunk: rows past its end read its last row instead
#pragma unroll
                for (int j = 0; j < KB8; ++j) {
                    const int b = ltid + 64 * j;
                    const int dg = b / 16, tq = b % 16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 4 * tq + i < last ? 4 * tq + i : last;
                        pk[j][i] = *(const u32x4 *)bytes(ck, (unsigned)t * rsK + 16 * dg);
                    }
                }
                if (!mpart) {
#pragma unroll
                    for (int j = 0; j < VB8; ++j)
                        if (vblock(j)) {
                            const int b = ltid + 64 * j;
                            const int dg = b / 16, tq = b % 16;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int t = 4 * tq + i < last ? 4 * tq + i : last;
                                pv[j][i] = *(const u32x4 *)bytes(cv, (unsigned)t * rsV + 16 * dg);
                            }
                        }
                }
            }
        };
        // K rows (internal token order), K^T (internal d_k order) and V^T of chunk c
        auto store = [&](auto stc, int c) {
            constexpr int ST = decltype(stc)::value;
            const int nv = nvalid_of(c);
            const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < KB8; ++j) {
                const int tq = (ltid + 64 * j) % 16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (4 * tq + i >= nv) pk[j][i] = z;
                    *(u32x4 *)(smem + lKr[j][i] + ST * L::stK) = pk[j][i];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    u32x2 col;
                    col[0] = __builtin_amdgcn_perm(pk[j][1][w], pk[j][0][w], sel);
                    col[1] = __builtin_amdgcn_perm(pk[j][3][w], pk[j][2][w], sel);
                    *(u32x2 *)(smem + lKt[j][e] + ST * L::stKt) = col;
                }
            }
#pragma unroll
            for (int j = 0; j < VB8; ++j) {
                if (!vblock(j)) continue;
                const int tq = (ltid + 64 * j) % 16;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (mpart || 4 * tq + i >= nv) pv[j][i] = z;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    u32x2 col;
                    col[0] = __builtin_amdgcn_perm(pv[j][1][w], pv[j][0][w], sel);
                    col[1] = __builtin_amdgcn_perm(pv[j][3][w], pv[j][2][w], sel);
                    *(u32x2 *)(smem + lVt[j][e] + ST * L::stV) = col;
                }
            }
        };
        if (nchunks > 0) {
            load(0);
            store(st0, 0);
            if (nchunks > 1) load(1);
            __syncthreads();
        }
        // iteration c stores chunk c+1 (stage (c+1) & 1) and loads chunk c+2
        for (int c = 0; c < nchunks; c += 2) {
            if (c + 1 < nchunks) {
                store(st1, c + 1);
                if (c + 2 < nchunks) load(c + 2);
            }
            __syncthreads();
            if (c + 1 < nchunks) {
                if (c + 2 < nchunks) {
                    store(st0, c + 2);
                    if (c + 3 < nchunks) load(c + 3);
                }
                __syncthreads();
            }
        }
        return;
    }

    // ================================================================ scan waves
    const int c0 = job.col0 + 16 * sw;     // first state column of this wave
    f32x4 S[MBK];
    {
        const float *src = nullptr;
        if (MODE == kModeScan) {
            if (job.seg == 0) {
                if (a.s0) src = a.s0 + ((long long)job.n * H + job.h) * DK * DV + c0;
            } else {
                src = a.segB + ((long long)(job.entry - 1) * H + job.h) * DK * DV + c0;
            }
        } else if (!mpart && job.seg == 0 && a.s0) {
            src = a.s0 + ((long long)job.n * H + job.h) * DK * DV + c0;
        }
        // register S[m][i] of lane (ln, lg) holds state row split_orig(16 m + 4 lg + i)
#pragma unroll
        for (int m = 0; m < MBK; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = split_orig(16 * m + 4 * lg + i);
                float x = 0.f;
                if (mpart) x = (row == c0 - DV + ln) ? 1.f : 0.f;
                else if (src) x = src[(long long)row * DV + ln];
                S[m][i] = x;
            }
    }
    auto chunk = [&](auto stc, int c) {
        constexpr int ST = decltype(stc)::value;
        const unsigned char *bKc = smem + L::sK + ST * L::stK;
        const unsigned char *bQc = smem + L::sQ + ST * L::stK;
        const unsigned char *bKt = smem + L::sKt + ST * L::stKt;
        const unsigned char *rec = smem + L::sRec + ST * L::stRec;
        const unsigned char *bTc = rec + kRecT;
        const unsigned char *bPc = rec + kRecP;
        const float *sGc = (const float *)(rec + kRecG);
        const unsigned char *bVc = smem + L::sV + ST * L::stV;
        const long long t0 = job.tok0 + (long long)c * kChunk;
        const int nv = nvalid_of(c);
        // Fragments are loaded one step ahead of the MFMAs that use them; the scheduling
        // fences keep the compiler from sinking each load next to its use.
        bf16x8 fk[2][4], fq[2][4], ft[6];
        auto ld_kq = [&](int kb, int buf) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                fk[buf][tb] = ldfrag<OP, DK>(bKc, tb * 16 + ln, kb * 32 + 8 * lg);
                if (kY) fq[buf][tb] = ldfrag<OP, DK>(bQc, tb * 16 + ln, kb * 32 + 8 * lg);
            }
        };
        auto frag64 = [&](const unsigned char *base, int row, int k0) {
            return ldfrag<OP, kChunk>(base, row, k0 + 8 * lg);
        };

        // ---- K S and S^T Q^T from the chunk-start state ----
        f32x4 accYt[4], acc_ks[4], vv[4], gam[4];
        bf16x8 Sb[KBD];
        ld_kq(0, 0);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            // rows of K S held by this lane: internal 16 tb + 4 lg + i, i.e. tokens o0 + i
            const int o0 = split_orig(tb * 16 + 4 * lg);
            vv[tb] = load4((const OP *)(bVc + swz<OP, kChunk>(16 * sw + ln, o0)));
            gam[tb] = *(const f32x4 *)(sGc + o0);
        }
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) Sb[kb] = pack8s(S[2 * kb], S[2 * kb + 1]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            acc_ks[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            accYt[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            if (kb + 1 < KBD) {
                ld_kq(kb + 1, (kb + 1) & 1);
            } else {
                // T' fragments for U = T' R: rows 0..31 use tokens 0..31 only
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) ft[mb] = frag64(bTc, mb * 16 + ln, 0);
                ft[4] = frag64(bTc, 32 + ln, 32);
                ft[5] = frag64(bTc, 48 + ln, 32);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                M::mma(acc_ks[tb], fk[kb & 1][tb], Sb[kb]);
                if (kY) M::mma(accYt[tb], Sb[kb], fq[kb & 1][tb]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- R = V - diag(gamma) K S;  U = T' R ----
        bf16x8 fkt[2][MBK];
#pragma unroll
        for (int m = 0; m < MBK; ++m) fkt[0][m] = frag64(bKt, m * 16 + ln, 0);
        f32x4 U[4];
        {
            f32x4 R[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) R[tb] = vv[tb] - exp2x4(gam[tb]) * acc_ks[tb];
            const bf16x8 Rb0 = pack8s(R[0], R[1]);
            const bf16x8 Rb1 = pack8s(R[2], R[3]);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                U[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
                M::mma(U[mb], ft[mb], Rb0);
            }
            M::mma(U[2], ft[4], Rb1);
            M::mma(U[3], ft[5], Rb1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < MBK; ++m) fkt[1][m] = frag64(bKt, m * 16 + ln, 32);
        __builtin_amdgcn_sched_barrier(0);

        // ---- S = gamma_C S + K^T diag(gamma_C / gamma) U ----
        const float gC = sGc[kChunk - 1];
        {
            f32x4 Us[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) Us[mb] = U[mb] * exp2x4(gC - gam[mb]);
            const bf16x8 Ub0 = pack8s(Us[0], Us[1]);
            const bf16x8 Ub1 = pack8s(Us[2], Us[3]);
            const float gamC = __builtin_amdgcn_exp2f(gC);
#pragma unroll
            for (int m = 0; m < MBK; ++m) {
                S[m] *= gamC;
                M::mma(S[m], fkt[0][m], Ub0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kY) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) ft[tb] = frag64(bPc, tb * 16 + ln, 0);
                ft[4] = frag64(bPc, 32 + ln, 32);
                ft[5] = frag64(bPc, 48 + ln, 32);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MBK; ++m) M::mma(S[m], fkt[1][m], Ub1);
        }

        // ---- Y^T = S^T Q^T diag(gamma) + U^T P^T ----
        if (kY) {
            const bf16x8 Uu0 = pack8s(U[0], U[1]);
            const bf16x8 Uu1 = pack8s(U[2], U[3]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                accYt[tb] *= __builtin_amdgcn_exp2f(sGc[tb * 16 + ln]);
                M::mma(accYt[tb], Uu0, ft[tb]);
            }
            M::mma(accYt[2], Uu1, ft[4]);
            M::mma(accYt[3], Uu1, ft[5]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = tb * 16 + ln;
                if (t < nv)
                    store4((OP *)a.y + ((t0 + t) * H + job.h) * (long long)DV + c0 + 4 * lg,
                           accYt[tb]);
            }
        }
        __syncthreads();
    };
    if (nchunks > 0) __syncthreads();     // the prologue's barrier (chunk 0 staged)
    for (int c = 0; c < nchunks; c += 2) {
        chunk(std::integral_constant<int, 0>{}, c);
        if (c + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, c + 1);
    }

    // ================================================================ state out
    {
        float *dst = nullptr;
        long long ld = DV;
        if (MODE == kModeScan) {
            if (job.seg == job.nseg - 1 && a.s_final)
                dst = a.s_final + ((long long)job.n * H + job.h) * DK * DV + c0;
        } else if (mpart) {
            dst = a.segM + ((long long)job.entry * H + job.h) * DK * DK + (c0 - DV);
            ld = DK;
        } else {
            dst = a.segB + ((long long)job.entry * H + job.h) * DK * DV + c0;
        }
        if (dst) {
#pragma unroll
            for (int m = 0; m < MBK; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(long long)split_orig(16 * m + 4 * lg + i) * ld + ln] = S[m][i];
        }
    }
}

// =========================================================================================
// Host side
// =========================================================================================
template <int DK>
hipError_t launch_chunk_prep(const PrefillArgs &args, long long nslots, hipStream_t stream)
{
    const long long groups = nslots * args.H;
    if (groups <= 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_prep_kernel<DK>), dim3((unsigned)groups), dim3(256), 0, stream,
                       args, nslots);
    return hipGetLastError();
}

template <int DK, int DVT, int MODE>
hipError_t launch_scan_split(const PrefillArgs &args, long long units, int ntiles,
                             hipStream_t stream)
{
    const long long groups = (units * args.H + 7) / 8 * 8 * ntiles;
    if (groups <= 0) return hipSuccess;
    PrefillArgs a2 = args;
    a2.units = units;
    a2.ntiles = ntiles;
    hipLaunchKernelGGL((scan_split_kernel<DK, DVT, MODE>), dim3((unsigned)groups),
                       dim3(64 * (DVT / 16 + loaders_for<DVT>())), 0, stream, a2);
    return hipGetLastError();
}

template hipError_t launch_chunk_prep<128>(const PrefillArgs &, long long, hipStream_t);
template hipError_t launch_chunk_prep<64>(const PrefillArgs &, long long, hipStream_t);

#define GDN_SPLIT_INST(DK, DVT)                                                               \
    template hipError_t launch_scan_split<DK, DVT, kModeScan>(const PrefillArgs &, long long, \
                                                              int, hipStream_t);              \
    template hipError_t launch_scan_split<DK, DVT, kModeAug>(const PrefillArgs &, long long,  \
                                                             int, hipStream_t);
GDN_SPLIT_INST(128, 16)
GDN_SPLIT_INST(128, 32)
GDN_SPLIT_INST(128, 64)
GDN_SPLIT_INST(64, 16)
GDN_SPLIT_INST(64, 32)
GDN_SPLIT_INST(64, 64)
#undef GDN_SPLIT_INST

}  // namespace gdn
