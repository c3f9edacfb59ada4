// gdn_prefill_ws.hip -- warp-specialised chunked prefill for bf16 inputs (gfx950).
//
// Same chunk algebra as gdn_prefill.hip (the WY / UT form of the reading notes'
// transition-matrix recurrence, section 2.1), split over two kinds of waves of one
// workgroup that own one (sequence, head, 16 x NSW state columns) chain:
//
//   producer waves (4): for chunk c+1 they stage K, Q, V and the gates in LDS, form the
//     decay-masked Gram matrices A and P, and invert the unit lower-triangular I + A
//     (T' = (I + A)^{-1} diag(beta)).  This is the latency-bound, state-independent part.
//   scan waves (NSW): each owns 16 state columns for all d_k rows, in MFMA accumulator
//     registers, and runs the state-dependent chunk update for chunk c entirely in
//     registers: R = V - diag(gamma) K S, U = T' R, S = gamma_C S + K^T diag(gamma_C/gamma) U,
//     Y^T = S^T Q^T diag(gamma) + U^T P^T.  Every intermediate that feeds the next product
//     stays in the accumulator layout, which is the operand layout of that product when the
//     contraction index of a 32-wide K-block is split as {4g..4g+3} U {16+4g..16+4g+3}
//     (g = lane / 16).  No LDS round trip and no barrier sit on the state's dependency chain.
//
// The two roles overlap: all waves meet at four barriers per chunk, and the chunk-c data the
// scan waves read is double-buffered (K, Q, P, g) or written by the producers only after the
// scan waves are past their last read of it (T', V^T, K^T).
#include "gdn_prefill_common.hpp"

namespace gdn {

constexpr int kProducers = 4;

template <int DK, int DVT>
struct LdsWs {
    static constexpr int al(int x) { return (x + 255) & ~255; }
    static constexpr int szRow = kChunk * DK * 2;        // [64][DK] bf16
    static constexpr int szPT = kChunk * kChunk * 2;     // [64][64] bf16
    static constexpr int szV = DVT * kChunk * 2;         // [DVT][64] bf16
    static constexpr int LDA = kChunk + 4;               // padded fp32 rows of A
    static constexpr int LDX = 20;                       // padded rows of a diagonal X block
    // double-buffered stages: K, Q rows, P, T', V^T, g
    static constexpr int oK0 = 0;
    static constexpr int oK1 = szRow;
    static constexpr int oQ0 = 2 * szRow;
    static constexpr int oQ1 = 3 * szRow;
    static constexpr int oP0 = 4 * szRow;
    static constexpr int oP1 = oP0 + szPT;
    static constexpr int oT0 = oP1 + szPT;
    static constexpr int oT1 = oT0 + szPT;
    static constexpr int oV0 = oT1 + szPT;
    static constexpr int oV1 = oV0 + szV;
    static constexpr int oG0 = oV1 + szV;
    static constexpr int oG1 = oG0 + kChunk * 4;
    // single buffers
    static constexpr int oKt = al(oG1 + kChunk * 4);
    static constexpr int oA = al(oKt + DK * kChunk * 2);
    static constexpr int oX = al(oA + kChunk * LDA * 4);
    static constexpr int oB = al(oX + 4 * 16 * LDX * 4);
    static constexpr int total = oB + kChunk * 4;
};

// Eight bf16 operand values from two 4-element runs of a swizzled row-major tile: elements
// k0 + 4g .. k0 + 4g + 3 and k0 + 16 + 4g .. + 3 of row `row` (the split K-block mapping).
template <int W>
__device__ __forceinline__ bf16x8 ldsplit(const unsigned char *base, int row, int k0, int lg)
{
    const u32x2 lo = *(const u32x2 *)(base + swz<uint16_t, W>(row, k0 + 4 * lg));
    const u32x2 hi = *(const u32x2 *)(base + swz<uint16_t, W>(row, k0 + 16 + 4 * lg));
    const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, w);
}

// Two accumulator blocks (rows 4g..4g+3 of blocks 2kb and 2kb+1) as one bf16 operand.
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b)
{
    const bf16x4 l = __builtin_convertvector(a, bf16x4);
    const bf16x4 h = __builtin_convertvector(b, bf16x4);
    return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
}

__device__ __forceinline__ f32x4 exp2v(f32x4 x)
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
__device__ __forceinline__ void mm16(f32x4 &c, f32x4 arow, f32x4 bcol)
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

__device__ __forceinline__ f32x4 mm16r(f32x4 arow, f32x4 bcol)
{
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    mm16(c, arow, bcol);
    return c;
}

template <int DK, int DVT, int MODE>
__global__ __launch_bounds__(64 * (DVT / 16 + kProducers)) void prefill_ws_kernel(PrefillArgs a)
{
    using L = LdsWs<DK, DVT>;
    using OP = uint16_t;
    using M = Mma<OP>;
    using Q4 = Quad<OP>;
    constexpr int NSW = DVT / 16;          // scan waves
    constexpr int MBK = DK / 16;           // 16-row blocks of the state
    constexpr int KBD = DK / 32;           // K-blocks over the key dimension
    constexpr int DQ = DK / 4;             // quads per key row
    constexpr int VQ = DVT / 4;            // quads per value-tile row
    constexpr int PT = kProducers * 64;    // producer threads
    constexpr int KBLK = (16 * DQ) / PT;   // 4x4 blocks of K / Q per producer thread
    constexpr int VBLK = (16 * VQ + PT - 1) / PT;
    constexpr bool kY = (MODE == kModeScan);
    static_assert((16 * DQ) % PT == 0, "K tile must split evenly over producer threads");

    __shared__ __align__(16) unsigned char smem[L::total];
    float *const sA = (float *)(smem + L::oA);
    float *const sX = (float *)(smem + L::oX);
    float *const sBeta = (float *)(smem + L::oB);
    unsigned char *const bKt = smem + L::oKt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index held in a scalar register: the role branches below are wave-uniform, and
    // both roles execute the same number of barriers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const bool producer = wave < kProducers;
    const int sw = wave - kProducers;      // scan wave index (scan waves only)

    // ---- job (same decoding as the 4-wave kernel) ----
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
    const OP *gq = (const OP *)a.q;
    const OP *gk = (const OP *)a.k;
    const OP *gv = (const OP *)a.v;
    const int nchunks = (job.len + kChunk - 1) / kChunk;
    auto nvalid_of = [&](int c) {
        const int r = job.len - c * kChunk;
        return r < kChunk ? r : kChunk;
    };

    // ================================================================ scan-wave state
    const int c0 = job.col0 + 16 * (producer ? 0 : sw);   // first state column of this wave
    f32x4 S[MBK];
    if (!producer) {
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
#pragma unroll
        for (int m = 0; m < MBK; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * m + 4 * lg + i;
                float x = 0.f;
                if (mpart) x = (row == c0 - DV + ln) ? 1.f : 0.f;
                else if (src) x = src[(long long)row * DV + ln];
                S[m][i] = x;
            }
    }

    // ================================================================ producer state
    Q4 pk[KBLK][4], pq[KBLK][4], pv[VBLK][4];
    float pa = 1.f;
    auto prefetch_kq = [&](int c) {
        const long long t0 = job.tok0 + (long long)c * kChunk;
        const int nv = nvalid_of(c);
        const OP *ck = gk + (t0 * H + job.h) * (long long)DK;
        const OP *cq = gq + (t0 * H + job.h) * (long long)DK;
#pragma unroll
        for (int j = 0; j < KBLK; ++j) {
            const int b = tid + PT * j;
            const int dq = b % DQ, tq = b / DQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * tq + i;
                const int tc = t < nv ? t : nv - 1;
                const int off = tc * H * DK + 4 * dq;
                pk[j][i] = Q4::load(ck + off);
                if (kY) pq[j][i] = Q4::load(cq + off);
            }
        }
        const int tc = lane < nv ? lane : nv - 1;
        const float *g = (wave == 0) ? a.alpha : a.beta;
        pa = g[(t0 + tc) * H + job.h];
    };
    auto prefetch_v = [&](int c) {
        if (mpart) {
#pragma unroll
            for (int j = 0; j < VBLK; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[j][i] = Q4::zero();
            return;
        }
        const long long t0 = job.tok0 + (long long)c * kChunk;
        const int nv = nvalid_of(c);
        const OP *cv = gv + (t0 * H + job.h) * (long long)DV + job.col0;
#pragma unroll
        for (int j = 0; j < VBLK; ++j) {
            const int b = (tid + PT * j) % (16 * VQ);
            const int dq = b % VQ, tq = b / VQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * tq + i;
                const int tc = t < nv ? t : nv - 1;
                pv[j][i] = Q4::load(cv + tc * H * DV + 4 * dq);
            }
        }
    };

    // P1: K, Q rows, V^T and the gates of chunk c into stage (c & 1)
    auto produce_stage = [&](int c) {
        const int st = c & 1;
        unsigned char *bK = smem + (st ? L::oK1 : L::oK0);
        unsigned char *bQ = smem + (st ? L::oQ1 : L::oQ0);
        unsigned char *bV = smem + (st ? L::oV1 : L::oV0);
        float *sG = (float *)(smem + (st ? L::oG1 : L::oG0));
        const int nv = nvalid_of(c);
#pragma unroll
        for (int j = 0; j < KBLK; ++j) {
            const int b = tid + PT * j;
            const int dq = b % DQ, tq = b / DQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned keep = (4 * tq + i < nv) ? 0xffffffffu : 0u;
                pk[j][i].mask(keep);
                pk[j][i].store((OP *)(bK + swz<OP, DK>(4 * tq + i, 4 * dq)));
                if (kY) {
                    pq[j][i].mask(keep);
                    pq[j][i].store((OP *)(bQ + swz<OP, DK>(4 * tq + i, 4 * dq)));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < VBLK; ++j) {
            const int b = tid + PT * j;
            if (b < 16 * VQ) {
                const int dq = b % VQ, tq = b / VQ;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pv[j][i].mask((4 * tq + i < nv && !mpart) ? 0xffffffffu : 0u);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    Q4::column(pv[j], jj).store((OP *)(bV + swz<OP, kChunk>(4 * dq + jj, 4 * tq)));
            }
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
    };

    // P2: Gram tiles of chunk c -> A (off-diagonal tiles, fp32) and P; wave w also inverts
    // the diagonal block w of I + A in registers:  with N the strictly lower part,
    // (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) exactly (N^16 = 0).  Both X and X^T
    // are carried in the accumulator layout: the accumulator layout of M^T is the row
    // layout of M, so every product has its operands at hand.  Wave w takes the diagonal
    // pair (w, w) and the off-diagonal pairs {(1,0),(3,0)}, {(2,0),(3,1)}, {(2,1)}, {(3,2)}.
    f32x4 xcol[4];
    auto produce_gram = [&](int c) {
        const int st = c & 1;
        const unsigned char *bK = smem + (st ? L::oK1 : L::oK0);
        const unsigned char *bQ = smem + (st ? L::oQ1 : L::oQ0);
        unsigned char *bP = smem + (st ? L::oP1 : L::oP0);
        unsigned char *bTs = smem + (st ? L::oT1 : L::oT0);
        const float *sG = (const float *)(smem + (st ? L::oG1 : L::oG0));
        // up to three tile pairs interleaved by K-block (independent accumulators back to back)
        auto gram3 = [&](const int (&tb)[3], const int (&ib)[3], int np, f32x4 (&accG)[3],
                         f32x4 (&accP)[3]) {
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
                        const auto ai = ldfrag<OP, DK>(bK, ib[p] * 16 + ln, kb * 32 + 8 * lg);
                        const auto bt = ldfrag<OP, DK>(bK, tb[p] * 16 + ln, kb * 32 + 8 * lg);
                        M::mma(accG[p], ai, bt);
                        if (kY) {
                            const auto bq = ldfrag<OP, DK>(bQ, tb[p] * 16 + ln, kb * 32 + 8 * lg);
                            M::mma(accP[p], ai, bq);
                        }
                    }
                }
            }
        };
        // accG[r] = k_i . k_t, accP[r] = k_i . q_t for i = ib*16 + 4lg + r, t = tb*16 + ln
        auto mask_store = [&](int tb, int ib, f32x4 accG, f32x4 accP) {
            const int t = tb * 16 + ln;
            const float gt = sG[t];
            const float bt_ = sBeta[t];
            const f32x4 gi = *(const f32x4 *)(sG + ib * 16 + 4 * lg);
            f32x4 av, pv4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ib * 16 + 4 * lg + r;
                const float dec = (i <= t) ? __builtin_amdgcn_exp2f(gt - gi[r]) : 0.f;
                av[r] = (i < t) ? bt_ * accG[r] * dec : 0.f;
                pv4[r] = accP[r] * dec;
            }
            if (tb != ib) *(f32x4 *)(sA + t * L::LDA + ib * 16 + 4 * lg) = av;
            if (kY) M::put4((OP *)(bP + swz<OP, kChunk>(t, ib * 16 + 4 * lg)), pv4);
            return av;
        };
        // diagonal pair first: its inverse is the long dependency chain
        const int d0 = wave * 16;
        // pairs of this wave: the diagonal one first, then the off-diagonal ones
        const int np = wave < 2 ? 3 : 2;
        const int tb0 = wave == 0 ? 1 : (wave == 1 ? 2 : (wave == 2 ? 2 : 3));
        const int ib0 = wave == 0 ? 0 : (wave == 1 ? 0 : (wave == 2 ? 1 : 2));
        const int ib1 = wave == 0 ? 0 : 1;
        const int tbs[3] = {wave, tb0, 3};
        const int ibs[3] = {wave, ib0, ib1};
        f32x4 accG[3], accP[3];
        gram3(tbs, ibs, np, accG, accP);
        const f32x4 gD = accG[0], pD = accP[0];
        // N^T and N of the diagonal block in the accumulator layout
        const f32x4 nT = mask_store(wave, wave, gD, pD);
        f32x4 nC;
        {
            const int t = d0 + ln;
            const float gt = sG[t];
            const f32x4 gi = *(const f32x4 *)(sG + d0 + 4 * lg);
            const f32x4 bi = *(const f32x4 *)(sBeta + d0 + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = d0 + 4 * lg + r;
                nC[r] = (t < i) ? bi[r] * gD[r] * __builtin_amdgcn_exp2f(gi[r] - gt) : 0.f;
            }
        }
        mask_store(tb0, ib0, accG[1], accP[1]);
        if (np == 3) mask_store(3, ib1, accG[2], accP[2]);
        if (kY && (wave == 0 || wave == 2))
            M::put4((OP *)(bP + swz<OP, kChunk>(d0 + ln, d0 + 16 + 4 * lg)),
                    f32x4{0.f, 0.f, 0.f, 0.f});
        // (I + N)^{-1} by doubling; C = accumulator layout of M, T = of M^T
        f32x4 eye;
#pragma unroll
        for (int r = 0; r < 4; ++r) eye[r] = (4 * lg + r == ln) ? 1.f : 0.f;
        const f32x4 n2C = mm16r(nT, nC), n2T = mm16r(nC, nT);
        const f32x4 m1C = mm16r(nT, n2C), m1T = mm16r(n2C, nT);      // N N^2 and its transpose
        const f32x4 n4C = mm16r(n2T, n2C), n4T = mm16r(n2C, n2T);
        const f32x4 p1C = eye - nC + n2C - m1C, p1T = eye - nT + n2T - m1T;
        const f32x4 n8C = mm16r(n4T, n4C);
        f32x4 p2C = p1C, p2T = p1T;
        mm16(p2C, p1T, n4C);
        mm16(p2T, n4C, p1T);
        f32x4 xC = p2C, xT = p2T;
        mm16(xC, p2T, n8C);
        mm16(xT, n8C, p2T);
#pragma unroll
        for (int m = 0; m < 4; ++m) xcol[m] = (m == wave) ? xC : f32x4{0.f, 0.f, 0.f, 0.f};
        // row layout of X_ww for the other block columns; T' diagonal block (row d0 + ln,
        // columns d0 + 4lg .. + 3, scaled by beta of the column)
        *(f32x4 *)(sX + (d0 + ln) * L::LDX + 4 * lg) = xT;
        const f32x4 bcol = *(const f32x4 *)(sBeta + d0 + 4 * lg);
        M::put4((OP *)(bTs + swz<OP, kChunk>(d0 + ln, d0 + 4 * lg)), xT * bcol);
        if (wave == 0 || wave == 2)
            M::put4((OP *)(bTs + swz<OP, kChunk>(d0 + ln, d0 + 16 + 4 * lg)),
                    f32x4{0.f, 0.f, 0.f, 0.f});
    };

    // P3: off-diagonal blocks of X down block column j = wave:
    // X_ij = -X_ii sum_{m=j}^{i-1} A_im X_mj, then T'; K^T of chunk c from its K rows.
    auto produce_offdiag = [&](int c) {
        const int st = c & 1;
        unsigned char *bTs = smem + (st ? L::oT1 : L::oT0);
        const int j = wave;
        const float bcol = sBeta[16 * j + ln];
        // A_im in the row layout and X_ii in the row layout, all loaded up front
        auto arow = [&](int i, int m) {
            return *(const f32x4 *)(sA + (16 * i + ln) * L::LDA + 16 * m + 4 * lg);
        };
        auto xrow = [&](int i) { return *(const f32x4 *)(sX + (16 * i + ln) * L::LDX + 4 * lg); };
        auto put_t = [&](int i, f32x4 z) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Elem<OP>::store((OP *)(bTs + swz<OP, kChunk>(16 * i + 4 * lg + r, 16 * j + ln)),
                                z[r] * bcol);
        };
        // products with the column's diagonal block first (independent of each other), then
        // the chain down the column, each new block feeding the rows below it
        if (j <= 2) {
            const f32x4 xjj = xcol[j];
            f32x4 acc1 = mm16r(arow(j + 1, j), xjj);
            f32x4 acc2 = {0.f, 0.f, 0.f, 0.f}, acc3 = {0.f, 0.f, 0.f, 0.f};
            if (j + 2 <= 3) acc2 = mm16r(arow(j + 2, j), xjj);
            if (j + 3 <= 3) acc3 = mm16r(arow(j + 3, j), xjj);
            const f32x4 x1 = -mm16r(xrow(j + 1), acc1);            // X_{j+1,j}
            put_t(j + 1, x1);
            if (j + 2 <= 3) {
                mm16(acc2, arow(j + 2, j + 1), x1);
                if (j + 3 <= 3) mm16(acc3, arow(j + 3, j + 1), x1);
                const f32x4 x2 = -mm16r(xrow(j + 2), acc2);        // X_{j+2,j}
                put_t(j + 2, x2);
                if (j + 3 <= 3) {
                    mm16(acc3, arow(j + 3, j + 2), x2);
                    const f32x4 x3 = -mm16r(xrow(j + 3), acc3);    // X_{j+3,j}
                    put_t(j + 3, x3);
                }
            }
        }
        const unsigned char *bK = smem + (st ? L::oK1 : L::oK0);
#pragma unroll
        for (int jb = 0; jb < KBLK; ++jb) {
            const int b = tid + PT * jb;
            const int dq = b % DQ, tq = b / DQ;
            Q4 rows[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rows[i] = Q4::load((const OP *)(bK + swz<OP, DK>(4 * tq + i, 4 * dq)));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Q4::column(rows, jj).store((OP *)(bKt + swz<OP, kChunk>(4 * dq + jj, 4 * tq)));
        }
    };

    // ================================================================ producer waves
    if (producer) {
        if (nchunks > 0) {
            prefetch_kq(0);
            prefetch_v(0);
            produce_stage(0);
            if (nchunks > 1) {
                prefetch_kq(1);
                prefetch_v(1);
            }
            __syncthreads();
            produce_gram(0);
            __syncthreads();
            produce_offdiag(0);
            __syncthreads();
        }
        for (int c = 0; c < nchunks; ++c) {
            const bool more = c + 1 < nchunks;
            if (more) {
                produce_stage(c + 1);
                if (c + 2 < nchunks) {
                    prefetch_kq(c + 2);
                    prefetch_v(c + 2);
                }
            }
            __syncthreads();
            if (more) produce_gram(c + 1);
            __syncthreads();
            if (more) produce_offdiag(c + 1);
            __syncthreads();
        }
        return;
    }

    // ================================================================ scan waves
    if (nchunks > 0) {
        // the prologue's three barriers (chunk 0 being produced)
        __syncthreads();
        __syncthreads();
        __syncthreads();
    }
    for (int c = 0; c < nchunks; ++c) {
        const int st = c & 1;
        const long long t0 = job.tok0 + (long long)c * kChunk;
        const int nv = nvalid_of(c);
        const unsigned char *bKc = smem + (st ? L::oK1 : L::oK0);
        const unsigned char *bQc = smem + (st ? L::oQ1 : L::oQ0);
        const unsigned char *bPc = smem + (st ? L::oP1 : L::oP0);
        const unsigned char *bTc = smem + (st ? L::oT1 : L::oT0);
        const unsigned char *bVc = smem + (st ? L::oV1 : L::oV0);
        const float *sGc = (const float *)(smem + (st ? L::oG1 : L::oG0));

        // ---- phase 1: K S, S^T Q^T (chunk-start state); R = V - diag(gamma) K S; U = T' R
        f32x4 accYt[4], U[4];
        {
            f32x4 acc_ks[4];
            bf16x8 Sb[KBD];
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) Sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                acc_ks[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                accYt[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // K-block outermost: consecutive MFMAs write different accumulators
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    M::mma(acc_ks[tb], ldsplit<DK>(bKc, tb * 16 + ln, kb * 32, lg), Sb[kb]);
                    if (kY) M::mma(accYt[tb], Sb[kb], ldsplit<DK>(bQc, tb * 16 + ln, kb * 32, lg));
                }
            }
            f32x4 R[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int trow = tb * 16 + 4 * lg;
                const f32x4 gam = exp2v(*(const f32x4 *)(sGc + trow));
                const f32x4 vv = load4((const OP *)(bVc + swz<OP, kChunk>(16 * sw + ln, trow)));
                R[tb] = vv - gam * acc_ks[tb];
            }
            const bf16x8 Rb0 = pack8(R[0], R[1]);
            const bf16x8 Rb1 = pack8(R[2], R[3]);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                U[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
                M::mma(U[mb], ldsplit<kChunk>(bTc, mb * 16 + ln, 0, lg), Rb0);
            }
            M::mma(U[2], ldsplit<kChunk>(bTc, 32 + ln, 32, lg), Rb1);
            M::mma(U[3], ldsplit<kChunk>(bTc, 48 + ln, 32, lg), Rb1);
        }
        __syncthreads();

        // ---- phase 2: S = gamma_C S + K^T diag(gamma_C / gamma) U; Y^T += U^T P^T ----
        {
            const float gC = sGc[kChunk - 1];
            f32x4 Us[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                Us[mb] = U[mb] * exp2v(gC - *(const f32x4 *)(sGc + mb * 16 + 4 * lg));
            const bf16x8 Ub0 = pack8(Us[0], Us[1]);
            const bf16x8 Ub1 = pack8(Us[2], Us[3]);
            const float gamC = __builtin_amdgcn_exp2f(gC);
#pragma unroll
            for (int m = 0; m < MBK; ++m) {
                S[m] *= gamC;
                M::mma(S[m], ldsplit<kChunk>(bKt, m * 16 + ln, 0, lg), Ub0);
            }
#pragma unroll
            for (int m = 0; m < MBK; ++m) M::mma(S[m], ldsplit<kChunk>(bKt, m * 16 + ln, 32, lg), Ub1);
            if (kY) {
                const bf16x8 Uu0 = pack8(U[0], U[1]);
                const bf16x8 Uu1 = pack8(U[2], U[3]);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    accYt[tb] *= __builtin_amdgcn_exp2f(sGc[tb * 16 + ln]);
                    M::mma(accYt[tb], Uu0, ldsplit<kChunk>(bPc, tb * 16 + ln, 0, lg));
                }
                M::mma(accYt[2], Uu1, ldsplit<kChunk>(bPc, 32 + ln, 32, lg));
                M::mma(accYt[3], Uu1, ldsplit<kChunk>(bPc, 48 + ln, 32, lg));
            }
        }
        __syncthreads();

        // ---- phase 3: y ----
        if (kY) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = tb * 16 + ln;
                if (t < nv)
                    store4((OP *)a.y + ((t0 + t) * H + job.h) * (long long)DV + c0 + 4 * lg,
                           accYt[tb]);
            }
        }
        __syncthreads();
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
                    dst[(long long)(16 * m + 4 * lg + i) * ld + ln] = S[m][i];
        }
    }
}

template <int DK, int DVT, int MODE>
hipError_t launch_scan_ws(const PrefillArgs &args, long long units, int ntiles,
                          hipStream_t stream)
{
    const long long groups = (units * args.H + 7) / 8 * 8 * ntiles;
    if (groups <= 0) return hipSuccess;
    PrefillArgs a2 = args;
    a2.units = units;
    a2.ntiles = ntiles;
    hipLaunchKernelGGL((prefill_ws_kernel<DK, DVT, MODE>), dim3((unsigned)groups),
                       dim3(64 * (DVT / 16 + kProducers)), 0, stream, a2);
    return hipGetLastError();
}

#define GDN_WS_INST(DK, DVT)                                                                \
    template hipError_t launch_scan_ws<DK, DVT, kModeScan>(const PrefillArgs &, long long, \
                                                           int, hipStream_t);              \
    template hipError_t launch_scan_ws<DK, DVT, kModeAug>(const PrefillArgs &, long long,  \
                                                          int, hipStream_t);
GDN_WS_INST(128, 32)
GDN_WS_INST(128, 64)
GDN_WS_INST(64, 32)
GDN_WS_INST(64, 64)
#undef GDN_WS_INST

}  // namespace gdn
