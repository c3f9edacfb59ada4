// gdn_prefill.hip -- chunked gated delta rule prefill for gfx950.
//
// Method (jianyuh.github.io reading notes on Qwen3.8-Next, section 2.1 "Gated DeltaNet",
// the boxed transition form S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
// y_t = S_t^T q_t).  Unrolling that form over a chunk of C = 64 tokens that starts at state
// S gives an exact chunk update (the WY / UT representation of a product of rank-one
// corrected identities).  With g_t the within-chunk prefix sum of log alpha,
// gamma_t = e^{g_t}, Gamma_ti = e^{g_t - g_i} (i <= t) and
//     A  = diag(beta) strictlower(K K^T o Gamma)            (decayed Gram, a1)
//     T' = (I + A)^{-1} diag(beta)                          (unit-lower solve, a2)
//     P  = lower(Q K^T o Gamma)                             (intra-chunk scores, a4)
// every chunk step is
//     R  = V - diag(gamma) K S                              (what the keys already hold)
//     U  = T' R                                             (the written residuals, a3)
//     Y  = diag(gamma) Q S + P U                            (outputs, a5)
//     S  = gamma_C S + (diag(gamma_C / gamma) K)^T U        (next chunk's state, a5)
// All decay factors come from differences of within-chunk log sums, so they are <= 1 and
// nothing overflows or underflows to 0/0.
//
// One workgroup (4 waves) owns one (sequence, head, column tile of the state) chain.  The
// fp32 state tile stays in the MFMA accumulator registers for the whole sequence; the
// chunk-local products (Gram, solve) are recomputed per column tile, which keeps every
// intermediate on chip (no workspace round trip through HBM).  Products run on
// v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation) for bf16 inputs and on
// v_mfma_f32_16x16x4_f32 for fp32 inputs.
//
// Long sequences are cut into segments (segment-parallel scan): phase A scans each segment
// from a zero state with the augmented state [S | M] (M starts at I with V = 0, giving the
// segment's transition matrix), phase B folds S_{p+1} = M_p S_p + B_p per sequence, and
// phase C rescans every segment from its true start state and writes y.  The composition
// is exact because the chunk update is affine in S.
#include "gdn_prefill_common.hpp"

namespace gdn {

// ---------------------------------------------------------------------------------------
// The chunked scan.  MODE == kModeScan: start from S0 (or a segment start state), write y
// and (for the last segment) the final state.  MODE == kModeAug: phase A of the segment
// scan; no y; columns col0 >= d_v belong to the transition part (V = 0, start = identity).
//
// Per chunk, six barriers separate the phases:
//   a  prefetched K, Q, V, gates -> LDS (K, Q row major; K, V transposed); log2 prefix of
//      alpha; issue the global loads of the next chunk
//   b  Gram tiles K K^T, K Q^T -> decay-masked A (fp32) and P; K S and S^T Q^T; R
//   c  R -> LDS; diagonal 16 x 16 blocks of X = (I + A)^{-1} by forward substitution
//   d  off-diagonal blocks of X on fp32 MFMA; T' = X diag(beta)
//   e  U = T' R
//   f  Y^T = S^T Q^T diag(gamma) + U^T P^T -> y; S = gamma_C S + K^T diag(gamma_C/gamma) U
// ---------------------------------------------------------------------------------------
template <int DK, int DVT, typename OP, int MODE>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a)
{
    using L = Lds<DK, DVT, OP>;
    using M = Mma<OP>;
    using Q4 = Quad<OP>;
    constexpr int NB = DVT / 16;          // 16-column blocks of the tile
    constexpr int KBD = DK / 32;          // K-blocks over the key dimension
    constexpr int MBS = DK / 64;          // 16-row blocks of S owned by each wave
    constexpr int DQ = DK / 4;            // quads per key row
    constexpr int VQ = DVT / 4;           // quads per value-tile row
    constexpr int KBLK = (16 * DQ + kThreads - 1) / kThreads;   // 4x4 blocks per thread
    constexpr int VBLK = (16 * VQ + kThreads - 1) / kThreads;
    constexpr bool kY = (MODE == kModeScan);

    __shared__ __align__(16) unsigned char smem[L::total];
    unsigned char *const bK = smem + L::oK;
    unsigned char *const bQ = smem + L::oQ;
    unsigned char *const bRt = smem + L::oRt;
    unsigned char *const bUt = smem + L::oUt;
    unsigned char *const bUs = smem + L::oUs;
    unsigned char *const bVt = smem + L::oVt;
    float *const sX = (float *)(smem + L::oX);
    unsigned char *const bKt = smem + L::oKt;
    float *const sA = (float *)(smem + L::oA);
    unsigned char *const bP = smem + L::oP;
    unsigned char *const bT = smem + L::oT;
    unsigned char *const bSt = smem + L::oSt;
    float *const sG = (float *)(smem + L::oG);
    float *const sBeta = (float *)(smem + L::oB);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;
    const int lg = lane >> 4;

    // ---- decode the job (XCD-aware: all column tiles of one unit share blockIdx % 8) ----
    const int xcd = blockIdx.x & 7;
    const int rest = blockIdx.x >> 3;
    const int tile = rest % a.ntiles;
    const long long uh = (long long)(rest / a.ntiles) * 8 + xcd;   // unit * H + head
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
        if (job.seg == job.nseg - 1) return;          // last segment: phase C finishes it
        if (mpart && job.seg == 0) return;            // first segment starts from the true S0
    }
    const int H = a.H;
    const int DV = a.dv;
    const OP *gq = (const OP *)a.q;
    const OP *gk = (const OP *)a.k;
    const OP *gv = (const OP *)a.v;

    // ---- initial state: S registers in the accumulator layout ----
    // wave w owns state rows [w*DK/4, (w+1)*DK/4), i.e. MBS 16-row blocks
    f32x4 S[MBS][NB];
    {
        const float *src = nullptr;
        if (MODE == kModeScan) {
            if (job.seg == 0) {
                if (a.s0) src = a.s0 + ((long long)job.n * H + job.h) * DK * DV + job.col0;
            } else {
                src = a.segB + ((long long)(job.entry - 1) * H + job.h) * DK * DV + job.col0;
            }
        } else if (!mpart && job.seg == 0 && a.s0) {
            src = a.s0 + ((long long)job.n * H + job.h) * DK * DV + job.col0;
        }
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = (wave * MBS + mb) * 16 + 4 * lg + i;
                    const int col = nb * 16 + ln;
                    float x = 0.f;
                    if (mpart) x = (row == job.col0 - DV + col) ? 1.f : 0.f;
                    else if (src) x = src[(long long)row * DV + col];
                    S[mb][nb][i] = x;
                }
    }

    // ---- global -> register prefetch of one chunk.  Rows past the end of the sequence are
    //      clamped to its last row (no load is predicated); they are zeroed when the
    //      registers are stored to LDS in the next iteration, so nothing here waits for the
    //      loads to return.
    Q4 pk[KBLK][4], pq[KBLK][4], pv[VBLK][4];
    float pa = 1.f;   // threads 0..63: alpha of token (tid); threads 64..127: beta
    auto prefetch = [&](long long t0, int nvalid) {
        const OP *ck = gk + (t0 * H + job.h) * (long long)DK;
        const OP *cq = gq + (t0 * H + job.h) * (long long)DK;
#pragma unroll
        for (int j = 0; j < KBLK; ++j) {
            const int b = tid + kThreads * j;
            const int dq = b % DQ, tq = b / DQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * tq + i;
                const int tc = t < nvalid ? t : nvalid - 1;
                const int off = tc * H * DK + 4 * dq;
                pk[j][i] = Q4::load(ck + off);
                if (kY) pq[j][i] = Q4::load(cq + off);
            }
        }
        // V tile (every thread loads; threads past the 16 x VQ blocks re-read a valid block
        // and never store it).  The transition columns of phase A have V = 0 (uniform per
        // workgroup).
        if (!mpart) {
            const OP *cv = gv + (t0 * H + job.h) * (long long)DV + job.col0;
#pragma unroll
            for (int j = 0; j < VBLK; ++j) {
                const int b = (tid + kThreads * j) % (16 * VQ);
                const int dq = b % VQ, tq = b / VQ;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * tq + i;
                    const int tc = t < nvalid ? t : nvalid - 1;
                    pv[j][i] = Q4::load(cv + tc * H * DV + 4 * dq);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < VBLK; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[j][i] = Q4::zero();
        }
        // gates: lanes of wave 0 read alpha, every other lane beta, of token (lane)
        {
            const int t = lane;
            const int tc = t < nvalid ? t : nvalid - 1;
            const float *g = (tid < 64) ? a.alpha : a.beta;
            pa = g[(t0 + tc) * H + job.h];
        }
    };

    // S -> LDS (transposed copy, the operand of K S and S^T Q^T)
    auto store_state_lds = [&]() {
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                M::put4((OP *)(bSt + swz<OP, DK>(nb * 16 + ln, (wave * MBS + mb) * 16 + 4 * lg)),
                        S[mb][nb]);
    };
    store_state_lds();

    const int nchunks = (job.len + kChunk - 1) / kChunk;
    if (nchunks > 0) prefetch(job.tok0, job.len < kChunk ? job.len : kChunk);

    const int trow = wave * 16 + 4 * lg;   // first token row of this lane in the acc layout

    for (int c = 0; c < nchunks; ++c) {
        const long long t0 = job.tok0 + (long long)c * kChunk;
        const int nvalid = (job.len - c * kChunk) < kChunk ? (job.len - c * kChunk) : kChunk;
        __syncthreads();   // the previous chunk is done with every LDS buffer

        // ---- a: registers -> LDS (rows past the end of the sequence become zeros) ----
#pragma unroll
        for (int j = 0; j < KBLK; ++j) {
            const int b = tid + kThreads * j;
            const int dq = b % DQ, tq = b / DQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned keep = (4 * tq + i < nvalid) ? 0xffffffffu : 0u;
                pk[j][i].mask(keep);
                pk[j][i].store((OP *)(bK + swz<OP, DK>(4 * tq + i, 4 * dq)));
                if (kY) {
                    pq[j][i].mask(keep);
                    pq[j][i].store((OP *)(bQ + swz<OP, DK>(4 * tq + i, 4 * dq)));
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Q4::column(pk[j], jj).store((OP *)(bKt + swz<OP, kChunk>(4 * dq + jj, 4 * tq)));
        }
#pragma unroll
        for (int j = 0; j < VBLK; ++j) {
            const int b = tid + kThreads * j;
            if (b < 16 * VQ) {
                const int dq = b % VQ, tq = b / VQ;
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[j][i].mask((4 * tq + i < nvalid) ? 0xffffffffu : 0u);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    Q4::column(pv[j], jj).store((OP *)(bVt + swz<OP, kChunk>(4 * dq + jj, 4 * tq)));
            }
        }
        if (wave == 0) {
            // inclusive prefix sum of log2 alpha over the chunk (lane = token): Hillis-Steele
            // within each 16-lane row by DPP row shifts, then across rows by row broadcasts
            float x = lane < nvalid ? fmaxf(__builtin_amdgcn_logf(pa), kLog2AlphaFloor) : 0.f;
            x += dpp_f32<0x111, 0xf>(x);   // row_shr:1
            x += dpp_f32<0x112, 0xf>(x);   // row_shr:2
            x += dpp_f32<0x114, 0xf>(x);   // row_shr:4
            x += dpp_f32<0x118, 0xf>(x);   // row_shr:8
            x += dpp_f32<0x142, 0xa>(x);   // row_bcast:15 -> rows 1, 3
            x += dpp_f32<0x143, 0xc>(x);   // row_bcast:31 -> rows 2, 3
            sG[lane] = x;
        } else if (wave == 1) {
            sBeta[lane] = lane < nvalid ? pa : 0.f;
        }
        if (c + 1 < nchunks) {
            const int nv = (job.len - (c + 1) * kChunk) < kChunk ? (job.len - (c + 1) * kChunk)
                                                                 : kChunk;
            prefetch(t0 + kChunk, nv);
        }
        __syncthreads();

        // ---- b: Gram tiles -> A, P (masked by the decay).  Pair p = (t-block, i-block):
        //      0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) 7:(3,1) 8:(3,2) 9:(3,3);
        //      wave w takes pairs w, w + 4 and (waves 0, 1) w + 8.  A diagonal tile also
        //      gets its strictly lower part mirrored into its upper half (column access
        //      for the substitution of phase c).
        auto gram_pair = [&](int p) {
            const int tb = p < 1 ? 0 : (p < 3 ? 1 : (p < 6 ? 2 : 3));
            const int ib = p - tb * (tb + 1) / 2;
            const int t = tb * 16 + ln;
            const float gt = sG[t];
            const float bt_ = sBeta[t];
            const f32x4 gi = *(const f32x4 *)(sG + ib * 16 + 4 * lg);
            f32x4 accG = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                const auto ai = ldfrag<OP, DK>(bK, ib * 16 + ln, kb * 32 + 8 * lg);
                const auto bt = ldfrag<OP, DK>(bK, tb * 16 + ln, kb * 32 + 8 * lg);
                M::mma(accG, ai, bt);
                if (kY) {
                    const auto bq = ldfrag<OP, DK>(bQ, tb * 16 + ln, kb * 32 + 8 * lg);
                    M::mma(accP, ai, bq);
                }
            }
            // accG[r] = k_i . k_t and accP[r] = k_i . q_t for i = ib*16 + 4lg + r
            f32x4 av, pv4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ib * 16 + 4 * lg + r;
                const float dec = (i <= t) ? __builtin_amdgcn_exp2f(gt - gi[r]) : 0.f;
                av[r] = (i < t) ? bt_ * accG[r] * dec : 0.f;
                pv4[r] = accP[r] * dec;
            }
            *(f32x4 *)(sA + t * L::LDA + ib * 16 + 4 * lg) = av;
            if (tb == ib) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ib * 16 + 4 * lg + r;
                    if (i < t) sA[i * L::LDA + t] = av[r];
                }
            }
            if (kY) M::put4((OP *)(bP + swz<OP, kChunk>(t, ib * 16 + 4 * lg)), pv4);
        };
        gram_pair(wave);
        gram_pair(wave + 4);
        if (wave < 2) gram_pair(wave + 8);
        // P blocks (0,1) and (2,3) lie inside the diagonal 32-wide K-blocks of U^T P^T
        if (kY && (wave == 0 || wave == 2)) {
            M::put4((OP *)(bP + swz<OP, kChunk>(wave * 16 + ln, wave * 16 + 16 + 4 * lg)),
                    f32x4{0.f, 0.f, 0.f, 0.f});
        }
        // ---- b: K S (rows 16w..) and S^T Q^T (tokens 16w..) ----
        f32x4 accKS[NB], accYt[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            accKS[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            accYt[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            const auto ak = ldfrag<OP, DK>(bK, wave * 16 + ln, kb * 32 + 8 * lg);
            typename M::frag bq;
            if (kY) bq = ldfrag<OP, DK>(bQ, wave * 16 + ln, kb * 32 + 8 * lg);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const auto bs = ldfrag<OP, DK>(bSt, nb * 16 + ln, kb * 32 + 8 * lg);
                M::mma(accKS[nb], ak, bs);
                if (kY) M::mma(accYt[nb], bs, bq);
            }
        }
        // ---- b: R = V - diag(gamma) K S   (wave w: token rows 16w .. 16w + 15) ----
        f32x4 gam;
#pragma unroll
        for (int r = 0; r < 4; ++r) gam[r] = __builtin_amdgcn_exp2f(sG[trow + r]);
        f32x4 R[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const f32x4 vv = M::get4((const OP *)(bVt + swz<OP, kChunk>(nb * 16 + ln, trow)));
            R[nb] = vv - gam * accKS[nb];
        }
        __syncthreads();   // K, Q row-major tiles and V^T are dead

        // ---- c: R -> LDS; diagonal blocks of X = (I + A)^{-1} ----
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            M::put4((OP *)(bRt + swz<OP, kChunk>(nb * 16 + ln, trow)), R[nb]);
        // wave w inverts diagonal block w by forward substitution, one column per lane (the
        // four 16-lane groups compute the same columns).  Each lane then keeps rows
        // 4 lg .. 4 lg + 3 of its column: the accumulator layout of that block.
        f32x4 xcol[4];
        {
            const int d0 = wave * 16;
            // right-looking: once x[c] is final, subtract its column from the rows below;
            // row c of the block's upper half holds A[r][c] for r > c (mirrored in phase b)
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == ln) ? 1.f : 0.f;
#pragma unroll
            for (int c = 0; c < 15; ++c) {
                const float *col = sA + (d0 + c) * L::LDA + d0;
#pragma unroll
                for (int q4 = (c + 1) / 4; q4 < 4; ++q4) {
                    const f32x4 a4 = *(const f32x4 *)(col + 4 * q4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * q4 + e > c) x[4 * q4 + e] -= a4[e] * x[c];
                }
            }
            f32x4 mine;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mine[i] = lg == 0 ? x[i] : (lg == 1 ? x[4 + i] : (lg == 2 ? x[8 + i] : x[12 + i]));
#pragma unroll
            for (int m = 0; m < 4; ++m) xcol[m] = (m == wave) ? mine : f32x4{0.f, 0.f, 0.f, 0.f};
            // row-major copy of the block (an MFMA A operand for the other block columns)
#pragma unroll
            for (int i = 0; i < 4; ++i) sX[(d0 + 4 * lg + i) * L::LDX + ln] = mine[i];
            const float bcol = sBeta[d0 + ln];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Elem<OP>::store((OP *)(bT + swz<OP, kChunk>(d0 + 4 * lg + i, d0 + ln)),
                                mine[i] * bcol);
            // zero the blocks of T' that the K-blocks of U = T' R read above the diagonal
            if (wave == 0 || wave == 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Elem<OP>::store((OP *)(bT + swz<OP, kChunk>(d0 + 4 * lg + i, d0 + 16 + ln)),
                                    0.f);
            }
        }
        __syncthreads();

        // ---- d: wave j walks down block column j: X_ij = -X_ii sum_{m=j}^{i-1} A_im X_mj.
        //      Every product runs on v_mfma_f32_16x16x4_f32; the column's blocks stay in the
        //      accumulator layout, which is the B-operand layout of the next product
        //      (contraction index 4 lg + s in step s).
        {
            const int j = wave;
            const float bcol = sBeta[16 * j + ln];
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                if (i > j) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < 3; ++m) {
                        if (m >= j && m < i) {
                            const f32x4 a4 = *(const f32x4 *)(sA + (16 * i + ln) * L::LDA +
                                                              16 * m + 4 * lg);
                            const f32x4 b4 = xcol[m];
#pragma unroll
                            for (int st = 0; st < 4; ++st)
                                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[st], b4[st], acc,
                                                                           0, 0, 0);
                        }
                    }
                    mfma_f32_drain();
                    const f32x4 xi = *(const f32x4 *)(sX + (16 * i + ln) * L::LDX + 4 * lg);
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < 4; ++st)
                        z = __builtin_amdgcn_mfma_f32_16x16x4f32(xi[st], acc[st], z, 0, 0, 0);
                    mfma_f32_drain();
                    xcol[i] = -z;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Elem<OP>::store((OP *)(bT + swz<OP, kChunk>(16 * i + 4 * lg + r,
                                                                    16 * j + ln)),
                                        -z[r] * bcol);
                }
            }
        }
        __syncthreads();

        // ---- e: U = T' R (lower triangular: K-blocks up to the diagonal) ----
        const float gC = sG[kChunk - 1];
        f32x4 accU[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) accU[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb <= (wave >> 1)) {
                const auto at = ldfrag<OP, kChunk>(bT, wave * 16 + ln, kb * 32 + 8 * lg);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const auto br = ldfrag<OP, kChunk>(bRt, nb * 16 + ln, kb * 32 + 8 * lg);
                    M::mma(accU[nb], at, br);
                }
            }
        }
        f32x4 tail;   // gamma_C / gamma_t
#pragma unroll
        for (int r = 0; r < 4; ++r) tail[r] = __builtin_amdgcn_exp2f(gC - sG[trow + r]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if (kY) M::put4((OP *)(bUt + swz<OP, kChunk>(nb * 16 + ln, trow)), accU[nb]);
            M::put4((OP *)(bUs + swz<OP, kChunk>(nb * 16 + ln, trow)), accU[nb] * tail);
        }
        __syncthreads();

        // ---- f: Y^T = S^T Q^T diag(gamma) + U^T P^T (tokens 16w .. 16w + 15) ----
        if (kY) {
            const float gtok = __builtin_amdgcn_exp2f(sG[wave * 16 + ln]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) accYt[nb] *= gtok;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb <= (wave >> 1)) {
                    const auto bp = ldfrag<OP, kChunk>(bP, wave * 16 + ln, kb * 32 + 8 * lg);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const auto au = ldfrag<OP, kChunk>(bUt, nb * 16 + ln, kb * 32 + 8 * lg);
                        M::mma(accYt[nb], au, bp);
                    }
                }
            }
            // lane (token 16w + ln) holds columns 4 lg .. 4 lg + 3 of each 16-column block
            const int t = wave * 16 + ln;
            if (t < nvalid) {
                OP *gy = (OP *)a.y + ((t0 + t) * H + job.h) * (long long)DV + job.col0 + 4 * lg;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) store4(gy + nb * 16, accYt[nb]);
            }
        }

        // ---- f: S = gamma_C S + (diag(gamma_C / gamma) K)^T U ----
        const float gamC = __builtin_amdgcn_exp2f(gC);
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb) {
            const int drow = (wave * MBS + mb) * 16;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) S[mb][nb] *= gamC;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const auto ak = ldfrag<OP, kChunk>(bKt, drow + ln, kb * 32 + 8 * lg);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const auto bu = ldfrag<OP, kChunk>(bUs, nb * 16 + ln, kb * 32 + 8 * lg);
                    M::mma(S[mb][nb], ak, bu);
                }
            }
        }
        store_state_lds();
    }

    // ---- write the state ----
    float *dst = nullptr;
    long long ld = DV;
    if (MODE == kModeScan) {
        if (job.seg == job.nseg - 1 && a.s_final)
            dst = a.s_final + ((long long)job.n * H + job.h) * DK * DV + job.col0;
    } else if (mpart) {
        dst = a.segM + ((long long)job.entry * H + job.h) * DK * DK + (job.col0 - DV);
        ld = DK;
    } else {
        dst = a.segB + ((long long)job.entry * H + job.h) * DK * DV + job.col0;
    }
    if (dst) {
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = (wave * MBS + mb) * 16 + 4 * lg + i;
                    dst[(long long)row * ld + nb * 16 + ln] = S[mb][nb][i];
                }
    }
}

// ---------------------------------------------------------------------------------------
// a0: segment table.  One workgroup: per sequence, the number of segments of seg_chunks
// chunks (at least one, so a zero-length sequence still returns its initial state), an
// exclusive prefix sum over sequences for the entry offsets, then one entry per segment.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void segment_table_kernel(PrefillArgs a, int seg_tokens,
                                                             SegEntry *table, int32_t *count,
                                                             int32_t *zero, long long nzero)
{
    __shared__ int32_t s_scan[1024];
    __shared__ int32_t s_base;
    const int tid = threadIdx.x;
    // words the next launch expects to start at zero (the wide scan's job counter and flags)
    for (long long i = tid; i < nzero; i += 1024) zero[i] = 0;
    if (tid == 0) s_base = 0;
    __syncthreads();
    for (int n0 = 0; n0 < a.num_seqs; n0 += 1024) {
        const int n = n0 + tid;
        long long t0 = 0;
        int len = 0, nseg = 0;
        if (n < a.num_seqs) {
            seq_bounds(a, n, t0, len);
            nseg = len > 0 ? (len + seg_tokens - 1) / seg_tokens : 1;
        }
        s_scan[tid] = nseg;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        const int base = s_base + s_scan[tid] - nseg;
        for (int p = 0; p < nseg; ++p) {
            SegEntry e;
            e.n = n;
            e.seg = p;
            e.nseg = nseg;
            e.tok0 = t0 + (long long)p * seg_tokens;
            const long long remain = (long long)len - (long long)p * seg_tokens;
            e.len = (int)(remain < seg_tokens ? remain : seg_tokens);
            table[base + p] = e;
        }
        __syncthreads();
        if (tid == 1023) s_base = base + nseg;
        __syncthreads();
    }
    if (tid == 0) *count = s_base;
}

// ---------------------------------------------------------------------------------------
// a6 phase B: per (sequence, head, 16-column tile) fold the segment maps in order,
// S_{p+1} = M_p S_p + B_p, overwriting B_p with S_{p+1} (the start state of segment p + 1).
// Segment 0's entry already holds the true S_1 (phase A started it from S0).
// Wave w computes state rows [w DK/4, (w+1) DK/4); the state tile lives in LDS.
// ---------------------------------------------------------------------------------------
template <int DK, typename OP>
__global__ __launch_bounds__(kThreads) void segment_combine_kernel(PrefillArgs a)
{
    using M = Mma<OP>;
    constexpr int LDK = DK + 16 / (int)sizeof(OP);
    constexpr int KBD = DK / 32;
    constexpr int MBS = DK / 64;
    __shared__ __align__(16) OP sSt[16 * LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lg = lane >> 4;
    const int ntile = a.dv / 16;
    const int tile = blockIdx.x % ntile;
    const long long nh = blockIdx.x / ntile;
    if (nh >= (long long)a.num_seqs * a.H) return;
    const int n = (int)(nh / a.H), h = (int)(nh % a.H);
    // locate the sequence's first entry (entries are in sequence order)
    const int cnt = *a.n_entries;
    int lo = 0, hi = cnt;   // first entry with e.n >= n
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a.table[mid].n < n) lo = mid + 1; else hi = mid;
    }
    if (lo >= cnt || a.table[lo].n != n) return;
    const int e0 = lo;
    const int nseg = a.table[e0].nseg;
    if (nseg <= 2) return;
    const int DV = a.dv;
    const int col0 = tile * 16;
    const long long stB = (long long)DK * DV, stM = (long long)DK * DK;
    // S_1 (fp32) from entry e0
    f32x4 S[MBS];
    {
        const float *src = a.segB + ((long long)e0 * a.H + h) * stB + col0;
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[mb][i] = src[(long long)((wave * MBS + mb) * 16 + 4 * lg + i) * DV + ln];
    }
    for (int p = 1; p < nseg - 1; ++p) {
        const int e = e0 + p;
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb)
            M::put4(sSt + ln * LDK + (wave * MBS + mb) * 16 + 4 * lg, S[mb]);
        __syncthreads();
        const float *Mp = a.segM + ((long long)e * a.H + h) * stM;
        float *Bp = a.segB + ((long long)e * a.H + h) * stB + col0;
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb) {
            const int row0 = (wave * MBS + mb) * 16;
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = Bp[(long long)(row0 + 4 * lg + i) * DV + ln];
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                // A fragment: row (row0 + ln) of M_p, 8 consecutive columns, fp32 -> OP
                const float *mrow = Mp + (long long)(row0 + ln) * DK + kb * 32 + 8 * lg;
                const auto am = M::from_f32(*(const f32x4 *)mrow, *(const f32x4 *)(mrow + 4));
                const auto bs = M::load(sSt + ln * LDK + kb * 32 + 8 * lg);
                M::mma(acc, am, bs);
            }
            S[mb] = acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) Bp[(long long)(row0 + 4 * lg + i) * DV + ln] = acc[i];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
static long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

template <int DK, int DVT, typename OP, int MODE>
static hipError_t launch_scan(const PrefillArgs &args, long long units, int ntiles,
                              hipStream_t stream)
{
    if constexpr (sizeof(OP) == 2 && DVT <= 64) {
        if (args.prep) return launch_scan_split<DK, DVT, MODE>(args, units, ntiles, stream);
    }
    const long long groups = cdiv(units * args.H, 8) * 8 * ntiles;
    if (groups <= 0) return hipSuccess;
    PrefillArgs a2 = args;
    a2.units = units;
    a2.ntiles = ntiles;
    hipLaunchKernelGGL((prefill_kernel<DK, DVT, OP, MODE>), dim3((unsigned)groups),
                       dim3(kThreads), 0, stream, a2);
    return hipGetLastError();
}

template <int DK, int DVT, typename OP>
static hipError_t run_prefill(const PrefillArgs &args, const PrefillPlan &plan,
                              long long max_entries, hipStream_t stream)
{
    const int dv = args.dv;
    if constexpr (sizeof(OP) == 2) {
        if (args.prep) {
            // records of every chunk (read by phase A and by the final scan)
            hipError_t err = launch_chunk_prep<DK>(args, plan.nslots, stream);
            if (err != hipSuccess) return err;
        }
    }
    if (plan.seg_chunks < 0) {
        return launch_scan<DK, DVT, OP, kModeScan>(args, args.num_seqs, dv / DVT, stream);
    }
    hipLaunchKernelGGL(segment_table_kernel, dim3(1), dim3(1024), 0, stream, args,
                       plan.seg_chunks * kChunk, (SegEntry *)args.table,
                       (int32_t *)args.n_entries, (int32_t *)nullptr, 0ll);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // phase A: [S | M] scans of every segment but the last of each sequence (bf16: 64-column
    // tiles, which halve the per-tile copies of the chunk's K, Q and record for the d_v + d_k
    // columns of [S | M]; phase C keeps the plan's tile)
    constexpr int DVTA = (sizeof(OP) == 2 && DVT == 32) ? 64 : DVT;
    if (dv % DVTA == 0)
        err = launch_scan<DK, DVTA, OP, kModeAug>(args, max_entries, (dv + DK) / DVTA, stream);
    else
        err = launch_scan<DK, DVT, OP, kModeAug>(args, max_entries, (dv + DK) / DVT, stream);
    if (err != hipSuccess) return err;
    // phase B: fold the segment maps
    {
        const long long groups = (long long)args.num_seqs * args.H * (dv / 16);
        hipLaunchKernelGGL((segment_combine_kernel<DK, OP>), dim3((unsigned)groups),
                           dim3(kThreads), 0, stream, args);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // phase C: every segment from its true start state, writing y
    return launch_scan<DK, DVT, OP, kModeScan>(args, max_entries, dv / DVT, stream);
}

template <typename OP, int DK, int DVT>
static hipError_t run_if_fits(const PrefillArgs &args, const PrefillPlan &plan,
                              long long max_entries, hipStream_t stream)
{
    if constexpr (Lds<DK, DVT, OP>::total <= 160 * 1024)
        return run_prefill<DK, DVT, OP>(args, plan, max_entries, stream);
    return hipErrorInvalidValue;
}

template <typename OP>
static hipError_t dispatch_dk_dvt(const PrefillArgs &args, const PrefillPlan &plan, int dk,
                                  long long max_entries, hipStream_t stream)
{
    const int t = plan.dv_tile;
    if (dk == 128) {
        if (t == 16) return run_if_fits<OP, 128, 16>(args, plan, max_entries, stream);
        if (t == 32) return run_if_fits<OP, 128, 32>(args, plan, max_entries, stream);
        if (t == 64) return run_if_fits<OP, 128, 64>(args, plan, max_entries, stream);
        if (t == 128) return run_if_fits<OP, 128, 128>(args, plan, max_entries, stream);
    } else {
        if (t == 16) return run_if_fits<OP, 64, 16>(args, plan, max_entries, stream);
        if (t == 32) return run_if_fits<OP, 64, 32>(args, plan, max_entries, stream);
        if (t == 64) return run_if_fits<OP, 64, 64>(args, plan, max_entries, stream);
        if (t == 128) return run_if_fits<OP, 64, 128>(args, plan, max_entries, stream);
    }
    return hipErrorInvalidValue;
}

// Column tiles whose kernel fits the 160 KiB of LDS of a gfx950 CU.
template <typename OP, int DK>
static constexpr bool fits(int t)
{
    return t == 16    ? Lds<DK, 16, OP>::total <= 160 * 1024
           : t == 32  ? Lds<DK, 32, OP>::total <= 160 * 1024
           : t == 64  ? Lds<DK, 64, OP>::total <= 160 * 1024
           : t == 128 ? Lds<DK, 128, OP>::total <= 160 * 1024
                      : false;
}

static bool tile_ok(int dtype, int dk, int dv, int t)
{
    if (t != 16 && t != 32 && t != 64 && t != 128) return false;
    if (dv % t != 0) return false;
    if (dtype == kDtypeF32) return dk == 128 ? fits<float, 128>(t) : fits<float, 64>(t);
    return dk == 128 ? fits<uint16_t, 128>(t) : fits<uint16_t, 64>(t);
}

static int largest_tile(int dtype, int dk, int dv)
{
    for (int t = 128; t >= 16; t >>= 1)
        if (tile_ok(dtype, dk, dv, t)) return t;
    return 0;
}

// The one-launch bf16 scan (gdn_prefill_wide.hip) for d_k = d_v = 128: one workgroup per
// (segment, head) with the whole state.  By default it serves the sequences that the
// column-split scan could only spread over the CUs with the segment phases (few chains of
// many chunks); they are split into one segment per CU's worth of work.
static bool use_wide_by_default(int num_seqs, long long total_T, int H)
{
    const long long chains = (long long)num_seqs * H;
    const long long avg_chunks = cdiv(total_T, (long long)num_seqs * kChunk);
    // few long chains: segments of them fill the chip
    if (chains * 4 < 256 && avg_chunks >= 64) return true;
    // plenty of work: once every CU has 128 or more chunk steps to run, the one-launch scan
    // (no chunk records through HBM) beats the two-launch path
    const long long total_chunks = cdiv(total_T, kChunk) + num_seqs;
    return total_chunks * H >= 128LL * 256 && avg_chunks >= 32;
}

static bool make_wide_plan(int num_seqs, long long total_T, int H, int seg_chunks_req,
                           PrefillPlan *plan)
{
    const long long chains = (long long)num_seqs * H;
    const long long total_chunks = cdiv(total_T, kChunk) + num_seqs;
    int seg = seg_chunks_req;
    if (seg == 0) {
        constexpr long long kJobs = 256;
        if (chains >= kJobs) {
            // about three jobs per CU, so that unequal lengths even out (on 32 packed
            // sequences of 512..16384 tokens: 82 chunks 1.37 ms, the 123 of two jobs per CU
            // 1.40 ms, 64 chunks 1.44 ms, 48 chunks 1.54 ms)
            long long s = cdiv(total_chunks * H, 3 * kJobs);
            if (s < 64) s = 64;
            if (s > (1 << 24)) s = 1 << 24;
            seg = (int)s;
        } else {
            long long s = cdiv(total_chunks * H, kJobs);
            if (s < 16) s = 16;
            if (s > (1 << 24)) s = 1 << 24;
            seg = (int)s;
            // equal lengths: no split when one segment holds a whole sequence
            if (total_T % num_seqs == 0 && cdiv(total_T / num_seqs, kChunk) <= seg) seg = -1;
        }
    }
    if (seg == 0 || seg < -1) return false;
    plan->wide = 1;
    plan->dv_tile = 128;
    plan->two_launch = 0;
    plan->seg_chunks = seg;
    plan->nslots = 0;
    plan->ws_prep = 0;
    plan->ws_seg = 0;
    if (seg < 0) {
        plan->max_segments = num_seqs;
        plan->ws_table = 0;
        plan->ws_wide = 0;
    } else {
        const long long max_entries = num_seqs + cdiv(total_T, (long long)seg * kChunk);
        plan->max_segments = max_entries;
        plan->ws_table = (size_t)(cdiv((long long)max_entries * sizeof(SegEntry) + 16, 256) * 256);
        // job counter and error word (256 bytes), flags [entries, H], end states
        const size_t flags = (size_t)cdiv(max_entries * H * 4, 256) * 256;
        plan->ws_wide = 256 + flags + (size_t)max_entries * H * 128 * 128 * 4;
    }
    return true;
}

bool make_plan(int num_seqs, long long total_T, int H, int dk, int dv, int dtype,
               int dv_tile_req, int seg_chunks_req, PrefillPlan *plan)
{
    plan->wide = 0;
    plan->ws_wide = 0;
    if (dtype == kDtypeBF16 && dk == 128 && dv == 128 &&
        (dv_tile_req == 128 || (dv_tile_req == 0 && use_wide_by_default(num_seqs, total_T, H))))
        return make_wide_plan(num_seqs, total_T, H, seg_chunks_req, plan);
    // Column tile: the chains (sequence, head) are independent; split the state columns
    // until there are enough workgroups to cover the 256 CUs, within the LDS budget.
    int tile = dv_tile_req;
    const long long chains = (long long)num_seqs * H;
    if (tile == 0) {
        tile = largest_tile(dtype, dk, dv);
        // the two-launch path; its pipelined scan takes 16 or 32 columns per workgroup
        if (dtype == kDtypeBF16 && tile > 32) tile = 32;
        while (tile > 32 && chains * (dv / tile) < 512) tile >>= 1;
    }
    if (!tile_ok(dtype, dk, dv, tile)) return false;
    plan->two_launch = (dtype == kDtypeBF16 && tile <= 64) ? 1 : 0;
    plan->nslots = total_T / kChunk + num_seqs;
    plan->ws_prep = plan->two_launch
                        ? (size_t)plan->nslots * H * kPrepRecordBytes
                        : 0;
    // Segments: split sequences when the chains alone cannot fill the chip and the average
    // sequence is long enough to pay for the extra phases.
    int seg = seg_chunks_req;
    const long long total_chunks = cdiv(total_T, kChunk) + num_seqs;
    if (seg == 0) {
        const long long groups = chains * (dv / tile);
        const long long avg_chunks = num_seqs > 0 ? cdiv(total_T, (long long)num_seqs * kChunk) : 0;
        if (groups >= 256 || avg_chunks < 64) {
            seg = -1;
        } else {
            // aim for ~1024 phase-C workgroups, segments of at least 32 chunks
            long long want_units = cdiv(1024, (long long)H * (dv / tile));
            long long s = cdiv(total_chunks, want_units);
            if (s < 32) s = 32;
            seg = (int)s;
        }
    }
    if (seg == 0 || seg < -1) return false;
    plan->dv_tile = tile;
    plan->seg_chunks = seg;
    if (seg < 0) {
        plan->max_segments = num_seqs;
        plan->ws_table = 0;
        plan->ws_seg = 0;
    } else {
        const long long max_entries = num_seqs + cdiv(total_T, (long long)seg * kChunk);
        plan->max_segments = max_entries;
        plan->ws_table = (size_t)(cdiv((long long)max_entries * sizeof(SegEntry) + 16, 256) * 256);
        plan->ws_seg = (size_t)max_entries * H * ((size_t)dk * dv + (size_t)dk * dk) * 4;
    }
    return true;
}

hipError_t launch_prefill(const PrefillProblem &p, const PrefillPlan &plan, void *workspace,
                          hipStream_t stream)
{
    PrefillArgs a{};
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.s0 = p.s0;
    a.cu = p.cu;
    a.num_seqs = p.num_seqs;
    a.total_T = p.total_T;
    a.H = p.H;
    a.dv = p.dv;
    a.y = p.y;
    a.s_final = p.s_final;
    a.og_z = p.og_z;
    a.og_w = p.og_w;
    a.og_eps = p.og_eps;
    if (plan.seg_chunks >= 0) {
        unsigned char *ws = (unsigned char *)workspace;
        a.table = (const SegEntry *)ws;
        a.n_entries = (const int32_t *)(ws + plan.max_segments * sizeof(SegEntry));
        float *seg = (float *)(ws + plan.ws_table);
        a.segB = seg;
        a.segM = seg + (size_t)plan.max_segments * p.H * p.dk * p.dv;
    }
    if (plan.two_launch) a.prep = (unsigned char *)workspace + plan.ws_table + plan.ws_seg;
    if (p.gated) {
        // only the record kernel and the wide scan read the gates
        if (!plan.two_launch && !plan.wide) return hipErrorInvalidValue;
        a.gate_A = p.gate_A;
        a.gate_b_alpha = p.gate_b_alpha;
    }
    if (plan.wide) {
        WideArgs w{};
        w.a = a;
        long long jobs = (long long)p.num_seqs * p.H;
        if (plan.seg_chunks >= 0) {
            unsigned char *ws = (unsigned char *)workspace;
            unsigned char *ctl = ws + plan.ws_table;
            w.counter = (int32_t *)ctl;
            w.error = (int32_t *)(ctl + 4);
            w.flags = (int32_t *)(ctl + 256);
            const size_t flags = (size_t)cdiv(plan.max_segments * p.H * 4, 256) * 256;
            w.seg_state = (float *)(ctl + 256 + flags);
            w.wmax = plan.seg_chunks;
            w.a.segB = nullptr;
            w.a.segM = nullptr;
            // the table, and zeros for the counter, the error word and the flags
            hipLaunchKernelGGL(segment_table_kernel, dim3(1), dim3(1024), 0, stream, a,
                               plan.seg_chunks * kChunk, (SegEntry *)a.table,
                               (int32_t *)a.n_entries, (int32_t *)ctl,
                               (long long)(256 + flags) / 4);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
            jobs = plan.max_segments * p.H;
        }
        return launch_wide_scan(w, jobs, stream);
    }
    if (p.dtype == kDtypeBF16)
        return dispatch_dk_dvt<uint16_t>(a, plan, p.dk, plan.max_segments, stream);
    return dispatch_dk_dvt<float>(a, plan, p.dk, plan.max_segments, stream);
}

}  // namespace gdn
