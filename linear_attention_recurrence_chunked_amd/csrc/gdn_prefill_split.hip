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
//   and writes T' and g to the workspace (8448 bytes per record).
//
//   scan_split_kernel (one workgroup per (sequence or segment, head, column tile)):
//     two loader waves copy K, Q, V and the record of a chunk into an LDS stage ahead of
//     use and form P = lower_incl(Q K^T (.) Gamma) there, while the scan waves apply the
//     current chunk to the state held in MFMA accumulator registers:
//     R = V - diag(gamma) K S,  U = T' R,  Y^T = S^T Q^T diag(gamma) + U^T P^T,
//     S = gamma_C S + K^T diag(gamma_C / gamma) U.   One barrier per chunk.
//
// Chunk slots: chunk c of sequence n (first row t0_n) has slot floor(t0_n / 64) + n + c.
// Slots of different chunks differ, and all are below floor(total_T / 64) + num_seqs.
#include <type_traits>

#include "gdn_prefill_ops.hpp"

namespace gdn {

// Record of one (slot, head): T' [64][64] bf16 (rows in the internal token order of
// gdn_prefill_ops.hpp) in the XOR-swizzled byte layout of a 64-wide LDS tile (so the scan
// copies it into LDS granule for granule), then g [64] fp32.
constexpr int kRecT = 0;
constexpr int kRecG = kChunk * kChunk * 2;
static_assert(kRecG + kChunk * 4 == kPrepRecordBytes, "record layout");


// =========================================================================================
// Launch 1: per (chunk slot, head) record T', g.  Four waves; wave w owns block row /
// column w of the 4 x 4 grid of 16 x 16 blocks.
// =========================================================================================
// T' goes from registers straight to the record in HBM (it is never read back here), so the
// LDS holds only g, beta, the decay factors and the K rows, later A and the X blocks: 17 KiB,
// eight workgroups per CU.
template <int DK>
struct LdsPrep {
    static constexpr int szRow = kChunk * DK * 2;
    static constexpr int LDB = 20;                  // padded fp32 rows of an A block
    static constexpr int LDX = 20;                  // padded rows of a diagonal X block
    static constexpr int oG = 0;
    static constexpr int oBeta = oG + kChunk * 4;
    static constexpr int oE = oBeta + 256;          // 2^g and 2^-g of the tokens
    static constexpr int oK = oE + 512;             // K rows (phases 1-2) ...
    static constexpr int oA = oK;                   // ... then A and the X blocks (phase 3)
    // the six strictly lower 16 x 16 blocks of A, block (i, m) at index i (i - 1) / 2 + m
    static constexpr int oX = oA + 6 * 16 * LDB * 4;
    static constexpr int total = oK + (szRow > 6 * 16 * LDB * 4 + 4 * 16 * LDX * 4
                                           ? szRow
                                           : 6 * 16 * LDB * 4 + 4 * 16 * LDX * 4);
};

template <int DK>
__global__ __launch_bounds__(256, 8) void chunk_prep_kernel(PrefillArgs a, long long nslots)
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
    float *const sE = (float *)(smem + L::oE);          // 2^g
    float *const sIE = sE + kChunk;                      // 2^-g
    float *const sA = (float *)(smem + L::oA);
    float *const sX = (float *)(smem + L::oX);
    unsigned char *const bK = smem + L::oK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    // every argument this kernel reads, fetched in one round of scalar loads
    const int H = a.H;
    const int32_t *const cu = a.cu;
    const long long totT = a.total_T;
    const int nseq = a.num_seqs;
    const OP *const gk = (const OP *)a.k;
    const float *const galpha = a.alpha, *const gbeta = a.beta;
    unsigned char *const gprep = (unsigned char *)a.prep;
    asm volatile("" ::"s"(H), "s"(cu), "s"(totT), "s"(nseq), "s"(gk), "s"(galpha), "s"(gbeta),
                 "s"(gprep), "s"(nslots));
    const long long slot = (long long)(blockIdx.x / (unsigned)H);
    const int h = (int)(blockIdx.x % (unsigned)H);
    if (slot >= nslots) return;
    // sequence of the slot: the last n with first_slot(n) <= slot (32-bit arithmetic and one
    // wave-wide vote where they suffice: this runs before anything else in the workgroup)
    long long per = 0;                     // tokens per sequence when all have one length
    if (!cu)
        per = totT < 0x7fffffffLL ? (long long)((unsigned)totT / (unsigned)nseq) : totT / nseq;
    auto row0 = [&](int m) -> long long { return cu ? cu[m] : per * m; };
    int n;
    if (cu && nseq <= 64) {
        const bool ok = lane < nseq && (cu[lane] >> 6) + lane <= slot;
        n = __popcll(__builtin_amdgcn_ballot_w64(ok)) - 1;
    } else {
        int lo = 0, hi = nseq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((row0(mid) >> 6) + mid <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
    }
    const long long st0 = row0(n);
    const int slen = (int)(cu ? cu[n + 1] - st0 : per);
    const long long c = slot - ((st0 >> 6) + n);
    if (c < 0 || c * kChunk >= slen) return;          // unused slot
    const long long t0 = st0 + c * kChunk;
    const int nv = (int)((slen - c * kChunk) < kChunk ? (slen - c * kChunk) : kChunk);
    // the record: T' (written block by block as it is formed), then g
    unsigned char *const bT = gprep + (slot * H + h) * (long long)kPrepRecordBytes;

    // ---- phase 1: K rows (zero beyond the chunk's last row), g, beta ----
    {
        u32x4 rk[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int idx = tid + 256 * j;
            const int row = idx / GR, gc = idx % GR;
            const int tc = row < nv ? row : nv - 1;
            const long long off = ((t0 + tc) * H + h) * (long long)DK + 8 * gc;
            rk[j] = ld16(gk + off);
        }
        // alpha and beta, or, from gate pre-activations (reading notes, "Gating dynamics"),
        // log2 alpha = -e^A softplus(a + b_alpha) / ln 2 with no exp/log round trip and
        // beta = sigmoid(b)
        const float *const gA = a.gate_A;
        float pa = 0.f;
        if (wave < 2) {
            const int tc = lane < nv ? lane : nv - 1;
            pa = (wave == 0 ? galpha : gbeta)[(t0 + tc) * H + h];
            if (gA) {
                if (wave == 0) {
                    const float u = pa + a.gate_b_alpha[h];
                    const float sp = u > 20.f ? u : log1pf(__expf(u));          // softplus
                    pa = -__expf(gA[h]) * sp * 1.44269504088896341f;
                } else {
                    pa = __builtin_amdgcn_rcpf(1.f + __expf(-pa));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int idx = tid + 256 * j;
            const int row = idx / GR, gc = idx % GR;
            const u32x4 z = {0u, 0u, 0u, 0u};
            *(u32x4 *)(bK + swz<OP, DK>(row, 8 * gc)) = row < nv ? rk[j] : z;
        }
        if (wave == 0) {
            float x = lane < nv ? fmaxf(gA ? pa : __builtin_amdgcn_logf(pa), kLog2AlphaFloor)
                                : 0.f;
            x += dpp_f32<0x111, 0xf>(x);
            x += dpp_f32<0x112, 0xf>(x);
            x += dpp_f32<0x114, 0xf>(x);
            x += dpp_f32<0x118, 0xf>(x);
            x += dpp_f32<0x142, 0xa>(x);
            x += dpp_f32<0x143, 0xc>(x);
            sG[lane] = x;
            ((float *)(bT + kRecG))[lane] = x;
            sE[lane] = __builtin_amdgcn_exp2f(x);
            sIE[lane] = __builtin_amdgcn_exp2f(-x);
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
    f32x4 accG[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) accG[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            if (p < np) {
                const auto ai = ldfrag<OP, DK>(bK, ibs[p] * 16 + ln, kb * 32 + 8 * lg);
                const auto bt = ldfrag<OP, DK>(bK, tbs[p] * 16 + ln, kb * 32 + 8 * lg);
                M::mma(accG[p], ai, bt);
            }
        }
    }
    // accG[p][r] = k_i . k_t for i = ib*16 + 4lg + r, t = tb*16 + ln.  Masked value: the A^T
    // block (row i, column t).  Gamma_ti = 2^(g_t - g_i): as 2^g_t 2^-g_i while the chunk's
    // total decay g_C stays at or above -60 (both factors then normal), else per element.
    const bool factored = __builtin_amdgcn_readfirstlane((int)(sG[kChunk - 1] >= -60.f));
    auto masked = [&](int tb, int ib, f32x4 g_, f32x4 &av) {
        const int t = tb * 16 + ln;
        const float bt_ = sBeta[t];
        if (factored) {
            const float cf = bt_ * sE[t];
            const f32x4 ie = *(const f32x4 *)(sIE + ib * 16 + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ib * 16 + 4 * lg + r;
                av[r] = (i < t) ? (cf * ie[r]) * g_[r] : 0.f;
            }
        } else {
            const float gt = sG[t];
            const f32x4 gi = *(const f32x4 *)(sG + ib * 16 + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ib * 16 + 4 * lg + r;
                av[r] = (i < t) ? bt_ * g_[r] * __builtin_amdgcn_exp2f(gt - gi[r]) : 0.f;
            }
        }
    };
    f32x4 nT, a1, a2;
    masked(wave, wave, accG[0], nT);
    masked(tb0, ib0, accG[1], a1);
    if (np == 3) masked(3, ib1, accG[2], a2);
    // N (accumulator layout of the strictly lower diagonal block, row i, column t)
    f32x4 nC;
    {
        const int t = d0 + ln;
        const f32x4 bi = *(const f32x4 *)(sBeta + d0 + 4 * lg);
        if (factored) {
            const float iet = sIE[t];
            const f32x4 ei = *(const f32x4 *)(sE + d0 + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = d0 + 4 * lg + r;
                nC[r] = (t < i) ? (bi[r] * (ei[r] * iet)) * accG[0][r] : 0.f;
            }
        } else {
            const float gt = sG[t];
            const f32x4 gi = *(const f32x4 *)(sG + d0 + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = d0 + 4 * lg + r;
                nC[r] = (t < i) ? bi[r] * accG[0][r] * __builtin_amdgcn_exp2f(gi[r] - gt) : 0.f;
            }
        }
    }
    // zero blocks above the diagonal of T': wave w clears blocks (w, j), j > w
#pragma unroll
    for (int j = 1; j < 4; ++j) {
        if (j > wave)
            M::put4((OP *)(bT + swz<OP, kChunk>(split_pos(d0 + ln), 16 * j + 4 * lg)),
                    f32x4{0.f, 0.f, 0.f, 0.f});
    }
    // (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since N^16 = 0.  C = the
    // accumulator layout of a block, T = of its transpose (which is the row layout of it).
    f32x4 eye;
#pragma unroll
    for (int r = 0; r < 4; ++r) eye[r] = (4 * lg + r == ln) ? 1.f : 0.f;
    const Sp snT = split4(nT), snC = split4(nC);
    const f32x4 n2C = mm3r(snT, snC), n2T = mm3r(snC, snT);
    const Sp sn2C = split4(n2C), sn2T = split4(n2T);
    const f32x4 m1C = mm3r(snT, sn2C), m1T = mm3r(sn2C, snT);
    const f32x4 n4C = mm3r(sn2T, sn2C), n4T = mm3r(sn2C, sn2T);
    const f32x4 p1C = eye - nC + n2C - m1C, p1T = eye - nT + n2T - m1T;
    const Sp sn4C = split4(n4C), sp1T = split4(p1T);
    const f32x4 n8C = mm3r(split4(n4T), sn4C);
    f32x4 p2C = p1C, p2T = p1T;
    mm3(p2C, sp1T, sn4C);
    mm3(p2T, sn4C, sp1T);
    const Sp sn8C = split4(n8C), sp2T = split4(p2T);
    f32x4 xC = p2C, xT = p2T;
    mm3(xC, sp2T, sn8C);
    mm3(xT, sn8C, sp2T);
    __syncthreads();   // K is dead: its space now holds A and the X blocks

    // ---- phase 3 (stores): A blocks, X_ww in the row layout, T' diagonal block ----
    auto ablk = [&](int i, int m) { return sA + ((i * (i - 1) / 2 + m) * 16 + ln) * L::LDB + 4 * lg; };
    *(f32x4 *)ablk(tb0, ib0) = a1;
    if (np == 3) *(f32x4 *)ablk(3, ib1) = a2;
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
        auto arow = [&](int i, int m) { return split4(*(const f32x4 *)ablk(i, m)); };
        auto xrow = [&](int i) {
            return split4(*(const f32x4 *)(sX + (16 * i + ln) * L::LDX + 4 * lg));
        };
        auto put_t = [&](int i, f32x4 z) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Elem<OP>::store((OP *)(bT + swz<OP, kChunk>(split_pos(16 * i + 4 * lg + r), 16 * j + ln)),
                                z[r] * bcol);
        };
        if (j <= 2) {
            const Sp xjj = split4(xC);
            f32x4 acc1 = mm3r(arow(j + 1, j), xjj);
            f32x4 acc2 = {0.f, 0.f, 0.f, 0.f}, acc3 = {0.f, 0.f, 0.f, 0.f};
            if (j + 2 <= 3) acc2 = mm3r(arow(j + 2, j), xjj);
            if (j + 3 <= 3) acc3 = mm3r(arow(j + 3, j), xjj);
            const f32x4 x1 = -mm3r(xrow(j + 1), split4(acc1));      // X_{j+1,j}
            put_t(j + 1, x1);
            if (j + 2 <= 3) {
                const Sp sx1 = split4(x1);
                mm3(acc2, arow(j + 2, j + 1), sx1);
                if (j + 3 <= 3) mm3(acc3, arow(j + 3, j + 1), sx1);
                const f32x4 x2 = -mm3r(xrow(j + 2), split4(acc2));  // X_{j+2,j}
                put_t(j + 2, x2);
                if (j + 3 <= 3) {
                    mm3(acc3, arow(j + 3, j + 2), split4(x2));
                    const f32x4 x3 = -mm3r(xrow(j + 3), split4(acc3));  // X_{j+3,j}
                    put_t(j + 3, x3);
                }
            }
        }
    }
}

// =========================================================================================
// Launch 2: the state scan.  Waves 0-1 copy, the others scan (16 or 32 columns each).
// =========================================================================================
constexpr int kLoaders = 2;

// One pipeline stage: K rows (internal token order, swizzled), Q rows (swizzled), the record
// (T', g), P and the decay factors (formed by the loader waves) and the V tile (rows =
// tokens, plain).  Three stages
// when they fit in LDS, so that the copies of a chunk have two chunk-steps to arrive; two
// otherwise.
template <int DK, int DVT>
struct LdsSplit {
    static constexpr int al(int x) { return (x + 255) & ~255; }
    static constexpr int szRow = kChunk * DK * 2;       // [64][DK] bf16
    static constexpr int szV = kChunk * DVT * 2;        // [64][DVT] bf16
    static constexpr int sK = 0;
    static constexpr int sQ = szRow;
    static constexpr int sRec = 2 * szRow;
    static constexpr int sP = sRec + kPrepRecordBytes;  // [64][64] bf16, swizzled
    static constexpr int sGam = sP + kChunk * kChunk * 2;   // gamma_t 2^ls, fp32
    static constexpr int sRho = sGam + kChunk * 4;          // gamma_C / gamma_t / 2^ls', fp32
    static constexpr int sV = sRho + kChunk * 4;
    static constexpr int stage = al(sV + szV);
    static constexpr int nst = 3 * stage + 16 <= 160 * 1024 ? 3 : 2;
    static constexpr int sFlag = nst * stage;                // two ints (two-stage loaders)
    static constexpr int total = sFlag + 16;
};


// Column groups (16 state columns each) per scan wave.  One group per wave is the faster
// shape (the chunk update is a latency-bound chain, so more waves beat longer ones); the
// 64-column tile takes two groups per wave so that the workgroup stays at four waves (one
// per SIMD, with the full register file each).
template <int DVT> constexpr int groups_per_wave() { return DVT >= 64 ? 2 : 1; }
template <int DVT> constexpr int scan_waves() { return DVT / (16 * groups_per_wave<DVT>()); }

template <int DK, int DVT, int MODE>
__global__ __launch_bounds__(64 * (scan_waves<DVT>() + kLoaders)) void scan_split_kernel(PrefillArgs a)
{
    using L = LdsSplit<DK, DVT>;
    constexpr int NG = groups_per_wave<DVT>();
    using OP = uint16_t;
    using M = Mma<OP>;
    constexpr int NST = L::nst;
    constexpr int MBK = DK / 16;           // 16-row blocks of the state
    constexpr int KBD = DK / 32;           // K-blocks over the key dimension
    constexpr int KG = DK / 8;             // 16-byte granules per key row
    constexpr int CK = L::szRow / 1024;    // 1 KiB copies per K (or Q) tile
    constexpr int CV = L::szV / 1024 > 0 ? L::szV / 1024 : 1;   // ... per V tile
    constexpr int CR = kRecG / 1024;       // ... per T'
    constexpr bool kY = (MODE == kModeScan);
    static_assert(CK % 2 == 0 && CR % 2 == 0, "copy split");

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
    if constexpr (NST == 2) {
        if (tid < 2) ((volatile int *)(smem + L::sFlag))[tid] = -1;
        __syncthreads();
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
        // Every operand tile is a set of whole token rows, copied global -> LDS by the
        // direct-to-LDS loads (16 bytes per lane; lane l lands at the wave's LDS pointer +
        // 16 l).  Copy j of a tile fills its bytes [1024 j, 1024 j + 1024); the lane's source
        // row and column follow from the destination through the swizzle and, for K, the
        // internal token order.  Rows past the end of the job repeat its last row: they meet
        // zero rows and columns of T'.  P = lower_incl(Q K^T (.) Gamma) is formed in LDS from
        // the copied K, Q and g.
        //   three stages: wave 0 only copies (chunk c+2 during iteration c, into the stage
        //     iteration c-1 finished reading; it makes no other LDS access, so nothing waits
        //     on these copies before the end of the iteration) and wave 1 only forms P of
        //     chunk c+1, whose copies completed before the barrier that began iteration c;
        //   two stages: both waves copy chunk c+1, wait for it, and form half of its P.
        typedef __attribute__((address_space(3))) void lds_void;
        constexpr int CW = NST == 3 ? 1 : 2;                  // copying waves
        const unsigned rsK = (unsigned)(H * DK) * 2, rsV = (unsigned)(H * DV) * 2;  // bytes
        const int vcol0 = mpart ? 0 : job.col0;   // the M part copies (unused) V columns
        auto copy = [&](auto stc, int c) {
            constexpr int ST = decltype(stc)::value;
            unsigned char *stg = smem + ST * L::stage;
            const long long t0 = job.tok0 + (long long)c * kChunk;
            const int last = nvalid_of(c) - 1;
            const unsigned char *ck = (const unsigned char *)a.k + (t0 * H + job.h) * (long long)DK * 2;
            const unsigned char *cq = (const unsigned char *)a.q + (t0 * H + job.h) * (long long)DK * 2;
            const unsigned char *cv = (const unsigned char *)a.v +
                                      ((t0 * H + job.h) * (long long)DV + vcol0) * 2;
            const unsigned char *rec = (const unsigned char *)a.prep +
                                       ((slot0 + c) * H + job.h) * (long long)kPrepRecordBytes;
#pragma unroll
            for (int j = 0; j < CK / CW; ++j) {
                const int jj = wave + CW * j;
                const int P = 64 * jj + lane;                      // granule of the tile
                const int r = P / KG, pg = P % KG;
                const int lgq = pg ^ swz_key<OP, DK>(r);           // logical granule
                const int rk = split_orig(r) < last ? split_orig(r) : last;
                __builtin_amdgcn_global_load_lds(
                    (const void *)(ck + (unsigned)rk * rsK + 16 * lgq),
                    (lds_void *)(stg + L::sK + 1024 * jj), 16, 0, 0);
                if (kY) {
                    const int rq = r < last ? r : last;
                    __builtin_amdgcn_global_load_lds(
                        (const void *)(cq + (unsigned)rq * rsK + 16 * lgq),
                        (lds_void *)(stg + L::sQ + 1024 * jj), 16, 0, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < CR / CW; ++j) {
                const int jj = wave + CW * j;
                __builtin_amdgcn_global_load_lds((const void *)(rec + 16 * (64 * jj + lane)),
                                                 (lds_void *)(stg + L::sRec + 1024 * jj), 16, 0, 0);
            }
            // g (with two copying waves both write the same 256 bytes)
            __builtin_amdgcn_global_load_lds((const void *)(rec + kRecG + 4 * lane),
                                             (lds_void *)(stg + L::sRec + kRecG), 4, 0, 0);
#pragma unroll
            for (int j = 0; j < (CV + CW - 1) / CW; ++j) {
                const int jj = wave + CW * j;
                if (jj < CV) {
                    const int byte = 1024 * jj + 16 * lane;
                    const int r0 = byte / (DVT * 2), cb = byte % (DVT * 2);
                    const int r = r0 < last ? r0 : last;
                    __builtin_amdgcn_global_load_lds(
                        (const void *)(cv + (unsigned)r * rsV + cb),
                        (lds_void *)(stg + L::sV + 1024 * jj), 16, 0, 0);
                }
            }
        };
        // P of the chunk in stage ST from its K and Q rows and g.  Blocks (t-block, i-block):
        // (0,0) (1,0) (1,1) (2,0) (3,0) (2,1) (2,2) (3,1) (3,2) (3,3), split in halves when
        // two waves share the work; the blocks (0,1) and (2,3) that the scan reads are zero.
        // Accumulator [r] = k_i . q_t, i = 16 ib + 4 lg + r, t = 16 tb + ln: row t, columns
        // i .. i + 3 of P.
        auto make_p = [&](auto stc, auto nwc, auto pwc) {
            constexpr int ST = decltype(stc)::value;
            constexpr int NB = 10 / decltype(nwc)::value;
            constexpr int pw = decltype(pwc)::value;
            unsigned char *stg = smem + ST * L::stage;
            const unsigned char *bK = stg + L::sK;
            const unsigned char *bQ = stg + L::sQ;
            const float *sG = (const float *)(stg + L::sRec + kRecG);
            unsigned char *bP = stg + L::sP;
            constexpr int kTb[10] = {0, 1, 1, 2, 3, 2, 2, 3, 3, 3};
            constexpr int kIb[10] = {0, 0, 1, 0, 0, 1, 2, 1, 2, 3};
            f32x4 acc[NB];
#pragma unroll
            for (int p = 0; p < NB; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
                for (int p = 0; p < NB; ++p) {
                    const int tb = kTb[pw * NB + p], ib = kIb[pw * NB + p];
                    M::mma(acc[p], ldfrag<OP, DK>(bK, split_pos(ib * 16 + ln), kb * 32 + 8 * lg),
                           ldfrag<OP, DK>(bQ, tb * 16 + ln, kb * 32 + 8 * lg));
                }
#pragma unroll
            for (int p = 0; p < NB; ++p) {
                const int tb = kTb[pw * NB + p], ib = kIb[pw * NB + p];
                const int t = tb * 16 + ln;
                const float gt = sG[t];
                const f32x4 gi = *(const f32x4 *)(sG + ib * 16 + 4 * lg);
                f32x4 pv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ib * 16 + 4 * lg + r;
                    pv[r] = (i <= t) ? acc[p][r] * __builtin_amdgcn_exp2f(gt - gi[r]) : 0.f;
                }
                M::put4((OP *)(bP + swz<OP, kChunk>(t, ib * 16 + 4 * lg)), pv);
            }
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            if (NB == 10 || pw == 0) M::put4((OP *)(bP + swz<OP, kChunk>(ln, 16 + 4 * lg)), z);
            if (NB == 10 || pw == 1) M::put4((OP *)(bP + swz<OP, kChunk>(32 + ln, 48 + 4 * lg)), z);
        };
        // The scan holds its state as S = 2^ls Shat.  ls starts at 0 and after each chunk
        // becomes ls + g_C, or 0 when that would fall below -32 (the scan then rescales Shat);
        // both sides follow the same rule on the same g_C, so they agree bit for bit.  The
        // loader folds 2^ls into the factors it leaves in the stage:
        //   sGam[t] = gamma_t 2^ls,  sRho[t] = (gamma_C / gamma_t) / 2^ls'
        // (ls of the chunk, ls' of the next).
        float lsl = 0.f;
        auto prepare = [&](auto stc, auto nwc, auto pwc) {
            constexpr bool gam_writer = decltype(pwc)::value == 0;
            constexpr int ST = decltype(stc)::value;
            unsigned char *stg = smem + ST * L::stage;
            const float *sG = (const float *)(stg + L::sRec + kRecG);
            const float gt = sG[lane], gC = sG[kChunk - 1];
            const float lsc = lsl;
            float lsn = lsc + gC;
            if (lsn < -32.f) lsn = 0.f;
            if (gam_writer) {
                ((float *)(stg + L::sGam))[lane] = __builtin_amdgcn_exp2f(gt + lsc);
                ((float *)(stg + L::sRho))[lane] = __builtin_amdgcn_exp2f((gC - gt) - lsn);
            }
            if (kY) make_p(stc, nwc, pwc);
            lsl = lsn;
        };
        const std::integral_constant<int, 0> s0{};
        const std::integral_constant<int, 1> s1{};
        const std::integral_constant<int, 2> s2{};
        const std::integral_constant<int, 0> w0{};    // (the wave index as a constant keeps
        const std::integral_constant<int, 1> w1{};    //  make_p's block tables in registers)
        if constexpr (NST == 3) {
            const std::integral_constant<int, 1> one{};
            if (wave == 0) {
                if (nchunks > 0) {
                    copy(s0, 0);
                    if (nchunks > 1) copy(s1, 1);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    __syncthreads();    // chunks 0 and 1 are in LDS
                    __syncthreads();    // chunk 0 has its P
                }
                auto step = [&](auto stc, int c) {
                    if (c + 2 < nchunks) copy(stc, c + 2);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    __syncthreads();
                };
                for (int c = 0; c < nchunks; c += 3) {
                    step(s2, c);
                    if (c + 1 < nchunks) step(s0, c + 1);
                    if (c + 2 < nchunks) step(s1, c + 2);
                }
            } else {
                if (nchunks > 0) {
                    __syncthreads();
                    prepare(s0, one, w0);
                    __syncthreads();
                }
                auto step = [&](auto stp, int c) {
                    if (c + 1 < nchunks) prepare(stp, one, w0);
                    __syncthreads();
                };
                for (int c = 0; c < nchunks; c += 3) {
                    step(s1, c);
                    if (c + 1 < nchunks) step(s2, c + 1);
                    if (c + 2 < nchunks) step(s0, c + 2);
                }
            }
        } else {
            const std::integral_constant<int, 2> two{};
            // the two waves copy alternate 1 KiB pieces of every tile, so each waits for the
            // other's copies (a flag per wave in LDS) before it reads the K and Q rows
            volatile int *flag = (volatile int *)(smem + L::sFlag);
            auto both_copied = [&](int c) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (lane == 0) flag[wave] = c;
                while (flag[1 - wave] < c) __builtin_amdgcn_s_sleep(1);
            };
            if (nchunks > 0) {
                copy(s0, 0);
                both_copied(0);
                if (wave == 0) prepare(s0, two, w0);
                else prepare(s0, two, w1);
                __syncthreads();
            }
            auto step = [&](auto stn, int c) {
                if (c + 1 < nchunks) {
                    copy(stn, c + 1);
                    both_copied(c + 1);
                    if (wave == 0) prepare(stn, two, w0);
                    else prepare(stn, two, w1);
                }
                __syncthreads();
            };
            for (int c = 0; c < nchunks; c += 2) {
                step(s1, c);
                if (c + 1 < nchunks) step(s0, c + 1);
            }
        }
        return;
    }

    // ================================================================ scan waves
    // this wave owns state columns c0 + 16 g + ln, g < NG
    const int c0 = job.col0 + 16 * NG * sw;
    f32x4 S[NG][MBK];
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
        // register S[g][m][i] of lane (ln, lg) holds state row split_orig(16 m + 4 lg + i)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int m = 0; m < MBK; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = split_orig(16 * m + 4 * lg + i);
                    const int col = 16 * g + ln;
                    float x = 0.f;
                    if (mpart) x = (row == c0 - DV + col) ? 1.f : 0.f;
                    else if (src) x = src[(long long)row * DV + col];
                    S[g][m][i] = x;
                }
    }
    // The state is held as S = 2^ls * Shat (ls uniform, in [-32, 0]): the per-chunk decay
    // gamma_C goes into ls instead of a pass over the registers, and Shat is rescaled only
    // when ls would fall below -32.
    float ls = 0.f;
    auto chunk = [&](auto stc, int c) {
        constexpr int ST = decltype(stc)::value;
        const unsigned char *stg = smem + ST * L::stage;
        const unsigned char *bKc = stg + L::sK;
        const unsigned char *bQc = stg + L::sQ;
        const unsigned char *bTc = stg + L::sRec + kRecT;
        const unsigned char *bPc = stg + L::sP;
        const float *sGc = (const float *)(stg + L::sRec + kRecG);
        const float *sGam = (const float *)(stg + L::sGam);
        const float *sRho = (const float *)(stg + L::sRho);
        const unsigned char *bVc = stg + L::sV;
        const long long t0 = job.tok0 + (long long)c * kChunk;
        const int nv = nvalid_of(c);
        // Fragments are loaded one step ahead of the MFMAs that use them; the scheduling
        // fences keep the compiler from sinking each load next to its use.
        bf16x8 fk[2][4], fq[2][4], ft[6];
        auto frag64 = [&](const unsigned char *base, int row, int k0) {
            return ldfrag<OP, kChunk>(base, row, k0 + 8 * lg);
        };
        // K^T fragment for the state update: A[row = state row 16 m + ln (internal)][k =
        // tokens 32 kt + 8 lg .. + 7] by two transposing reads of the K rows.  Lane ln of the
        // group addresses token 32 kt + 8 lg + (ln / 4) (+ 4) and the four key columns that
        // lanes 4 (ln % 4) .. + 3 receive.
        auto frag_kt = [&](int m, int kt) {
            const int col = 32 * (m >> 1) + 8 * (ln & 3) + 4 * (m & 1);
            const int t = 32 * kt + 8 * lg + (ln >> 2);
            const bf16x4 lo = ldtr(bKc + swz<OP, DK>(split_pos(t), col));
            const bf16x4 hi = ldtr(bKc + swz<OP, DK>(split_pos(t + 4), col));
            return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };

        // ---- K S from the chunk-start state (the head of the state chain) ----
        f32x4 accYt[NG][4], acc_ks[NG][4];
        bf16x8 Sb[NG][KBD];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) fk[0][tb] = ldfrag<OP, DK>(bKc, tb * 16 + ln, 8 * lg);
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) Sb[g][kb] = pack8s(S[g][2 * kb], S[g][2 * kb + 1]);
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc_ks[g][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            if (kb + 1 < KBD) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    fk[(kb + 1) & 1][tb] = ldfrag<OP, DK>(bKc, tb * 16 + ln, (kb + 1) * 32 + 8 * lg);
            } else {
                // T' fragments for U = T' R: rows 0..31 use tokens 0..31 only
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) ft[mb] = frag64(bTc, mb * 16 + ln, 0);
                ft[4] = frag64(bTc, 32 + ln, 32);
                ft[5] = frag64(bTc, 48 + ln, 32);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int g = 0; g < NG; ++g) M::mma(acc_ks[g][tb], fk[kb & 1][tb], Sb[g][kb]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- R = V - diag(gamma 2^ls) K Shat;  U = T' R ----
        // the rows of K S this lane holds are internal 16 tb + 4 lg + i, i.e. tokens o0 + i
        f32x4 gam[4], rho[4];
        f32x4 U[NG][4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int o0 = split_orig(tb * 16 + 4 * lg);
            gam[tb] = *(const f32x4 *)(sGam + o0);
            rho[tb] = *(const f32x4 *)(sRho + o0);
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            f32x4 R[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                // V[o0 .. o0 + 3][column] by one transposing read of the V rows
                const int o0 = split_orig(tb * 16 + 4 * lg);
                const int col = c0 - job.col0 + 16 * g + 4 * (ln & 3);
                const bf16x4 v4 = ldtr(bVc + ((o0 + (ln >> 2)) * DVT + col) * 2);
                const f32x4 vv =
                    mpart ? f32x4{0.f, 0.f, 0.f, 0.f} : __builtin_convertvector(v4, f32x4);
                R[tb] = vv - gam[tb] * acc_ks[g][tb];
            }
            const bf16x8 Rb0 = pack8s(R[0], R[1]);
            const bf16x8 Rb1 = pack8s(R[2], R[3]);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                U[g][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
                M::mma(U[g][mb], ft[mb], Rb0);
            }
            M::mma(U[g][2], ft[4], Rb1);
            M::mma(U[g][3], ft[5], Rb1);
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- S^T Q^T from the chunk-start state (off the state chain: fills U's latency) ----
        bf16x8 fkt[2][MBK];
        float gy[4];
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) accYt[g][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (kY) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) fq[0][tb] = ldfrag<OP, DK>(bQc, tb * 16 + ln, 8 * lg);
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                if (kb + 1 < KBD) {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
                        fq[(kb + 1) & 1][tb] =
                            ldfrag<OP, DK>(bQc, tb * 16 + ln, (kb + 1) * 32 + 8 * lg);
                } else {
                    // K^T for the first half of the update, P for U^T P^T, gamma_t 2^ls
#pragma unroll
                    for (int m = 0; m < MBK; ++m) fkt[0][m] = frag_kt(m, 0);
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) ft[tb] = frag64(bPc, tb * 16 + ln, 0);
                    ft[4] = frag64(bPc, 32 + ln, 32);
                    ft[5] = frag64(bPc, 48 + ln, 32);
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) gy[tb] = sGam[tb * 16 + ln];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                    for (int g = 0; g < NG; ++g) M::mma(accYt[g][tb], Sb[g][kb], fq[kb & 1][tb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int m = 0; m < MBK; ++m) fkt[0][m] = frag_kt(m, 0);
        }

        // ---- U^T P^T (before the update, so that the output's epilogue runs while the
        //      update's products are in flight) ----
        f32x4 accPU[NG][4];
        if (kY) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const bf16x8 Uu0 = pack8s(U[g][0], U[g][1]);
                const bf16x8 Uu1 = pack8s(U[g][2], U[g][3]);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    accPU[g][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    M::mma(accPU[g][tb], Uu0, ft[tb]);
                }
                M::mma(accPU[g][2], Uu1, ft[4]);
                M::mma(accPU[g][3], Uu1, ft[5]);
            }
        }

        // ---- S = gamma_C S + K^T diag(gamma_C / gamma) U, as Shat += K^T diag(rho) U ----
        {
            float ln_ = ls + sGc[kChunk - 1];
            ln_ = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ln_)));
            if (ln_ < -32.f) {                     // fold the scale into Shat (rare)
                const float f = __builtin_amdgcn_exp2f(ln_);
#pragma unroll
                for (int g = 0; g < NG; ++g)
#pragma unroll
                    for (int m = 0; m < MBK; ++m) S[g][m] *= f;
                ln_ = 0.f;
            }
            ls = ln_;
            bf16x8 Ub0[NG], Ub1[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                f32x4 Us[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) Us[mb] = U[g][mb] * rho[mb];
                Ub0[g] = pack8s(Us[0], Us[1]);
                Ub1[g] = pack8s(Us[2], Us[3]);
            }
#pragma unroll
            for (int m = 0; m < MBK; ++m)
#pragma unroll
                for (int g = 0; g < NG; ++g) M::mma(S[g][m], fkt[0][m], Ub0[g]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MBK; ++m) fkt[1][m] = frag_kt(m, 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MBK; ++m)
#pragma unroll
                for (int g = 0; g < NG; ++g) M::mma(S[g][m], fkt[1][m], Ub1[g]);
        }

        // ---- Y^T = Shat^T Q^T diag(gamma 2^ls) + U^T P^T ----
        if (kY) {
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const int t = tb * 16 + ln;
                    const f32x4 yv = accYt[g][tb] * gy[tb] + accPU[g][tb];
                    if (t < nv)
                        store4((OP *)a.y + ((t0 + t) * H + job.h) * (long long)DV + c0 + 16 * g +
                                   4 * lg,
                               yv);
                }
        }
        __syncthreads();
    };
    if (nchunks > 0) {                    // the prologue's barriers (chunk 0 staged)
        __syncthreads();
        if (NST == 3) __syncthreads();
    }
    if constexpr (NST == 3) {
        for (int c = 0; c < nchunks; c += 3) {
            chunk(std::integral_constant<int, 0>{}, c);
            if (c + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, c + 1);
            if (c + 2 < nchunks) chunk(std::integral_constant<int, 2>{}, c + 2);
        }
    } else {
        for (int c = 0; c < nchunks; c += 2) {
            chunk(std::integral_constant<int, 0>{}, c);
            if (c + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, c + 1);
        }
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
            const float sp = __builtin_amdgcn_exp2f(ls);
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int m = 0; m < MBK; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[(long long)split_orig(16 * m + 4 * lg + i) * ld + 16 * g + ln] =
                            S[g][m][i] * sp;
        }
    }
}

// =========================================================================================
// Launch 2, pipelined form (bf16, 16 or 32 state columns per workgroup).  The output
// products leave the state chain: each 16-column group has a chain wave that carries the
// state and an output wave that forms Y, and the two meet in LDS.  During chunk step c:
//   copiers A, B   issue the copies of chunk c+2 (A: K in the internal token order and T';
//                  B: Q, V and g of chunk c+3) and wait only for their own copies of the
//                  step before, so that every copy has two chunk-steps to arrive
//   P wave         forms P of chunk c as six operand fragments
//   chain waves    R = V - diag(gamma 2^ls) K Shat, U = T' R and the state update of chunk
//                  c; they leave bf16 U and bf16 Shat (start of chunk c+1) in LDS
//   output waves   Shat^T Q^T of chunk c, then Y of chunk c-1 = diag(gamma 2^ls) Q Shat
//                  + P U, stored to y; the first also forms the decay factors of chunk c+1
// One barrier per chunk step.  P has two LDS buffers, by chunk parity, ordered by the step
// barriers; U and Shat have one each: the output wave raises a flag once it holds its copy
// in registers, and the chain wave waits for that flag before it writes the next value.
// =========================================================================================

template <int DK, int DVT>
struct LdsPipe {
    static constexpr int al(int x) { return (x + 255) & ~255; }
    static constexpr int NS = DVT / 16;               // 16-column groups
    static constexpr int szRow = kChunk * DK * 2;     // [64][DK] bf16
    static constexpr int szV = kChunk * DVT * 2;      // [64][DVT] bf16
    static constexpr int szP = 6 * 1024;              // six bf16 operand fragments of P
    static constexpr int szSb = DK * 16 * 2;          // bf16 Shat of a group, lane-linear
    static constexpr int szU = kChunk * 16 * 2;       // bf16 U of a group, lane-linear
    static constexpr int sK = 0;
    static constexpr int sQ = szRow;
    static constexpr int sRec = 2 * szRow;                  // T'
    static constexpr int sGam = sRec + kRecG;               // gamma_t 2^ls, fp32
    static constexpr int sRho = sGam + kChunk * 4;          // gamma_C / gamma_t / 2^ls', fp32
    static constexpr int sV = sRho + kChunk * 4;
    static constexpr int stage = al(sV + szV);        // three stages: chunk c in stage c % 3
    static constexpr int sG = 3 * stage;              // g of chunk c in slot c % 4 (fp32)
    static constexpr int sPb = sG + 4 * kChunk * 4;   // P of chunk c in buffer c & 1
    static constexpr int sSb = sPb + 2 * szP;
    static constexpr int sUb = sSb + NS * szSb;
    static constexpr int sFlag = sUb + NS * szU;      // [2][NS][NS] ints: Shat, U taken
    static constexpr int total = sFlag + 2 * NS * NS * 4;
    static_assert(total <= 160 * 1024, "LDS");
};

template <int DK, int DVT>
__global__ __launch_bounds__(64 * (3 + 2 * (DVT / 16))) void scan_pipe_kernel(PrefillArgs a)
{
    using L = LdsPipe<DK, DVT>;
    constexpr int NS = L::NS;
    using OP = uint16_t;
    using M = Mma<OP>;
    constexpr int MBK = DK / 16;           // 16-row blocks of the state
    constexpr int KBD = DK / 32;           // K-blocks over the key dimension
    constexpr int KG = DK / 8;             // 16-byte granules per key row
    constexpr int CK = L::szRow / 1024;    // 1 KiB copies per K or Q tile
    constexpr int CV = L::szV / 1024;      // ... per V tile
    constexpr int CR = kRecG / 1024;       // ... per T'
    constexpr int kCopiesA = CK + CR;      // copy instructions per chunk: K and T' (copier A)
    constexpr int kCopiesB = CK + CV;      // ... Q and V (copier B, plus one for g)
    // two chunks of copies in flight per copier stay below the 63 its counter holds
    static_assert(L::szV % 1024 == 0 && 2 * kCopiesA < 64 && 2 * (kCopiesB + 1) < 64, "copies");

    __shared__ __align__(16) unsigned char smem[L::total];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // role of the wave: 0 copier A, 1 P, 2 .. 1 + NS chains, 2 + NS .. 1 + 2 NS output,
    // 2 + 2 NS copier B.  Waves w and w + 4 share a SIMD: with two groups the P wave (the
    // longest step) has a SIMD of its own, each chain wave pairs with a copier and the two
    // output waves pair (wave -> role: 0 -> 0, 1 -> 4, 2 -> 2, 3 -> 1, 4 -> 3, 5 -> 5,
    // 6 -> 6).
    const int role = NS == 2 ? (wave == 1 ? 4 : wave == 3 ? 1 : wave == 4 ? 3 : wave) : wave;
    const int ln = lane & 15;
    const int lg = lane >> 4;

    // ---- job (as in scan_split_kernel) ----
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
    const int H = a.H;
    const int DV = a.dv;
    const int nchunks = (job.len + kChunk - 1) / kChunk;
    const long long srow0 = first_row(a, job.n);
    const long long slot0 = (srow0 >> 6) + job.n + (job.tok0 - srow0) / kChunk;
    auto nvalid_of = [&](int c) {
        const int r = job.len - c * kChunk;
        return r < kChunk ? r : kChunk;
    };
    // (LDS-qualified, so that the flags take LDS instructions and no memory-counter waits)
    typedef __attribute__((address_space(3))) volatile int lds_flag;
    // flag[g * NS + w]: output wave w holds the chain group g's Shat (flagS) or U (flagU)
    lds_flag *flagS = (lds_flag *)(smem + L::sFlag);
    lds_flag *flagU = flagS + NS * NS;
    if (tid < 2 * NS * NS) flagS[tid] = -1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // wait until flag[i] >= v (the output waves raise these early in every chunk step)
    auto wait_flag = [&](lds_flag *f, int v) {
        while (*f < v) __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");
    };
    const std::integral_constant<int, 0> s0{};
    const std::integral_constant<int, 1> s1{};
    const std::integral_constant<int, 2> s2{};
    // The step barrier orders LDS only: no wave reads another wave's global stores (y) during
    // the scan, so the barrier waits for this wave's LDS operations and not for its stores.
    auto lds_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    // Decay factors of chunk c into its stage (formed by the first output wave, a step ahead).
    // The scan holds its state as S = 2^ls Shat: ls starts at 0 and after each chunk becomes
    // ls + g_C, or 0 when that would fall below -32 (the chain waves then rescale Shat); both
    // follow the same rule on the same g_C, so they agree bit for bit.  The factors carry
    // 2^ls:  sGam[t] = gamma_t 2^ls,  sRho[t] = (gamma_C / gamma_t) / 2^ls'  (ls of the
    // chunk, ls' of the next).
    float lsl = 0.f;
    auto factors = [&](auto stc, int c) {
        constexpr int ST = decltype(stc)::value;
        unsigned char *stg = smem + ST * L::stage;
        const float *gc = (const float *)(smem + L::sG + (c & 3) * kChunk * 4);
        const float gt = gc[lane], gC = gc[kChunk - 1];
        const float lsc = lsl;
        float lsn = lsc + gC;
        if (lsn < -32.f) lsn = 0.f;
        ((float *)(stg + L::sGam))[lane] = __builtin_amdgcn_exp2f(gt + lsc);
        ((float *)(stg + L::sRho))[lane] = __builtin_amdgcn_exp2f((gC - gt) - lsn);
        lsl = lsn;
    };

    // ================================================================ copy waves
    // Two waves issue the copies, so that each stays within the 63 outstanding vector
    // memory instructions a wave can count: copier A the K tile and T', copier B the Q tile,
    // V and g.  Copy j of a tile fills its bytes [1024 j, 1024 j + 1024); each lane's source row
    // and column follow from its destination through the swizzle and, for K, the internal
    // token order.  Rows past the end of the job repeat its last row.  In step c a copier
    // issues its copies of chunk c+2 (copier B also g of chunk c+3), then waits only for
    // those it issued in the step before; the barrier needs no fence, as each copier's
    // copies are ordered by its counter alone.
    if (role == 0 || role == 2 + 2 * NS) {
        typedef __attribute__((address_space(3))) void lds_void;
        const bool is_a = role == 0;
        const unsigned rsK = (unsigned)(H * DK) * 2, rsV = (unsigned)(H * DV) * 2;   // bytes
        auto rec_of = [&](int c) {
            return (const unsigned char *)a.prep +
                   ((slot0 + c) * H + job.h) * (long long)kPrepRecordBytes;
        };
        // copier A: the K tile (rows in the internal token order) and T'
        auto copy_a = [&](auto stc, int c) {
            constexpr int ST = decltype(stc)::value;
            unsigned char *stg = smem + ST * L::stage;
            const long long t0 = job.tok0 + (long long)c * kChunk;
            const int last = nvalid_of(c) - 1;
            const unsigned char *ck = (const unsigned char *)a.k + (t0 * H + job.h) * (long long)DK * 2;
            const unsigned char *rec = rec_of(c);
#pragma unroll
            for (int j = 0; j < CK; ++j) {
                const int P = 64 * j + lane;                       // granule of the tile
                const int r = P / KG, pg = P % KG;
                const int rk = split_orig(r) < last ? split_orig(r) : last;
                __builtin_amdgcn_global_load_lds(
                    (const void *)(ck + (unsigned)rk * rsK + 16 * kq_logical<DK>(r, pg)),
                    (lds_void *)(stg + L::sK + 1024 * j), 16, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < CR; ++j)
                __builtin_amdgcn_global_load_lds((const void *)(rec + 16 * (64 * j + lane)),
                                                 (lds_void *)(stg + L::sRec + 1024 * j), 16, 0, 0);
        };
        // copier B: the Q tile and the V tile
        auto copy_b = [&](auto stc, int c) {
            constexpr int ST = decltype(stc)::value;
            unsigned char *stg = smem + ST * L::stage;
            const long long t0 = job.tok0 + (long long)c * kChunk;
            const int last = nvalid_of(c) - 1;
            const unsigned char *cq = (const unsigned char *)a.q + (t0 * H + job.h) * (long long)DK * 2;
            const unsigned char *cv = (const unsigned char *)a.v +
                                      ((t0 * H + job.h) * (long long)DV + job.col0) * 2;
#pragma unroll
            for (int j = 0; j < CK; ++j) {
                const int P = 64 * j + lane;
                const int r = P / KG, pg = P % KG;
                const int rq = r < last ? r : last;
                __builtin_amdgcn_global_load_lds(
                    (const void *)(cq + (unsigned)rq * rsK + 16 * kq_logical<DK>(r, pg)),
                    (lds_void *)(stg + L::sQ + 1024 * j), 16, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < CV; ++j) {
                const int byte = 1024 * j + 16 * lane;
                const int r0 = byte / (DVT * 2), cb = byte % (DVT * 2);
                const int r = r0 < last ? r0 : last;
                __builtin_amdgcn_global_load_lds((const void *)(cv + (unsigned)r * rsV + cb),
                                                 (lds_void *)(stg + L::sV + 1024 * j), 16, 0, 0);
            }
        };
        // g of chunk c (one copy instruction), a step earlier than the rest of its data
        auto copy_g = [&](int c) {
            __builtin_amdgcn_global_load_lds((const void *)(rec_of(c) + kRecG + 4 * lane),
                                             (lds_void *)(smem + L::sG + (c & 3) * kChunk * 4),
                                             4, 0, 0);
        };
        if (is_a) {
            if (nchunks > 0) {
                copy_a(s0, 0);
                if (nchunks > 1) {
                    copy_a(s1, 1);
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopiesA) : "memory");   // all but chunk 1
                } else {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_s_barrier();
            }
            auto step = [&](auto stc, int c) {
                if (c + 2 < nchunks) {
                    copy_a(stc, c + 2);
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopiesA) : "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                __builtin_amdgcn_s_barrier();
            };
            for (int c = 0; c < nchunks; c += 3) {
                step(s2, c);
                if (c + 1 < nchunks) step(s0, c + 1);
                if (c + 2 < nchunks) step(s1, c + 2);
            }
        } else {
            if (nchunks > 0) {
                copy_g(0);
                if (nchunks > 1) copy_g(1);
                if (nchunks > 2) copy_g(2);
                copy_b(s0, 0);
                if (nchunks > 1) {
                    copy_b(s1, 1);
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopiesB) : "memory");   // all but chunk 1
                } else {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_s_barrier();
            }
            auto step = [&](auto stc, int c) {
                if (c + 3 < nchunks) {
                    copy_b(stc, c + 2);
                    copy_g(c + 3);
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopiesB + 1) : "memory");
                } else if (c + 2 < nchunks) {
                    copy_b(stc, c + 2);
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopiesB) : "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                __builtin_amdgcn_s_barrier();
            };
            for (int c = 0; c < nchunks; c += 3) {
                step(s2, c);
                if (c + 1 < nchunks) step(s0, c + 1);
                if (c + 2 < nchunks) step(s1, c + 2);
            }
        }
        return;
    }

    // ================================================================ P wave
    if (role == 1) {
        // P = lower_incl(Q K^T (.) Gamma) of chunk c as the six operand fragments the output
        // waves read: fragment f < 4 holds rows 16 f .. 16 f + 15 and columns 0 .. 31,
        // fragments 4 and 5 rows 32 .. 47 and 48 .. 63 and columns 32 .. 63 (the rest of P is
        // zero); lane (ln, lg) holds row r0 + ln, columns c0 + 8 lg .. c0 + 8 lg + 7.  The K
        // operand takes the tile's rows as they lie (the internal token order), so the two
        // accumulator blocks of a 32-column half pack into a fragment directly: accumulator
        // [r] of block (tb, ib) = k_i . q_t, t = 16 tb + ln, i = original token of internal
        // row 16 ib + 4 lg + r, which is 32 (ib / 2) + 8 lg + 4 (ib % 2) + r.
        // Gamma_ti = 2^(g_t - g_i): formed as 2^g_t 2^-g_i while the chunk's total decay g_C
        // stays at or above -60 (both factors then normal floats), else per element.
        auto make_p = [&](auto stc, int c) {
            constexpr int ST = decltype(stc)::value;
            const unsigned char *stg = smem + ST * L::stage;
            const float *gc = (const float *)(smem + L::sG + (c & 3) * kChunk * 4);
            const unsigned char *bK = stg + L::sK;
            const unsigned char *bQ = stg + L::sQ;
            unsigned char *bP = smem + L::sPb + (c & 1) * L::szP;
            // blocks (tb, ib) in fragment order: (f, 0), (f, 1) for f < 4, then (2, 2) (2, 3)
            // (3, 2) (3, 3)
            constexpr int kTb[12] = {0, 0, 1, 1, 2, 2, 3, 3, 2, 2, 3, 3};
            constexpr int kIb[12] = {0, 1, 0, 1, 0, 1, 0, 1, 2, 3, 2, 3};
            bf16x8 fkb[KBD][4], fqb[KBD][4];
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fkb[kb][i] = ldfrag_kq<DK>(bK, i * 16 + ln, kb * 32 + 8 * lg);
                    fqb[kb][i] = ldfrag_kq<DK>(bQ, i * 16 + ln, kb * 32 + 8 * lg);
                }
            float gt[4];
            f32x4 gi[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gt[i] = gc[i * 16 + ln];
                gi[i] = *(const f32x4 *)(gc + 32 * (i >> 1) + 8 * lg + 4 * (i & 1));
            }
            f32x4 acc[12];
#pragma unroll
            for (int p = 0; p < 12; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
                for (int p = 0; p < 12; ++p) M::mma(acc[p], fkb[kb][kIb[p]], fqb[kb][kTb[p]]);
            // Gamma_ti = 2^(g_t - g_i).  g is non-increasing inside a chunk, so when the
            // chunk's total decay g_C stays above -60 both 2^g_t and 2^-g_i are normal and
            // their product (formed before it meets the accumulator) costs 8 exponentials;
            // below, 2^g_t would underflow and 2^-g_i overflow (0 * inf), so every element
            // takes its own 2^(g_t - g_i).  The branch is uniform over the wave.
            // g_C from the register lane 63 already holds (gi[3][3] there is g[63])
            const float gC = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gi[3][3]), 63));
            const bool factored = gC >= -60.f;
            f32x4 pv[12];
            if (factored) {
                float et[4];
                f32x4 ei[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    et[i] = __builtin_amdgcn_exp2f(gt[i]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) ei[i][r] = __builtin_amdgcn_exp2f(-gi[i][r]);
                }
#pragma unroll
                for (int p = 0; p < 12; ++p) {
                    const int tb = kTb[p], ib = kIb[p];
                    const int t = tb * 16 + ln;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 32 * (ib >> 1) + 8 * lg + 4 * (ib & 1) + r;
                        pv[p][r] = (i <= t) ? acc[p][r] * (et[tb] * ei[ib][r]) : 0.f;
                    }
                }
            } else {
#pragma unroll
                for (int p = 0; p < 12; ++p) {
                    const int tb = kTb[p], ib = kIb[p];
                    const int t = tb * 16 + ln;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 32 * (ib >> 1) + 8 * lg + 4 * (ib & 1) + r;
                        pv[p][r] = (i <= t)
                                       ? acc[p][r] * __builtin_amdgcn_exp2f(gt[tb] - gi[ib][r])
                                       : 0.f;
                    }
                }
            }
#pragma unroll
            for (int f = 0; f < 6; ++f)
                *(bf16x8 *)(bP + (f * 64 + lane) * 16) = pack8s(pv[2 * f], pv[2 * f + 1]);
        };
        if (nchunks > 0) {
            lds_barrier();
            lds_barrier();
        }
        // step c: P of chunk c (stage STc)
        auto step = [&](auto stc, int c) {
            make_p(stc, c);
            lds_barrier();
        };
        for (int c = 0; c < nchunks; c += 3) {
            step(s0, c);
            if (c + 1 < nchunks) step(s1, c + 1);
            if (c + 2 < nchunks) step(s2, c + 2);
        }
        return;
    }

    // ================================================================ chain waves
    if (role < 2 + NS) {
        const int sw = role - 2;
        // this wave owns the state columns col0 + kq(sw, ln): its 16 columns interleave with
        // the other group's in runs of four, so that the output waves hold, per lane, NS runs
        // of four that are adjacent in the row (one 16-byte store at NS = 2)
        const int c0 = job.col0 + 4 * NS * (ln >> 2) + 4 * sw + (ln & 3);
        f32x4 S[MBK];
        {
            const float *src = nullptr;
            if (job.seg == 0) {
                if (a.s0) src = a.s0 + ((long long)job.n * H + job.h) * DK * DV + c0;
            } else {
                src = a.segB + ((long long)(job.entry - 1) * H + job.h) * DK * DV + c0;
            }
            // register S[m][i] of lane (ln, lg) holds state row split_orig(16 m + 4 lg + i)
#pragma unroll
            for (int m = 0; m < MBK; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[m][i] = src ? src[(long long)split_orig(16 * m + 4 * lg + i) * DV] : 0.f;
        }
        unsigned char *sb = smem + L::sSb + sw * L::szSb;
        unsigned char *ub = smem + L::sUb + sw * L::szU;
        bf16x8 Sb[KBD];
        // bf16 Shat for the state products of a chunk, also left in LDS (lane-linear) for
        // the output wave of this group
        auto pack_state = [&]() {
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) Sb[kb] = pack8s(S[2 * kb], S[2 * kb + 1]);
        };
        auto put_state = [&]() {
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) *(bf16x8 *)(sb + (kb * 64 + lane) * 16) = Sb[kb];
        };
        float ls = 0.f;
        pack_state();
        put_state();
        auto chunk = [&](auto stc, int c) {
            constexpr int ST = decltype(stc)::value;
            const unsigned char *stg = smem + ST * L::stage;
            const unsigned char *bKc = stg + L::sK;
            const unsigned char *bTc = stg + L::sRec + kRecT;
            const float *sGc = (const float *)(smem + L::sG + (c & 3) * kChunk * 4);
            const float *sGam = (const float *)(stg + L::sGam);
            const float *sRho = (const float *)(stg + L::sRho);
            const unsigned char *bVc = stg + L::sV;
            auto frag64 = [&](const unsigned char *base, int row, int k0) {
                return ldfrag<OP, kChunk>(base, row, k0 + 8 * lg);
            };
            // K^T fragment for the state update: A[row = state row 16 m + ln (internal)][k =
            // tokens 32 kt + 8 lg .. + 7] by two transposing reads of the K rows.
            auto frag_kt = [&](int m, int kt) {
                const int col = 32 * (m >> 1) + 8 * (ln & 3) + 4 * (m & 1);
                const int t = 32 * kt + 8 * lg + (ln >> 2);
                const bf16x4 lo = ldtr(bKc + swz_kq<DK>(split_pos(t), col));
                const bf16x4 hi = ldtr(bKc + swz_kq<DK>(split_pos(t + 4), col));
                return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            };

            // ---- K S from the chunk-start state (the head of the state chain) ----
            bf16x8 fk[2][4], ft[6];
            f32x4 acc_ks[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) fk[0][tb] = ldfrag_kq<DK>(bKc, tb * 16 + ln, 8 * lg);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc_ks[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                if (kb + 1 < KBD) {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
                        fk[(kb + 1) & 1][tb] =
                            ldfrag_kq<DK>(bKc, tb * 16 + ln, (kb + 1) * 32 + 8 * lg);
                } else {
                    // T' fragments for U = T' R: rows 0..31 use tokens 0..31 only
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) ft[mb] = frag64(bTc, mb * 16 + ln, 0);
                    ft[4] = frag64(bTc, 32 + ln, 32);
                    ft[5] = frag64(bTc, 48 + ln, 32);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) M::mma(acc_ks[tb], fk[kb & 1][tb], Sb[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }

            // ---- R = V - diag(gamma 2^ls) K Shat;  U = T' R ----
            // the rows of K S this lane holds are internal 16 tb + 4 lg + i: tokens o0 + i
            f32x4 gam[4], rho[4], U[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int o0 = split_orig(tb * 16 + 4 * lg);
                gam[tb] = *(const f32x4 *)(sGam + o0);
                rho[tb] = *(const f32x4 *)(sRho + o0);
            }
            {
                f32x4 R[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    // V[o0 .. o0 + 3][column] by one transposing read of the V rows
                    const int o0 = split_orig(tb * 16 + 4 * lg);
                    // (lane j receives column 4 NS (j / 4) + 4 sw + j % 4 of tile rows o0..o0+3)
                    const int col = 4 * NS * (ln & 3) + 4 * sw;
                    const bf16x4 v4 = ldtr(bVc + ((o0 + (ln >> 2)) * DVT + col) * 2);
                    R[tb] = __builtin_convertvector(v4, f32x4) - gam[tb] * acc_ks[tb];
                }
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
            bf16x8 fkt[2][MBK];
#pragma unroll
            for (int m = 0; m < MBK; ++m) fkt[0][m] = frag_kt(m, 0);
            __builtin_amdgcn_sched_barrier(0);

            // ---- bf16 U for the output wave (which holds U of chunk c-1 by now) ----
            {
                const bf16x8 Uu0 = pack8s(U[0], U[1]);
                const bf16x8 Uu1 = pack8s(U[2], U[3]);
                if (c > 0)
                    for (int w = 0; w < NS; ++w) wait_flag(flagU + sw * NS + w, c - 1);
                *(bf16x8 *)(ub + lane * 16) = Uu0;
                *(bf16x8 *)(ub + 1024 + lane * 16) = Uu1;
            }
            // ---- S = gamma_C S + K^T diag(gamma_C / gamma) U, as Shat += K^T diag(rho) U ----
            float ln_ = ls + sGc[kChunk - 1];
            ln_ = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ln_)));
            if (ln_ < -32.f) {                     // fold the scale into Shat (rare)
                const float f = __builtin_amdgcn_exp2f(ln_);
#pragma unroll
                for (int m = 0; m < MBK; ++m) S[m] *= f;
                ln_ = 0.f;
            }
            ls = ln_;
            bf16x8 Ub0, Ub1;
            {
                f32x4 Us[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) Us[mb] = U[mb] * rho[mb];
                Ub0 = pack8s(Us[0], Us[1]);
                Ub1 = pack8s(Us[2], Us[3]);
            }
#pragma unroll
            for (int m = 0; m < MBK; ++m) M::mma(S[m], fkt[0][m], Ub0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MBK; ++m) fkt[1][m] = frag_kt(m, 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MBK; ++m) M::mma(S[m], fkt[1][m], Ub1);
            pack_state();
            // every output wave holds Shat of chunk c
            for (int w = 0; w < NS; ++w) wait_flag(flagS + sw * NS + w, c);
            put_state();
            lds_barrier();
        };
        if (nchunks > 0) {                // the prologue's barriers (chunk 0 staged)
            lds_barrier();
            lds_barrier();
        }
        for (int c = 0; c < nchunks; c += 3) {
            chunk(s0, c);
            if (c + 1 < nchunks) chunk(s1, c + 1);
            if (c + 2 < nchunks) chunk(s2, c + 2);
        }
        if (job.seg == job.nseg - 1 && a.s_final) {
            float *dst = a.s_final + ((long long)job.n * H + job.h) * DK * DV + c0;
            const float sp = __builtin_amdgcn_exp2f(ls);
#pragma unroll
            for (int m = 0; m < MBK; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(long long)split_orig(16 * m + 4 * lg + i) * DV] = S[m][i] * sp;
        }
        return;
    }

    // ================================================================ output waves
    // Output wave w forms y for tokens 64 w / NS .. 64 (w + 1) / NS - 1 of every chunk and
    // all DVT columns: per 16-token block and column group g, Shat_g^T Q^T and U_g^T P^T in
    // the accumulator layout (lane (ln, lg): token ln, the group's columns 4 lg .. 4 lg + 3,
    // i.e. tile columns 4 NS lg + 4 g .. + 3), so that a lane's NS runs of four are adjacent.
    {
        const int yw = role - 2 - NS;
        constexpr int TPW = 4 / NS;                   // 16-token blocks per output wave
        const int tbw = TPW * yw;                     // this wave's first block
        f32x4 accYp[NS][TPW];
        float gyp[TPW];
        // U of every group and the P fragments of this wave's token blocks, chunk c
        bf16x8 Uu0[NS], Uu1[NS], fp[TPW][2];
        auto take_up = [&](int c) {
#pragma unroll
            for (int g = 0; g < NS; ++g) {
                const unsigned char *ub = smem + L::sUb + g * L::szU;
                Uu0[g] = *(const bf16x8 *)(ub + lane * 16);
                Uu1[g] = *(const bf16x8 *)(ub + 1024 + lane * 16);
            }
            const unsigned char *bP = smem + L::sPb + (c & 1) * L::szP;
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int tb = tbw + u;
                fp[u][0] = *(const bf16x8 *)(bP + (tb * 64 + lane) * 16);
                if (tb >= 2) fp[u][1] = *(const bf16x8 *)(bP + ((tb + 2) * 64 + lane) * 16);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0)
                for (int g = 0; g < NS; ++g) flagU[g * NS + yw] = c;
        };
        // Y of chunk c = diag(gamma 2^ls) (Shat^T Q^T)^T (accYp, gyp) + P U
        auto finish = [&](int c) {
            const long long t0 = job.tok0 + (long long)c * kChunk;
            const int nv = nvalid_of(c);
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int tb = tbw + u;
                f32x4 yv[NS];
#pragma unroll
                for (int g = 0; g < NS; ++g) {
                    f32x4 pu = {0.f, 0.f, 0.f, 0.f};
                    M::mma(pu, Uu0[g], fp[u][0]);
                    if (tb >= 2) M::mma(pu, Uu1[g], fp[u][1]);
                    yv[g] = accYp[g][u] * gyp[u] + pu;
                }
                const int t = tb * 16 + ln;
                OP *dst = (OP *)a.y + ((t0 + t) * H + job.h) * (long long)DV + job.col0 + 4 * NS * lg;
                if (t < nv) {
                    if constexpr (NS == 2) *(bf16x8 *)dst = pack8s(yv[0], yv[1]);
                    else store4(dst, yv[0]);
                }
            }
        };
        auto step = [&](auto stc, int c) {
            constexpr int ST = decltype(stc)::value;
            const unsigned char *stg = smem + ST * L::stage;
            const float *sGam = (const float *)(stg + L::sGam);
            const unsigned char *bQ = stg + L::sQ;
            if (c > 0) take_up(c - 1);
            bf16x8 Sb[NS][KBD];
#pragma unroll
            for (int g = 0; g < NS; ++g) {
                const unsigned char *sb = smem + L::sSb + g * L::szSb;
#pragma unroll
                for (int kb = 0; kb < KBD; ++kb) Sb[g][kb] = *(const bf16x8 *)(sb + (kb * 64 + lane) * 16);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0)
                for (int g = 0; g < NS; ++g) flagS[g * NS + yw] = c;
            f32x4 accQ[NS][TPW];
#pragma unroll
            for (int g = 0; g < NS; ++g)
#pragma unroll
                for (int u = 0; u < TPW; ++u) accQ[g][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    const bf16x8 qf = ldfrag_kq<DK>(bQ, (tbw + u) * 16 + ln, kb * 32 + 8 * lg);
#pragma unroll
                    for (int g = 0; g < NS; ++g) M::mma(accQ[g][u], Sb[g][kb], qf);
                }
            float gy[TPW];
#pragma unroll
            for (int u = 0; u < TPW; ++u) gy[u] = sGam[(tbw + u) * 16 + ln];
            __builtin_amdgcn_sched_barrier(0);
            if (c > 0) finish(c - 1);
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
#pragma unroll
                for (int g = 0; g < NS; ++g) accYp[g][u] = accQ[g][u];
                gyp[u] = gy[u];
            }
            if (yw == 0 && c + 1 < nchunks) factors(std::integral_constant<int, (ST + 1) % 3>{}, c + 1);
            lds_barrier();
        };
        if (nchunks > 0) {
            lds_barrier();
            if (yw == 0) factors(s0, 0);
            lds_barrier();
        }
        for (int c = 0; c < nchunks; c += 3) {
            step(s0, c);
            if (c + 1 < nchunks) step(s1, c + 1);
            if (c + 2 < nchunks) step(s2, c + 2);
        }
        if (nchunks > 0) {
            take_up(nchunks - 1);
            finish(nchunks - 1);
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
    if constexpr (MODE == kModeScan && DVT <= 32) {
        hipLaunchKernelGGL((scan_pipe_kernel<DK, DVT>), dim3((unsigned)groups),
                           dim3(64 * (3 + 2 * (DVT / 16))), 0, stream, a2);
    } else {
        hipLaunchKernelGGL((scan_split_kernel<DK, DVT, MODE>), dim3((unsigned)groups),
                           dim3(64 * (scan_waves<DVT>() + kLoaders)), 0, stream, a2);
    }
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
