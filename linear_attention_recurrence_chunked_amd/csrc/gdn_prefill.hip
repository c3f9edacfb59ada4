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
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

constexpr int kThreads = 256;
constexpr float kLogAlphaFloor = -87.0f;   // log alpha clamp: keeps alpha = 0 finite

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
        u32x2 w;
        w[0] = pack_bf16x2(x[0], x[1]);
        w[1] = pack_bf16x2(x[2], x[3]);
        *(u32x2 *)p = w;
    }
    static __device__ __forceinline__ f32x4 get4(const uint16_t *p) { return load4(p); }
    static __device__ __forceinline__ frag from_f32(f32x4 lo, f32x4 hi) {
        u32x4 w;
        w[0] = pack_bf16x2(lo[0], lo[1]);
        w[1] = pack_bf16x2(lo[2], lo[3]);
        w[2] = pack_bf16x2(hi[0], hi[1]);
        w[3] = pack_bf16x2(hi[2], hi[3]);
        return __builtin_bit_cast(frag, w);
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
// LDS carve-up.  Rows are padded by 16 bytes so that the 16-lane groups of a fragment load
// fall on different banks.  Region R1 is time-shared by (i) the row-major Q and K tiles,
// (ii) the fp32 solve buffers and (iii) the transposed R / U / scaled-U tiles.
// ---------------------------------------------------------------------------------------
template <int DK, int DVT, typename OP>
struct Lds {
    static constexpr int E = sizeof(OP);
    static constexpr int LDK = DK + 16 / E;      // row length of [*, DK] tiles
    static constexpr int LDT = kChunk + 16 / E;  // row length of [*, 64 tokens] tiles
    static constexpr int LDA = kChunk + 4;       // fp32 solve rows
    static constexpr int al(int x) { return (x + 15) & ~15; }
    static constexpr int mx(int a, int b) { return a > b ? a : b; }
    static constexpr int szQK = 2 * kChunk * LDK * E;
    static constexpr int szSolve = 2 * kChunk * LDA * 4 + 3 * 16 * 16 * 4;
    static constexpr int szRU = 3 * DVT * LDT * E;
    static constexpr int R1 = al(mx(szQK, mx(szSolve, szRU)));
    static constexpr int oQ = 0;
    static constexpr int oK = kChunk * LDK * E;
    static constexpr int oA = 0;
    static constexpr int oX = kChunk * LDA * 4;
    static constexpr int oY = 2 * kChunk * LDA * 4;
    static constexpr int oRt = 0;
    static constexpr int oUt = DVT * LDT * E;
    static constexpr int oUs = 2 * DVT * LDT * E;
    static constexpr int oKt = R1;
    static constexpr int oVt = al(oKt + DK * LDT * E);
    static constexpr int oP = al(oVt + DVT * LDT * E);
    static constexpr int oT = al(oP + kChunk * LDT * E);
    static constexpr int oSt = al(oT + kChunk * LDT * E);
    static constexpr int oG = al(oSt + DVT * LDK * E);
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
};

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

// ---------------------------------------------------------------------------------------
// The chunked scan.  MODE == kModeScan: start from S0 (or a segment start state), write y
// and (for the last segment) the final state.  MODE == kModeAug: phase A of the segment
// scan; no y; columns col0 >= d_v belong to the transition part (V = 0, start = identity).
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
    constexpr int KBLK = (16 * DQ + kThreads - 1) / kThreads;   // 4x4 blocks per thread (q, k)
    constexpr int VBLK = (16 * VQ + kThreads - 1) / kThreads;   // 4x4 blocks per thread (v)
    constexpr bool kWantY = (MODE == kModeScan);

    __shared__ __align__(16) unsigned char smem[L::total];
    OP *sQ = (OP *)(smem + L::oQ);
    OP *sK = (OP *)(smem + L::oK);
    float *sA = (float *)(smem + L::oA);
    float *sX = (float *)(smem + L::oX);
    float *sY = (float *)(smem + L::oY);
    OP *sRt = (OP *)(smem + L::oRt);
    OP *sUt = (OP *)(smem + L::oUt);
    OP *sUs = (OP *)(smem + L::oUs);
    OP *sKt = (OP *)(smem + L::oKt);
    OP *sVt = (OP *)(smem + L::oVt);
    OP *sP = (OP *)(smem + L::oP);
    OP *sT = (OP *)(smem + L::oT);
    OP *sSt = (OP *)(smem + L::oSt);
    float *sG = (float *)(smem + L::oG);
    float *sBeta = (float *)(smem + L::oB);

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
        long long ld = DV;
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
                    else if (src) x = src[(long long)row * ld + col];
                    S[mb][nb][i] = x;
                }
    }

    // ---- global -> register prefetch of one chunk ----
    Q4 pk[KBLK][4], pq[KBLK][4], pv[VBLK][4];
    float pa = 1.f;   // threads 0..63: alpha of token (tid); threads 64..127: beta of token
    auto prefetch = [&](long long t0, int nvalid) {
#pragma unroll
        for (int j = 0; j < KBLK; ++j) {
            const int b = tid + kThreads * j;
            const int dq = b % DQ, tq = b / DQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * tq + i;
                if (b < 16 * DQ && t < nvalid) {
                    const long long off = ((t0 + t) * H + job.h) * (long long)DK + 4 * dq;
                    pk[j][i] = Q4::load(gk + off);
                    if (kWantY) pq[j][i] = Q4::load(gq + off);
                } else {
                    pk[j][i] = Q4::zero();
                    if (kWantY) pq[j][i] = Q4::zero();
                }
            }
        }
#pragma unroll
        for (int j = 0; j < VBLK; ++j) {
            const int b = tid + kThreads * j;
            const int dq = b % VQ, tq = b / VQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * tq + i;
                if (!mpart && b < 16 * VQ && t < nvalid) {
                    const long long off =
                        ((t0 + t) * H + job.h) * (long long)DV + job.col0 + 4 * dq;
                    pv[j][i] = Q4::load(gv + off);
                } else {
                    pv[j][i] = Q4::zero();
                }
            }
        }
        if (tid < 64) {
            pa = (tid < nvalid) ? a.alpha[(t0 + tid) * H + job.h] : 1.f;
        } else if (tid < 128) {
            const int t = tid - 64;
            pa = (t < nvalid) ? a.beta[(t0 + t) * H + job.h] : 0.f;
        }
    };

    // S -> LDS (transposed bf16/fp32 copy used as the B operand of [K; Q] S)
    auto store_state_lds = [&]() {
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = (wave * MBS + mb) * 16 + 4 * lg;
                M::put4(sSt + (nb * 16 + ln) * L::LDK + row, S[mb][nb]);
            }
    };
    store_state_lds();

    const int nchunks = (job.len + kChunk - 1) / kChunk;
    if (nchunks > 0) prefetch(job.tok0, job.len < kChunk ? job.len : kChunk);

    // Gram tile pairs (t-block, i-block) with i-block <= t-block, spread over the waves
    constexpr int kPairs = 10;
    constexpr int kPairsPerWave = 3;

    for (int c = 0; c < nchunks; ++c) {
        const long long t0 = job.tok0 + (long long)c * kChunk;
        const int nvalid = (job.len - c * kChunk) < kChunk ? (job.len - c * kChunk) : kChunk;
        __syncthreads();   // the previous chunk is done with every LDS buffer

        // ---- registers -> LDS: Q, K row major; K, V transposed; g; beta ----
#pragma unroll
        for (int j = 0; j < KBLK; ++j) {
            const int b = tid + kThreads * j;
            if (b < 16 * DQ) {
                const int dq = b % DQ, tq = b / DQ;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pk[j][i].store(sK + (4 * tq + i) * L::LDK + 4 * dq);
                    if (kWantY) pq[j][i].store(sQ + (4 * tq + i) * L::LDK + 4 * dq);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    Q4::column(pk[j], jj).store(sKt + (4 * dq + jj) * L::LDT + 4 * tq);
            }
        }
#pragma unroll
        for (int j = 0; j < VBLK; ++j) {
            const int b = tid + kThreads * j;
            if (b < 16 * VQ) {
                const int dq = b % VQ, tq = b / VQ;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    Q4::column(pv[j], jj).store(sVt + (4 * dq + jj) * L::LDT + 4 * tq);
            }
        }
        if (wave == 0) {
            // inclusive prefix sum of log alpha over the chunk (lane = token)
            float x = fmaxf(logf(pa), kLogAlphaFloor);
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            sG[lane] = x;
        } else if (wave == 1) {
            sBeta[lane] = pa;
        }
        if (c + 1 < nchunks) {
            const int nv = (job.len - (c + 1) * kChunk) < kChunk ? (job.len - (c + 1) * kChunk)
                                                                 : kChunk;
            prefetch(t0 + kChunk, nv);
        }
        __syncthreads();

        // ---- a1/a4: Gram tiles (K K^T and K Q^T, lower pairs), and [K; Q] S ----
        f32x4 accG[kPairsPerWave], accP[kPairsPerWave];
#pragma unroll
        for (int pi = 0; pi < kPairsPerWave; ++pi) {
            const int p = wave + 4 * pi;
            accG[pi] = f32x4{0.f, 0.f, 0.f, 0.f};
            accP[pi] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p < kPairs) {
                // pair p -> (tb, ib): 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) ...
                const int tb = p < 1 ? 0 : (p < 3 ? 1 : (p < 6 ? 2 : 3));
                const int ib = p - tb * (tb + 1) / 2;
#pragma unroll
                for (int kb = 0; kb < KBD; ++kb) {
                    const auto ai = M::load(sK + (ib * 16 + ln) * L::LDK + kb * 32 + 8 * lg);
                    const auto bt = M::load(sK + (tb * 16 + ln) * L::LDK + kb * 32 + 8 * lg);
                    M::mma(accG[pi], ai, bt);
                    if (kWantY) {
                        const auto bq = M::load(sQ + (tb * 16 + ln) * L::LDK + kb * 32 + 8 * lg);
                        M::mma(accP[pi], ai, bq);
                    }
                }
            }
        }
        f32x4 accKS[NB], accQS[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            accKS[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            accQS[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            const auto ak = M::load(sK + (wave * 16 + ln) * L::LDK + kb * 32 + 8 * lg);
            typename M::frag aq;
            if (kWantY) aq = M::load(sQ + (wave * 16 + ln) * L::LDK + kb * 32 + 8 * lg);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const auto bs = M::load(sSt + (nb * 16 + ln) * L::LDK + kb * 32 + 8 * lg);
                M::mma(accKS[nb], ak, bs);
                if (kWantY) M::mma(accQS[nb], aq, bs);
            }
        }
        __syncthreads();   // Q and K row-major tiles are dead; R1 becomes the solve area

        // ---- decay masks: A (fp32, strictly lower, rows scaled by beta) and P ----
#pragma unroll
        for (int pi = 0; pi < kPairsPerWave; ++pi) {
            const int p = wave + 4 * pi;
            if (p < kPairs) {
                const int tb = p < 1 ? 0 : (p < 3 ? 1 : (p < 6 ? 2 : 3));
                const int ib = p - tb * (tb + 1) / 2;
                const int t = tb * 16 + ln;
                const float gt = sG[t];
                const float bt = sBeta[t];
                f32x4 av, pv4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ib * 16 + 4 * lg + r;
                    const float dec = (i <= t) ? expf(gt - sG[i]) : 0.f;
                    av[r] = (i < t) ? bt * accG[pi][r] * dec : 0.f;
                    pv4[r] = accP[pi][r] * dec;
                }
                *(f32x4 *)(sA + t * L::LDA + ib * 16 + 4 * lg) = av;
                if (kWantY) M::put4(sP + t * L::LDT + ib * 16 + 4 * lg, pv4);
            }
        }
        // upper tiles (i-block > t-block) are zero
#pragma unroll
        for (int ui = 0; ui < 2; ++ui) {
            const int u = wave + 4 * ui;
            if (u < 6) {
                // 0:(0,1) 1:(0,2) 2:(0,3) 3:(1,2) 4:(1,3) 5:(2,3)
                const int tb = u < 3 ? 0 : (u < 5 ? 1 : 2);
                const int ib = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
                const int t = tb * 16 + ln;
                *(f32x4 *)(sA + t * L::LDA + ib * 16 + 4 * lg) = f32x4{0.f, 0.f, 0.f, 0.f};
                if (kWantY) M::put4(sP + t * L::LDT + ib * 16 + 4 * lg, f32x4{0.f, 0.f, 0.f, 0.f});
            }
        }
        __syncthreads();

        // ---- a2: X = (I + A)^{-1}, blocked by 16 ----
        {
            // diagonal blocks: wave w inverts block w by forward substitution, one column
            // per lane (the four 16-lane groups compute the same columns; group 0 stores)
            const int d0 = wave * 16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == ln) ? 1.f : 0.f;
#pragma unroll
                for (int cc = 0; cc < r; ++cc) acc -= sA[(d0 + r) * L::LDA + d0 + cc] * x[cc];
                x[r] = acc;
            }
            if (lg == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sX[(d0 + r) * L::LDA + d0 + ln] = x[r];
            }
        }
        __syncthreads();
        // off-diagonal blocks by distance: X_ij = -X_ii * sum_{m in blocks j..i-1} A_im X_mj
        {
            const int r = tid >> 4, cc = tid & 15;
#pragma unroll
            for (int dist = 1; dist <= 3; ++dist) {
                const int npairs = 4 - dist;
                // Y_ij[r][cc] = sum_m A[16i + r][m] X[m][16j + cc]
                for (int pj = 0; pj < npairs; ++pj) {
                    const int j = pj, i = pj + dist;
                    float acc = 0.f;
                    for (int m = 16 * j; m < 16 * i; ++m)
                        acc += sA[(16 * i + r) * L::LDA + m] * sX[m * L::LDA + 16 * j + cc];
                    sY[(pj * 16 + r) * 16 + cc] = acc;
                }
                __syncthreads();
                for (int pj = 0; pj < npairs; ++pj) {
                    const int j = pj, i = pj + dist;
                    float acc = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        acc += sX[(16 * i + r) * L::LDA + 16 * i + m] * sY[(pj * 16 + m) * 16 + cc];
                    sX[(16 * i + r) * L::LDA + 16 * j + cc] = -acc;
                }
                __syncthreads();
            }
        }
        // T' = X diag(beta) (unit diagonal of X -> beta_t), lower triangle only
        {
            const int t = tid >> 2;
            const int i0 = (tid & 3) * 16;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 tv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + 4 * q4 + e;
                    tv[e] = (i < t) ? sX[t * L::LDA + i] * sBeta[i] : (i == t ? sBeta[t] : 0.f);
                }
                M::put4(sT + t * L::LDT + i0 + 4 * q4, tv);
            }
        }
        __syncthreads();   // solve buffers are dead; R1 becomes the R / U area

        // ---- R = V - diag(gamma) K S   (wave w: token rows 16w .. 16w + 15) ----
        const int trow = wave * 16 + 4 * lg;
        f32x4 gam;
#pragma unroll
        for (int r = 0; r < 4; ++r) gam[r] = expf(sG[trow + r]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int col = nb * 16 + ln;
            const f32x4 vv = M::get4(sVt + col * L::LDT + trow);
            M::put4(sRt + col * L::LDT + trow, vv - gam * accKS[nb]);
        }
        __syncthreads();

        // ---- U = T' R (lower triangular: K-blocks up to the diagonal) ----
        const float gC = sG[kChunk - 1];
        f32x4 accU[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) accU[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb <= (wave >> 1)) {
                const auto at = M::load(sT + (wave * 16 + ln) * L::LDT + kb * 32 + 8 * lg);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const auto br = M::load(sRt + (nb * 16 + ln) * L::LDT + kb * 32 + 8 * lg);
                    M::mma(accU[nb], at, br);
                }
            }
        }
        f32x4 tail;   // gamma_C / gamma_t
#pragma unroll
        for (int r = 0; r < 4; ++r) tail[r] = expf(gC - sG[trow + r]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int col = nb * 16 + ln;
            if (kWantY) M::put4(sUt + col * L::LDT + trow, accU[nb]);
            M::put4(sUs + col * L::LDT + trow, accU[nb] * tail);
        }
        __syncthreads();

        // ---- Y = diag(gamma) Q S + P U ----
        if (kWantY) {
            f32x4 accY[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) accY[nb] = gam * accQS[nb];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb <= (wave >> 1)) {
                    const auto ap = M::load(sP + (wave * 16 + ln) * L::LDT + kb * 32 + 8 * lg);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const auto bu = M::load(sUt + (nb * 16 + ln) * L::LDT + kb * 32 + 8 * lg);
                        M::mma(accY[nb], ap, bu);
                    }
                }
            }
            OP *gy = (OP *)a.y;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = trow + r;
                    if (t < nvalid)
                        Elem<OP>::store(gy + ((t0 + t) * H + job.h) * (long long)DV + job.col0 +
                                            nb * 16 + ln,
                                        accY[nb][r]);
                }
        }

        // ---- S = gamma_C S + (diag(gamma_C / gamma) K)^T U ----
        const float gamC = expf(gC);
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb) {
            const int drow = (wave * MBS + mb) * 16;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) S[mb][nb] *= gamC;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const auto ak = M::load(sKt + (drow + ln) * L::LDT + kb * 32 + 8 * lg);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const auto bu = M::load(sUs + (nb * 16 + ln) * L::LDT + kb * 32 + 8 * lg);
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
                                                             SegEntry *table, int32_t *count)
{
    __shared__ int32_t s_scan[1024];
    __shared__ int32_t s_base;
    const int tid = threadIdx.x;
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
    if (plan.seg_chunks < 0) {
        return launch_scan<DK, DVT, OP, kModeScan>(args, args.num_seqs, dv / DVT, stream);
    }
    hipLaunchKernelGGL(segment_table_kernel, dim3(1), dim3(1024), 0, stream, args,
                       plan.seg_chunks * kChunk, (SegEntry *)args.table,
                       (int32_t *)args.n_entries);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // phase A: [S | M] scans of every segment but the last of each sequence
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

// Tiles each dtype supports (LDS budget): bf16 16..128, fp32 16..64.
static bool tile_ok(int dtype, int dk, int dv, int t)
{
    if (t != 16 && t != 32 && t != 64 && t != 128) return false;
    if (dv % t != 0) return false;
    if (dtype == kDtypeF32 && (t > 64 || (dk == 128 && t > 32))) return false;
    return true;
}

bool make_plan(int num_seqs, long long total_T, int H, int dk, int dv, int dtype,
               int dv_tile_req, int seg_chunks_req, PrefillPlan *plan)
{
    // Column tile: the chains (sequence, head) are independent; split the state columns
    // until there are enough workgroups to cover the 256 CUs, within the LDS budget.
    int tile = dv_tile_req;
    const long long chains = (long long)num_seqs * H;
    if (tile == 0) {
        tile = (dtype == kDtypeF32) ? (dk == 128 ? 32 : 64) : dv;
        while (tile > 32 && chains * (dv / tile) < 512) tile >>= 1;
        if (!tile_ok(dtype, dk, dv, tile)) tile = 32;
    }
    if (!tile_ok(dtype, dk, dv, tile)) return false;
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
    if (plan.seg_chunks >= 0) {
        unsigned char *ws = (unsigned char *)workspace;
        a.table = (const SegEntry *)ws;
        a.n_entries = (const int32_t *)(ws + plan.max_segments * sizeof(SegEntry));
        float *seg = (float *)(ws + plan.ws_table);
        a.segB = seg;
        a.segM = seg + (size_t)plan.max_segments * p.H * p.dk * p.dv;
    }
    if (p.dtype == kDtypeBF16)
        return dispatch_dk_dvt<uint16_t>(a, plan, p.dk, plan.max_segments, stream);
    return dispatch_dk_dvt<float>(a, plan, p.dk, plan.max_segments, stream);
}

}  // namespace gdn
