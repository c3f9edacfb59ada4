// gdn_qsa.hip -- the compressed block indexer of the sparse attention (gfx950).
//
// The reading notes' "compressed lightweight indexer" (Qwen3.8-Next, QSA): an MQA indexer
// with 4 query heads and one shared key head of 128 dimensions.  For one sequence of n
// tokens:
//   q_i^h  = PRoPE(RMSNorm(q_i^h), i)                 (queries, per head)
//   kb_b   = PRoPE(RMSNorm(mean(k_{4b} .. k_{4b+3})), 4b)   (pooled block keys)
//   I_ib   = sum_h ReLU(<q_i^h, kb_b>)  for 4b + 3 <= i
//   B_i    = the K_B highest-scoring blocks (ties to the lower index), expanded to their
//            tokens and joined with the tail {floor((i+1)/4) 4 .. i}.
// PRoPE rotates dims (m, m + 32), m < 32, by pos * 10000^(-2m/64); dims 64..127 pass.
// RMSNorm(x) = x / sqrt(mean(x^2) + 1e-6), no scale.
//
// Two launches, no score matrix (workspace O(n): the prepared queries and block keys):
//   qsa_prep_kernel    one wave per query row (token, head) or per key block: normalise,
//                      rotate (angles and their sines in fp64: positions reach 10^6 radians),
//                      store bf16.
//   qsa_select_kernel  QN queries per workgroup against all their visible blocks on 16x16x32
//                      bf16 MFMAs, the queries' fragments held in registers and the block keys
//                      streamed from L2 one step ahead: the four heads of a query are four
//                      consecutive accumulator rows, i.e. the four values one lane holds, so
//                      the ReLU head-sum needs no exchange.  Each score is compared with its
//                      query's running threshold as it is formed; the few that pass go to the
//                      query's candidate list in LDS, in block order, and a list that fills up
//                      is trimmed to the K_B best (an exact selection over at most a few
//                      thousand entries), which raises the threshold.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kQH = 4;          // query heads
constexpr int kQD = 128;        // head dimension
constexpr int kQR = 4;          // tokens per key block
constexpr float kQEps = 1e-6f;

struct QsaArgs {
    const void *q, *k;
    long long n;
    int kb;                     // block budget
    uint16_t *qr;               // [n, 4, 128] bf16
    uint16_t *kbk;              // [nb, 128] bf16
    int32_t *blocks;            // [n, kb] or null
    int32_t *tokens;            // [n, kb * 4 + 3] or null
};

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// RMSNorm and partial RoPE of one 128-element row held as (x0 = dim lane, x1 = dim 64+lane);
// writes the bf16 row.
__device__ __forceinline__ void norm_rotate_store(float x0, float x1, double pos, uint16_t *dst)
{
    const int lane = threadIdx.x & 63;
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float sc = 1.0f / sqrtf(ss * (1.0f / kQD) + kQEps);
    x0 *= sc;
    x1 *= sc;
    const float other = __shfl_xor(x0, 32, kWave);          // the partner of the pair
    const int m = lane & 31;
    const double ang = pos * exp(-(2.0 * m / 64.0) * log(10000.0));
    double sd, cd;
    sincos(ang, &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    const float out0 = lane < 32 ? x0 * c - other * s : other * s + x0 * c;
    Elem<uint16_t>::store(dst + lane, out0);
    Elem<uint16_t>::store(dst + 64 + lane, x1);
}

template <typename T>
__global__ __launch_bounds__(256) void qsa_prep_kernel(QsaArgs a)
{
    const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long long nq = a.n * kQH, nb = a.n / kQR;
    const T *q = (const T *)a.q, *k = (const T *)a.k;
    if (w < nq) {
        const long long row = w;                                // token * 4 + head
        const float x0 = Elem<T>::load(q + row * kQD + lane);
        const float x1 = Elem<T>::load(q + row * kQD + 64 + lane);
        norm_rotate_store(x0, x1, (double)(row / kQH), a.qr + row * kQD);
    } else if (w < nq + nb) {
        const long long b = w - nq;
        float x0 = 0.f, x1 = 0.f;
#pragma unroll
        for (int t = 0; t < kQR; ++t) {
            x0 += Elem<T>::load(k + (b * kQR + t) * kQD + lane);
            x1 += Elem<T>::load(k + (b * kQR + t) * kQD + 64 + lane);
        }
        norm_rotate_store(x0 * 0.25f, x1 * 0.25f, (double)(b * kQR), a.kbk + b * kQD);
    }
}

// The 16-lane group g's bits of a ballot (lanes 16 g .. 16 g + 15).
__device__ __forceinline__ uint32_t group_bits(uint64_t m, int g)
{
    return (uint32_t)(m >> (16 * g)) & 0xffffu;
}

// DPP lane moves within rows of 16 (row_shr:n shifts in zeros; the four butterfly patterns
// give every lane its row's reduction)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, true);
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, Op op)
{
    x = op(x, dpp_u32<0xb1>(x));            // quad_perm [1, 0, 3, 2]
    x = op(x, dpp_u32<0x4e>(x));            // quad_perm [2, 3, 0, 1]
    x = op(x, dpp_u32<0x141>(x));           // row_half_mirror
    x = op(x, dpp_u32<0x140>(x));           // row_mirror
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return op(op(r0, r1), op(r2, r3));
}

// Exclusive prefix sum over the wave's lanes (lane order), and the wave total.
__device__ __forceinline__ int wave_excl_scan(int x, int &total)
{
    const int lane = threadIdx.x & 63;
    uint32_t v = (uint32_t)x;
    v += dpp_u32<0x111>(v);                 // row_shr:1
    v += dpp_u32<0x112>(v);                 // row_shr:2
    v += dpp_u32<0x114>(v);                 // row_shr:4
    v += dpp_u32<0x118>(v);                 // row_shr:8
    const int t0 = __builtin_amdgcn_readlane((int)v, 15);
    const int t1 = __builtin_amdgcn_readlane((int)v, 31);
    const int t2 = __builtin_amdgcn_readlane((int)v, 47);
    const int t3 = __builtin_amdgcn_readlane((int)v, 63);
    const int row = lane >> 4;
    const int off = row == 0 ? 0 : row == 1 ? t0 : row == 2 ? t0 + t1 : t0 + t1 + t2;
    total = t0 + t1 + t2 + t3;
    return off + (int)v - x;
}

// The k-th largest (1 <= k <= number of flagged keys) of the keys that src flags, and how
// many keys equal to it are among the k largest (need_eq).  src.load(gi, key, use) gives
// group gi of the keys, 16 per lane (src.groups() groups).  The key range [lo, hi] starts at
// the flagged keys' minimum and maximum; each round counts the keys of the range in 256 bins
// of (key - lo) >> sh and narrows the range to the bin holding the rank still wanted; a bin of
// at most 64 keys is ranked pairwise, a range of one value ends the search.  scr: 256 ints,
// cand: 64 words of this wave's LDS.
template <typename Src>
__device__ __forceinline__ uint32_t kth_largest(const Src &src, int k, int *scr, uint32_t *cand,
                                                int &need_eq)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[16];
    bool use[16];
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (int gi = 0; gi < src.groups(); ++gi) {
        src.load(gi, key, use);
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (use[u]) {
                lo = min(lo, key[u]);
                hi = max(hi, key[u]);
            }
    }
    lo = wave_reduce_u32(lo, [](uint32_t a, uint32_t b) { return min(a, b); });
    hi = wave_reduce_u32(hi, [](uint32_t a, uint32_t b) { return max(a, b); });
    int need = k;
#pragma unroll 1
    for (int it = 0; it < 8; ++it) {
        if (lo == hi) break;
        const uint32_t span = hi - lo;
        const int sh = max(0, 32 - (int)__builtin_clz(span) - 8);   // span >> sh <= 255
#pragma unroll
        for (int v = 0; v < 4; ++v) scr[4 * lane + v] = 0;
        __builtin_amdgcn_wave_barrier();
        for (int gi = 0; gi < src.groups(); ++gi) {
            src.load(gi, key, use);
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (use[u] && key[u] >= lo && key[u] <= hi) atomicAdd(&scr[(key[u] - lo) >> sh], 1);
        }
        __builtin_amdgcn_wave_barrier();
        // lane L holds bins 255 - 4 L - v (descending); excl = keys in higher bins
        int hv[4], tot = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            hv[v] = scr[255 - 4 * lane - v];
            tot += hv[v];
        }
        int all_;
        int excl = wave_excl_scan(tot, all_);
        int fbin = -1, fabove = 0, fcnt = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (excl < need && excl + hv[v] >= need) {
                fbin = 255 - 4 * lane - v;
                fabove = excl;
                fcnt = hv[v];
            }
            excl += hv[v];
        }
        const uint64_t fm = __builtin_amdgcn_ballot_w64(fbin >= 0);
        const int fsrc = (int)__builtin_ctzll(fm);
        const int bin = __builtin_amdgcn_readlane(fbin, fsrc);
        const int bcnt = __builtin_amdgcn_readlane(fcnt, fsrc);
        need -= __builtin_amdgcn_readlane(fabove, fsrc);
        const uint32_t nlo = lo + ((uint32_t)bin << sh);
        const unsigned long long top = (unsigned long long)nlo + ((1ull << sh) - 1ull);
        hi = top < (unsigned long long)hi ? (uint32_t)top : hi;
        lo = nlo;
        __builtin_amdgcn_wave_barrier();
        if (bcnt <= 64) {
            // the bin's keys into cand, then their pairwise ranks
            int mine = 0;
            for (int gi = 0; gi < src.groups(); ++gi) {
                src.load(gi, key, use);
#pragma unroll
                for (int u = 0; u < 16; ++u) mine += use[u] && key[u] >= lo && key[u] <= hi;
            }
            int tot2;
            int off = wave_excl_scan(mine, tot2);
            for (int gi = 0; gi < src.groups(); ++gi) {
                src.load(gi, key, use);
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (use[u] && key[u] >= lo && key[u] <= hi) cand[off++] = key[u];
            }
            __builtin_amdgcn_wave_barrier();
            const uint32_t xl = lane < bcnt ? cand[lane] : 0u;
            int gt = 0, eq = 0;
            for (int j = 0; j < bcnt; ++j) {
                const uint32_t xj = (uint32_t)__builtin_amdgcn_readlane((int)xl, j);
                gt += xj > xl;
                eq += xj == xl;
            }
            const bool hit = lane < bcnt && gt < need && need <= gt + eq;
            const uint64_t hm = __builtin_amdgcn_ballot_w64(hit);
            const int hs = (int)__builtin_ctzll(hm);
            need_eq = need - __builtin_amdgcn_readlane(gt, hs);
            const uint32_t tau = (uint32_t)__builtin_amdgcn_readlane((int)xl, hs);
            __builtin_amdgcn_wave_barrier();
            return tau;
        }
    }
    need_eq = need;
    return lo;
}

// Entry j of a list, 16 per lane per group of 1,024: idx = 1024 gi + 64 u + lane.
struct ListKeys {          // the score patterns of entries 0 .. c - 1
    const u32x2 *e;
    int c;
    __device__ int groups() const { return (c + 1023) >> 10; }
    __device__ void load(int gi, uint32_t (&key)[16], bool (&use)[16]) const
    {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int idx = 1024 * gi + 64 * u + lane;
            use[u] = idx < c;
            key[u] = use[u] ? e[idx].x : 0u;
        }
    }
};
struct TieBlocks {         // the complemented blocks of the entries scoring exactly tau
    const u32x2 *e;
    int c;
    uint32_t tau;
    __device__ int groups() const { return (c + 1023) >> 10; }
    __device__ void load(int gi, uint32_t (&key)[16], bool (&use)[16]) const
    {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int idx = 1024 * gi + 64 * u + lane;
            const u32x2 v = idx < c ? e[idx] : u32x2{0u, 0u};
            use[u] = idx < c && v.x == tau;
            key[u] = ~v.y;
        }
    }
};

// One wave trims a query's candidate list e[0 .. c) (entries {score bit pattern, block}, in
// no particular order) to its K best in the order (score descending, block ascending) and
// returns the bit pattern tau of the K-th best score.  Scores are sums of ReLUs (never -0), so
// their bit patterns order like the values.  Of the entries scoring exactly tau, the need_eq
// with the lowest blocks are kept (a second selection, on the complemented block index, when
// more than need_eq tie).  The kept entries are packed group by group: a group's entries land
// below the next group's, which is read before anything is written over it.
__device__ __forceinline__ uint32_t trim_list(u32x2 *e, int c, int K, int *scr, uint32_t *cand)
{
    const int lane = threadIdx.x & 63;
    int need_eq;
    const uint32_t tau = kth_largest(ListKeys{e, c}, K, scr, cand, need_eq);
    const int ngroups = (c + 1023) >> 10;
    int neq = 0;
    for (int gi = 0; gi < ngroups; ++gi)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int idx = 1024 * gi + 64 * u + lane;
            neq += idx < c && e[idx].x == tau;
        }
    int tot_eq;
    wave_excl_scan(neq, tot_eq);
    uint32_t bmax = 0xffffffffu;          // tau entries kept: block <= bmax
    if (tot_eq > need_eq) {
        int dummy;
        bmax = ~kth_largest(TieBlocks{e, c, tau}, need_eq, scr, cand, dummy);
    }
    int out = 0;
    for (int gi = 0; gi < ngroups; ++gi) {
        u32x2 v[16];
        bool keep[16];
        int mine = 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int idx = 1024 * gi + 64 * u + lane;
            v[u] = idx < c ? e[idx] : u32x2{0u, 0u};
            keep[u] = idx < c && (v[u].x > tau || (v[u].x == tau && v[u].y <= bmax));
            mine += keep[u];
        }
        int tot;
        int off = out + wave_excl_scan(mine, tot);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (keep[u]) e[off++] = v[u];
        __builtin_amdgcn_wave_barrier();
        out += tot;
    }
    return tau;
}

// The blocks of a query's final list (at most K, R per lane, any order) in ascending order
// into out[0 .. c): the rank of a block is the number of listed blocks below it, counted on a
// bitmap of the visible blocks (bm: NW words, 32 NW blocks at a time) with per-word prefix
// counts (pre: NW words).
template <int R, int NW>
__device__ __forceinline__ void sort_blocks(const u32x2 *e, int c, int nvis, uint32_t *out,
                                            uint32_t *bm, uint32_t *pre)
{
    const int lane = threadIdx.x & 63;
    uint32_t blk[R];
#pragma unroll
    for (int u = 0; u < R; ++u) blk[u] = 64 * u + lane < c ? e[64 * u + lane].y : 0xffffffffu;
    __builtin_amdgcn_wave_barrier();
    int base = 0;                               // listed blocks below the current window
    for (int w0 = 0; w0 < nvis; w0 += 32 * NW) {
        for (int i = lane; i < NW; i += 64) bm[i] = 0u;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const uint32_t d = blk[u] - (uint32_t)w0;
            if (d < 32u * NW) atomicOr(&bm[d >> 5], 1u << (d & 31));
        }
        __builtin_amdgcn_wave_barrier();
        // lane L owns words NW/64 L .. NW/64 (L + 1) - 1
        constexpr int PW = NW / 64;
        int s = 0;
        uint32_t wv[PW];
#pragma unroll
        for (int v = 0; v < PW; ++v) {
            wv[v] = bm[PW * lane + v];
            s += __builtin_popcount(wv[v]);
        }
        int tot;
        int run = base + wave_excl_scan(s, tot);
#pragma unroll
        for (int v = 0; v < PW; ++v) {
            pre[PW * lane + v] = (uint32_t)run;
            run += __builtin_popcount(wv[v]);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const uint32_t d = blk[u] - (uint32_t)w0;
            if (d < 32u * NW) {
                const uint32_t word = bm[d >> 5];
                out[pre[d >> 5] + __builtin_popcount(word & ((1u << (d & 31)) - 1u))] = blk[u];
            }
        }
        __builtin_amdgcn_wave_barrier();
        base += tot;
    }
}

constexpr int kSelWaves = 8;                    // waves of a selection workgroup
constexpr int kStepBlocks = 256;                // blocks per step: 8 waves x 2 tiles of 16
constexpr int kSelTiles = kStepBlocks / 16 / kSelWaves;
constexpr int kSelEntries = 16384;              // candidate entries of a workgroup (128 KiB)
constexpr int kSelMaxBudget = kSelEntries / 4 / 2;   // 2,048 blocks with 4 queries
constexpr int kBins = 1024;                     // score histogram: bins of 1/2 over [0, 512)

// Scores are sums over 4 heads of ReLU(<q, kb>) with both vectors of norm at most sqrt(128)
// (RMS-normalised, then rotated), so they lie in [0, 512] (a little above at most, by the
// bf16 rounding of the operands): bin = floor(2 score), the last bin open-ended.  Monotone
// in the score.
__device__ __forceinline__ int score_bin(float v)
{
    return min(kBins - 1, (int)(v * 2.0f));
}

// Scores and selection without a score matrix.  A workgroup takes QN queries (QN / 4 tiles of
// 16 MFMA rows: 4 tokens x 4 heads, the queries' fragments held in registers) and streams the
// blocks visible to its last query twice, in steps of 256: wave w scores blocks 64 w ..
// 64 w + 63 of each step (the next step's keys in flight meanwhile).
//   Pass 1 counts each query's scores in a histogram of kBins bins (LDS atomics); the bin
//   holding the K-th best score, b*, follows from a scan down from the top.
//   Pass 2 scores again and lists, per query, the blocks whose score falls in b* or above:
//   the K best and the rest of b*'s bin, in LDS (CAP = 16,384 / QN entries, one LDS atomic
//   per query and tile reserving their places).  Where a histogram says that a list could
//   outgrow CAP (a crowded bin), the pass also syncs after every step and trims a list that
//   could overflow in the next one (more than CAP - 256 entries) to its K best (trim_list);
//   blocks are then taken only when they also beat the K-th best so far, tau (a block of a
//   later step that only ties it ranks below the K entries that hold it).
// Finally every list longer than K is trimmed to its K best, sorted by block and written out.
// Query tiles run last-first: the longest rows start first.
template <int QN>
__global__ __launch_bounds__(64 * kSelWaves) void qsa_select_kernel(QsaArgs a)
{
    constexpr int AT = QN / 4;
    constexpr int CAP = kSelEntries / QN;
    constexpr int RK = CAP / 128;                // final entries per lane (K <= CAP / 2)
    static_assert(QN * kBins * 4 <= kSelEntries * 8, "histograms share the lists' LDS");
    __shared__ __align__(16) u32x2 list[QN * CAP];
    __shared__ int cnt_s[QN];                    // list lengths (append counters)
    __shared__ int bmin_s[QN];                   // b*: the lowest bin a block may come from
    __shared__ float thr_s[QN];
    __shared__ int crowded_s;
    __shared__ int scr[kSelWaves][256];
    __shared__ uint32_t cand[kSelWaves][64];
    int *hist = (int *)list;                     // pass 1: [QN][kBins]
    const long long nb = a.n / kQR;
    const long long qtiles = (a.n + QN - 1) / QN;
    const long long i0 = (qtiles - 1 - (long long)blockIdx.x) * QN;
    const long long ilast = i0 + QN - 1 < a.n - 1 ? i0 + QN - 1 : a.n - 1;
    const int nvis = (int)((ilast + 1) / kQR < nb ? (ilast + 1) / kQR : nb);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int KB = a.kb;
    const bool all = nvis <= KB;                 // every query takes all its blocks
    if (!all) {
        for (int i = threadIdx.x; i < QN * kBins; i += 64 * kSelWaves) hist[i] = 0;
        if (threadIdx.x < QN) {
            cnt_s[threadIdx.x] = 0;
            thr_s[threadIdx.x] = -1.f;
        }
        if (threadIdx.x == 0) crowded_s = 0;
        int nv[AT];
#pragma unroll
        for (int t = 0; t < AT; ++t) {
            const long long i = i0 + 4 * t + g;
            nv[t] = i < a.n ? (int)((i + 1) / kQR < nb ? (i + 1) / kQR : nb) : 0;
        }
        bf16x8 fa[AT][4];
#pragma unroll
        for (int t = 0; t < AT; ++t) {
            const long long qrow = i0 * kQH + 16 * t + r;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (qrow < a.n * kQH) x = *(const u32x4 *)(a.qr + qrow * kQD + 32 * kk + 8 * g);
                fa[t][kk] = __builtin_bit_cast(bf16x8, x);
            }
        }
        // blocks past the last visible one read that block's key (no lane takes them), so the
        // next step's keys are fetched unconditionally, also after the last step: no branch
        // around the loads, whose wait counts then stay exact.  The keys of a step arrive in
        // one of two register sets while the other feeds the MFMAs: a load never targets
        // registers that an issued MFMA may still have to read.
        u32x4 fbA[kSelTiles][4], fbB[kSelTiles][4];
        auto load_b = [&](int step, u32x4 (&fb)[kSelTiles][4]) {
#pragma unroll
            for (int st = 0; st < kSelTiles; ++st) {
                const int b = min(step * kStepBlocks + (wave * kSelTiles + st) * 16 + r, nvis - 1);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    fb[st][kk] = *(const u32x4 *)(a.kbk + (long long)b * kQD + 32 * kk + 8 * g);
            }
        };
        const int nsteps = (nvis + kStepBlocks - 1) / kStepBlocks;
        // the step's scores: visit(st, t, blk, v) for lane (r, g) of tile t: query 4 t + g
        // (heads in acc[st][t][0..3]), block blk.  v is exact up to the sign of a zero.
        auto scores = [&](int s, u32x4 (&fb)[kSelTiles][4], u32x4 (&fn)[kSelTiles][4],
                          auto &&visit) {
            load_b(s + 1, fn);
            // the loads stay ahead of this step's MFMAs (into the other register set)
            __builtin_amdgcn_sched_barrier(0);
            f32x4 acc[kSelTiles][AT];
#pragma unroll
            for (int st = 0; st < kSelTiles; ++st)
#pragma unroll
                for (int t = 0; t < AT; ++t) acc[st][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int st = 0; st < kSelTiles; ++st) {
                    const bf16x8 b8 = __builtin_bit_cast(bf16x8, fb[st][kk]);
#pragma unroll
                    for (int t = 0; t < AT; ++t)
                        acc[st][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[t][kk], b8, acc[st][t], 0, 0, 0);
                }
#pragma unroll
            for (int st = 0; st < kSelTiles; ++st) {
                const int blk = s * kStepBlocks + (wave * kSelTiles + st) * 16 + r;
#pragma unroll
                for (int t = 0; t < AT; ++t) {
                    const f32x4 c4 = acc[st][t];
                    const float v = __builtin_amdgcn_fmed3f(c4[0], 0.f, 3.0e38f) +
                                    __builtin_amdgcn_fmed3f(c4[1], 0.f, 3.0e38f) +
                                    __builtin_amdgcn_fmed3f(c4[2], 0.f, 3.0e38f) +
                                    __builtin_amdgcn_fmed3f(c4[3], 0.f, 3.0e38f);
                    visit(st, t, blk, v);
                }
            }
        };
        // ---- pass 1: histograms
        load_b(0, fbA);
        __syncthreads();
        auto count = [&](int, int t, int blk, float v) {
            if (blk < nv[t]) atomicAdd(&hist[(4 * t + g) * kBins + score_bin(v)], 1);
        };
        int s1 = 0;
#pragma unroll 1
        for (; s1 + 1 < nsteps; s1 += 2) {
            scores(s1, fbA, fbB, count);
            scores(s1 + 1, fbB, fbA, count);
        }
        if (s1 < nsteps) scores(s1, fbA, fbB, count);
        load_b(0, fbA);
        __syncthreads();
        // b* per query (its owner wave): lane L holds bins kBins - 1 - 16 L - v, descending
        for (int q = wave; q < QN; q += kSelWaves) {
            int hv[16], tot = 0;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                hv[v] = hist[q * kBins + kBins - 1 - 16 * lane - v];
                tot += hv[v];
            }
            int all_;
            int excl = wave_excl_scan(tot, all_);
            int fb_ = -1, fabove = 0, fcnt = 0;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if (excl < KB && excl + hv[v] >= KB) {
                    fb_ = kBins - 1 - 16 * lane - v;
                    fabove = excl;
                    fcnt = hv[v];
                }
                excl += hv[v];
            }
            const uint64_t fm = __builtin_amdgcn_ballot_w64(fb_ >= 0);
            int bstar = 0, pred = all_;                 // fewer than K blocks: all of them
            if (fm != 0) {
                const int fs = (int)__builtin_ctzll(fm);
                bstar = __builtin_amdgcn_readlane(fb_, fs);
                pred = __builtin_amdgcn_readlane(fabove, fs) + __builtin_amdgcn_readlane(fcnt, fs);
            }
            if (lane == 0) {
                bmin_s[q] = bstar;
                if (pred > CAP - kStepBlocks) crowded_s = 1;
            }
        }
        __syncthreads();
        int bmin[AT];
        float thr[AT];
#pragma unroll
        for (int t = 0; t < AT; ++t) {
            bmin[t] = bmin_s[4 * t + g];
            thr[t] = -1.f;
        }
        const bool crowded = crowded_s != 0;
        __syncthreads();                          // the histograms are read: lists may start
        // ---- pass 2: lists
        auto collect = [&](int, int t, int blk, float v) {
            const bool take = blk < nv[t] && score_bin(v) >= bmin[t] && v > thr[t];
            const uint64_t m = __builtin_amdgcn_ballot_w64(take);
            if (m == 0) return;                       // the common case: one scalar branch
            const uint32_t bits = group_bits(m, g);
            if (bits != 0u) {
                // the group's lowest taking lane reserves the places
                const int lead = __builtin_ctz(bits);
                int base = 0;
                if (r == lead) base = atomicAdd(&cnt_s[4 * t + g], __builtin_popcount(bits));
                base = __shfl(base, 16 * g + lead, kWave);
                // + 0: a zero score's bit pattern is +0 (patterns must order like values)
                if (take)
                    list[(4 * t + g) * CAP + base + __builtin_popcount(bits & ((1u << r) - 1u))] =
                        u32x2{__float_as_uint(v + 0.f), (uint32_t)blk};
            }
        };
        auto sync_trim = [&]() {
            __syncthreads();
            // lane q < QN holds list q's length, the same in every wave: no wave appends or
            // trims before all have read them
            const int cl = lane < QN ? cnt_s[lane] : 0;
            const uint64_t over = __builtin_amdgcn_ballot_w64(cl > CAP - kStepBlocks);
            __syncthreads();
            if (over != 0) {
                for (int q = wave; q < QN; q += kSelWaves) {
                    const int cq = __builtin_amdgcn_readlane(cl, q);
                    if (cq > CAP - kStepBlocks) {
                        const uint32_t tau = trim_list(list + q * CAP, cq, KB, scr[wave], cand[wave]);
                        if (lane == 0) {
                            thr_s[q] = __uint_as_float(tau);
                            cnt_s[q] = KB;
                        }
                    }
                }
                __syncthreads();
#pragma unroll
                for (int t = 0; t < AT; ++t) thr[t] = thr_s[4 * t + g];
            }
        };
        int s2 = 0;
#pragma unroll 1
        for (; s2 + 1 < nsteps; s2 += 2) {
            scores(s2, fbA, fbB, collect);
            if (crowded) sync_trim();
            scores(s2 + 1, fbB, fbA, collect);
            if (crowded) sync_trim();
        }
        if (s2 < nsteps) {
            scores(s2, fbA, fbB, collect);
            if (crowded) sync_trim();
        }
        __syncthreads();
    }
    // output: query q by wave q % 4; the selected blocks ascending with their tokens, then the
    // tail of the incomplete block and -1 padding
    const int W = KB * kQR + kQR - 1;
    for (int q = wave; q < QN; q += kSelWaves) {
        const long long i = i0 + q;
        if (i >= a.n) break;
        const int nvq = (int)((i + 1) / kQR < nb ? (i + 1) / kQR : nb);
        int nsel = nvq;
        uint32_t *sorted = (uint32_t *)(list + q * CAP);        // first CAP / 2 words
        if (!all) {
            const int cq = __builtin_amdgcn_readfirstlane(cnt_s[q]);
            if (cq > KB) trim_list(list + q * CAP, cq, KB, scr[wave], cand[wave]);
            nsel = cq < KB ? cq : KB;
            // the bitmap and prefix counts take the second and third quarter words of the
            // list, the sorted blocks the first (the entries are in registers meanwhile)
            sort_blocks<RK, CAP / 2>(list + q * CAP, nsel, nvq, sorted, sorted + CAP / 2,
                                     sorted + CAP);
        }
        if (a.blocks) {
            int32_t *blk = a.blocks + i * KB;
            for (int p = lane; p < KB; p += kWave)
                blk[p] = p < nsel ? (all ? p : (int32_t)sorted[p]) : -1;
        }
        if (a.tokens) {
            int32_t *tok = a.tokens + i * W;
            const long long tail0 = ((i + 1) / kQR) * kQR;
            const int ntail = (int)(i + 1 - tail0);
            for (int p = lane; p < W; p += kWave) {
                const int u = p >> 2;
                int32_t v;
                if (u < nsel) {
                    v = kQR * (all ? u : (int32_t)sorted[u]) + (p & 3);
                } else {
                    const int o = p - kQR * nsel;
                    v = o < ntail ? (int32_t)(tail0 + o) : -1;
                }
                tok[p] = v;
            }
        }
    }
}

}  // namespace

size_t qsa_workspace_bytes(long long n)
{
    const long long nb = n / kQR;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al((size_t)n * kQH * kQD * 2) + al((size_t)(nb > 0 ? nb : 1) * kQD * 2);
}

long long qsa_max_tokens() { return 1LL << 20; }

bool qsa_budget_supported(long long n, int block_budget)
{
    return block_budget <= kSelMaxBudget || n / kQR <= block_budget;
}

hipError_t launch_qsa(const QsaProblem &p, void *workspace, hipStream_t stream)
{
    const long long nb = p.n / kQR;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    QsaArgs a;
    a.q = p.q;
    a.k = p.k;
    a.n = p.n;
    a.kb = p.block_budget;
    unsigned char *ws = (unsigned char *)workspace;
    a.qr = (uint16_t *)ws;
    a.kbk = (uint16_t *)(ws + al((size_t)p.n * kQH * kQD * 2));
    a.blocks = p.blocks;
    a.tokens = p.tokens;
    const long long waves = p.n * kQH + nb;
    const unsigned prep_blocks = (unsigned)((waves + 3) / 4);
    if (p.dtype == kDtypeBF16)
        hipLaunchKernelGGL(qsa_prep_kernel<uint16_t>, dim3(prep_blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(qsa_prep_kernel<float>, dim3(prep_blocks), dim3(256), 0, stream, a);
    // lists of 2 x budget entries at least: 16 queries per workgroup up to a budget of 512,
    // 8 up to 1,024, 4 up to 2,048 (a larger budget only where it covers every row)
    const int kb = p.block_budget;
    if (kb <= kSelEntries / 16 / 2 || nb <= kb)
        hipLaunchKernelGGL(qsa_select_kernel<16>, dim3((unsigned)((p.n + 15) / 16)),
                           dim3(64 * kSelWaves), 0, stream, a);
    else if (kb <= kSelEntries / 8 / 2)
        hipLaunchKernelGGL(qsa_select_kernel<8>, dim3((unsigned)((p.n + 7) / 8)),
                           dim3(64 * kSelWaves), 0, stream, a);
    else
        hipLaunchKernelGGL(qsa_select_kernel<4>, dim3((unsigned)((p.n + 3) / 4)),
                           dim3(64 * kSelWaves), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gdn
