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
// Three launches:
//   qsa_prep_kernel   one wave per query row (token, head) or per key block: normalise,
//                     rotate (angles and their sines in fp64: positions reach 10^5 radians),
//                     store bf16.
//   qsa_score_kernel  16 queries per workgroup against all their visible blocks on 16x16x32
//                     bf16 MFMAs, the queries' fragments held in registers and the block
//                     keys streamed from L2 one 16-block tile ahead: the four heads of a
//                     query are four consecutive accumulator rows, i.e. the four values one
//                     lane holds, so the ReLU head-sum needs no exchange.
//   qsa_topk_kernel   one workgroup per query: the row's scores in LDS (16-byte loads, eight
//                     in flight); a 2,048-bin histogram of a digit linear in the score up to
//                     the row maximum (scores of one magnitude spread over many bins) and a
//                     scan over it find the bin holding the K_B-th largest score; the scores in
//                     that bin (a few dozen, typically) are ranked pairwise to find it exactly,
//                     or, in a crowded bin, by a radix select on 11, 11 and 10 bits of their
//                     patterns (scores are sums of ReLUs, so their bit patterns order like the
//                     values).  Ties at the threshold are taken in index order; each wave
//                     places its range's selected blocks, ascending, by a packed prefix sum of
//                     (greater, equal) counts, with their tokens, then the tail and padding.
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
    float *scores;              // [n, ld]
    long long ld;               // score row stride: nb rounded up to 4 (16-byte rows)
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

// 16 queries (64 rows of qr, token-major, head-minor) against every block visible to the
// last of them, in tiles of 16 blocks; wave w takes tiles w, w + 4, ...  The queries'
// MFMA fragments stay in registers for the whole row; the block keys (at most 4 MB, resident
// in L2) stream in one tile ahead.  Query tiles run last-first: the longest rows start first.
__global__ __launch_bounds__(256) void qsa_score_kernel(QsaArgs a)
{
    const long long nb = a.n / kQR;
    const long long qtiles = (a.n + 15) / 16;
    const long long i0 = (qtiles - 1 - (long long)blockIdx.x) * 16;
    const long long ilast = i0 + 15 < a.n - 1 ? i0 + 15 : a.n - 1;
    const long long nvis = (ilast + 1) / kQR < nb ? (ilast + 1) / kQR : nb;
    const int ntiles = (int)((nvis + 15) / 16);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    // per wave: its 16 x 16 score tile, rows 16-byte aligned, to turn four 4-byte stores per
    // lane into one 16-byte store
    __shared__ __align__(16) float sT[4][16 * 20];
    if (wave >= ntiles) return;               // no barriers below
    // A fragments: tile t holds rows 16 t .. 16 t + 15 (tokens i0 + 4 t .. i0 + 4 t + 3)
    bf16x8 fa[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const long long qrow = i0 * kQH + 16 * t + r;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow < a.n * kQH) x = *(const u32x4 *)(a.qr + qrow * kQD + 32 * kk + 8 * g);
            fa[t][kk] = __builtin_bit_cast(bf16x8, x);
        }
    }
    u32x4 fb[4], fn[4];
    auto load_b = [&](int tile, u32x4 (&f)[4]) {
        const long long b = (long long)tile * 16 + r;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            f[kk] = u32x4{0u, 0u, 0u, 0u};
            if (b < nb) f[kk] = *(const u32x4 *)(a.kbk + b * kQD + 32 * kk + 8 * g);
        }
    };
    load_b(wave, fb);
#pragma unroll 1
    for (int tile = wave; tile < ntiles; tile += 4) {
        if (tile + 4 < ntiles) load_b(tile + 4, fn);
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 b8 = __builtin_bit_cast(bf16x8, fb[kk]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[t][kk], b8, acc[t], 0, 0, 0);
        }
        // tile t, lane (r, g): rows 16 t + 4 g + h (token i0 + 4 t + g, head h), block r.
        // + 0: a sum of four -0 becomes +0 (bit patterns must order like values)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            sT[wave][(4 * t + g) * 20 + r] = fmaxf(acc[t][0], 0.f) + fmaxf(acc[t][1], 0.f) +
                                             fmaxf(acc[t][2], 0.f) + fmaxf(acc[t][3], 0.f) + 0.f;
        __builtin_amdgcn_wave_barrier();
        {
            // lane l: token i0 + l / 4, blocks 16 tile + 4 (l % 4) .. + 3 (a row's padding
            // to a multiple of 4 blocks absorbs the last group's overhang)
            const f32x4 v = *(const f32x4 *)&sT[wave][(lane >> 2) * 20 + 4 * (lane & 3)];
            const long long i = i0 + (lane >> 2);
            const long long b = (long long)tile * 16 + 4 * (lane & 3);
            if (i < a.n && b < nb) __builtin_nontemporal_store(v, (f32x4 *)(a.scores + i * a.ld + b));
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) fb[kk] = fn[kk];
    }
}

constexpr int kTK = 1024;       // threads of a top-k workgroup
constexpr int kTW = kTK / kWave;

// Exclusive prefix sum of one value per thread over a workgroup of kTK threads.
__device__ __forceinline__ int block_excl_scan(int x, int *tmp)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int v = x;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const int o = __shfl_up(v, m, kWave);
        if (lane >= m) v += o;
    }
    if (lane == 63) tmp[wave] = v;
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wave; ++w) off += tmp[w];   // wave-uniform
    __syncthreads();
    return off + v - x;
}

// blocks per row held in LDS: 16,384 (64 KiB, two workgroups per CU) up to 65,536 tokens,
// 32,768 (128 KiB, one per CU) up to 131,072
constexpr int kMaxRowSmall = 16384;
constexpr int kMaxRow = 32768;

// First radix digit of a score x >= lo: (x - lo) scaled linearly onto 2,048 bins.  Monotone
// in x (a rounded subtraction and multiply, then a floor), so ordering by (digit, bit
// pattern) orders like the scores, and scores of one magnitude spread over many bins.
__device__ __forceinline__ uint32_t lin_digit(uint32_t x, float lo, float s)
{
    const float v = (__uint_as_float(x) - lo) * s;
    return v < 2047.f ? (uint32_t)v : 2047u;
}

// number of lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

constexpr int kCand = 256;      // a threshold bin this small is resolved by pairwise ranks

// One workgroup per query, longest rows first.
//
// The K_B-th largest score tau is at least the smallest of the maxima of any K_B disjoint
// groups of the row (those maxima are K_B scores at least that large), so scores below that
// bound take no part in the search.  A block is taken when its score is above tau, or equal to
// it and not after b_last, the index of the last equal score that still fits the budget.
template <int MAXROW>
__global__ __launch_bounds__(kTK) void qsa_topk_kernel(QsaArgs a)
{
    __shared__ __align__(16) uint32_t row[MAXROW];
    __shared__ int hist[2048];
    __shared__ uint32_t cx[kCand];
    __shared__ int cb[kCand];
    __shared__ int tmp[kTW];
    __shared__ int wcount[kTW];
    __shared__ float wmax[kTW], wmin[kTW];
    __shared__ uint32_t sh_prefix, sh_need, sh_c1;
    __shared__ int sh_cnt, sh_fill, sh_blast;
    const long long i = a.n - 1 - (long long)blockIdx.x;
    const long long nb = a.n / kQR;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nvalid = (int)((i + 1) / kQR < nb ? (i + 1) / kQR : nb);
    const int KB = a.kb;
    const bool all = nvalid <= KB;            // uniform over the workgroup
    const int n4 = (nvalid + 3) >> 2;
    const u32x4 *row4 = (const u32x4 *)row;

    uint32_t tau = 0;         // the bit pattern of the K_B-th largest score (when !all)
    int b_last = -1;          // the last taken block among those scoring exactly tau
    if (!all) {
        // the row's visible scores into LDS: 16-byte loads, all of a thread's in flight
        const u32x4 *src = (const u32x4 *)(a.scores + i * a.ld);
        {
            u32x4 v[MAXROW / 4 / kTK];
#pragma unroll
            for (int u = 0; u < MAXROW / 4 / kTK; ++u) {
                const int c = u * kTK + tid;
                v[u] = u32x4{0u, 0u, 0u, 0u};
                if (c < n4) v[u] = src[c];
            }
#pragma unroll
            for (int u = 0; u < MAXROW / 4 / kTK; ++u) {
                const int c = u * kTK + tid;
                if (c < n4) *(u32x4 *)(row + 4 * c) = v[u];
            }
        }
        hist[2 * tid] = 0;
        hist[2 * tid + 1] = 0;
        if (tid == 0) {
            sh_prefix = 0;
            sh_need = (uint32_t)KB;
            sh_fill = 0;
        }
        __syncthreads();
        // group g = the blocks b = g (mod K_B), halved between threads 2g' and 2g' + 1 of a
        // pair: the row maximum and the smallest group maximum
        float mx = 0.f, mn = 3.0e38f;
        for (int g0 = 0; g0 < KB; g0 += kTK / 2) {
            const int g = g0 + (tid >> 1);
            float m = 0.f;
            if (g < KB)
                for (int b = g + (tid & 1) * KB; b < nvalid; b += 2 * KB)
                    m = fmaxf(m, __uint_as_float(row[b]));
            m = fmaxf(m, __shfl_xor(m, 1, kWave));
            if (g < KB) {
                mx = fmaxf(mx, m);
                mn = fminf(mn, m);
            }
        }
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) {
            mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
            mn = fminf(mn, __shfl_xor(mn, m, kWave));
        }
        if (lane == 0) {
            wmax[wave] = mx;
            wmin[wave] = mn;
        }
        __syncthreads();
        float lo = wmin[0];
        mx = wmax[0];
#pragma unroll
        for (int w = 1; w < kTW; ++w) {
            mx = fmaxf(mx, wmax[w]);
            lo = fminf(lo, wmin[w]);
        }
        const uint32_t lo_bits = __float_as_uint(lo);
        const float s = mx > lo ? fminf(2047.f / (mx - lo), 1e30f) : 0.f;
        // first digit over the scores >= lo
#pragma unroll 2
        for (int c = tid; c < n4; c += kTK) {
            const u32x4 x = row4[c];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * c + e < nvalid && x[e] >= lo_bits)
                    atomicAdd(&hist[lin_digit(x[e], lo, s)], 1);
        }
        __syncthreads();
        // thread t looks at digits 2047 - 2t - j (descending); gt = how many values have a
        // larger digit; the digit where the rank falls is unique
        {
            int c[2], tot = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                c[j] = hist[2047 - 2 * tid - j];
                tot += c[j];
            }
            const uint32_t need = sh_need;
            int gt = block_excl_scan(tot, tmp);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if ((uint32_t)gt < need && (uint32_t)(gt + c[j]) >= need) {
                    sh_c1 = (uint32_t)(2047 - 2 * tid - j);
                    sh_need = need - (uint32_t)gt;
                    sh_cnt = c[j];
                }
                gt += c[j];
            }
            __syncthreads();
        }
        const uint32_t c1 = sh_c1, need = sh_need;
        const int cnt = sh_cnt;
        if (cnt <= kCand) {
            // gather the bin's scores; the one whose rank among them holds `need` (the first
            // in index order among equals) is tau; then the need_eq-th equal in index order
#pragma unroll 2
            for (int c = tid; c < n4; c += kTK) {
                const u32x4 x = row4[c];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * c + e < nvalid && x[e] >= lo_bits && lin_digit(x[e], lo, s) == c1) {
                        const int slot = atomicAdd(&sh_fill, 1);
                        cx[slot] = x[e];
                        cb[slot] = 4 * c + e;
                    }
            }
            __syncthreads();
            if (tid < cnt) {
                const uint32_t xj = cx[tid];
                const int bj = cb[tid];
                int above = 0, same = 0, same_first = 1;
                for (int k = 0; k < cnt; ++k) {
                    const uint32_t xk = cx[k];
                    above += xk > xj;
                    same += xk == xj;
                    if (xk == xj && cb[k] < bj) same_first = 0;
                }
                if (same_first && (uint32_t)above < need && need <= (uint32_t)(above + same)) {
                    sh_prefix = xj;
                    sh_need = need - (uint32_t)above;
                }
            }
            __syncthreads();
            tau = sh_prefix;
            const int need_eq = (int)sh_need;
            if (tid < cnt && cx[tid] == tau) {
                const int bj = cb[tid];
                int before = 0;
                for (int k = 0; k < cnt; ++k) before += cx[k] == tau && cb[k] < bj;
                if (before == need_eq - 1) sh_blast = bj;
            }
            __syncthreads();
        } else {
            // a crowded bin (many equal scores): bits 31..21, 20..10, 9..0 of its scores
#pragma unroll 1
            for (int pass = 0; pass < 3; ++pass) {
                const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
                const int bits = pass == 2 ? 10 : 11;
                const uint32_t dmask = (1u << bits) - 1;
                const uint32_t mask = pass == 0 ? 0u : (0xffffffffu << (shift + bits));
                hist[2 * tid] = 0;
                hist[2 * tid + 1] = 0;
                __syncthreads();
                const uint32_t pre = sh_prefix;
                for (int b = tid; b < nvalid; b += kTK) {
                    const uint32_t x = row[b];
                    if (x >= lo_bits && lin_digit(x, lo, s) == c1 && (x & mask) == pre)
                        atomicAdd(&hist[(x >> shift) & dmask], 1);
                }
                __syncthreads();
                int c[2], tot = 0;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    c[j] = hist[2047 - 2 * tid - j];
                    tot += c[j];
                }
                const uint32_t nd = sh_need;
                int gt = block_excl_scan(tot, tmp);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if ((uint32_t)gt < nd && (uint32_t)(gt + c[j]) >= nd) {
                        sh_prefix = pre | ((uint32_t)(2047 - 2 * tid - j) << shift);
                        sh_need = nd - (uint32_t)gt;
                    }
                    gt += c[j];
                }
                __syncthreads();
            }
            tau = sh_prefix;
            const int need_eq = (int)sh_need;
            // the need_eq-th score equal to tau in index order: contiguous ranges per thread
            const int chunk = (nvalid + kTK - 1) / kTK;
            const int b0 = tid * chunk, b1 = b0 + chunk < nvalid ? b0 + chunk : nvalid;
            int eq = 0;
            for (int b = b0; b < b1; ++b) eq += row[b] == tau;
            int before = block_excl_scan(eq, tmp);
            if (before < need_eq && before + eq >= need_eq)
                for (int b = b0; b < b1; ++b)
                    if (row[b] == tau && ++before == need_eq) sh_blast = b;
            __syncthreads();
        }
        b_last = sh_blast;
    }

    // selection in index order: wave w takes a contiguous range of the row (a multiple of
    // 256 blocks), lane l the four blocks 4 l .. 4 l + 3 of each 256-block step; ballots of
    // the four slots place every taken block
    const int per = ((nvalid + kTW * 256 - 1) / (kTW * 256)) * 256;
    const int lo_b = wave * per, hi_b = lo_b + per < nvalid ? lo_b + per : nvalid;
    auto taken = [&](uint32_t x, int b) { return x > tau || (x == tau && b <= b_last); };
    if (!all) {
        int count = 0;
#pragma unroll 2
        for (int b0 = lo_b; b0 < hi_b; b0 += 256) {
            const int b = b0 + 4 * lane;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (b < hi_b) x = *(const u32x4 *)(row + b);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                count += __popcll(__builtin_amdgcn_ballot_w64(b + u < hi_b && taken(x[u], b + u)));
        }
        if (lane == 0) wcount[wave] = count;
    }
    __syncthreads();
    int pos = lo_b;
    if (!all) {
        pos = 0;
        for (int w = 0; w < wave; ++w) pos += wcount[w];
    }
    const int W = KB * kQR + kQR - 1;
    int32_t *blk = a.blocks ? a.blocks + i * KB : nullptr;
    int32_t *tok = a.tokens ? a.tokens + i * W : nullptr;
#pragma unroll 2
    for (int b0 = lo_b; b0 < hi_b; b0 += 256) {
        const int b = b0 + 4 * lane;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (!all && b < hi_b) x = *(const u32x4 *)(row + b);
        bool t[4];
        uint64_t m[4];
        int p = pos;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            t[u] = b + u < hi_b && (all || taken(x[u], b + u));
            m[u] = __builtin_amdgcn_ballot_w64(t[u]);
            p += lanes_below(m[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (t[u]) {
                if (blk) blk[p] = b + u;
                if (tok) {
#pragma unroll
                    for (int v = 0; v < kQR; ++v) tok[kQR * p + v] = kQR * (b + u) + v;
                }
                ++p;
            }
            pos += __popcll(m[u]);
        }
    }
    // padding, and the tail of the incomplete block after the selected tokens
    const int nsel = all ? nvalid : KB;
    if (blk)
        for (int p = nsel + tid; p < KB; p += kTK) blk[p] = -1;
    if (tok) {
        const long long tail0 = ((i + 1) / kQR) * kQR;
        const int ntail = (int)(i + 1 - tail0);
        for (int p = kQR * nsel + tid; p < W; p += kTK) {
            const int u = p - kQR * nsel;
            tok[p] = u < ntail ? (int32_t)(tail0 + u) : -1;
        }
    }
}

}  // namespace

static long long score_ld(long long nb) { return ((nb > 0 ? nb : 1) + 3) & ~3LL; }

size_t qsa_workspace_bytes(long long n)
{
    const long long nb = n / kQR;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al((size_t)n * kQH * kQD * 2) + al((size_t)(nb > 0 ? nb : 1) * kQD * 2) +
           al((size_t)n * score_ld(nb) * 4);
}

long long qsa_max_tokens() { return (long long)kMaxRow * kQR; }

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
    a.scores = (float *)(ws + al((size_t)p.n * kQH * kQD * 2) +
                         al((size_t)(nb > 0 ? nb : 1) * kQD * 2));
    a.ld = score_ld(nb);
    a.blocks = p.blocks;
    a.tokens = p.tokens;
    const long long waves = p.n * kQH + nb;
    const unsigned prep_blocks = (unsigned)((waves + 3) / 4);
    if (p.dtype == kDtypeBF16)
        hipLaunchKernelGGL(qsa_prep_kernel<uint16_t>, dim3(prep_blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(qsa_prep_kernel<float>, dim3(prep_blocks), dim3(256), 0, stream, a);
    if (nb > 0) {
        hipLaunchKernelGGL(qsa_score_kernel, dim3((unsigned)((p.n + 15) / 16)), dim3(256), 0,
                           stream, a);
    }
    if (nb <= kMaxRowSmall)
        hipLaunchKernelGGL(qsa_topk_kernel<kMaxRowSmall>, dim3((unsigned)p.n), dim3(kTK), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(qsa_topk_kernel<kMaxRow>, dim3((unsigned)p.n), dim3(kTK), 0, stream,
                           a);
    return hipGetLastError();
}

}  // namespace gdn
