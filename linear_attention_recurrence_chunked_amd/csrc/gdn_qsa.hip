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
//   qsa_score_kernel  16 queries x 64 blocks per workgroup on 16x16x32 bf16 MFMAs: the four
//                     heads of a query are four consecutive accumulator rows, i.e. the four
//                     values one lane holds, so the ReLU head-sum needs no exchange; tiles
//                     entirely after their queries' causal limit are skipped.
//   qsa_topk_kernel   one workgroup per query: the row's scores in LDS, a radix select of
//                     the K_B-th largest in three passes of 11, 11 and 10 bits (scores are
//                     sums of ReLUs, so their bit patterns order like the values; 11-bit
//                     first digits keep scores of one magnitude from crowding a few bins;
//                     the digit holding the rank is found over a scan of the histogram),
//                     ties at the threshold taken in index order, then the ascending block
//                     list and the expanded token list.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kQH = 4;          // query heads
constexpr int kQD = 128;        // head dimension
constexpr int kQR = 4;          // tokens per key block
constexpr float kQEps = 1e-6f;
constexpr int kLQ = kQD + 8;    // bf16 LDS row stride

struct QsaArgs {
    const void *q, *k;
    long long n;
    int kb;                     // block budget
    uint16_t *qr;               // [n, 4, 128] bf16
    uint16_t *kbk;              // [nb, 128] bf16
    float *scores;              // [n, nb]
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

// 16 queries (64 rows of qr) x 64 blocks; wave w takes blocks 16 w .. 16 w + 15.
__global__ __launch_bounds__(256) void qsa_score_kernel(QsaArgs a)
{
    __shared__ __align__(16) uint16_t sA[64 * kLQ];
    __shared__ __align__(16) uint16_t sB[64 * kLQ];
    const long long nb = a.n / kQR;
    const long long btiles = (nb + 63) / 64;
    const long long qt = blockIdx.x / btiles, bt = blockIdx.x % btiles;
    const long long i0 = qt * 16, b0 = bt * 64;
    // the tile's earliest block must be complete before its last query
    if (b0 * kQR + kQR - 1 > i0 + 15) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int p = tid; p < 64 * kQD / 8; p += 256) {
        const int r = p / (kQD / 8), c = 8 * (p % (kQD / 8));
        u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
        if (i0 * kQH + r < a.n * kQH) xa = *(const u32x4 *)(a.qr + (i0 * kQH + r) * kQD + c);
        if (b0 + r < nb) xb = *(const u32x4 *)(a.kbk + (b0 + r) * kQD + c);
        *(u32x4 *)(sA + r * kLQ + c) = xa;
        *(u32x4 *)(sB + r * kLQ + c) = xb;
    }
    __syncthreads();
    const int r = lane & 15, g = lane >> 4;
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < kQD; k0 += 32) {
        const bf16x8 fb = *(const bf16x8 *)(sB + (16 * wave + r) * kLQ + k0 + 8 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8 fa = *(const bf16x8 *)(sA + (16 * t + r) * kLQ + k0 + 8 * g);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc[t], 0, 0, 0);
        }
    }
    // tile t, lane (r, g): rows 16 t + 4 g + h (query 4 t + g, head h), block column r
    const long long b = b0 + 16 * wave + r;
    if (b < nb) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const long long i = i0 + 4 * t + g;
            if (i < a.n) {
                const float sc = fmaxf(acc[t][0], 0.f) + fmaxf(acc[t][1], 0.f) +
                                 fmaxf(acc[t][2], 0.f) + fmaxf(acc[t][3], 0.f);
                a.scores[i * nb + b] = sc;
            }
        }
    }
}

// Exclusive prefix sum of one value per thread over the workgroup (256 threads).
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
    for (int w = 0; w < wave; ++w) off += tmp[w];
    __syncthreads();
    return off + v - x;
}

constexpr int kMaxRow = 16384;  // blocks per row held in LDS (n <= 65536)

__global__ __launch_bounds__(256) void qsa_topk_kernel(QsaArgs a)
{
    __shared__ uint32_t row[kMaxRow];
    __shared__ int hist[2048];
    __shared__ int tmp[8];
    __shared__ uint32_t sh_prefix, sh_need;
    const long long i = blockIdx.x;
    const long long nb = a.n / kQR;
    const int tid = threadIdx.x;
    const int nvalid = (int)((i + 1) / kQR < nb ? (i + 1) / kQR : nb);
    const int KB = a.kb;
    const int chunk = (nvalid + 255) / 256;
    const int lo = tid * chunk, hi = lo + chunk < nvalid ? lo + chunk : nvalid;

    uint32_t tau = 0;         // the K_B-th largest bit pattern (only when nvalid > KB)
    int need_eq = 0;          // elements equal to tau to take, in index order
    const bool all = nvalid <= KB;
    if (!all) {
        for (int b = tid; b < nvalid; b += 256) row[b] = __float_as_uint(a.scores[i * nb + b]);
        if (tid == 0) {
            sh_prefix = 0;
            sh_need = (uint32_t)KB;
        }
        __syncthreads();
        // three passes (bits 31..21, 20..10, 9..0): 11-bit first digits spread scores of one
        // magnitude over many bins; find the digit holding the remaining rank
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
            const int bits = pass == 2 ? 10 : 11;
            const uint32_t dmask = (1u << bits) - 1;
            const uint32_t mask = pass == 0 ? 0u : (0xffffffffu << (shift + bits));
#pragma unroll
            for (int j = 0; j < 8; ++j) hist[8 * tid + j] = 0;
            __syncthreads();
            const uint32_t pre = sh_prefix;
            for (int b = tid; b < nvalid; b += 256) {
                const uint32_t x = row[b];
                if ((x & mask) == pre) atomicAdd(&hist[(x >> shift) & dmask], 1);
            }
            __syncthreads();
            // thread t looks at digits 2047 - 8t - j (descending); gt = how many matching
            // values have a larger digit; the digit where the remaining rank falls is unique
            int c[8], tot = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                c[j] = hist[2047 - 8 * tid - j];
                tot += c[j];
            }
            const uint32_t need = sh_need;
            int gt = block_excl_scan(tot, tmp);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if ((uint32_t)gt < need && (uint32_t)(gt + c[j]) >= need) {
                    sh_prefix = pre | ((uint32_t)(2047 - 8 * tid - j) << shift);
                    sh_need = need - (uint32_t)gt;
                }
                gt += c[j];
            }
            __syncthreads();
        }
        tau = sh_prefix;
        need_eq = (int)sh_need;      // how many of the elements equal to tau are taken
    }
    // selection flags in index order: chunk per thread, prefix counts of equals and of takes
    int eq = 0;
    if (!all)
        for (int b = lo; b < hi; ++b) eq += row[b] == tau;
    const int eq_before = all ? 0 : block_excl_scan(eq, tmp);
    int take = 0;
    {
        int e = eq_before;
        for (int b = lo; b < hi; ++b) {
            bool t = all;
            if (!all) {
                const uint32_t x = row[b];
                t = x > tau || (x == tau && e < need_eq);
                e += x == tau;
            }
            take += t;
        }
    }
    const int pos0 = block_excl_scan(take, tmp);
    const int W = KB * kQR + kQR - 1;
    const int nsel = all ? nvalid : KB;
    // write the selected blocks and their tokens in ascending order
    {
        int e = eq_before, pos = pos0;
        for (int b = lo; b < hi; ++b) {
            bool t = all;
            if (!all) {
                const uint32_t x = row[b];
                t = x > tau || (x == tau && e < need_eq);
                e += x == tau;
            }
            if (t) {
                if (a.blocks) a.blocks[i * KB + pos] = b;
                if (a.tokens) {
                    int32_t *tk = a.tokens + i * W + kQR * pos;
#pragma unroll
                    for (int u = 0; u < kQR; ++u) tk[u] = kQR * b + u;
                }
                ++pos;
            }
        }
    }
    // padding, and the tail of the incomplete block after the selected tokens
    if (a.blocks)
        for (int p = nsel + tid; p < KB; p += 256) a.blocks[i * KB + p] = -1;
    if (a.tokens) {
        const long long tail0 = ((i + 1) / kQR) * kQR;
        const int ntail = (int)(i + 1 - tail0);
        for (int p = kQR * nsel + tid; p < W; p += 256) {
            const int u = p - kQR * nsel;
            a.tokens[i * W + p] = u < ntail ? (int32_t)(tail0 + u) : -1;
        }
    }
}

}  // namespace

size_t qsa_workspace_bytes(long long n)
{
    const long long nb = n / kQR;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al((size_t)n * kQH * kQD * 2) + al((size_t)(nb > 0 ? nb : 1) * kQD * 2) +
           al((size_t)n * (nb > 0 ? nb : 1) * 4);
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
    a.blocks = p.blocks;
    a.tokens = p.tokens;
    const long long waves = p.n * kQH + nb;
    const unsigned prep_blocks = (unsigned)((waves + 3) / 4);
    if (p.dtype == kDtypeBF16)
        hipLaunchKernelGGL(qsa_prep_kernel<uint16_t>, dim3(prep_blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(qsa_prep_kernel<float>, dim3(prep_blocks), dim3(256), 0, stream, a);
    if (nb > 0) {
        const long long grid = ((p.n + 15) / 16) * ((nb + 63) / 64);
        hipLaunchKernelGGL(qsa_score_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
    }
    hipLaunchKernelGGL(qsa_topk_kernel, dim3((unsigned)p.n), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gdn
