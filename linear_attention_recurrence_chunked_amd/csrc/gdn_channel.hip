// gdn_channel.hip -- channel-wise gated variants of the rule, token by token (gfx950).
//
// The reading notes mention two successors of Gated DeltaNet only in a sentence each (Kimi
// Delta Attention: a gate per feature channel; Gated DeltaNet-2: separate channel-wise erase
// and write gates).  The form implemented covers both and keeps the rule as a special case:
//
//     S~ = Diag(a_t) S,   e = (w_t .* v_t) - (b_t .* (S~^T k_t)),   S = S~ + k_t e^T,
//     y_t = S^T q_t
//
// with a_t in (0, 1]^{d_k} (decay per key channel) and b_t, w_t in [0, 1]^{d_v} (erase and
// write gates per value channel).  Uniform gates a_t = alpha_t, b_t = w_t = beta_t give the
// gated delta rule.
//
// Both kernels keep each (sequence, head) state column in fp32 registers across the whole
// sequence, split over lanes by rows; per token a lane decays its rows and forms its parts of
// S~^T k and S^T q, and the lanes of a column add their parts.
//
// channel_gated_kernel (sequences of 16 or more tokens on average): eight waves per
// (sequence, head, 32 value columns); lane (j = lane / 16, g = lane % 16) holds rows
// g d_k/16 .. of column 4 w + j, so a column's sums stay inside one 16-lane row and take four
// DPP rotations.  The workgroup stages blocks of 32 tokens (k, q and decay rows, v and the
// gates of its columns) in LDS, fetching the next block into registers while the current one
// is processed: global latency is paid once per block, with one barrier per block.
//
// channel_step_kernel (short sequences): four waves per (sequence, head, 32 columns), lane
// (g = lane / 8, j = lane % 8) holds rows g d_k/8 .. of column 8 w + j, inputs loaded
// straight from memory one token ahead, no LDS and no barriers.
//
// channel_decode_kernel (one token per sequence, the state carried in place): one streaming
// pass over the state (below).
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kGroups = 8;      // row groups per wave of the step kernel
constexpr int kCols = 8;        // value columns per wave of the step kernel
constexpr int kWgCols = 32;     // value columns per workgroup (both kernels)

struct ChanArgs {
    const void *q, *k, *v;
    const float *a, *b, *w;
    const float *s0;
    const int32_t *cu;
    int num_seqs;
    long long total_T;
    int H, dv;
    void *y;
    float *s_final;
};

// Sum over a 16-lane row, every lane receiving the total (four DPP rotations).
__device__ __forceinline__ float row_sum16(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
    return x;
}

// R consecutive elements as floats (R a multiple of 8; 16-byte aligned).
template <int R>
__device__ __forceinline__ void load_row(const float *p, float *o)
{
#pragma unroll
    for (int i = 0; i < R / 4; ++i) {
        const f32x4 x = *(const f32x4 *)(p + 4 * i);
        o[4 * i] = x[0];
        o[4 * i + 1] = x[1];
        o[4 * i + 2] = x[2];
        o[4 * i + 3] = x[3];
    }
}
template <int R>
__device__ __forceinline__ void load_row(const uint16_t *p, float *o)
{
#pragma unroll
    for (int i = 0; i < R / 8; ++i) {
        const u32x4 x = *(const u32x4 *)(p + 8 * i);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            o[8 * i + 2 * w] = __uint_as_float(x[w] << 16);
            o[8 * i + 2 * w + 1] = __uint_as_float(x[w] & 0xffff0000u);
        }
    }
}

// Sum over the eight row groups (lanes j, j + 8, ..., j + 56): the partner 8 lanes away
// within a row by a DPP rotation of the row by 8 (lane i meets lane (i + 8) mod 16 = i ^ 8),
// then across the four rows.
__device__ __forceinline__ float sum_groups(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, true));
    return row_sum4(x);
}

template <int R>
struct Tok {
    float k[R], q[R], a[R];
    float v, b, w;
};

// The job of this workgroup: (sequence, head) unit, then column tile.  Workgroups are dealt
// to the eight XCDs in turn (block b to XCD b % 8); when the grid divides evenly, the column
// tiles of a unit get block indices of one residue mod 8, so the k, q and decay rows that they
// all read are fetched into one L2 instead of four.
__device__ __forceinline__ int tile_job(int tiles)
{
    const int b = blockIdx.x, G = gridDim.x;
    return G % (8 * tiles) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
}

template <int DK, typename T>
__global__ __launch_bounds__(256) void channel_step_kernel(ChanArgs p)
{
    constexpr int R = DK / kGroups;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 3, j = lane & 7;
    const int H = p.H, dv = p.dv;
    const int tiles = dv / kWgCols;
    const int job = tile_job(tiles);
    const int tile = job % tiles;
    const int h = (job / tiles) % H;
    const int n = job / (tiles * H);
    const int col = tile * kWgCols + wave * kCols + j;
    long long t0;
    int len;
    if (p.cu) {
        t0 = p.cu[n];
        len = (int)(p.cu[n + 1] - p.cu[n]);
    } else {
        const long long per = p.total_T / p.num_seqs;
        t0 = per * n;
        len = (int)per;
    }
    const T *gq = (const T *)p.q, *gk = (const T *)p.k, *gv = (const T *)p.v;
    T *gy = (T *)p.y;

    float s[R];
    const long long sbase = (((long long)n * H + h) * DK + g * R) * dv + col;
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = p.s0 ? p.s0[sbase + (long long)i * dv] : 0.f;

    auto fetch = [&](Tok<R> &x, int t) {
        const long long row = t0 + t;
        const long long kq = (row * H + h) * DK + g * R;
        const long long vv = (row * H + h) * (long long)dv + col;
        load_row<R>(gk + kq, x.k);
        load_row<R>(gq + kq, x.q);
        load_row<R>(p.a + kq, x.a);
        x.v = Elem<T>::load(gv + vv);
        x.b = p.b[vv];
        x.w = p.w[vv];
    };
    auto step = [&](const Tok<R> &x, int t) {
        float r = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            s[i] *= x.a[i];
            r += s[i] * x.k[i];
        }
        r = sum_groups(r);
        const float e = x.w * x.v - x.b * r;
        float yo = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            s[i] += x.k[i] * e;
            yo += s[i] * x.q[i];
        }
        yo = sum_groups(yo);
        if (g == 0) Elem<T>::store(gy + ((t0 + t) * H + h) * (long long)dv + col, yo);
    };

    Tok<R> ta, tb;
    if (len > 0) fetch(ta, 0);
    for (int t = 0; t < len; t += 2) {
        if (t + 1 < len) fetch(tb, t + 1);
        step(ta, t);
        if (t + 1 < len) {
            if (t + 2 < len) fetch(ta, t + 2);
            step(tb, t + 1);
        }
    }
    if (p.s_final) {
#pragma unroll
        for (int i = 0; i < R; ++i) p.s_final[sbase + (long long)i * dv] = s[i];
    }
}

constexpr int TB = 32;          // tokens per staged block

template <int DK>
struct ChanLds {
    static constexpr int oK = 0;                          // [TB][DK] fp32 k
    static constexpr int oQ = oK + TB * DK * 4;           // [TB][DK] fp32 q
    static constexpr int oA = oQ + TB * DK * 4;           // [TB][DK] fp32 decay
    static constexpr int oV = oA + TB * DK * 4;           // [TB][32] fp32 v
    static constexpr int oB = oV + TB * kWgCols * 4;      // [TB][32] fp32 erase gate
    static constexpr int oW = oB + TB * kWgCols * 4;      // [TB][32] fp32 write gate
    static constexpr int buf = oW + TB * kWgCols * 4;
    static constexpr int total = 2 * buf;
};

// 16-byte pieces of a staged block held in registers: k and q rows (dtype), decay rows,
// then the workgroup's 32 columns of v and of the two gates.
template <int DK, typename T>
struct Stage {
    static constexpr int E = (int)sizeof(T);
    static constexpr int KP = TB * DK * E / 16;           // pieces of k (and of q)
    static constexpr int AP = TB * DK / 4;                // pieces of the decay rows
    static constexpr int VP = TB * kWgCols * E / 16;      // pieces of v
    static constexpr int GP = TB * kWgCols / 4;           // pieces of each gate
    static constexpr int N = 2 * KP + AP + VP + 2 * GP;
    static constexpr int PER = (N + 511) / 512;
    u32x4 x[PER];
};

template <int DK, typename T>
__global__ __launch_bounds__(512) void channel_gated_kernel(ChanArgs p)
{
    constexpr int R = DK / 16;
    using L = ChanLds<DK>;
    using S = Stage<DK, T>;
    constexpr int EP = 16 / S::E;                         // elements per piece (dtype)
    __shared__ __align__(16) unsigned char smem[L::total];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane & 15, j = lane >> 4;
    const int H = p.H, dv = p.dv;
    const int tiles = dv / kWgCols;
    const int job = tile_job(tiles);
    const int tile = job % tiles;
    const int h = (job / tiles) % H;
    const int n = job / (tiles * H);
    const int col0 = tile * kWgCols;
    const int cl = wave * 4 + j;                          // this lane's column in the tile
    long long t0;
    int len;
    if (p.cu) {
        t0 = p.cu[n];
        len = (int)(p.cu[n + 1] - p.cu[n]);
    } else {
        const long long per = p.total_T / p.num_seqs;
        t0 = per * n;
        len = (int)per;
    }
    const T *gq = (const T *)p.q, *gk = (const T *)p.k, *gv = (const T *)p.v;
    T *gy = (T *)p.y;

    float s[R];
    const long long sbase = (((long long)n * H + h) * DK + g * R) * dv + col0 + cl;
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = p.s0 ? p.s0[sbase + (long long)i * dv] : 0.f;

    // piece id -> (kind, token, offset); tokens past the sequence read as zero
    S st;
    auto fetch = [&](int blk) {
#pragma unroll
        for (int u = 0; u < S::PER; ++u) {
            int i = tid + 512 * u;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (i < 2 * S::KP) {
                const T *src = i < S::KP ? gk : gq;
                const int ii = i % S::KP, per = DK / EP, t = ii / per, c = ii % per;
                if (blk * TB + t < len)
                    x = *(const u32x4 *)(src + ((t0 + blk * TB + t) * H + h) * DK + c * EP);
            } else if ((i -= 2 * S::KP) < S::AP) {
                const int per = DK / 4, t = i / per, c = i % per;
                if (blk * TB + t < len)
                    x = *(const u32x4 *)(p.a + ((t0 + blk * TB + t) * H + h) * DK + c * 4);
            } else if ((i -= S::AP) < S::VP) {
                const int per = kWgCols / EP, t = i / per, c = i % per;
                if (blk * TB + t < len)
                    x = *(const u32x4 *)(gv + ((t0 + blk * TB + t) * H + h) * (long long)dv +
                                         col0 + c * EP);
            } else if ((i -= S::VP) < 2 * S::GP) {
                const float *src = i < S::GP ? p.b : p.w;
                const int ii = i % S::GP, per = kWgCols / 4, t = ii / per, c = ii % per;
                if (blk * TB + t < len)
                    x = *(const u32x4 *)(src + ((t0 + blk * TB + t) * H + h) * (long long)dv +
                                         col0 + c * 4);
            }
            st.x[u] = x;
        }
    };
    // write a piece as fp32 into LDS: dtype pieces widen to two 16-byte stores for bf16
    auto put = [&](float *dst, u32x4 x) {
        if constexpr (S::E == 2) {
            f32x4 lo, hi;
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                lo[2 * w] = __uint_as_float(x[w] << 16);
                lo[2 * w + 1] = __uint_as_float(x[w] & 0xffff0000u);
                hi[2 * w] = __uint_as_float(x[2 + w] << 16);
                hi[2 * w + 1] = __uint_as_float(x[2 + w] & 0xffff0000u);
            }
            *(f32x4 *)dst = lo;
            *(f32x4 *)(dst + 4) = hi;
        } else {
            *(u32x4 *)dst = x;
        }
    };
    auto commit = [&](int buf) {
        unsigned char *base = smem + buf * L::buf;
#pragma unroll
        for (int u = 0; u < S::PER; ++u) {
            int i = tid + 512 * u;
            const u32x4 x = st.x[u];
            if (i < 2 * S::KP) {
                float *dst = (float *)(base + (i < S::KP ? L::oK : L::oQ));
                const int ii = i % S::KP, per = DK / EP, t = ii / per, c = ii % per;
                put(dst + t * DK + c * EP, x);
            } else if ((i -= 2 * S::KP) < S::AP) {
                const int per = DK / 4, t = i / per, c = i % per;
                *(u32x4 *)((float *)(base + L::oA) + t * DK + c * 4) = x;
            } else if ((i -= S::AP) < S::VP) {
                const int per = kWgCols / EP, t = i / per, c = i % per;
                put((float *)(base + L::oV) + t * kWgCols + c * EP, x);
            } else if ((i -= S::VP) < 2 * S::GP) {
                float *dst = (float *)(base + (i < S::GP ? L::oB : L::oW));
                const int ii = i % S::GP, per = kWgCols / 4, t = ii / per, c = ii % per;
                *(u32x4 *)(dst + t * kWgCols + c * 4) = x;
            }
        }
    };

    const int nblk = (len + TB - 1) / TB;
    if (nblk > 0) {
        fetch(0);
        commit(0);
    }
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
        if (blk + 1 < nblk) fetch(blk + 1);
        const unsigned char *base = smem + (blk & 1) * L::buf;
        const float *sk = (const float *)(base + L::oK), *sq = (const float *)(base + L::oQ);
        const float *sa = (const float *)(base + L::oA), *sv = (const float *)(base + L::oV);
        const float *sb = (const float *)(base + L::oB), *sw = (const float *)(base + L::oW);
        const int nt = len - blk * TB < TB ? len - blk * TB : TB;
#pragma unroll 2
        for (int t = 0; t < nt; ++t) {
            float kr[R], qr[R], ar[R];
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const f32x4 k4 = *(const f32x4 *)(sk + t * DK + g * R + i);
                const f32x4 q4 = *(const f32x4 *)(sq + t * DK + g * R + i);
                const f32x4 a4 = *(const f32x4 *)(sa + t * DK + g * R + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kr[i + e] = k4[e];
                    qr[i + e] = q4[e];
                    ar[i + e] = a4[e];
                }
            }
            const float vv = sv[t * kWgCols + cl], bb = sb[t * kWgCols + cl];
            const float ww = sw[t * kWgCols + cl];
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int i = 0; i < R; i += 2) {
                s[i] *= ar[i];
                s[i + 1] *= ar[i + 1];
                r0 += s[i] * kr[i];
                r1 += s[i + 1] * kr[i + 1];
            }
            const float r = row_sum16(r0 + r1);
            const float e = ww * vv - bb * r;
            float y0 = 0.f, y1 = 0.f;
#pragma unroll
            for (int i = 0; i < R; i += 2) {
                s[i] += kr[i] * e;
                s[i + 1] += kr[i + 1] * e;
                y0 += s[i] * qr[i];
                y1 += s[i + 1] * qr[i + 1];
            }
            const float yo = row_sum16(y0 + y1);
            if (g == 0)
                Elem<T>::store(gy + ((t0 + blk * TB + t) * H + h) * (long long)dv + col0 + cl, yo);
        }
        if (blk + 1 < nblk) commit((blk + 1) & 1);
        __syncthreads();
    }
    if (p.s_final) {
#pragma unroll
        for (int i = 0; i < R; ++i) p.s_final[sbase + (long long)i * dv] = s[i];
    }
}

// channel_decode_kernel: every sequence has exactly one token (a decode step).  One pass over
// the state: with the decay folded into the key and the query,
//     r = S^T (a .* k),  s = S^T (a .* q),  e = w .* v - b .* r,
//     y = s + (k . q) e,  S <- Diag(a) S + k e^T,
// each workgroup streams a 64-column slice of one head's state once in and once out with
// 16-byte non-temporal accesses (lane: 4 columns, 16 row groups), reducing over the key
// dimension with shuffles and a small LDS exchange.
template <int DK, int DV, typename T>
__global__ __launch_bounds__(256) void channel_decode_kernel(ChanArgs p)
{
    constexpr int NCT = DV / 64;
    constexpr int RPT = DK / 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid & 15, rg = tid >> 4;
    const int slice = blockIdx.x % NCT;
    const long long bh = blockIdx.x / NCT;
    const int col = slice * 64 + cg * 4;
    const T *gq = (const T *)p.q, *gk = (const T *)p.k, *gv = (const T *)p.v;
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = p.s0 ? __builtin_nontemporal_load(
                          (const f32x4 *)(p.s0 + (bh * DK + rg + 16 * i) * DV + col))
                    : f32x4{0.f, 0.f, 0.f, 0.f};
    float kr[RPT], ka[RPT], qa[RPT], ar[RPT];
    float pkq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const long long o = bh * DK + rg + 16 * i;
        kr[i] = Elem<T>::load(gk + o);
        const float qv = Elem<T>::load(gq + o);
        ar[i] = p.a[o];
        ka[i] = ar[i] * kr[i];
        qa[i] = ar[i] * qv;
        pkq += kr[i] * qv;
    }
    f32x4 pr = {0.f, 0.f, 0.f, 0.f}, ps = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        pr += s[i] * ka[i];
        ps += s[i] * qa[i];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        pr[c] = row_sum4(pr[c]);
        ps[c] = row_sum4(ps[c]);
    }
    pkq = row_sum4(pkq);
    __shared__ f32x4 red_r[4][16], red_s[4][16];
    __shared__ float red_kq[4];
    if (lane < 16) {
        red_r[wave][lane] = pr;
        red_s[wave][lane] = ps;
    }
    if (lane == 0) red_kq[wave] = pkq;
    __syncthreads();
    const f32x4 r = red_r[0][cg] + red_r[1][cg] + red_r[2][cg] + red_r[3][cg];
    const f32x4 sq = red_s[0][cg] + red_s[1][cg] + red_s[2][cg] + red_s[3][cg];
    const float kq = red_kq[0] + red_kq[1] + red_kq[2] + red_kq[3];
    const long long vo = bh * DV + col;
    const f32x4 e = *(const f32x4 *)(p.w + vo) * load4(gv + vo) - *(const f32x4 *)(p.b + vo) * r;
    if (rg == 0) store4((T *)p.y + vo, sq + kq * e);
    if (p.s_final) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            __builtin_nontemporal_store(ar[i] * s[i] + kr[i] * e,
                                        (f32x4 *)(p.s_final + (bh * DK + rg + 16 * i) * DV + col));
    }
}

template <typename T>
hipError_t launch_decode_kernel(const ChanArgs &p, int dk, int dv, hipStream_t stream)
{
    const unsigned grid = (unsigned)((long long)p.num_seqs * p.H * (dv / 64));
    if (dk == 128 && dv == 128)
        hipLaunchKernelGGL((channel_decode_kernel<128, 128, T>), dim3(grid), dim3(256), 0, stream, p);
    else if (dk == 128)
        hipLaunchKernelGGL((channel_decode_kernel<128, 64, T>), dim3(grid), dim3(256), 0, stream, p);
    else if (dv == 128)
        hipLaunchKernelGGL((channel_decode_kernel<64, 128, T>), dim3(grid), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((channel_decode_kernel<64, 64, T>), dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_channel_gated(const ChannelProblem &c, hipStream_t stream)
{
    ChanArgs p;
    p.q = c.q;
    p.k = c.k;
    p.v = c.v;
    p.a = c.a;
    p.b = c.b;
    p.w = c.w;
    p.s0 = c.s0;
    p.cu = c.cu;
    p.num_seqs = c.num_seqs;
    p.total_T = c.total_T;
    p.H = c.H;
    p.dv = c.dv;
    p.y = c.y;
    p.s_final = c.s_final;
    const bool bf = c.dtype == kDtypeBF16;
    if (!c.cu && c.total_T == c.num_seqs)     // one token per sequence: a decode step
        return bf ? launch_decode_kernel<uint16_t>(p, c.dk, c.dv, stream)
                  : launch_decode_kernel<float>(p, c.dk, c.dv, stream);
    const unsigned grid = (unsigned)((long long)c.num_seqs * c.H * (c.dv / kWgCols));
    // staging pays off from about one block of tokens per sequence on
    const bool staged = c.total_T >= 16LL * c.num_seqs;
    if (staged) {
        if (c.dk == 128) {
            if (bf) hipLaunchKernelGGL((channel_gated_kernel<128, uint16_t>), dim3(grid), dim3(512), 0, stream, p);
            else hipLaunchKernelGGL((channel_gated_kernel<128, float>), dim3(grid), dim3(512), 0, stream, p);
        } else {
            if (bf) hipLaunchKernelGGL((channel_gated_kernel<64, uint16_t>), dim3(grid), dim3(512), 0, stream, p);
            else hipLaunchKernelGGL((channel_gated_kernel<64, float>), dim3(grid), dim3(512), 0, stream, p);
        }
    } else {
        if (c.dk == 128) {
            if (bf) hipLaunchKernelGGL((channel_step_kernel<128, uint16_t>), dim3(grid), dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((channel_step_kernel<128, float>), dim3(grid), dim3(256), 0, stream, p);
        } else {
            if (bf) hipLaunchKernelGGL((channel_step_kernel<64, uint16_t>), dim3(grid), dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((channel_step_kernel<64, float>), dim3(grid), dim3(256), 0, stream, p);
        }
    }
    return hipGetLastError();
}

}  // namespace gdn
