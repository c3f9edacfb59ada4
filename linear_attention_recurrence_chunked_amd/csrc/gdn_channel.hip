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
// channel_gated_kernel: one wave per (sequence, head, 8 value columns), four waves per
// workgroup.  Lane (g = lane / 8, j = lane % 8) keeps rows g R .. g R + R - 1 (R = d_k / 8) of
// column j of the fp32 state in registers for the whole sequence; per token it decays its
// rows, forms its part of S~^T k and of S^T q and the wave adds the eight parts with three
// shuffles.  There are no barriers: every wave runs its own chain.  The next token's inputs
// are loaded while the current one is computed.  A decode step is a call with one token per
// sequence and the state carried in place.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int kGroups = 8;      // row groups per wave
constexpr int kCols = 8;        // value columns per wave
constexpr int kWgCols = 4 * kCols;

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

// Sum over the eight row groups (lanes j, j + 8, ..., j + 56).
__device__ __forceinline__ float sum_groups(float x)
{
    x += __shfl_xor(x, 8, kWave);
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

template <int R>
struct Tok {
    float k[R], q[R], a[R];
    float v, b, w;
};

template <int DK, typename T>
__global__ __launch_bounds__(256) void channel_gated_kernel(ChanArgs p)
{
    constexpr int R = DK / kGroups;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 3, j = lane & 7;
    const int H = p.H, dv = p.dv;
    const int tiles = dv / kWgCols;
    const int tile = blockIdx.x % tiles;
    const int h = (blockIdx.x / tiles) % H;
    const int n = blockIdx.x / (tiles * H);
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
    const unsigned grid = (unsigned)((long long)c.num_seqs * c.H * (c.dv / kWgCols));
    const bool bf = c.dtype == kDtypeBF16;
    if (c.dk == 128) {
        if (bf) hipLaunchKernelGGL((channel_gated_kernel<128, uint16_t>), dim3(grid), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((channel_gated_kernel<128, float>), dim3(grid), dim3(256), 0, stream, p);
    } else {
        if (bf) hipLaunchKernelGGL((channel_gated_kernel<64, uint16_t>), dim3(grid), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((channel_gated_kernel<64, float>), dim3(grid), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace gdn
