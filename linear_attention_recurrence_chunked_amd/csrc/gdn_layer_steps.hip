// gdn_layer_steps.hip -- the elementwise steps either side of the gated delta rule (gfx950).
//
// The jianyuh.github.io reading notes on Qwen3.8-Next (section 2.1 "Gated DeltaNet",
// "Feature parameterization", "Gating dynamics" and the output equation after them) put
// three steps around the recurrence:
//   features  q, k = L2Norm(SiLU(ShortConv(.))),  v = SiLU(ShortConv(.))   (per head)
//   gates     beta = sigmoid(b),  alpha = exp(-exp(A) softplus(a + b_alpha))
//   output    o = sigmoid(z) (.) RMSNorm(y), the RMSNorm scale stored as an offset from one
// All three stream their operands once and are HBM-bound, so each kernel moves 16 bytes per
// lane per access (eight bf16 or, in two halves, eight fp32 values) along contiguous rows.
//
// Short convolution: out[t, c] = sum_j w[c, j] x[t - (W-1) + j, c] over the tokens of t's
// own sequence, the W-1 inputs before a sequence's first token coming from a carried state
// [N, C, W-1] (oldest first) or zero.  A wave takes 8 consecutive tokens of 512 channels and
// keeps the 8 + W - 1 input rows it needs in registers.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

constexpr int kLsThreads = 256;
constexpr int kConvTokens = 8;             // tokens per wave
constexpr float kLsEps = 1e-6f;

__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// Eight consecutive elements (16 bytes of bf16, 32 of fp32) as floats, and back.
template <typename T> struct Oct;
template <> struct Oct<uint16_t> {
    typedef u32x4 raw;
    static __device__ __forceinline__ raw load(const uint16_t *p) { return *(const u32x4 *)p; }
    static __device__ __forceinline__ float get(const raw &r, int e) {
        const uint32_t w = r[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    static __device__ __forceinline__ raw zero() { return u32x4{0u, 0u, 0u, 0u}; }
    static __device__ __forceinline__ void store(uint16_t *p, const float *x) {
        *(bf16x8 *)p = bf16x8{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                              (__bf16)x[4], (__bf16)x[5], (__bf16)x[6], (__bf16)x[7]};
    }
};
template <> struct Oct<float> {
    struct raw { f32x4 lo, hi; };
    static __device__ __forceinline__ raw load(const float *p) {
        return raw{*(const f32x4 *)p, *(const f32x4 *)(p + 4)};
    }
    static __device__ __forceinline__ float get(const raw &r, int e) {
        return e < 4 ? r.lo[e] : r.hi[e - 4];
    }
    static __device__ __forceinline__ raw zero() {
        return raw{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    }
    static __device__ __forceinline__ void store(float *p, const float *x) {
        *(f32x4 *)p = f32x4{x[0], x[1], x[2], x[3]};
        *(f32x4 *)(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
};

// sequence n containing row t: the last n with cu[n] <= t (row0 of n = per * n without cu)
__device__ __forceinline__ int seq_of(const int32_t *cu, int nseq, long long per, long long t)
{
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const long long r = cu ? (long long)cu[mid] : per * mid;
        if (r <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Sum over the LPH lanes of one head (lanes LPH h .. LPH h + LPH - 1).
template <int LPH>
__device__ __forceinline__ float head_sum(float x)
{
#pragma unroll
    for (int m = 1; m < LPH; m <<= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// One wave: 8 consecutive tokens of 512 channels, eight per lane; HD = 0 (no normalisation),
// 64 or 128 channels per head (8 or 16 lanes).
template <typename T, int W, int HD>
__global__ __launch_bounds__(kLsThreads) void short_conv_kernel(
    const T *__restrict__ x, const float *__restrict__ wgt, const int32_t *__restrict__ cu,
    int nseq, long long total_T, int C, const float *__restrict__ state_in, T *__restrict__ out)
{
    using O = Oct<T>;
    const int lane = threadIdx.x & 63;
    const int groups = (C + 511) / 512;
    const long long wid = (long long)blockIdx.x * (kLsThreads / 64) + (threadIdx.x >> 6);
    const long long tb = wid / groups;
    const int c = (int)(wid % groups) * 512 + 8 * lane;           // this lane's 8 channels
    const long long t0 = tb * kConvTokens;
    if (t0 >= total_T) return;
    const bool live = c < C;
    const int cc = live ? c : 0;                                   // in-bounds for every lane
    const long long per = cu ? 0 : total_T / nseq;
    // rows t0 - (W-1) .. t0 + kConvTokens - 1, each loaded from a row clamped into
    // [0, total_T): rows outside it are never used (the token loop stops at total_T and the
    // rows before a sequence come from the carried state)
    constexpr int NR = kConvTokens + W - 1;
    float xr[NR][8];
    {
        typename O::raw r[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            long long t = t0 - (W - 1) + i;
            t = t < 0 ? 0 : (t >= total_T ? total_T - 1 : t);
            r[i] = O::load(x + t * C + cc);
        }
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[i][e] = O::get(r[i], e);
    }
    float w[8][W];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < W; ++j) w[e][j] = wgt[(long long)(cc + e) * W + j];
    int n = seq_of(cu, nseq, per, t0);
    long long s_n = cu ? (long long)cu[n] : per * n;
    long long e_n = cu ? (long long)cu[n + 1] : per * (n + 1);
#pragma unroll
    for (int i = 0; i < kConvTokens; ++i) {
        const long long t = t0 + i;
        if (t >= total_T) break;
        while (t >= e_n) {                                    // next sequence (skip empty ones)
            ++n;
            s_n = e_n;
            e_n = cu ? (long long)cu[n + 1] : per * (n + 1);
        }
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const long long tj = t - (W - 1) + j;
            if (tj >= s_n) {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += w[e][j] * xr[i + j][e];
            } else if (state_in) {                             // before the sequence: state
                const long long sidx = (W - 1) + (tj - s_n);
                const float *sp = state_in + ((long long)n * C + cc) * (W - 1) + sidx;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += w[e][j] * sp[e * (W - 1)];
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // SiLU: x sigmoid(x) with the hardware reciprocal (about 1 ulp)
            o[e] = o[e] * __builtin_amdgcn_rcpf(1.f + __expf(-o[e]));
            ss += o[e] * o[e];
        }
        if constexpr (HD > 0) {
            const float f = __builtin_amdgcn_rsqf(head_sum<HD / 8>(ss) + kLsEps);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= f;
        }
        if (live) O::store(out + t * C + c, o);
    }
}

// state_out[n][c][j] = ext(L_n - (W-1) + j), ext(i) = x[s_n + i][c] for i >= 0, else the
// incoming state state_in[n][c][(W-1) + i] (or zero).  One thread per (sequence, channel);
// it reads its own incoming state before writing, so state_out may be state_in.
template <typename T, int W>
__global__ __launch_bounds__(kLsThreads) void conv_state_kernel(
    const T *__restrict__ x, const int32_t *__restrict__ cu, int nseq, long long total_T,
    int C, const float *state_in, float *state_out)
{
    const long long idx = (long long)blockIdx.x * kLsThreads + threadIdx.x;
    if (idx >= (long long)nseq * C) return;
    const int n = (int)(idx / C), c = (int)(idx % C);
    const long long per = cu ? 0 : total_T / nseq;
    const long long s_n = cu ? (long long)cu[n] : per * n;
    const long long L = (cu ? (long long)cu[n + 1] : per * (n + 1)) - s_n;
    float v[W > 1 ? W - 1 : 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const long long i = L - (W - 1) + j;
        v[j] = i >= 0 ? Elem<T>::load(x + (s_n + i) * C + c)
                      : (state_in ? state_in[idx * (W - 1) + (W - 1) + i] : 0.f);
    }
#pragma unroll
    for (int j = 0; j < W - 1; ++j) state_out[idx * (W - 1) + j] = v[j];
}

// alpha = exp(-exp(A_h) softplus(a + b_alpha_h)), beta = sigmoid(b); one element per thread
__global__ __launch_bounds__(kLsThreads) void gates_kernel(
    const float *__restrict__ a, const float *__restrict__ b, const float *__restrict__ A,
    const float *__restrict__ b_alpha, long long n, int H, float *__restrict__ alpha,
    float *__restrict__ beta)
{
    const long long i = (long long)blockIdx.x * kLsThreads + threadIdx.x;
    if (i >= n) return;
    const int h = (int)(i % H);
    const float u = a[i] + b_alpha[h];
    const float sp = u > 20.f ? u : log1pf(__expf(u));          // softplus
    alpha[i] = __expf(-__expf(A[h]) * sp);
    beta[i] = sigmoidf_(b[i]);
}

// out = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w) over each row of DV values.  Eight
// values per lane, DV / 8 lanes per row, 64 * 8 / DV rows per wave and step; two steps in
// flight per iteration.  out may be y (each lane reads its values before it writes them).
template <typename T, int DV>
__global__ __launch_bounds__(kLsThreads) void output_gate_kernel(
    const T *y, const T *__restrict__ z, const float *__restrict__ w, long long rows,
    float eps, T *out)
{
    using O = Oct<T>;
    constexpr int LPR = DV / 8;                                  // lanes per row
    constexpr int RPW = 64 / LPR;                                // rows per wave and step
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR, col = 8 * (lane % LPR);
    const long long wid = (long long)blockIdx.x * (kLsThreads / 64) + (threadIdx.x >> 6);
    const long long nw = (long long)gridDim.x * (kLsThreads / 64);
    float ws[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ws[e] = 1.f + w[col + e];
    for (long long r0 = 2 * wid * RPW; r0 < rows; r0 += 2 * nw * RPW) {
        typename O::raw yv[2], zv[2];
        long long row[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            row[u] = r0 + u * RPW + sub;
            if (row[u] < rows) {
                yv[u] = O::load(y + row[u] * DV + col);
                zv[u] = O::load(z + row[u] * DV + col);
            } else {
                yv[u] = O::zero();
                zv[u] = O::zero();
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += O::get(yv[u], e) * O::get(yv[u], e);
            ss = head_sum<LPR>(ss);
            const float inv = __builtin_amdgcn_rsqf(ss * (1.f / DV) + eps);
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = O::get(yv[u], e) * inv * ws[e] * sigmoidf_(O::get(zv[u], e));
            if (row[u] < rows) O::store(out + row[u] * DV + col, o);
        }
    }
}

// ------------------------------------------------------------------------------ launchers
template <typename T, int W>
static hipError_t launch_conv_w(const void *x, const float *w, const int32_t *cu, int nseq,
                                long long total_T, int C, int head_dim, const float *sin,
                                float *sout, void *out, hipStream_t st)
{
    const long long waves = (total_T + kConvTokens - 1) / kConvTokens * ((C + 511) / 512);
    const long long blocks = (waves + 3) / 4;
    if (blocks > 0) {
        if (head_dim == 128)
            hipLaunchKernelGGL((short_conv_kernel<T, W, 128>), dim3((unsigned)blocks),
                               dim3(kLsThreads), 0, st, (const T *)x, w, cu, nseq, total_T, C,
                               sin, (T *)out);
        else if (head_dim == 64)
            hipLaunchKernelGGL((short_conv_kernel<T, W, 64>), dim3((unsigned)blocks),
                               dim3(kLsThreads), 0, st, (const T *)x, w, cu, nseq, total_T, C,
                               sin, (T *)out);
        else
            hipLaunchKernelGGL((short_conv_kernel<T, W, 0>), dim3((unsigned)blocks),
                               dim3(kLsThreads), 0, st, (const T *)x, w, cu, nseq, total_T, C,
                               sin, (T *)out);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (sout && W > 1) {
        const long long n = (long long)nseq * C;
        hipLaunchKernelGGL((conv_state_kernel<T, W>), dim3((unsigned)((n + kLsThreads - 1) / kLsThreads)),
                           dim3(kLsThreads), 0, st, (const T *)x, cu, nseq, total_T, C, sin,
                           sout);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T>
static hipError_t launch_conv_t(const void *x, const float *w, const int32_t *cu, int nseq,
                                long long total_T, int C, int W, int head_dim, const float *sin,
                                float *sout, void *out, hipStream_t st)
{
    switch (W) {
    case 1: return launch_conv_w<T, 1>(x, w, cu, nseq, total_T, C, head_dim, sin, sout, out, st);
    case 2: return launch_conv_w<T, 2>(x, w, cu, nseq, total_T, C, head_dim, sin, sout, out, st);
    case 3: return launch_conv_w<T, 3>(x, w, cu, nseq, total_T, C, head_dim, sin, sout, out, st);
    default: return launch_conv_w<T, 4>(x, w, cu, nseq, total_T, C, head_dim, sin, sout, out, st);
    }
}

hipError_t launch_short_conv(const void *x, const float *w, const int32_t *cu, int nseq,
                             long long total_T, int C, int W, int head_dim, int dtype,
                             const float *state_in, float *state_out, void *out,
                             hipStream_t stream)
{
    if (dtype == kDtypeBF16)
        return launch_conv_t<uint16_t>(x, w, cu, nseq, total_T, C, W, head_dim, state_in,
                                       state_out, out, stream);
    return launch_conv_t<float>(x, w, cu, nseq, total_T, C, W, head_dim, state_in, state_out,
                                out, stream);
}

hipError_t launch_gates(const float *a, const float *b, const float *A, const float *b_alpha,
                        long long total_T, int H, float *alpha, float *beta, hipStream_t stream)
{
    const long long n = total_T * H;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(gates_kernel, dim3((unsigned)((n + kLsThreads - 1) / kLsThreads)),
                       dim3(kLsThreads), 0, stream, a, b, A, b_alpha, n, H, alpha, beta);
    return hipGetLastError();
}

hipError_t launch_output_gate(const void *y, const void *z, const float *w, long long rows,
                              int dv, float eps, int dtype, void *out, hipStream_t stream)
{
    if (rows <= 0) return hipSuccess;
    // two steps of 64 * 8 / dv rows per wave and iteration; at most 8192 workgroups of four
    // waves (32 per CU), each looping over its share
    const long long per_wave = 2 * (64 * 8 / dv);
    long long blocks = (rows + 4 * per_wave - 1) / (4 * per_wave);
    if (blocks > 8192) blocks = 8192;
#define GDN_OG(T, DV)                                                                       \
    hipLaunchKernelGGL((output_gate_kernel<T, DV>), dim3((unsigned)blocks), dim3(kLsThreads), \
                       0, stream, (const T *)y, (const T *)z, w, rows, eps, (T *)out)
    if (dtype == kDtypeBF16) {
        if (dv == 128) GDN_OG(uint16_t, 128); else GDN_OG(uint16_t, 64);
    } else {
        if (dv == 128) GDN_OG(float, 128); else GDN_OG(float, 64);
    }
#undef GDN_OG
    return hipGetLastError();
}

}  // namespace gdn
