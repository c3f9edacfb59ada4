// gdn_layer_steps.hip -- the elementwise steps either side of the gated delta rule (gfx950).
//
// The jianyuh.github.io reading notes on Qwen3.8-Next (section 2.1 "Gated DeltaNet",
// "Feature parameterization", "Gating dynamics" and the output equation after them) put
// three steps around the recurrence:
//   features  q, k = L2Norm(SiLU(ShortConv(.))),  v = SiLU(ShortConv(.))   (per head)
//   gates     beta = sigmoid(b),  alpha = exp(-exp(A) softplus(a + b_alpha))
//   output    o = sigmoid(z) (.) RMSNorm(y), the RMSNorm scale stored as an offset from one
// All three stream their operands once and are HBM-bound, so each kernel is laid out for
// coalesced rows: one wave owns 128 consecutive channels (two per lane) of a row.
//
// Short convolution: out[t, c] = sum_j w[c, j] x[t - (W-1) + j, c] over the tokens of t's
// own sequence, the W-1 inputs before a sequence's first token coming from a carried state
// [N, C, W-1] (oldest first) or zero.  A wave takes 16 consecutive tokens of its 128 channels
// and keeps the 16 + W - 1 input rows it needs in registers.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

constexpr int kLsThreads = 256;
constexpr int kConvTokens = 16;            // tokens per wave
constexpr float kLsEps = 1e-6f;

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

template <typename T> struct Pair;
template <> struct Pair<float> {
    static __device__ __forceinline__ f32x2 load(const float *p) { return *(const f32x2 *)p; }
    static __device__ __forceinline__ void store(float *p, f32x2 x) { *(f32x2 *)p = x; }
};
template <> struct Pair<uint16_t> {
    static __device__ __forceinline__ f32x2 load(const uint16_t *p) {
        const uint32_t w = *(const uint32_t *)p;
        return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
    }
    static __device__ __forceinline__ void store(uint16_t *p, f32x2 x) {
        *(bf16x2 *)p = __builtin_convertvector(x, bf16x2);
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

// Sum over lanes of one head: 64 lanes (128 channels) or each 32-lane half (64 channels).
template <int HD>
__device__ __forceinline__ float head_sum(float x)
{
    x += __shfl_xor(x, 1, kWave);
    x += __shfl_xor(x, 2, kWave);
    x += __shfl_xor(x, 4, kWave);
    x += __shfl_xor(x, 8, kWave);
    x += __shfl_xor(x, 16, kWave);
    if constexpr (HD == 128) x += __shfl_xor(x, 32, kWave);
    return x;
}

// HD: 0 (no normalisation), 64 or 128 channels per head.
template <typename T, int W, int HD>
__global__ __launch_bounds__(kLsThreads) void short_conv_kernel(
    const T *__restrict__ x, const float *__restrict__ wgt, const int32_t *__restrict__ cu,
    int nseq, long long total_T, int C, const float *__restrict__ state_in, T *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int groups = (C + 127) / 128;
    const long long wid = (long long)blockIdx.x * (kLsThreads / 64) + (threadIdx.x >> 6);
    const long long tb = wid / groups;
    const int c = (int)(wid % groups) * 128 + 2 * lane;           // this lane's two channels
    const long long t0 = tb * kConvTokens;
    if (t0 >= total_T) return;
    const bool live = c < C;
    const long long per = cu ? 0 : total_T / nseq;
    // weights of the two channels
    f32x2 w[W];
#pragma unroll
    for (int j = 0; j < W; ++j)
        w[j] = live ? f32x2{wgt[(long long)c * W + j], wgt[(long long)(c + 1) * W + j]}
                    : f32x2{0.f, 0.f};
    // rows t0 - (W-1) .. t0 + 15 (rows outside [0, total_T) are never used)
    f32x2 r[kConvTokens + W - 1];
#pragma unroll
    for (int i = 0; i < kConvTokens + W - 1; ++i) {
        const long long t = t0 - (W - 1) + i;
        r[i] = (live && t >= 0 && t < total_T) ? Pair<T>::load(x + t * C + c) : f32x2{0.f, 0.f};
    }
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
        f32x2 acc = {0.f, 0.f};
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const long long tj = t - (W - 1) + j;
            f32x2 xv = r[i + j];
            if (tj < s_n) {                                    // before the sequence: state
                xv = f32x2{0.f, 0.f};
                if (state_in && live) {
                    const long long sidx = (W - 1) + (tj - s_n);   // index into the state row
                    const float *sp = state_in + ((long long)n * C + c) * (W - 1) + sidx;
                    xv = f32x2{sp[0], sp[W - 1]};
                }
            }
            acc += w[j] * xv;
        }
        f32x2 o = acc / (1.f + f32x2{__expf(-acc[0]), __expf(-acc[1])});   // SiLU
        if constexpr (HD > 0) {
            const float ss = head_sum<HD>(o[0] * o[0] + o[1] * o[1]);
            o *= __builtin_amdgcn_rsqf(ss + kLsEps);
        }
        if (live) Pair<T>::store(out + t * C + c, o);
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

// out = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w) over each row of DV values; one
// wave per row, rows strided over the grid.  out may be y.
template <typename T, int DV>
__global__ __launch_bounds__(kLsThreads) void output_gate_kernel(
    const T *y, const T *__restrict__ z, const float *__restrict__ w, long long rows,
    float eps, T *out)
{
    constexpr int PER = DV / 64;                                 // 1 or 2 values per lane
    const int lane = threadIdx.x & 63;
    const long long wid = (long long)blockIdx.x * (kLsThreads / 64) + (threadIdx.x >> 6);
    const long long nw = (long long)gridDim.x * (kLsThreads / 64);
    float ws[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) ws[p] = 1.f + w[PER * lane + p];
    for (long long row = wid; row < rows; row += nw) {
        const long long base = row * DV + PER * lane;
        float yv[PER], zv[PER];
        if constexpr (PER == 2) {
            const f32x2 a2 = Pair<T>::load(y + base), b2 = Pair<T>::load(z + base);
            yv[0] = a2[0]; yv[1] = a2[1]; zv[0] = b2[0]; zv[1] = b2[1];
        } else {
            yv[0] = Elem<T>::load(y + base);
            zv[0] = Elem<T>::load(z + base);
        }
        float ss = 0.f;
#pragma unroll
        for (int p = 0; p < PER; ++p) ss += yv[p] * yv[p];
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m, kWave);
        const float inv = __builtin_amdgcn_rsqf(ss / DV + eps);
        float o[PER];
#pragma unroll
        for (int p = 0; p < PER; ++p) o[p] = yv[p] * inv * ws[p] * sigmoidf_(zv[p]);
        if constexpr (PER == 2) Pair<T>::store(out + base, f32x2{o[0], o[1]});
        else Elem<T>::store(out + base, o[0]);
    }
}

// ------------------------------------------------------------------------------ launchers
template <typename T, int W>
static hipError_t launch_conv_w(const void *x, const float *w, const int32_t *cu, int nseq,
                                long long total_T, int C, int head_dim, const float *sin,
                                float *sout, void *out, hipStream_t st)
{
    const long long waves = (total_T + kConvTokens - 1) / kConvTokens * ((C + 127) / 128);
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
    // a few rows per wave: at most 2^16 workgroups of four waves
    long long blocks = (rows + 3) / 4;
    if (blocks > 65536) blocks = 65536;
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
