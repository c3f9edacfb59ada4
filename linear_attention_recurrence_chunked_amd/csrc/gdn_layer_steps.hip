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
// [N, C, W-1] (oldest first) or zero.  A wave takes 32 consecutive tokens of 512 channels in
// steps, keeping the step's input rows and the W - 1 before them in registers and loading the
// next step's rows while it computes.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

constexpr int kLsThreads = 256;
constexpr int kConvTokens = 32;            // tokens per wave
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

// The outgoing convolution state of one (sequence n, channel c), idx = n C + c:
// state_out[n][c][j] = ext(L_n - (W-1) + j), ext(i) = x[s_n + i][c] for i >= 0, else the
// incoming state state_in[n][c][(W-1) + i] (or zero).  It reads its own incoming state before
// writing, so state_out may be state_in when nothing else reads the incoming state meanwhile.
template <typename T, int W>
__device__ __forceinline__ void conv_state_item(long long idx, const T *x, const int32_t *cu,
                                                int nseq, long long total_T, int C,
                                                const float *state_in, float *state_out)
{
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

// Sum over the LPH (8 or 16) lanes of one head with DPP moves inside a row of 16 lanes: swap
// neighbours, swap pairs, mirror each half-row (lane i <-> 7 - i), then, for 16, the row
// (i <-> 15 - i); every lane ends with the head's total.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int LPH>
__device__ __forceinline__ float head_sum_dpp(float x)
{
    x += dpp_mov<0xb1>(x);                                // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4e>(x);                                // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x141>(x);                               // row_half_mirror
    if constexpr (LPH == 16) x += dpp_mov<0x140>(x);      // row_mirror
    return x;
}

// One wave: kConvTokens consecutive tokens of 512 channels, eight per lane, in steps of S
// tokens (four); the next step's rows load while the current step computes,
// and the last W-1 rows of a step carry over as the window of the next.  HD = 0 (no
// normalisation), 64 or 128 channels per head (8 or 16 lanes).  Workgroups from conv_blocks
// on write the outgoing state instead (state_out distinct from state_in, else null).
template <typename T, int W, int HD>
__global__ __launch_bounds__(kLsThreads) void short_conv_kernel(
    const T *__restrict__ x, const float *__restrict__ wgt, const int32_t *__restrict__ cu,
    int nseq, long long total_T, int C, const float *__restrict__ state_in, T *__restrict__ out,
    long long conv_blocks, float *__restrict__ state_out)
{
    if ((long long)blockIdx.x >= conv_blocks) {
        conv_state_item<T, W>(((long long)blockIdx.x - conv_blocks) * kLsThreads + threadIdx.x,
                              x, cu, nseq, total_T, C, state_in, state_out);
        return;
    }
    using O = Oct<T>;
    constexpr int S = 4;                                           // tokens per step
    constexpr int NW = W > 1 ? W - 1 : 1;                          // window rows kept
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
    // every row is loaded from a row clamped into [0, total_T): rows outside it are never
    // used (the token loop stops at total_T and the rows before a sequence come from the
    // carried state)
    auto row_at = [&](long long t) {
        t = t < 0 ? 0 : (t >= total_T ? total_T - 1 : t);
        return O::load(x + t * C + cc);
    };
    int n = seq_of(cu, nseq, per, t0);
    long long s_n = cu ? (long long)cu[n] : per * n;
    long long e_n = cu ? (long long)cu[n + 1] : per * (n + 1);
    const int n0 = n;                                              // t0's sequence
    // window: inputs t0 - (W-1) .. t0 - 1 of t0's sequence, from x or, before the sequence's
    // first token, from the incoming state (loaded here, beside the rows, not per token)
    float win[NW][8];
    {
        typename O::raw r[NW];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) r[i] = row_at(t0 - (W - 1) + i);
        // all W-1 state slots of the lane's channels in one batch of loads (a branch per
        // element would wait for each load in turn)
        float sv[NW][8];
#pragma unroll
        for (int k = 0; k < W - 1; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[k][e] = 0.f;
        const long long lag = t0 - s_n;                        // 0 .. W-2 when slots are used
        if (state_in && lag < W - 1) {
            const float *sb = state_in + ((long long)n * C + cc) * (W - 1);
#pragma unroll
            for (int k = 0; k < W - 1; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) sv[k][e] = sb[e * (W - 1) + k];
        }
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            // row t0 - (W-1) + i lies before the sequence when i + lag < W - 1; it is then
            // state slot i + lag
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = O::get(r[i], e);
#pragma unroll
                for (int k = 0; k < W - 1; ++k)
                    if (i + lag == k) v = sv[k][e];
                win[i][e] = v;
            }
        }
    }
    typename O::raw cur[S];
#pragma unroll
    for (int i = 0; i < S; ++i) cur[i] = row_at(t0 + i);
    float w[8][W];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < W; ++j) w[e][j] = wgt[(long long)(cc + e) * W + j];
#pragma unroll 1
    for (int st = 0; st < kConvTokens / S; ++st) {
        const long long ts = t0 + (long long)st * S;
        if (ts >= total_T) break;
        typename O::raw nxt[S];
        if (st + 1 < kConvTokens / S) {
#pragma unroll
            for (int i = 0; i < S; ++i) nxt[i] = row_at(ts + S + i);
        }
        // rows ts - (W-1) .. ts + S - 1
        float xr[W - 1 + S][8];
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[i][e] = win[i][e];
#pragma unroll
        for (int i = 0; i < S; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[W - 1 + i][e] = O::get(cur[i], e);
        // the sequence of each token (tokens past total_T keep the last one; never stored)
        long long sn[S];
        int nn[S];
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const long long t = ts + i;
            while (t < total_T && t >= e_n) {                 // next sequence (skip empty ones)
                ++n;
                s_n = e_n;
                e_n = cu ? (long long)cu[n + 1] : per * (n + 1);
            }
            sn[i] = s_n;
            nn[i] = n;
        }
        // every token's convolution and SiLU, then the head sums side by side
        float o[S][8], ss[S];
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const long long t = ts + i;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
#pragma unroll
            for (int j = 0; j < W; ++j) {
                const long long tj = t - (W - 1) + j;
                // rows of t0's sequence are all in xr (the window holds its state part); a
                // sequence starting later in the range reads its incoming state here
                if (tj >= sn[i] || nn[i] == n0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[i][e] += w[e][j] * xr[i + j][e];
                } else if (state_in) {                         // before the sequence: state
                    const long long sidx = (W - 1) + (tj - sn[i]);
                    const float *sp = state_in + ((long long)nn[i] * C + cc) * (W - 1) + sidx;
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[i][e] += w[e][j] * sp[e * (W - 1)];
                }
            }
            ss[i] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // SiLU: x sigmoid(x) with the hardware reciprocal (about 1 ulp)
                o[i][e] = o[i][e] * __builtin_amdgcn_rcpf(1.f + __expf(-o[i][e]));
                ss[i] += o[i][e] * o[i][e];
            }
        }
        if constexpr (HD > 0) {
#pragma unroll
            for (int i = 0; i < S; ++i) {
                const float f = __builtin_amdgcn_rsqf(head_sum_dpp<HD / 8>(ss[i]) + kLsEps);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[i][e] *= f;
            }
        }
#pragma unroll
        for (int i = 0; i < S; ++i)
            if (live && ts + i < total_T) O::store(out + (ts + i) * C + c, o[i]);
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) win[i][e] = xr[S + i][e];
#pragma unroll
        for (int i = 0; i < S; ++i) cur[i] = nxt[i];
    }
}

// state_out[n][c][j] = ext(L_n - (W-1) + j), ext(i) = x[s_n + i][c] for i >= 0, else the
// incoming state state_in[n][c][(W-1) + i] (or zero); its own launch, after the convolution,
// when state_out is state_in.
template <typename T, int W>
__global__ __launch_bounds__(kLsThreads) void conv_state_kernel(
    const T *__restrict__ x, const int32_t *__restrict__ cu, int nseq, long long total_T,
    int C, const float *state_in, float *state_out)
{
    conv_state_item<T, W>((long long)blockIdx.x * kLsThreads + threadIdx.x, x, cu, nseq,
                          total_T, C, state_in, state_out);
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
    // a distinct outgoing state is written by extra workgroups of the same launch; in place,
    // it waits for the convolution (which reads the incoming state) in a launch of its own
    const bool fused = sout && W > 1 && sout != sin;
    const long long sblocks = ((long long)nseq * C + kLsThreads - 1) / kLsThreads;
    const long long grid = blocks + (fused ? sblocks : 0);
    if (grid > 0) {
        float *fs = fused ? sout : nullptr;
        if (head_dim == 128)
            hipLaunchKernelGGL((short_conv_kernel<T, W, 128>), dim3((unsigned)grid),
                               dim3(kLsThreads), 0, st, (const T *)x, w, cu, nseq, total_T, C,
                               sin, (T *)out, blocks, fs);
        else if (head_dim == 64)
            hipLaunchKernelGGL((short_conv_kernel<T, W, 64>), dim3((unsigned)grid),
                               dim3(kLsThreads), 0, st, (const T *)x, w, cu, nseq, total_T, C,
                               sin, (T *)out, blocks, fs);
        else
            hipLaunchKernelGGL((short_conv_kernel<T, W, 0>), dim3((unsigned)grid),
                               dim3(kLsThreads), 0, st, (const T *)x, w, cu, nseq, total_T, C,
                               sin, (T *)out, blocks, fs);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (sout && W > 1 && !fused) {
        hipLaunchKernelGGL((conv_state_kernel<T, W>), dim3((unsigned)sblocks), dim3(kLsThreads),
                           0, st, (const T *)x, cu, nseq, total_T, C, sin, sout);
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
