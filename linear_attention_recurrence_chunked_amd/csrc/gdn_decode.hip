// gdn_decode.hip -- one gated delta rule step per (sequence, head), state in place.
//
// The step is the recurrence of the jianyuh.github.io reading notes on Qwen3.8-Next,
// section 2.1 ("Gated DeltaNet"), for a single token:
//     r = S^T k,  s = S^T q            (one read of S)
//     e = v - alpha r                   (residual against the decayed state)
//     y = alpha s + beta (k.q) e        (= S_t^T q, since S_t = alpha S + beta k e^T)
//     S <- alpha S + beta k e^T         (one write of S)
// The step is HBM-bound (about 0.9 flop per byte), so the design is about bytes: each
// workgroup owns a 64-column slice of one head's state, loads it into registers with
// 16-byte coalesced loads, reduces S^T k and S^T q over the key dimension with wavefront
// shuffles and a 1 KiB LDS exchange, and stores the updated slice once.  The state is read
// and written with non-temporal hints: a layer's state is touched once per step, and a
// model's states together do not stay in the caches between steps.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

constexpr int kDecThreads = 256;
constexpr int kDecCols = 64;      // state columns per workgroup: 16 lanes x float4

template <int DK, int DV, typename TIn>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    float *__restrict__ state, TIn *__restrict__ y)
{
    constexpr int NCT = DV / kDecCols;       // column slices per head
    constexpr int RPT = DK / 16;             // state rows per thread
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = tid & 15;                 // column group: 4 columns
    const int rg = tid >> 4;                 // row group 0..15; rows rg + 16 i
    const int slice = blockIdx.x % NCT;
    const long bh = blockIdx.x / NCT;        // b * H + h
    const int col = slice * kDecCols + cg * 4;

    float *S = state + bh * (long)DK * DV;
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = __builtin_nontemporal_load((const f32x4 *)(S + (long)(rg + 16 * i) * DV + col));

    float kr[RPT], qr[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        kr[i] = Elem<TIn>::load(k + bh * DK + rg + 16 * i);
        qr[i] = Elem<TIn>::load(q + bh * DK + rg + 16 * i);
    }
    const f32x4 vv = load4(v + bh * DV + col);
    const float a = alpha[bh];
    const float b = beta[bh];

    f32x4 pr = {0.f, 0.f, 0.f, 0.f}, ps = {0.f, 0.f, 0.f, 0.f};
    float pkq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        pr += s[i] * kr[i];
        ps += s[i] * qr[i];
        pkq += kr[i] * qr[i];
    }
    // reduce over the four row groups of this wave (lane bits 4 and 5)
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pr[c] += wave_xor(pr[c], m);
            ps[c] += wave_xor(ps[c], m);
        }
        pkq += wave_xor(pkq, m);
    }
    __shared__ f32x4 red_r[4][16];
    __shared__ f32x4 red_s[4][16];
    __shared__ float red_kq[4];
    if (lane < 16) {
        red_r[wave][lane] = pr;
        red_s[wave][lane] = ps;
    }
    if (lane == 0) red_kq[wave] = pkq;
    __syncthreads();
    f32x4 r = red_r[0][cg] + red_r[1][cg] + red_r[2][cg] + red_r[3][cg];
    f32x4 sq = red_s[0][cg] + red_s[1][cg] + red_s[2][cg] + red_s[3][cg];
    const float kq = red_kq[0] + red_kq[1] + red_kq[2] + red_kq[3];

    const f32x4 e = vv - a * r;
    if (rg == 0) store4(y + bh * DV + col, a * sq + (b * kq) * e);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float bk = b * kr[i];
        __builtin_nontemporal_store(a * s[i] + bk * e, (f32x4 *)(S + (long)(rg + 16 * i) * DV + col));
    }
}

template <int DK, int DV, typename TIn>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v,
                                  const float *alpha, const float *beta, float *state,
                                  void *y, int B, int H, hipStream_t stream)
{
    const long blocks = (long)B * H * (DV / kDecCols);
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, TIn>), dim3((unsigned)blocks),
                       dim3(kDecThreads), 0, stream, (const TIn *)q, (const TIn *)k,
                       (const TIn *)v, alpha, beta, state, (TIn *)y);
    return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_decode_dt(const void *q, const void *k, const void *v,
                                   const float *alpha, const float *beta, float *state,
                                   void *y, int B, int H, int dk, int dv, hipStream_t st)
{
    if (dk == 128 && dv == 128)
        return launch_decode_t<128, 128, TIn>(q, k, v, alpha, beta, state, y, B, H, st);
    if (dk == 128 && dv == 64)
        return launch_decode_t<128, 64, TIn>(q, k, v, alpha, beta, state, y, B, H, st);
    if (dk == 64 && dv == 128)
        return launch_decode_t<64, 128, TIn>(q, k, v, alpha, beta, state, y, B, H, st);
    return launch_decode_t<64, 64, TIn>(q, k, v, alpha, beta, state, y, B, H, st);
}

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *alpha,
                         const float *beta, float *state, void *y, int B, int H, int dk,
                         int dv, int dtype, hipStream_t stream)
{
    if (dtype == kDtypeBF16)
        return launch_decode_dt<uint16_t>(q, k, v, alpha, beta, state, y, B, H, dk, dv,
                                          stream);
    return launch_decode_dt<float>(q, k, v, alpha, beta, state, y, B, H, dk, dv, stream);
}

}  // namespace gdn
