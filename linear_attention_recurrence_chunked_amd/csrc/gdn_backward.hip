// gdn_backward.hip -- chunked backward (training) of the gated delta rule on gfx950.
//
// For L = <dy, y> + <dS_T, S_T> the library returns dq, dk, dv, dalpha, dbeta and dS_0.  The
// derivative is taken through the chunked (WY / UT) form of the recurrence of the reading
// notes (Gated DeltaNet, section 2.1).  Per chunk of c <= 64 tokens that starts with state S
// (g = within-chunk prefix of log alpha, gamma = e^g, gamma_C = gamma of the last token,
// Gamma_ti = e^{g_t - g_i} for i <= t):
//
//   L  = strictlower(K K^T (.) Gamma),   T' = (I + diag(beta) L)^{-1} diag(beta),
//   P  = lower_incl(Q K^T (.) Gamma),    R = V - diag(gamma) K S,   U = T' R,
//   Y  = diag(gamma) Q S + P U,          S_next = gamma_C S + K^T diag(gamma_C / gamma) U.
//
// Taken backwards with D = the adjoint of S_next (dY given):
//
//   dU = P^T dY + diag(gamma_C/gamma) K D      Z = T'^T dU  (= dV)      E = dU - L^T Z
//   adjoint of S  = gamma_C D + Q^T diag(gamma) dY - K^T diag(gamma) Z
//   dQ = diag(gamma) dY S^T + (dP (.) Gamma) K,          dP = lower_incl(dY U^T)
//   dK = -diag(gamma) Z S^T + diag(gamma_C/gamma) U D^T + (dP (.) Gamma)^T Q
//        + (dL (.) Gamma) K + (dL (.) Gamma)^T K,        dL = -diag(beta) strictlower(E U^T)
//   dbeta_t = sum_j E_tj R_tj - sum_i L_ti (E U^T)_ti
//   dg_t    = sum_i (Q (.) Gq)_ti + (K (.) GkA)_ti - (K (.) GkB)_ti
//             + sum_i (dP (.) P + dL (.) L)_ti - sum_s (dP (.) P + dL (.) L)_st
//             + [t = last] (gamma_C <S, D> + sum_{s,i} (K (.) GkB)_si)
//   with Gq = diag(gamma) dY S^T, GkA = -diag(gamma) Z S^T, GkB = diag(gamma_C/gamma) U D^T;
//   dlog alpha_s = sum_{t >= s in the chunk} dg_t,  dalpha = dlog alpha / alpha.
//
// Four launches:
//   bwd_prep_kernel     (chunk slot, head): T' and P (fp32) and g into a record.
//   bwd_states_kernel   (sequence, head, 32 state columns): the forward scan, keeping S at
//                       the start of every chunk.
//   bwd_dstates_kernel  (sequence, head, 32 state columns): the adjoint scan from the last
//                       chunk to the first, keeping D at the end of every chunk; dS_0.
//   bwd_chunk_kernel    (chunk slot, head): everything else, from the kept S and D.
// Every product runs on 16x16x16 bf16 MFMAs with fp32 operands split into two bf16 halves
// (hi + lo; three products per step, two when one operand is exactly bf16).
//
// Chunk slots are the prefill's: chunk c of sequence n (first row t0_n) has slot
// floor(t0_n / 64) + n + c, below floor(total_T / 64) + num_seqs.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int C = kChunk;
constexpr float kLnAlphaFloor = -87.0f;   // e^-87 is still a normal fp32
constexpr int LDC = C + 4;                 // padded fp32 rows of a 64 x 64 matrix
constexpr int kRecFloats = 2 * C * C + C;  // T' [64][64], P [64][64], g [64]
constexpr int DVT = 32;                    // state columns per workgroup of the scans
constexpr int LDT = DVT + 4;
constexpr int DVB = 16;                    // value columns per pass of the chunk kernel
constexpr int LDB = DVB + 4;

typedef short v4s __attribute__((ext_vector_type(4)));

struct Split {
    v4s hi, lo;
};
__device__ __forceinline__ Split split(f32x4 x)
{
    const bf16x4 h = __builtin_convertvector(x, bf16x4);
    const bf16x4 l = __builtin_convertvector(x - __builtin_convertvector(h, f32x4), bf16x4);
    return Split{__builtin_bit_cast(v4s, h), __builtin_bit_cast(v4s, l)};
}

__device__ __forceinline__ float ldsf(const float *p) { return *p; }
__device__ __forceinline__ float ldsf(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ f32x4 lds4(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ f32x4 lds4(const uint16_t *p) { return load4(p); }

// acc += opA[m0 .. m0+15][0 .. kd) * opB[0 .. kd)[n0 .. n0+15] with
//   opA(m, k) = TA ? A[k * lda + m] : A[m * lda + k],
//   opB(k, n) = TB ? B[n * ldb + k] : B[k * ldb + n].
// Lane (r = lane % 16, q = lane / 16) feeds row m0 + r of opA and column n0 + r of opB with
// contraction indices k0 + 4q .. k0 + 4q + 3; the accumulator holds rows m0 + 4q + i,
// column n0 + r.  XA / XB: the operand holds bf16 values exactly (its low half is zero).
template <bool TA, bool TB, bool XA, bool XB, typename EA, typename EB>
__device__ __forceinline__ void mm(f32x4 &acc, const EA *A, int lda, const EB *B, int ldb,
                                   int m0, int n0, int kd)
{
    const int lane = threadIdx.x & 63, r = lane & 15, q4 = (lane >> 4) * 4;
    for (int k0 = 0; k0 < kd; k0 += 16) {
        f32x4 a, b;
        if constexpr (!TA) {
            a = lds4(A + (m0 + r) * lda + k0 + q4);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = ldsf(A + (k0 + q4 + i) * lda + m0 + r);
        }
        if constexpr (TB) {
            b = lds4(B + (n0 + r) * ldb + k0 + q4);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) b[i] = ldsf(B + (k0 + q4 + i) * ldb + n0 + r);
        }
        const Split sa = split(a), sb = split(b);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sa.hi, sb.hi, acc, 0, 0, 0);
        if constexpr (!XA) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sa.lo, sb.hi, acc, 0, 0, 0);
        if constexpr (!XB) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sa.hi, sb.lo, acc, 0, 0, 0);
    }
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Sum over the 16 lanes that share lane / 16.
__device__ __forceinline__ float sum16(float x)
{
    x += __shfl_xor(x, 1, kWave);
    x += __shfl_xor(x, 2, kWave);
    x += __shfl_xor(x, 4, kWave);
    x += __shfl_xor(x, 8, kWave);
    return x;
}

struct BwdArgs {
    const uint16_t *q, *k, *v, *dy;
    const float *alpha, *beta;
    const float *s0, *ds_final;
    const int32_t *cu;
    int num_seqs;
    long long total_T;
    int H;
    uint16_t *dq, *dk, *dv;
    float *dalpha, *dbeta, *ds0;
    float *rec;        // [nslots, H, kRecFloats]
    float *hs;         // [nslots, H, DK, DV]  state at the start of each chunk
    float *dhs;        // [nslots, H, DK, DV]  adjoint of the state at the end of each chunk
    long long nslots;
};

__device__ __forceinline__ long long row0_of(const BwdArgs &a, int n)
{
    return a.cu ? (long long)a.cu[n] : (a.total_T / a.num_seqs) * n;
}
__device__ __forceinline__ int len_of(const BwdArgs &a, int n)
{
    return a.cu ? (int)(a.cu[n + 1] - a.cu[n]) : (int)(a.total_T / a.num_seqs);
}
__device__ __forceinline__ long long slot_of(const BwdArgs &a, int n, int c)
{
    return (row0_of(a, n) >> 6) + n + c;
}

// (sequence, chunk) of a slot, or false for a slot no chunk uses.
__device__ __forceinline__ bool decode_slot(const BwdArgs &a, long long slot, int &n, int &c,
                                            long long &t0, int &nv)
{
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((row0_of(a, mid) >> 6) + mid <= slot) lo = mid; else hi = mid - 1;
    }
    n = lo;
    const long long r0 = row0_of(a, n);
    const int len = len_of(a, n);
    const long long cc = slot - ((r0 >> 6) + n);
    if (cc < 0 || cc * C >= len) return false;
    c = (int)cc;
    t0 = r0 + cc * C;
    nv = len - c * C < C ? len - c * C : C;
    return true;
}

// Rows [t0, t0 + nv) of a [rows, H, W] bf16 tensor (head h) into LDS as bf16 [64][ld], rows
// nv .. 63 zero.  16-byte pieces, all threads.
template <int W>
__device__ __forceinline__ void load_rows_bf16(uint16_t *dst, int ld, const uint16_t *src,
                                               long long t0, int nv, int H, int h)
{
    constexpr int P = W / 8;
    for (int i = threadIdx.x; i < C * P; i += blockDim.x) {
        const int t = i / P, p = i % P;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (t < nv) x = *(const u32x4 *)(src + ((t0 + t) * H + h) * (long long)W + 8 * p);
        *(u32x2 *)(dst + t * ld + 8 * p) = u32x2{x[0], x[1]};
        *(u32x2 *)(dst + t * ld + 8 * p + 4) = u32x2{x[2], x[3]};
    }
}

// Columns [col0, col0 + NC) of rows [t0, t0 + nv) of a [rows, H, W] bf16 tensor into LDS as
// fp32 [64][ld]; rows nv .. 63 zero.
template <int W, int NC>
__device__ __forceinline__ void load_cols_f32(float *dst, int ld, const uint16_t *src,
                                              long long t0, int nv, int H, int h, int col0)
{
    constexpr int P = NC / 4;
    for (int i = threadIdx.x; i < C * P; i += blockDim.x) {
        const int t = i / P, p = i % P;
        f32x4 x = zero4();
        if (t < nv) x = load4(src + ((t0 + t) * H + h) * (long long)W + col0 + 4 * p);
        *(f32x4 *)(dst + t * ld + 4 * p) = x;
    }
}

// A [64][64] fp32 block of global memory (row stride 64) into LDS [64][LDC].
__device__ __forceinline__ void load_mat64(float *dst, const float *src)
{
    for (int i = threadIdx.x; i < C * C / 4; i += blockDim.x) {
        const int t = i / (C / 4), p = i % (C / 4);
        *(f32x4 *)(dst + t * LDC + 4 * p) = *(const f32x4 *)(src + t * C + 4 * p);
    }
}

// Rows x cols fp32 sub-block (cols a multiple of 4) between global (row stride gs) and LDS.
__device__ __forceinline__ void load_blk(float *dst, int ld, const float *src, long long gs,
                                         int rows, int cols)
{
    const int P = cols / 4;
    for (int i = threadIdx.x; i < rows * P; i += blockDim.x) {
        const int r = i / P, p = i % P;
        *(f32x4 *)(dst + r * ld + 4 * p) = *(const f32x4 *)(src + r * gs + 4 * p);
    }
}
__device__ __forceinline__ void store_blk(float *dst, long long gs, const float *src, int ld,
                                          int rows, int cols)
{
    const int P = cols / 4;
    for (int i = threadIdx.x; i < rows * P; i += blockDim.x) {
        const int r = i / P, p = i % P;
        *(f32x4 *)(dst + r * gs + 4 * p) = *(const f32x4 *)(src + r * ld + 4 * p);
    }
}

// g (within-chunk prefix of the floored log alpha; 0 beyond nv), gamma = e^g and
// rat = e^{g_last - g} into LDS, by the first wave.  g_last is g[63]: tokens beyond nv add 0.
__device__ __forceinline__ void gate_prefix(float *g, float *gam, float *rat, float *bet,
                                            const float *alpha, const float *beta,
                                            long long t0, int nv, int H, int h)
{
    if (threadIdx.x >= kWave) return;
    const int t = threadIdx.x;
    float la = 0.f, b = 0.f;
    if (t < nv) {
        la = fmaxf(__logf(alpha[(t0 + t) * H + h]), kLnAlphaFloor);
        b = beta[(t0 + t) * H + h];
    }
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
        const float o = __shfl_up(la, s, kWave);
        if (t >= s) la += o;
    }
    const float last = __shfl(la, kWave - 1, kWave);
    g[t] = la;
    gam[t] = __expf(la);
    rat[t] = __expf(last - la);
    if (bet) bet[t] = b;
}

// Gamma_ti = e^{g_t - g_i} for i <= t, else 0.
__device__ __forceinline__ float decay(const float *g, int t, int i)
{
    return i <= t ? __expf(g[t] - g[i]) : 0.f;
}

// ======================================================================================
// bwd_prep_kernel: per (chunk slot, head) T' = (I + diag(beta) L)^{-1} diag(beta) by forward
// substitution, P = lower_incl(Q K^T (.) Gamma), g.
// ======================================================================================
template <int DK>
struct PrepLds {
    static constexpr int LDK = DK + 8;
    static constexpr int oK = 0;
    static constexpr int oQ = oK + C * LDK * 2;
    static constexpr int oL = oQ + C * LDK * 2;
    static constexpr int oG = oL + C * LDC * 4;
    static constexpr int oGam = oG + C * 4;
    static constexpr int oRat = oGam + C * 4;
    static constexpr int oBet = oRat + C * 4;
    static constexpr int total = oBet + C * 4;
};

template <int DK>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a)
{
    using L = PrepLds<DK>;
    __shared__ __align__(16) unsigned char smem[L::total];
    uint16_t *sK = (uint16_t *)(smem + L::oK), *sQ = (uint16_t *)(smem + L::oQ);
    float *sL = (float *)(smem + L::oL);
    float *g = (float *)(smem + L::oG), *gam = (float *)(smem + L::oGam);
    float *rat = (float *)(smem + L::oRat), *bet = (float *)(smem + L::oBet);
    const int H = a.H;
    const long long slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int n, c, nv;
    long long t0;
    if (!decode_slot(a, slot, n, c, t0, nv)) return;
    float *rec = a.rec + (slot * H + h) * (long long)kRecFloats;

    load_rows_bf16<DK>(sK, L::LDK, a.k, t0, nv, H, h);
    load_rows_bf16<DK>(sQ, L::LDK, a.q, t0, nv, H, h);
    gate_prefix(g, gam, rat, bet, a.alpha, a.beta, t0, nv, H, h);
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, q4 = (lane >> 4) * 4;
    // L (to LDS) and P (to the record): 16 tiles each, four per wave
    for (int tile = wave; tile < 16; tile += 4) {
        const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
        f32x4 kk = zero4(), qk = zero4();
        mm<false, true, true, true>(kk, sK, L::LDK, sK, L::LDK, m0, n0, DK);
        mm<false, true, true, true>(qk, sQ, L::LDK, sK, L::LDK, m0, n0, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = m0 + q4 + i, s = n0 + r;
            const float G = decay(g, t, s);
            sL[t * LDC + s] = s < t ? kk[i] * G : 0.f;
            rec[C * C + t * C + s] = qk[i] * G;
        }
    }
    __syncthreads();

    // forward substitution, one column per lane group: wave w owns columns 16w .. 16w+15;
    // lane (j = 16w + r, p = lane / 16) keeps rows i = 4m + p of its column in registers.
    const int j = 16 * wave + r, p = lane >> 4;
    float col[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) col[m] = 0.f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            if (4 * m < t) {
                const int i = 4 * m + p;
                if (i < t) s += sL[t * LDC + i] * col[m];
            }
        }
        s += __shfl_xor(s, 16, kWave);
        s += __shfl_xor(s, 32, kWave);
        const float val = bet[t] * ((t == j ? 1.f : 0.f) - s);
        if (p == (t & 3)) {
            col[t >> 2] = val;
            rec[t * C + j] = val;
        }
    }
    if (threadIdx.x < C) rec[2 * C * C + threadIdx.x] = g[threadIdx.x];
}

// ======================================================================================
// bwd_states_kernel: S at the start of every chunk of (sequence, head), 32 columns.
// ======================================================================================
template <int DK>
struct ScanLds {
    static constexpr int LDK = DK + 8;
    static constexpr int oS = 0;                              // [DK][LDT] fp32
    static constexpr int oK = oS + DK * LDT * 4;              // [64][LDK] bf16
    static constexpr int oQ = oK + C * LDK * 2;               // [64][LDK] bf16 (adjoint scan)
    static constexpr int oT = oQ + C * LDK * 2;               // [64][LDC] fp32
    static constexpr int oP = oT + C * LDC * 4;               // [64][LDC] fp32 (adjoint scan)
    static constexpr int oA = oP + C * LDC * 4;               // [64][LDT] fp32 (V or dY)
    static constexpr int oB = oA + C * LDT * 4;               // [64][LDT] fp32
    static constexpr int oX = oB + C * LDT * 4;               // [64][LDT] fp32
    static constexpr int oG = oX + C * LDT * 4;
    static constexpr int oGam = oG + C * 4;
    static constexpr int oRat = oGam + C * 4;
    static constexpr int total = oRat + C * 4;
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void bwd_states_kernel(BwdArgs a)
{
    using L = ScanLds<DK>;
    constexpr int NT = DV / DVT;
    __shared__ __align__(16) unsigned char smem[L::total];
    float *sS = (float *)(smem + L::oS);
    uint16_t *sK = (uint16_t *)(smem + L::oK);
    float *sT = (float *)(smem + L::oT), *sV = (float *)(smem + L::oA);
    float *sU = (float *)(smem + L::oB), *sX = (float *)(smem + L::oX);
    float *g = (float *)(smem + L::oG), *gam = (float *)(smem + L::oGam);
    float *rat = (float *)(smem + L::oRat);
    const int H = a.H;
    const int tile = blockIdx.x % NT;
    const int h = (blockIdx.x / NT) % H;
    const int n = blockIdx.x / (NT * H);
    const int col0 = tile * DVT;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, q4 = (lane >> 4) * 4;

    if (a.s0) load_blk(sS, LDT, a.s0 + ((long long)n * H + h) * DK * DV + col0, DV, DK, DVT);
    else
        for (int i = threadIdx.x; i < DK * LDT; i += blockDim.x) sS[i] = 0.f;
    const long long r0 = row0_of(a, n);
    const int len = len_of(a, n);
    const int nch = (len + C - 1) / C;
    for (int c = 0; c < nch; ++c) {
        const long long slot = slot_of(a, n, c);
        const long long t0 = r0 + (long long)c * C;
        const int nv = len - c * C < C ? len - c * C : C;
        const float *rec = a.rec + (slot * H + h) * (long long)kRecFloats;
        load_rows_bf16<DK>(sK, L::LDK, a.k, t0, nv, H, h);
        load_cols_f32<DV, DVT>(sV, LDT, a.v, t0, nv, H, h, col0);
        load_mat64(sT, rec);
        if (threadIdx.x < C) {
            const float gt = rec[2 * C * C + threadIdx.x], gl = rec[2 * C * C + C - 1];
            g[threadIdx.x] = gt;
            gam[threadIdx.x] = __expf(gt);
            rat[threadIdx.x] = __expf(gl - gt);
        }
        __syncthreads();
        store_blk(a.hs + ((slot * H + h) * DK) * (long long)DV + col0, DV, sS, LDT, DK, DVT);
        // X = V - diag(gamma) K S   (4 x 2 tiles)
        for (int tl = wave; tl < 8; tl += 4) {
            const int m0 = 16 * (tl >> 1), n0 = 16 * (tl & 1);
            f32x4 acc = zero4();
            mm<false, false, true, false>(acc, sK, L::LDK, sS, LDT, m0, n0, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = m0 + q4 + i;
                sX[t * LDT + n0 + r] = sV[t * LDT + n0 + r] - gam[t] * acc[i];
            }
        }
        __syncthreads();
        // U = T' X, kept as diag(gamma_C / gamma) U
        for (int tl = wave; tl < 8; tl += 4) {
            const int m0 = 16 * (tl >> 1), n0 = 16 * (tl & 1);
            f32x4 acc = zero4();
            mm<false, false, false, false>(acc, sT, LDC, sX, LDT, m0, n0, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = m0 + q4 + i;
                sU[t * LDT + n0 + r] = rat[t] * acc[i];
            }
        }
        __syncthreads();
        // S = gamma_C S + K^T (diag(gamma_C / gamma) U)   (DK/16 x 2 tiles)
        const float gC = gam[C - 1];
        for (int tl = wave; tl < (DK / 16) * 2; tl += 4) {
            const int m0 = 16 * (tl >> 1), n0 = 16 * (tl & 1);
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = gC * sS[(m0 + q4 + i) * LDT + n0 + r];
            mm<true, false, true, false>(acc, sK, L::LDK, sU, LDT, m0, n0, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) sS[(m0 + q4 + i) * LDT + n0 + r] = acc[i];
        }
        __syncthreads();
    }
}

// ======================================================================================
// bwd_dstates_kernel: the adjoint D of the state at the end of every chunk, last chunk
// first; dS_0 after the first chunk.
// ======================================================================================
template <int DK, int DV>
__global__ __launch_bounds__(256) void bwd_dstates_kernel(BwdArgs a)
{
    using L = ScanLds<DK>;
    constexpr int NT = DV / DVT;
    __shared__ __align__(16) unsigned char smem[L::total];
    float *sD = (float *)(smem + L::oS);
    uint16_t *sK = (uint16_t *)(smem + L::oK), *sQ = (uint16_t *)(smem + L::oQ);
    float *sT = (float *)(smem + L::oT), *sP = (float *)(smem + L::oP);
    float *sY = (float *)(smem + L::oA), *sZ = (float *)(smem + L::oB);
    float *sX = (float *)(smem + L::oX);
    float *g = (float *)(smem + L::oG), *gam = (float *)(smem + L::oGam);
    float *rat = (float *)(smem + L::oRat);
    const int H = a.H;
    const int tile = blockIdx.x % NT;
    const int h = (blockIdx.x / NT) % H;
    const int n = blockIdx.x / (NT * H);
    const int col0 = tile * DVT;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, q4 = (lane >> 4) * 4;

    if (a.ds_final)
        load_blk(sD, LDT, a.ds_final + ((long long)n * H + h) * DK * DV + col0, DV, DK, DVT);
    else
        for (int i = threadIdx.x; i < DK * LDT; i += blockDim.x) sD[i] = 0.f;
    const long long r0 = row0_of(a, n);
    const int len = len_of(a, n);
    const int nch = (len + C - 1) / C;
    for (int c = nch - 1; c >= 0; --c) {
        const long long slot = slot_of(a, n, c);
        const long long t0 = r0 + (long long)c * C;
        const int nv = len - c * C < C ? len - c * C : C;
        const float *rec = a.rec + (slot * H + h) * (long long)kRecFloats;
        load_rows_bf16<DK>(sK, L::LDK, a.k, t0, nv, H, h);
        load_rows_bf16<DK>(sQ, L::LDK, a.q, t0, nv, H, h);
        load_cols_f32<DV, DVT>(sY, LDT, a.dy, t0, nv, H, h, col0);
        load_mat64(sT, rec);
        load_mat64(sP, rec + C * C);
        if (threadIdx.x < C) {
            const float gt = rec[2 * C * C + threadIdx.x], gl = rec[2 * C * C + C - 1];
            g[threadIdx.x] = gt;
            gam[threadIdx.x] = __expf(gt);
            rat[threadIdx.x] = __expf(gl - gt);
        }
        __syncthreads();
        store_blk(a.dhs + ((slot * H + h) * DK) * (long long)DV + col0, DV, sD, LDT, DK, DVT);
        // X = P^T dY + diag(gamma_C / gamma) K D
        for (int tl = wave; tl < 8; tl += 4) {
            const int m0 = 16 * (tl >> 1), n0 = 16 * (tl & 1);
            f32x4 a1 = zero4(), a2 = zero4();
            mm<true, false, false, true>(a1, sP, LDC, sY, LDT, m0, n0, C);
            mm<false, false, true, false>(a2, sK, L::LDK, sD, LDT, m0, n0, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = m0 + q4 + i;
                sX[t * LDT + n0 + r] = a1[i] + rat[t] * a2[i];
            }
        }
        __syncthreads();
        // Z = T'^T X, kept as -diag(gamma) Z
        for (int tl = wave; tl < 8; tl += 4) {
            const int m0 = 16 * (tl >> 1), n0 = 16 * (tl & 1);
            f32x4 acc = zero4();
            mm<true, false, false, false>(acc, sT, LDC, sX, LDT, m0, n0, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = m0 + q4 + i;
                sZ[t * LDT + n0 + r] = -gam[t] * acc[i];
            }
        }
        // diag(gamma) dY in place (P^T dY above was the last use of dY itself)
        for (int i = threadIdx.x; i < C * DVT; i += blockDim.x) {
            const int t = i / DVT, jj = i % DVT;
            sY[t * LDT + jj] *= gam[t];
        }
        __syncthreads();
        // D = gamma_C D + Q^T (diag(gamma) dY) + K^T (-diag(gamma) Z)
        const float gC = gam[C - 1];
        for (int tl = wave; tl < (DK / 16) * 2; tl += 4) {
            const int m0 = 16 * (tl >> 1), n0 = 16 * (tl & 1);
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = gC * sD[(m0 + q4 + i) * LDT + n0 + r];
            mm<true, false, true, false>(acc, sQ, L::LDK, sY, LDT, m0, n0, C);
            mm<true, false, true, false>(acc, sK, L::LDK, sZ, LDT, m0, n0, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) sD[(m0 + q4 + i) * LDT + n0 + r] = acc[i];
        }
        __syncthreads();
    }
    if (a.ds0) store_blk(a.ds0 + ((long long)n * H + h) * DK * DV + col0, DV, sD, LDT, DK, DVT);
}

// ======================================================================================
// bwd_chunk_kernel: per (chunk slot, head), eight waves.  Passes over the value columns in
// blocks of 16 accumulate the products that contract over d_v; the rest follows.
// ======================================================================================
template <int DK>
struct ChunkLds {
    static constexpr int LDK = DK + 8;
    static constexpr int oK = 0;
    static constexpr int oQ = oK + C * LDK * 2;
    static constexpr int oT = oQ + C * LDK * 2;
    static constexpr int oP = oT + C * LDC * 4;
    static constexpr int oL = oP + C * LDC * 4;
    static constexpr int oBlk = oL + C * LDC * 4;             // per-pass region
    static constexpr int oS = oBlk;                           // [DK][LDB] state block
    static constexpr int oD = oS + DK * LDB * 4;              // [DK][LDB] adjoint block
    static constexpr int oV = oD + DK * LDB * 4;              // [64][LDB] each below
    static constexpr int oY = oV + C * LDB * 4;
    static constexpr int oR = oY + C * LDB * 4;
    static constexpr int oDU = oR + C * LDB * 4;
    static constexpr int oU = oDU + C * LDB * 4;
    static constexpr int oZ = oU + C * LDB * 4;
    static constexpr int oE = oZ + C * LDB * 4;
    static constexpr int blkEnd = oE + C * LDB * 4;
    static constexpr int oDP = oBlk;                          // after the passes
    static constexpr int oDL = oDP + C * LDC * 4;
    static constexpr int oPart = oDL + C * LDC * 4;          // row-sum partials
    static_assert(oPart + (20 * C + 40) * 4 <= blkEnd, "dP, dL and partials fit");
    static constexpr int oG = blkEnd;
    static constexpr int oGam = oG + C * 4;
    static constexpr int oRat = oGam + C * 4;
    static constexpr int oBet = oRat + C * 4;
    static constexpr int oDb = oBet + C * 4;
    static constexpr int total = oDb + C * 4;
};

template <int DK, int DV>
__global__ __launch_bounds__(512) void bwd_chunk_kernel(BwdArgs a)
{
    using L = ChunkLds<DK>;
    constexpr int LDK = L::LDK;
    constexpr int KT = DK / 16;                 // 16-column tiles of d_k
    __shared__ __align__(16) unsigned char smem[L::total];
    uint16_t *sK = (uint16_t *)(smem + L::oK), *sQ = (uint16_t *)(smem + L::oQ);
    float *sT = (float *)(smem + L::oT), *sP = (float *)(smem + L::oP);
    float *sL = (float *)(smem + L::oL);
    float *sS = (float *)(smem + L::oS), *sD = (float *)(smem + L::oD);
    float *sV = (float *)(smem + L::oV), *sY = (float *)(smem + L::oY);
    float *sR = (float *)(smem + L::oR), *sDU = (float *)(smem + L::oDU);
    float *sU = (float *)(smem + L::oU), *sZ = (float *)(smem + L::oZ);
    float *sE = (float *)(smem + L::oE);
    float *sDP = (float *)(smem + L::oDP), *sDL = (float *)(smem + L::oDL);
    float *g = (float *)(smem + L::oG), *gam = (float *)(smem + L::oGam);
    float *rat = (float *)(smem + L::oRat), *bet = (float *)(smem + L::oBet);
    float *db = (float *)(smem + L::oDb);

    const int H = a.H;
    const long long slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int n, c, nv;
    long long t0;
    if (!decode_slot(a, slot, n, c, t0, nv)) return;
    const float *rec = a.rec + (slot * H + h) * (long long)kRecFloats;
    const float *hs = a.hs + (slot * H + h) * (long long)DK * DV;
    const float *dhs = a.dhs + (slot * H + h) * (long long)DK * DV;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, q4 = (lane >> 4) * 4;

    load_rows_bf16<DK>(sK, LDK, a.k, t0, nv, H, h);
    load_rows_bf16<DK>(sQ, LDK, a.q, t0, nv, H, h);
    load_mat64(sT, rec);
    load_mat64(sP, rec + C * C);
    if (threadIdx.x < C) {
        const int t = threadIdx.x;
        const float gt = rec[2 * C * C + t], gl = rec[2 * C * C + C - 1];
        g[t] = gt;
        gam[t] = __expf(gt);
        rat[t] = __expf(gl - gt);
        bet[t] = t < nv ? a.beta[(t0 + t) * H + h] : 0.f;
        db[t] = 0.f;
    }
    __syncthreads();
    // L = strictlower(K K^T (.) Gamma): 16 tiles, two per wave
    for (int tile = wave; tile < 16; tile += 8) {
        const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
        f32x4 kk = zero4();
        mm<false, true, true, true>(kk, sK, LDK, sK, LDK, m0, n0, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = m0 + q4 + i, s = n0 + r;
            sL[t * LDC + s] = s < t ? kk[i] * decay(g, t, s) : 0.f;
        }
    }

    // accumulators over the passes (tile ids: c x c tiles w, w + 8; c x d_k tiles w + 8 j)
    constexpr int NQ = 4 * KT / 8;              // c x d_k tiles per wave
    f32x4 accM[2], accEu[2], accGq[NQ], accGa[NQ], accGb[NQ];
#pragma unroll
    for (int i = 0; i < 2; ++i) accM[i] = accEu[i] = zero4();
#pragma unroll
    for (int i = 0; i < NQ; ++i) accGq[i] = accGa[i] = accGb[i] = zero4();
    float sd = 0.f;                             // partial <S, D>

    for (int col0 = 0; col0 < DV; col0 += DVB) {
        __syncthreads();   // previous pass done (and L written before the first)
        load_blk(sS, LDB, hs + col0, DV, DK, DVB);
        load_blk(sD, LDB, dhs + col0, DV, DK, DVB);
        load_cols_f32<DV, DVB>(sV, LDB, a.v, t0, nv, H, h, col0);
        load_cols_f32<DV, DVB>(sY, LDB, a.dy, t0, nv, H, h, col0);
        for (int i = threadIdx.x; i < DK * DVB / 4; i += blockDim.x) {
            const int rr = i / (DVB / 4), p = i % (DVB / 4);
            const f32x4 s4 = *(const f32x4 *)(hs + rr * DV + col0 + 4 * p);
            const f32x4 d4 = *(const f32x4 *)(dhs + rr * DV + col0 + 4 * p);
            sd += s4[0] * d4[0] + s4[1] * d4[1] + s4[2] * d4[2] + s4[3] * d4[3];
        }
        __syncthreads();
        // phase 1: R = V - diag(gamma) K S (waves 0-3), diag(gamma_C/gamma) K D (waves 4-7)
        {
            const int m0 = 16 * (wave & 3);
            f32x4 acc = zero4();
            if (wave < 4) {
                mm<false, false, true, false>(acc, sK, LDK, sS, LDB, m0, 0, DK);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = m0 + q4 + i;
                    sR[t * LDB + r] = sV[t * LDB + r] - gam[t] * acc[i];
                }
            } else {
                mm<false, false, true, false>(acc, sK, LDK, sD, LDB, m0, 0, DK);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = m0 + q4 + i;
                    sDU[t * LDB + r] = rat[t] * acc[i];
                }
            }
        }
        __syncthreads();
        // phase 2: U = T' R (waves 0-3), dU = P^T dY + that (waves 4-7)
        {
            const int m0 = 16 * (wave & 3);
            if (wave < 4) {
                f32x4 acc = zero4();
                mm<false, false, false, false>(acc, sT, LDC, sR, LDB, m0, 0, C);
#pragma unroll
                for (int i = 0; i < 4; ++i) sU[(m0 + q4 + i) * LDB + r] = acc[i];
            } else {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = sDU[(m0 + q4 + i) * LDB + r];
                mm<true, false, false, true>(acc, sP, LDC, sY, LDB, m0, 0, C);
#pragma unroll
                for (int i = 0; i < 4; ++i) sDU[(m0 + q4 + i) * LDB + r] = acc[i];
            }
        }
        __syncthreads();
        // phase 3: Z = T'^T dU (= dV)
        if (wave < 4) {
            const int m0 = 16 * wave;
            f32x4 acc = zero4();
            mm<true, false, false, false>(acc, sT, LDC, sDU, LDB, m0, 0, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = m0 + q4 + i;
                sZ[t * LDB + r] = acc[i];
                if (t < nv) Elem<uint16_t>::store(a.dv + ((t0 + t) * H + h) * (long long)DV + col0 + r, acc[i]);
            }
        }
        __syncthreads();
        // phase 4: E = dU - L^T Z;  dbeta_t += sum_j E_tj R_tj
        if (wave < 4) {
            const int m0 = 16 * wave;
            f32x4 acc = zero4();
            mm<true, false, false, false>(acc, sL, LDC, sZ, LDB, m0, 0, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = m0 + q4 + i;
                const float e = sDU[t * LDB + r] - acc[i];
                sE[t * LDB + r] = e;
                const float s = sum16(e * sR[t * LDB + r]);
                if (r == 0) db[t] += s;     // one lane per row: no other writer
            }
        }
        __syncthreads();
        // phase 5: M += dY U^T, Eu += E U^T (c x c); Gq += dY S^T, Ga += Z S^T, Gb += U D^T
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + 8 * i;
            const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
            mm<false, true, false, false>(accM[i], sY, LDB, sU, LDB, m0, n0, DVB);
            mm<false, true, false, false>(accEu[i], sE, LDB, sU, LDB, m0, n0, DVB);
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int tile = wave + 8 * i;
            const int m0 = 16 * (tile / KT), n0 = 16 * (tile % KT);
            mm<false, true, false, false>(accGq[i], sY, LDB, sS, LDB, m0, n0, DVB);
            mm<false, true, false, false>(accGa[i], sZ, LDB, sS, LDB, m0, n0, DVB);
            mm<false, true, false, false>(accGb[i], sU, LDB, sD, LDB, m0, n0, DVB);
        }
    }
    __syncthreads();   // the per-pass region becomes dP and dL

    // Row sums below are written per source tile into the free part of the per-pass region
    // and added in a fixed order afterwards, so every output is bitwise repeatable.
    //   pG[kt][t]  row dot of the c x d_k accumulators, column tile kt
    //   pR[ct][t]  row sums of dP (.) P + dL (.) L over column tile ct
    //   pC[rt][s]  column sums of the same over row tile rt
    //   pB[ct][t]  row sums of L (.) Eu over column tile ct
    //   pX[...]    per-tile sums of K (.) Gb (32) and per-wave partials of <S, D> (8)
    float *pG = (float *)(smem + L::oPart);
    float *pR = pG + 8 * C, *pC = pR + 4 * C, *pB = pC + 4 * C, *pX = pB + 4 * C;
    // scale the c x d_k accumulators by their row factors; their row dots with Q and K
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile / KT), n0 = 16 * (tile % KT);
        float xs = 0.f;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = m0 + q4 + ii, col = n0 + r;
            accGq[i][ii] *= gam[t];
            accGa[i][ii] *= -gam[t];
            accGb[i][ii] *= rat[t];
            const float qv = ldsf(sQ + t * LDK + col), kv = ldsf(sK + t * LDK + col);
            const float xb = kv * accGb[i][ii];
            const float d = sum16(qv * accGq[i][ii] + kv * accGa[i][ii] - xb);
            if (r == 0) pG[(n0 / 16) * C + t] = d;
            xs += xb;
        }
        xs = sum16(xs);
        xs += __shfl_xor(xs, 16, kWave);
        xs += __shfl_xor(xs, 32, kWave);
        if (lane == 0) pX[tile] = xs;
    }
    // <S, D> over the chunk
    {
        float s = sd;
        s += __shfl_xor(s, 1, kWave);
        s += __shfl_xor(s, 2, kWave);
        s += __shfl_xor(s, 4, kWave);
        s += __shfl_xor(s, 8, kWave);
        s += __shfl_xor(s, 16, kWave);
        s += __shfl_xor(s, 32, kWave);
        if (lane == 0) pX[32 + wave] = s;
    }
    // dP = lower_incl(M), dL = -diag(beta) strictlower(Eu); their decayed forms to LDS;
    // dg from (dP (.) P + dL (.) L): + row sums, - column sums;  dbeta -= sum_i L (.) Eu
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
        float cs = 0.f;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = m0 + q4 + ii, s = n0 + r;
            const float G = decay(g, t, s);
            const float dP = s <= t ? accM[i][ii] : 0.f;
            const float lv = sL[t * LDC + s];
            const float dL = s < t ? -bet[t] * accEu[i][ii] : 0.f;
            sDP[t * LDC + s] = dP * G;
            sDL[t * LDC + s] = dL * G;
            const float w = dP * sP[t * LDC + s] + dL * lv;
            const float rs = sum16(w);
            const float bsum = sum16(s < t ? lv * accEu[i][ii] : 0.f);
            if (r == 0) {
                pR[(n0 / 16) * C + t] = rs;
                pB[(n0 / 16) * C + t] = bsum;
            }
            cs += w;
        }
        cs += __shfl_xor(cs, 16, kWave);
        cs += __shfl_xor(cs, 32, kWave);
        if (lane < 16) pC[(m0 / 16) * C + n0 + r] = cs;
    }
    __syncthreads();
    // dQ = Gq + (dP (.) Gamma) K;  dK = Ga + Gb + (dP (.) Gamma)^T Q + (dL (.) Gamma) K
    //                                     + (dL (.) Gamma)^T K
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile / KT), n0 = 16 * (tile % KT);
        f32x4 aq = accGq[i];
        mm<false, false, false, true>(aq, sDP, LDC, sK, LDK, m0, n0, C);
        f32x4 ak = accGa[i] + accGb[i];
        mm<true, false, false, true>(ak, sDP, LDC, sQ, LDK, m0, n0, C);
        mm<false, false, false, true>(ak, sDL, LDC, sK, LDK, m0, n0, C);
        mm<true, false, false, true>(ak, sDL, LDC, sK, LDK, m0, n0, C);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = m0 + q4 + ii;
            if (t < nv) {
                const long long o = ((t0 + t) * H + h) * (long long)DK + n0 + r;
                Elem<uint16_t>::store(a.dq + o, aq[ii]);
                Elem<uint16_t>::store(a.dk + o, ak[ii]);
            }
        }
    }
    __syncthreads();
    // dlog alpha = reverse prefix of dg (the chunk-end terms land on the last slot)
    if (threadIdx.x < C) {
        const int t = threadIdx.x;
        float x = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) x += pG[kt * C + t];
        float bt = db[t];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            x += pR[ct * C + t] - pC[ct * C + t];
            bt -= pB[ct * C + t];
        }
        if (t == C - 1) {
            float xb = 0.f, sdt = 0.f;
            for (int i = 0; i < 4 * KT; ++i) xb += pX[i];
            for (int w = 0; w < 8; ++w) sdt += pX[32 + w];
            x += xb + gam[C - 1] * sdt;
        }
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const float o = __shfl_down(x, s, kWave);
            if (t + s < kWave) x += o;
        }
        if (t < nv) {
            const long long o = (t0 + t) * H + h;
            const float al = a.alpha[o];
            a.dalpha[o] = __logf(al) > kLnAlphaFloor ? x / al : 0.f;
            a.dbeta[o] = bt;
        }
    }
}

template <int DK, int DV>
hipError_t launch_bwd_dims(const BwdArgs &a, hipStream_t stream)
{
    const long long units = (long long)a.num_seqs * a.H;
    const long long slots = a.nslots * a.H;
    hipLaunchKernelGGL(bwd_prep_kernel<DK>, dim3((unsigned)slots), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((bwd_states_kernel<DK, DV>), dim3((unsigned)(units * (DV / DVT))),
                       dim3(256), 0, stream, a);
    hipLaunchKernelGGL((bwd_dstates_kernel<DK, DV>), dim3((unsigned)(units * (DV / DVT))),
                       dim3(256), 0, stream, a);
    hipLaunchKernelGGL((bwd_chunk_kernel<DK, DV>), dim3((unsigned)slots), dim3(512), 0, stream,
                       a);
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t backward_workspace_bytes(int num_seqs, long long total_T, int H, int dk, int dv)
{
    const long long nslots = total_T / kChunk + num_seqs;
    const size_t rec = align256((size_t)nslots * H * kRecFloats * 4);
    const size_t st = align256((size_t)nslots * H * dk * dv * 4);
    return rec + 2 * st;
}

hipError_t launch_backward(const BackwardProblem &p, void *workspace, hipStream_t stream)
{
    BwdArgs a;
    a.q = (const uint16_t *)p.q;
    a.k = (const uint16_t *)p.k;
    a.v = (const uint16_t *)p.v;
    a.dy = (const uint16_t *)p.dy;
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.s0 = p.s0;
    a.ds_final = p.ds_final;
    a.cu = p.cu;
    a.num_seqs = p.num_seqs;
    a.total_T = p.total_T;
    a.H = p.H;
    a.dq = (uint16_t *)p.dq;
    a.dk = (uint16_t *)p.dk_out;
    a.dv = (uint16_t *)p.dv_out;
    a.dalpha = p.dalpha;
    a.dbeta = p.dbeta;
    a.ds0 = p.ds0;
    a.nslots = p.total_T / kChunk + p.num_seqs;
    const size_t rec = align256((size_t)a.nslots * p.H * kRecFloats * 4);
    const size_t st = align256((size_t)a.nslots * p.H * p.dk * p.dv * 4);
    a.rec = (float *)workspace;
    a.hs = (float *)((unsigned char *)workspace + rec);
    a.dhs = (float *)((unsigned char *)workspace + rec + st);
    if (p.dk == 128 && p.dv == 128) return launch_bwd_dims<128, 128>(a, stream);
    if (p.dk == 128 && p.dv == 64) return launch_bwd_dims<128, 64>(a, stream);
    if (p.dk == 64 && p.dv == 128) return launch_bwd_dims<64, 128>(a, stream);
    return launch_bwd_dims<64, 64>(a, stream);
}

}  // namespace gdn
