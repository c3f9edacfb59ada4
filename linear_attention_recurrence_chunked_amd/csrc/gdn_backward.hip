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
//   dg_t    = sum_i (Q (.) Gq)_ti + (K (.) Ga)_ti - (K (.) Gb)_ti
//             + sum_i (dP (.) P + dL (.) L)_ti - sum_s (dP (.) P + dL (.) L)_st
//             + [t = last] (gamma_C <S, D> + sum_{s,i} (K (.) Gb)_si)
//   with Gq = diag(gamma) dY S^T, Ga = -diag(gamma) Z S^T, Gb = diag(gamma_C/gamma) U D^T;
//   dlog alpha_s = sum_{t >= s in the chunk} dg_t,  dalpha = dlog alpha / alpha.
//
// Four launches:
//   bwd_prep_kernel     (chunk slot, head): T' (blocked inversion, split-bf16 MFMAs) and P^T,
//                       bf16, and g into a record.
//   bwd_states_kernel   (sequence, head, 32 state columns): the forward scan, keeping S at
//                       the start of every chunk.
//   bwd_dstates_kernel  (sequence, head, 32 state columns): the adjoint scan from the last
//                       chunk to the first, keeping D at the end of every chunk; dS_0.
//   bwd_chunk_kernel    (chunk slot, head): everything else, from the kept S and D.
// Products run on 16x16x32 bf16 MFMAs with fp32 accumulation, operands rounded once to bf16
// (as in the forward), except where short sequences make the gradient a small difference of
// large terms: U = T' R, dY U^T and the three products with S and D take their right operand
// as bf16 hi + lo.  Tiles live in LDS in one orientation; an operand that is the
// transpose of a stored tile is read with the transposing LDS read.  The two scans keep
// their fp32 state in MFMA accumulators across chunks and fetch the next chunk's inputs into
// registers while the current one is computed.
//
// Chunk slots are the prefill's: chunk c of sequence n (first row t0_n) has slot
// floor(t0_n / 64) + n + c, below floor(total_T / 64) + num_seqs.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn_split_bf16.hpp"

namespace gdn {
namespace {

constexpr int C = kChunk;
constexpr float kLnAlphaFloor = -87.0f;   // e^-87 is still a normal fp32
constexpr int L64 = C + 8;                 // bf16 row stride of a [.][64] LDS tile
constexpr int DVT = 32;                    // state columns per workgroup of the two scans
constexpr int LVT = DVT + 8;               // bf16 row stride of a [.][32] LDS tile
constexpr int DVB = 32;                    // value columns per pass of the chunk kernel
constexpr int LF = C + 4;                  // fp32 row stride of the prep kernel's T'
constexpr int LNB = 20;                    // fp32 row stride of its 16 x 16 blocks
// Record of one (chunk slot, head), in bf16 units: T' [64][64], P^T [64][64], then the 64
// within-chunk log-decay prefixes g as fp32.
constexpr int kRT = 0, kRP = C * C, kRG = 2 * C * C;
constexpr int kRecHalfs = 2 * C * C + 2 * C;
constexpr int kThreadsScan = 512;
constexpr int LSF = DVT + 4;               // fp32 row stride of a kept state block in LDS

// An accumulator tile into a row-major fp32 [.][LSF] block, and the block's 16-byte pieces
// (row i / (DVT / 4), columns 4 (i % (DVT / 4)) ..) to a [DK][DV] state in HBM: the state
// leaves in whole pieces rather than one word per lane, and non-temporally, so the kept states
// (read back by a later launch) do not push the chunk inputs that the other column tiles of
// the same head still read out of L2.
__device__ __forceinline__ void put_f(float *D, int m0, int n0, f32x4 v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) D[(m0 + 4 * (lane >> 4) + i) * LSF + n0 + (lane & 15)] = v[i];
}
template <int DK, int DV>
__device__ __forceinline__ void store_state(float *dst, const float *Sf)
{
    constexpr int PR = DVT / 4, NPC = DK * PR / kThreadsScan;
    static_assert(DK * PR % kThreadsScan == 0, "whole pieces per thread");
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
        const int i = threadIdx.x + kThreadsScan * j, row = i / PR, c4 = 4 * (i % PR);
        __builtin_nontemporal_store(*(const f32x4 *)(Sf + row * LSF + c4),
                                    (f32x4 *)(dst + row * DV + c4));
    }
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float bf(const uint16_t *p) { return bf16_to_f32(*p); }

// Four bf16 values by the transposing LDS read: within each group of 16 lanes, lane j
// receives element j % 4 of the 8-byte rows addressed by lanes j / 4 + 4 s, s = 0..3.
__device__ __forceinline__ bf16x4 ldtr(const uint16_t *p)
{
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)p);
    return __builtin_bit_cast(bf16x4, r);
}

// MFMA operand fragments (16x16x32): lane (r = lane % 16, g = lane / 16) supplies the eight
// contraction indices k0 + 8 g .. k0 + 8 g + 7 of row m0 + r of the operand.
//   frag_r: the operand is stored row major, [m][ld] with k contiguous (one 16-byte read);
//   frag_c: the operand is the transpose of a stored [k][ld] tile (two transposing reads).
__device__ __forceinline__ bf16x8 frag_r(const uint16_t *X, int ld, int m0, int k0)
{
    const int lane = threadIdx.x & 63;
    return *(const bf16x8 *)(X + (m0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
__device__ __forceinline__ bf16x8 frag_c(const uint16_t *X, int ld, int m0, int k0)
{
    const int lane = threadIdx.x & 63, l = lane & 15;
    const uint16_t *p = X + (k0 + 8 * (lane >> 4) + (l >> 2)) * ld + m0 + 4 * (l & 3);
    const bf16x4 lo = ldtr(p), hi = ldtr(p + 4 * ld);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// acc += opA[m0 .. m0+15][0 .. kd) opB[0 .. kd)[n0 .. n0+15].
//   AT = false: A stored [m][k];  AT = true: A stored [k][m] (opA is its transpose).
//   BT = true:  B stored [n][k];  BT = false: B stored [k][n].
// The accumulator holds rows m0 + 4 (lane / 16) + i, column n0 + lane % 16.
template <bool AT, bool BT>
__device__ __forceinline__ void mm(f32x4 &acc, const uint16_t *A, int lda, const uint16_t *B,
                                   int ldb, int m0, int n0, int kd)
{
    for (int k0 = 0; k0 < kd; k0 += 32) {
        const bf16x8 a = AT ? frag_c(A, lda, m0, k0) : frag_r(A, lda, m0, k0);
        const bf16x8 b = BT ? frag_r(B, ldb, n0, k0) : frag_c(B, ldb, n0, k0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
}

// The same with the B operand held as two bf16 tiles, hi + lo (an fp32 value to about 16
// significant bits): two products per step.
template <bool AT, bool BT>
__device__ __forceinline__ void mm2(f32x4 &acc, const uint16_t *A, int lda, const uint16_t *Bh,
                                    const uint16_t *Bl, int ldb, int m0, int n0, int kd)
{
    for (int k0 = 0; k0 < kd; k0 += 32) {
        const bf16x8 a = AT ? frag_c(A, lda, m0, k0) : frag_r(A, lda, m0, k0);
        const bf16x8 bh = BT ? frag_r(Bh, ldb, n0, k0) : frag_c(Bh, ldb, n0, k0);
        const bf16x8 bl = BT ? frag_r(Bl, ldb, n0, k0) : frag_c(Bl, ldb, n0, k0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc, 0, 0, 0);
    }
}

// An accumulator tile (rows m0 + 4 g + i, column n0 + r) stored transposed into a bf16
// [n][ld] tile: one 8-byte store per lane.  put_t2 also stores the rounding remainder.
__device__ __forceinline__ void put_t(uint16_t *D, int ld, int m0, int n0, f32x4 v)
{
    const int lane = threadIdx.x & 63;
    *(bf16x4 *)(D + (n0 + (lane & 15)) * ld + m0 + 4 * (lane >> 4)) =
        __builtin_convertvector(v, bf16x4);
}
__device__ __forceinline__ void put_t2(uint16_t *Dh, uint16_t *Dl, int ld, int m0, int n0,
                                       f32x4 v)
{
    const int lane = threadIdx.x & 63;
    const int o = (n0 + (lane & 15)) * ld + m0 + 4 * (lane >> 4);
    const bf16x4 h = __builtin_convertvector(v, bf16x4);
    *(bf16x4 *)(Dh + o) = h;
    *(bf16x4 *)(Dl + o) = __builtin_convertvector(v - __builtin_convertvector(h, f32x4), bf16x4);
}

// Sum over the 16 lanes that share lane / 16 (DPP moves within the row: neighbour and pair
// swaps, then half-row and row mirrors, which meet lanes already holding equal sums), and
// over the whole wave.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum16(float x)
{
    x += dpp_f<0xb1>(x);                    // quad_perm [1, 0, 3, 2]: lane ^ 1
    x += dpp_f<0x4e>(x);                    // quad_perm [2, 3, 0, 1]: lane ^ 2
    x += dpp_f<0x141>(x);                   // row_half_mirror
    x += dpp_f<0x140>(x);                   // row_mirror
    return x;
}
__device__ __forceinline__ float sum64(float x) { return row_sum4(sum16(x)); }
// Sum over lanes l .. 63 (a reverse prefix): within each 16-lane row by DPP row shifts (lane
// l adds lane l + n of its row, 0 past the row's end), then the totals of the later rows,
// read from their first lanes.
__device__ __forceinline__ float suffix_sum64(float x)
{
    x += dpp_f<0x101>(x);                   // row_shl:1
    x += dpp_f<0x102>(x);                   // row_shl:2
    x += dpp_f<0x104>(x);                   // row_shl:4
    x += dpp_f<0x108>(x);                   // row_shl:8
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    const int row = (threadIdx.x & 63) >> 4;
    const float later = row == 0 ? r1 + (r2 + r3) : row == 1 ? r2 + r3 : row == 2 ? r3 : 0.f;
    return x + later;
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
    uint16_t *rec;     // [nslots, H, kRecHalfs]
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

// (unit = sequence * H + head, column tile) of a scan workgroup.  Workgroups are dealt to the
// eight XCDs in turn (block b to XCD b % 8); when the grid divides evenly, the NT column
// tiles of a unit get block indices of one residue mod 8, so the K, Q and record bytes they
// all read are fetched into one L2.
template <int NT>
__device__ __forceinline__ void scan_job(int &unit, int &tile)
{
    const int b = blockIdx.x, G = gridDim.x;
    int idx = b;
    if (G % (8 * NT) == 0) idx = (b & 7) * (G >> 3) + (b >> 3);
    unit = idx / NT;
    tile = idx % NT;
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

// Piece i (16 bytes: row i / (NC / 8), columns col0 + 8 (i % (NC / 8)) ..) of the rows
// [t0, t0 + nv) of a [rows, H, W] bf16 tensor, head h; zero beyond nv.
template <int W, int NC>
__device__ __forceinline__ u32x4 piece(const uint16_t *src, long long t0, int nv, int H, int h,
                                       int col0, int i)
{
    constexpr int P = NC / 8;
    const int t = i / P, p = i % P;
    if (t >= nv) return u32x4{0u, 0u, 0u, 0u};
    return *(const u32x4 *)(src + ((t0 + t) * H + h) * (long long)W + col0 + 8 * p);
}
// The same piece from the chunk's row base (first row, head h: one 64-bit address per chunk,
// shared by the wave) and the thread's offset within the chunk (fixed for a thread), so a
// scan's per-chunk fetch adds one offset per piece instead of forming each address anew.
template <int W, int NC>
__device__ __forceinline__ int piece_off(int H, int col0, int i)
{
    constexpr int P = NC / 8;
    return (i / P) * H * W + col0 + 8 * (i % P);
}
template <int NC>
__device__ __forceinline__ u32x4 piece_at(const uint16_t *base, int off, int nv, int i)
{
    if (i / (NC / 8) >= nv) return u32x4{0u, 0u, 0u, 0u};
    return *(const u32x4 *)(base + off);
}
// The same piece loaded from a row clamped into the chunk (nv >= 1), without a branch: for
// batches of loads that all go out before any is used; piece_keep() zeroes it past nv when
// it is stored.
template <int W, int NC>
__device__ __forceinline__ u32x4 piece_clamped(const uint16_t *src, long long t0, int nv, int H,
                                               int h, int col0, int i)
{
    constexpr int P = NC / 8;
    const int t = i / P, p = i % P;
    const int tc = t < nv ? t : nv - 1;
    return *(const u32x4 *)(src + ((t0 + tc) * H + h) * (long long)W + col0 + 8 * p);
}
template <int NC>
__device__ __forceinline__ u32x4 piece_keep(u32x4 x, int nv, int i)
{
    return i / (NC / 8) < nv ? x : u32x4{0u, 0u, 0u, 0u};
}

template <int NC>
__device__ __forceinline__ void put_piece(uint16_t *dst, int ld, int i, u32x4 x)
{
    constexpr int P = NC / 8;
    *(u32x4 *)(dst + (i / P) * ld + 8 * (i % P)) = x;
}

// Eight bf16 (one piece) times a scalar, rounded back to bf16.
__device__ __forceinline__ u32x4 scale_piece(u32x4 x, float s)
{
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float lo = __uint_as_float(x[w] << 16) * s;
        const float hi = __uint_as_float(x[w] & 0xffff0000u) * s;
        const bf16x2 b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
        o[w] = __builtin_bit_cast(uint32_t, b);
    }
    return o;
}

// Gamma_ti = e^{g_t - g_i} for i <= t, else 0.  The exponent is capped at 0 (g falls with t,
// so only the masked entries reach the cap) and the power is taken for every entry, so the
// mask is a select rather than a branch around the reads of g.
__device__ __forceinline__ float decay(const float *g, int t, int i)
{
    const float e = __expf(fminf(g[t] - g[i], 0.f));
    return i <= t ? e : 0.f;
}

// Record pieces (16 bytes of a [64][64] bf16 matrix) and their place in an LDS tile
// [64][L64].
__device__ __forceinline__ u32x4 rec_piece(const uint16_t *rec, int off, int i)
{
    return *(const u32x4 *)(rec + off + 8 * i);
}
__device__ __forceinline__ void put_rec_piece(uint16_t *dst, int i, u32x4 x)
{
    *(u32x4 *)(dst + (i >> 3) * L64 + 8 * (i & 7)) = x;
}

// ======================================================================================
// bwd_prep_kernel: per (chunk slot, head) T' = (I + N)^{-1} diag(beta) with N = diag(beta) L,
// P = lower_incl(Q K^T (.) Gamma), g.  Four waves; wave w owns block column w of the 4 x 4 grid
// of 16 x 16 blocks.  The diagonal blocks of (I + N)^{-1} come by doubling (exact, since a
// strictly lower 16 x 16 block has N^16 = 0), the blocks below them by block substitution;
// every product of the solve runs on bf16 MFMAs with its operands split into high parts and
// remainders (about 2^-16 relative).
// ======================================================================================
// N and the diagonal inverses take the place of Q once the products are done, T' that of K,
// and P^T goes to the record from the accumulators, so four workgroups fit in a CU's LDS.
template <int DK>
struct PrepLds {
    static constexpr int mx(int a, int b) { return a > b ? a : b; }
    static constexpr int LK = DK + 8;
    static constexpr int oK = 0;
    static constexpr int oT = 0;                    // [64][LF] fp32 T', after the products
    static constexpr int oQ = oK + C * LK * 2;
    static constexpr int oN = mx(oQ, C * LF * 4);   // six [16][LNB] fp32 blocks of N, and
    static constexpr int oX = oN + 6 * 16 * LNB * 4;    // four of X_ii, after the products
    static constexpr int oG = mx(oQ + C * LK * 2, oX + 4 * 16 * LNB * 4);
    static constexpr int oBet = oG + C * 4;
    static constexpr int total = oBet + C * 4;
};

template <int DK>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a)
{
    using L = PrepLds<DK>;
    constexpr int LK = L::LK;
    __shared__ __align__(16) unsigned char smem[L::total];
    uint16_t *sK = (uint16_t *)(smem + L::oK), *sQ = (uint16_t *)(smem + L::oQ);
    float *sN = (float *)(smem + L::oN), *sX = (float *)(smem + L::oX);
    float *sT = (float *)(smem + L::oT);
    float *g = (float *)(smem + L::oG), *bet = (float *)(smem + L::oBet);
    const int H = a.H;
    const long long slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int n, c, nv;
    long long t0;
    if (!decode_slot(a, slot, n, c, t0, nv)) return;
    uint16_t *rec = a.rec + (slot * H + h) * (long long)kRecHalfs;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q4 = (lane >> 4) * 4;

    // the gates, then every piece of K and Q, all in flight at once
    float la = 0.f, bta = 0.f;
    if (tid < C && tid < nv) {
        la = a.alpha[(t0 + tid) * H + h];
        bta = a.beta[(t0 + tid) * H + h];
    }
    {
        constexpr int NP = C * DK / 8 / 256;
        u32x4 kx[NP], qx[NP];
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            kx[u] = piece_clamped<DK, DK>(a.k, t0, nv, H, h, 0, tid + 256 * u);
            qx[u] = piece_clamped<DK, DK>(a.q, t0, nv, H, h, 0, tid + 256 * u);
        }
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            put_piece<DK>(sK, LK, tid + 256 * u, piece_keep<DK>(kx[u], nv, tid + 256 * u));
            put_piece<DK>(sQ, LK, tid + 256 * u, piece_keep<DK>(qx[u], nv, tid + 256 * u));
        }
    }
    if (tid < C) {
        float b = 0.f;
        if (tid < nv) {
            la = fmaxf(__logf(la), kLnAlphaFloor);
            b = bta;
        }
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const float o = __shfl_up(la, s, kWave);
            if (tid >= s) la += o;
        }
        g[tid] = la;
        bet[tid] = b;
        ((float *)(rec + kRG))[tid] = la;
    }
    __syncthreads();

    // N = diag(beta) L (fp32) and P (bf16, to the record): 16 tiles each, four per wave.  Wave w
    // takes block column w: tile (u, w) of N in the accumulator layout (lane (r, p) holds rows
    // 16u + 4p .. + 3 of column 16w + r).  The diagonal block also in the layout of its
    // transpose, from the same entries of the symmetric K K^T block.
    f32x4 nb[4], nT;
    const int w16 = 16 * wave;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int m0 = 16 * u;
        f32x4 kk = zero4(), qk = zero4();
        mm<false, true>(kk, sK, LK, sK, LK, m0, w16, DK);
        mm<false, true>(qk, sQ, LK, sK, LK, m0, w16, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = m0 + q4 + i, s = w16 + r;
            const float G = decay(g, t, s);
            nb[u][i] = s < t ? bet[t] * kk[i] * G : 0.f;
            qk[i] *= G;
        }
        if (u == wave) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = w16 + r, s = w16 + q4 + i;
                nT[i] = s < t ? bet[t] * kk[i] * decay(g, t, s) : 0.f;
            }
        }
        // P^T to the record: rows w16 + r, four adjacent columns m0 + q4 .. per lane
        *(bf16x4 *)(rec + kRP + (w16 + r) * C + m0 + q4) = __builtin_convertvector(qk, bf16x4);
    }
    // (I + N)^{-1} of the diagonal block by doubling, (I - N)(I + N^2)(I + N^4)(I + N^8)
    // (exact: N^16 = 0), with split-bf16 products; C = the accumulator layout of a block, T =
    // that of its transpose
    f32x4 nC = nb[0];
#pragma unroll
    for (int u = 1; u < 4; ++u)
        if (u == wave) nC = nb[u];
    f32x4 eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) eye[i] = q4 + i == r ? 1.f : 0.f;
    const Sp snT = split4(nT), snC = split4(nC);
    const f32x4 n2C = mm3r(snT, snC), n2T = mm3r(snC, snT);
    const Sp sn2C = split4(n2C), sn2T = split4(n2T);
    const f32x4 m1C = mm3r(snT, sn2C), m1T = mm3r(sn2C, snT);
    const f32x4 n4C = mm3r(sn2T, sn2C), n4T = mm3r(sn2C, sn2T);
    const f32x4 p1C = eye - nC + n2C - m1C, p1T = eye - nT + n2T - m1T;
    const Sp sn4C = split4(n4C), sp1T = split4(p1T);
    const f32x4 n8C = mm3r(split4(n4T), sn4C);
    f32x4 p2C = p1C, p2T = p1T;
    mm3(p2C, sp1T, sn4C);
    mm3(p2T, sn4C, sp1T);
    const Sp sn8C = split4(n8C), sp2T = split4(p2T);
    f32x4 xC = p2C, xT = p2T;
    mm3(xC, sp2T, sn8C);
    mm3(xT, sn8C, sp2T);
    __syncthreads();   // every wave is done with K and Q: T' goes over K, N and X over Q

    // the strictly lower blocks of N row-major (block (i, m) at index i (i - 1) / 2 + m), the
    // diagonal inverses X_ii row-major, T'_ww = X_ww diag(beta) and zeros above the diagonal
    auto nblk = [&](int i, int m) { return sN + (i * (i - 1) / 2 + m) * 16 * LNB; };
#pragma unroll
    for (int u = 1; u < 4; ++u)
        if (u > wave) {
#pragma unroll
            for (int i = 0; i < 4; ++i) nblk(u, wave)[(q4 + i) * LNB + r] = nb[u][i];
        }
    *(f32x4 *)(sX + (w16 + r) * LNB + q4) = xT;
    const float bcol = bet[w16 + r];
#pragma unroll
    for (int i = 0; i < 4; ++i) sT[(w16 + q4 + i) * LF + w16 + r] = xC[i] * bcol;
#pragma unroll
    for (int j = 1; j < 4; ++j)
        if (j > wave) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(w16 + q4 + i) * LF + 16 * j + r] = 0.f;
        }
    __syncthreads();

    // the blocks below the diagonal of block column j = w:
    // X_ij = -X_ii sum_{m=j}^{i-1} N_im X_mj,  T'_ij = X_ij diag(beta_j)
    {
        const int j = wave;
        auto arow = [&](int i, int m) {
            return split4(*(const f32x4 *)(nblk(i, m) + r * LNB + q4));
        };
        auto xrow = [&](int i) { return split4(*(const f32x4 *)(sX + (16 * i + r) * LNB + q4)); };
        auto put_tb = [&](int i, f32x4 x) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * i + q4 + e) * LF + w16 + r] = x[e] * bcol;
        };
        if (j <= 2) {
            const Sp xjj = split4(xC);
            f32x4 acc1 = mm3r(arow(j + 1, j), xjj);
            f32x4 acc2 = zero4(), acc3 = zero4();
            if (j + 2 <= 3) acc2 = mm3r(arow(j + 2, j), xjj);
            if (j + 3 <= 3) acc3 = mm3r(arow(j + 3, j), xjj);
            const f32x4 x1 = -mm3r(xrow(j + 1), split4(acc1));
            put_tb(j + 1, x1);
            if (j + 2 <= 3) {
                const Sp sx1 = split4(x1);
                mm3(acc2, arow(j + 2, j + 1), sx1);
                if (j + 3 <= 3) mm3(acc3, arow(j + 3, j + 1), sx1);
                const f32x4 x2 = -mm3r(xrow(j + 2), split4(acc2));
                put_tb(j + 2, x2);
                if (j + 3 <= 3) {
                    mm3(acc3, arow(j + 3, j + 2), split4(x2));
                    const f32x4 x3 = -mm3r(xrow(j + 3), split4(acc3));
                    put_tb(j + 3, x3);
                }
            }
        }
    }
    __syncthreads();
    // T' to the record in 16-byte pieces
    for (int i = tid; i < C * C / 8; i += 256) {
        const int t = i >> 3, c8 = 8 * (i & 7);
        const f32x4 lo = *(const f32x4 *)(sT + t * LF + c8);
        const f32x4 hi = *(const f32x4 *)(sT + t * LF + c8 + 4);
        const bf16x4 bl = __builtin_convertvector(lo, bf16x4);
        const bf16x4 bh = __builtin_convertvector(hi, bf16x4);
        *(bf16x8 *)(rec + kRT + t * C + c8) =
            bf16x8{bl[0], bl[1], bl[2], bl[3], bh[0], bh[1], bh[2], bh[3]};
    }
}

// ======================================================================================
// bwd_states_kernel: S at the start of every chunk of (sequence, head), 32 columns.
// Eight waves; wave w keeps state tiles w, w + 8, ... (16 x 16, row block id / 2, column
// block id % 2) in fp32 accumulators.  Per chunk:
//   X = V - diag(gamma) K S;  U = T' X;  S = gamma_C S + K^T diag(gamma_C / gamma) U
// ======================================================================================
template <int DK>
struct StLds {
    static constexpr int LK = DK + 8;
    // a chunk's inputs, in one of two sets by chunk parity (set stride SET)
    static constexpr int oK = 0;                         // [64][LK]   K
    static constexpr int oT = oK + C * LK * 2;           // [64][L64]  T'
    static constexpr int oV = oT + C * L64 * 2;          // [64][LVT]  V columns
    static constexpr int oGam = oV + C * LVT * 2;
    static constexpr int oRat = oGam + C * 4;
    static constexpr int SET = oRat + C * 4;
    static constexpr int oSt = 2 * SET;                  // [DVT][LK]  S^T (bf16)
    static constexpr int oXt = oSt + DVT * LK * 2;       // [DVT][L64] X^T
    static constexpr int oUt = oXt + DVT * L64 * 2;      // [DVT][L64] (diag(rho) U)^T
    static constexpr int oSf = oUt + DVT * L64 * 2;      // [DK][LSF]  S (fp32), to HBM
    static constexpr int total = oSf + DK * LSF * 4;
};

template <int DK, int DV>
__global__ __launch_bounds__(kThreadsScan) void bwd_states_kernel(BwdArgs a)
{
    using L = StLds<DK>;
    constexpr int LK = L::LK, NT = DV / DVT;
    constexpr int KP = C * DK / 8;                     // 16-byte pieces of K
    constexpr int KPT = (KP + kThreadsScan - 1) / kThreadsScan;
    constexpr int VP = C * DVT / 8;                    // pieces of the V columns
    constexpr int SPW = DK / 64;                       // state tiles per wave
    __shared__ __align__(16) unsigned char smem[L::total];
    uint16_t *sSt = (uint16_t *)(smem + L::oSt);
    uint16_t *sXt = (uint16_t *)(smem + L::oXt), *sUt = (uint16_t *)(smem + L::oUt);
    float *sSf = (float *)(smem + L::oSf);
    const int H = a.H;
    int unit, tile;
    scan_job<NT>(unit, tile);
    const int h = unit % H;
    const int n = unit / H;
    const int col0 = tile * DVT;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q4 = (lane >> 4) * 4;
    const long long r0 = row0_of(a, n);
    const long long slot0 = slot_of(a, n, 0);   // chunk c has slot slot0 + c
    const int len = len_of(a, n);
    const int nch = (len + C - 1) / C;

    f32x4 S[SPW];
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
        const int id = wave + 8 * k, mi = id >> 1, nt = id & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[k][i] = a.s0 ? a.s0[(((long long)n * H + h) * DK + 16 * mi + q4 + i) * DV + col0 +
                                  16 * nt + r]
                           : 0.f;
        put_t(sSt, LK, 16 * mi, 16 * nt, S[k]);
        put_f(sSf, 16 * mi, 16 * nt, S[k]);
    }

    // inputs of a later chunk, fetched two chunks ahead into one of two register sets
    struct Pre {
        u32x4 pk[KPT], pt, pv;
        float pg, pgl;
    };
    Pre ra, rb;
    auto fetch = [&](Pre &R, int c) {
        const long long slot = slot0 + c;
        const long long t0 = r0 + (long long)c * C;
        const int nv = len - c * C < C ? len - c * C : C;
        const uint16_t *rec = a.rec + (slot * H + h) * (long long)kRecHalfs;
        const uint16_t *kb = a.k + (t0 * H + h) * (long long)DK;
        const uint16_t *vb = a.v + (t0 * H + h) * (long long)DV;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = tid + kThreadsScan * j;
            if (i < KP) R.pk[j] = piece_at<DK>(kb, piece_off<DK, DK>(H, 0, i), nv, i);
        }
        R.pt = rec_piece(rec, kRT, tid);
        if (tid < VP) R.pv = piece_at<DVT>(vb, piece_off<DV, DVT>(H, col0, tid), nv, tid);
        if (tid < C) {
            R.pg = ((const float *)(rec + kRG))[tid];
            R.pgl = ((const float *)(rec + kRG))[C - 1];
        }
    };
    // the input set of chunk c
    auto set_of = [&](int c) { return smem + (c & 1) * L::SET; };
    auto commit = [&](const Pre &R, int c) {
        unsigned char *st = set_of(c);
        uint16_t *sK = (uint16_t *)(st + L::oK), *sT = (uint16_t *)(st + L::oT);
        uint16_t *sV = (uint16_t *)(st + L::oV);
        float *gam = (float *)(st + L::oGam), *rat = (float *)(st + L::oRat);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = tid + kThreadsScan * j;
            if (i < KP) put_piece<DK>(sK, LK, i, R.pk[j]);
        }
        put_rec_piece(sT, tid, R.pt);
        if (tid < VP) put_piece<DVT>(sV, LVT, tid, R.pv);
        if (tid < C) {
            gam[tid] = __expf(R.pg);
            rat[tid] = __expf(R.pgl - R.pg);
        }
    };

    if (nch > 0) {
        fetch(ra, 0);
        commit(ra, 0);
    }
    if (nch > 1) fetch(ra, 1);
    __syncthreads();
    const int mt = wave >> 1, nt = wave & 1;          // this wave's c x 32 tile
    // chunk c: LDS set c % 2 holds chunk c, cur holds chunk c + 1 (written into the other set
    // during the state update, that set's last reader being chunk c - 1), nxt receives c + 2
    auto step = [&](int c, Pre &cur, Pre &nxt) {
        const long long slot = slot0 + c;
        unsigned char *st = set_of(c);
        const uint16_t *sK = (const uint16_t *)(st + L::oK), *sT = (const uint16_t *)(st + L::oT);
        const uint16_t *sV = (const uint16_t *)(st + L::oV);
        const float *gam = (const float *)(st + L::oGam), *rat = (const float *)(st + L::oRat);
        if (c + 2 < nch) fetch(nxt, c + 2);
        store_state<DK, DV>(a.hs + ((slot * H + h) * DK) * (long long)DV + col0, sSf);
        // X = V - diag(gamma) K S
        {
            f32x4 acc = zero4();
            mm<false, true>(acc, sK, LK, sSt, LK, 16 * mt, 16 * nt, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + q4 + i;
                acc[i] = bf(sV + t * LVT + 16 * nt + r) - gam[t] * acc[i];
            }
            put_t(sXt, L64, 16 * mt, 16 * nt, acc);
        }
        __syncthreads();
        // U = T' X, kept as diag(gamma_C / gamma) U
        {
            f32x4 acc = zero4();
            mm<false, true>(acc, sT, L64, sXt, L64, 16 * mt, 16 * nt, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= rat[16 * mt + q4 + i];
            put_t(sUt, L64, 16 * mt, 16 * nt, acc);
        }
        __syncthreads();
        // S = gamma_C S + K^T (diag(gamma_C / gamma) U)
        const float gC = gam[C - 1];
#pragma unroll
        for (int k = 0; k < SPW; ++k) {
            const int id = wave + 8 * k, mi = id >> 1, nk = id & 1;
            S[k] *= gC;
            mm<true, true>(S[k], sK, LK, sUt, L64, 16 * mi, 16 * nk, C);
            put_t(sSt, LK, 16 * mi, 16 * nk, S[k]);
            put_f(sSf, 16 * mi, 16 * nk, S[k]);
        }
        if (c + 1 < nch) commit(cur, c + 1);
        __syncthreads();
    };
    for (int c = 0; c < nch; c += 2) {
        step(c, ra, rb);
        if (c + 1 < nch) step(c + 1, rb, ra);
    }
}

// ======================================================================================
// bwd_dstates_kernel: the adjoint D of the state at the end of every chunk, last chunk
// first; dS_0 after the first chunk.  Per chunk:
//   X = P^T dY + diag(gamma_C / gamma) K D;  Z = T'^T X;
//   D = gamma_C D + Q^T diag(gamma) dY - K^T diag(gamma) Z
// ======================================================================================
template <int DK>
struct DsLds {
    static constexpr int LK = DK + 8;
    static constexpr int oK = 0;                         // [64][LK]   K
    static constexpr int oQ = oK + C * LK * 2;           // [64][LK]   Q
    static constexpr int oP = oQ + C * LK * 2;           // [64][L64]  P^T
    static constexpr int oT = oP + C * L64 * 2;          // [64][L64]  T'
    static constexpr int oY = oT + C * L64 * 2;          // [64][LVT]  dY columns
    static constexpr int oYg = oY + C * LVT * 2;         // [64][LVT]  diag(gamma) dY
    static constexpr int oDt = oYg + C * LVT * 2;        // [DVT][LK]  D^T (bf16)
    static constexpr int oXt = oDt + DVT * LK * 2;       // [DVT][L64] X^T
    static constexpr int oZt = oXt + DVT * L64 * 2;      // [DVT][L64] (-diag(gamma) Z)^T
    static constexpr int oGam = oZt + DVT * L64 * 2;
    static constexpr int oRat = oGam + C * 4;
    static constexpr int oDf = oRat + C * 4;             // [DK][LSF]  D (fp32), to HBM
    static constexpr int total = oDf + DK * LSF * 4;
};

template <int DK, int DV>
__global__ __launch_bounds__(kThreadsScan) void bwd_dstates_kernel(BwdArgs a)
{
    using L = DsLds<DK>;
    constexpr int LK = L::LK, NT = DV / DVT;
    constexpr int KP = C * DK / 8;
    constexpr int KPT = (KP + kThreadsScan - 1) / kThreadsScan;
    constexpr int VP = C * DVT / 8;
    constexpr int SPW = DK / 64;
    __shared__ __align__(16) unsigned char smem[L::total];
    uint16_t *sK = (uint16_t *)(smem + L::oK), *sQ = (uint16_t *)(smem + L::oQ);
    uint16_t *sP = (uint16_t *)(smem + L::oP), *sT = (uint16_t *)(smem + L::oT);
    uint16_t *sY = (uint16_t *)(smem + L::oY), *sYg = (uint16_t *)(smem + L::oYg);
    uint16_t *sDt = (uint16_t *)(smem + L::oDt), *sXt = (uint16_t *)(smem + L::oXt);
    uint16_t *sZt = (uint16_t *)(smem + L::oZt);
    float *gam = (float *)(smem + L::oGam), *rat = (float *)(smem + L::oRat);
    float *sDf = (float *)(smem + L::oDf);
    const int H = a.H;
    int unit, tile;
    scan_job<NT>(unit, tile);
    const int h = unit % H;
    const int n = unit / H;
    const int col0 = tile * DVT;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q4 = (lane >> 4) * 4;
    const long long r0 = row0_of(a, n);
    const long long slot0 = slot_of(a, n, 0);   // chunk c has slot slot0 + c
    const int len = len_of(a, n);
    const int nch = (len + C - 1) / C;

    f32x4 D[SPW];
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
        const int id = wave + 8 * k, mi = id >> 1, nt = id & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            D[k][i] = a.ds_final ? a.ds_final[(((long long)n * H + h) * DK + 16 * mi + q4 + i) *
                                                  DV + col0 + 16 * nt + r]
                                 : 0.f;
        put_t(sDt, LK, 16 * mi, 16 * nt, D[k]);
        put_f(sDf, 16 * mi, 16 * nt, D[k]);
    }

    struct Pre {
        u32x4 pk[KPT], pq[KPT], pp, pt, py;
        float pg, pgl, pgy;
    };
    Pre ra, rb;
    auto fetch = [&](Pre &R, int c) {
        const long long slot = slot0 + c;
        const long long t0 = r0 + (long long)c * C;
        const int nv = len - c * C < C ? len - c * C : C;
        const uint16_t *rec = a.rec + (slot * H + h) * (long long)kRecHalfs;
        const float *rg = (const float *)(rec + kRG);
        const long long rb = (t0 * H + h) * (long long)DK;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = tid + kThreadsScan * j;
            if (i < KP) {
                const int o = piece_off<DK, DK>(H, 0, i);
                R.pk[j] = piece_at<DK>(a.k + rb, o, nv, i);
                R.pq[j] = piece_at<DK>(a.q + rb, o, nv, i);
            }
        }
        R.pp = rec_piece(rec, kRP, tid);
        R.pt = rec_piece(rec, kRT, tid);
        if (tid < VP) {
            R.py = piece_at<DVT>(a.dy + (t0 * H + h) * (long long)DV,
                                 piece_off<DV, DVT>(H, col0, tid), nv, tid);
            R.pgy = rg[tid / (DVT / 8)];
        }
        if (tid < C) {
            R.pg = rg[tid];
            R.pgl = rg[C - 1];
        }
    };
    auto commit = [&](const Pre &R) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = tid + kThreadsScan * j;
            if (i < KP) {
                put_piece<DK>(sK, LK, i, R.pk[j]);
                put_piece<DK>(sQ, LK, i, R.pq[j]);
            }
        }
        put_rec_piece(sP, tid, R.pp);
        put_rec_piece(sT, tid, R.pt);
        if (tid < VP) {
            put_piece<DVT>(sY, LVT, tid, R.py);
            put_piece<DVT>(sYg, LVT, tid, scale_piece(R.py, __expf(R.pgy)));
        }
        if (tid < C) {
            gam[tid] = __expf(R.pg);
            rat[tid] = __expf(R.pgl - R.pg);
        }
    };

    if (nch > 0) {
        fetch(ra, nch - 1);
        commit(ra);
    }
    if (nch > 1) fetch(ra, nch - 2);
    __syncthreads();
    const int mt = wave >> 1, nt = wave & 1;
    // chunk c: LDS holds chunk c, cur holds chunk c - 1, nxt receives chunk c - 2
    auto step = [&](int c, Pre &cur, Pre &nxt) {
        const long long slot = slot0 + c;
        if (c >= 2) fetch(nxt, c - 2);
        store_state<DK, DV>(a.dhs + ((slot * H + h) * DK) * (long long)DV + col0, sDf);
        // X = P^T dY + diag(gamma_C / gamma) K D
        {
            f32x4 a1 = zero4(), a2 = zero4();
            mm<false, false>(a1, sP, L64, sY, LVT, 16 * mt, 16 * nt, C);
            mm<false, true>(a2, sK, LK, sDt, LK, 16 * mt, 16 * nt, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i) a1[i] += rat[16 * mt + q4 + i] * a2[i];
            put_t(sXt, L64, 16 * mt, 16 * nt, a1);
        }
        __syncthreads();
        // Z = T'^T X, kept as -diag(gamma) Z
        {
            f32x4 acc = zero4();
            mm<true, true>(acc, sT, L64, sXt, L64, 16 * mt, 16 * nt, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= -gam[16 * mt + q4 + i];
            put_t(sZt, L64, 16 * mt, 16 * nt, acc);
        }
        __syncthreads();
        // D = gamma_C D + Q^T (diag(gamma) dY) + K^T (-diag(gamma) Z)
        const float gC = gam[C - 1];
#pragma unroll
        for (int k = 0; k < SPW; ++k) {
            const int id = wave + 8 * k, mi = id >> 1, nk = id & 1;
            D[k] *= gC;
            mm<true, false>(D[k], sQ, LK, sYg, LVT, 16 * mi, 16 * nk, C);
            mm<true, true>(D[k], sK, LK, sZt, L64, 16 * mi, 16 * nk, C);
            put_t(sDt, LK, 16 * mi, 16 * nk, D[k]);
            put_f(sDf, 16 * mi, 16 * nk, D[k]);
        }
        __syncthreads();
        if (c > 0) commit(cur);
        __syncthreads();
    };
    for (int c = nch - 1; c >= 0; c -= 2) {
        step(c, ra, rb);
        if (c >= 1) step(c - 1, rb, ra);
    }
    if (a.ds0) {
#pragma unroll
        for (int k = 0; k < SPW; ++k) {
            const int id = wave + 8 * k, mi = id >> 1, nk = id & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.ds0[(((long long)n * H + h) * DK + 16 * mi + q4 + i) * DV + col0 + 16 * nk +
                      r] = D[k][i];
        }
    }
}

// ======================================================================================
// bwd_chunk_kernel: per (chunk slot, head), eight waves.  Passes over the value columns in
// blocks of 32 accumulate the products that contract over d_v; the rest follows.
// ======================================================================================
template <int DK>
struct CkLds {
    static constexpr int LK = DK + 8;
    // kept for the whole chunk
    static constexpr int oK = 0;                          // [64][LK]   K
    static constexpr int oT = oK + C * LK * 2;            // [64][L64]  T'
    static constexpr int oP = oT + C * L64 * 2;           // [64][L64]  P^T
    static constexpr int oLt = oP + C * L64 * 2;          // [64][L64]  L^T
    static constexpr int oG = oLt + C * L64 * 2;          // g, gamma, rho, beta [64] fp32
    static constexpr int oGam = oG + C * 4;
    static constexpr int oRat = oGam + C * 4;
    static constexpr int oBet = oRat + C * 4;
    static constexpr int oDbp = oBet + C * 4;             // [2][64] dbeta partials
    static constexpr int oBlk = oDbp + 2 * C * 4;
    // one pass over 32 value columns
    // (S, D, R and U also as the remainders of their bf16 rounding: *l)
    static constexpr int oS = oBlk;                       // [DK][LVT]  S columns
    static constexpr int oSl = oS + DK * LVT * 2;
    static constexpr int oD = oSl + DK * LVT * 2;         // [DK][LVT]  D columns
    static constexpr int oDl = oD + DK * LVT * 2;
    static constexpr int oV = oDl + DK * LVT * 2;         // [64][LVT]  V columns
    static constexpr int oY = oV + C * LVT * 2;           // [64][LVT]  dY columns
    static constexpr int oRt = oY + C * LVT * 2;          // [32][L64]  R^T
    static constexpr int oRtl = oRt + DVB * L64 * 2;
    static constexpr int oUt = oRtl + DVB * L64 * 2;      // U^T
    static constexpr int oUtl = oUt + DVB * L64 * 2;
    static constexpr int oDUt = oUtl + DVB * L64 * 2;     // dU^T
    static constexpr int oZt = oDUt + DVB * L64 * 2;      // Z^T
    static constexpr int oEt = oZt + DVB * L64 * 2;       // E^T
    static constexpr int blkEnd = oEt + DVB * L64 * 2;
    // after the passes (the pass region is free)
    static constexpr int oQ = oBlk;                       // [64][LK]   Q
    static constexpr int oDPt = oQ + C * LK * 2;          // [64][L64]  (dP (.) Gamma)^T
    static constexpr int oDLt = oDPt + C * L64 * 2;       // [64][L64]  (dL (.) Gamma)^T
    static constexpr int oPart = oDLt + C * L64 * 2;      // row-sum partials (fp32)
    static constexpr int partFloats = 20 * C + 40;
    // each wave's dq and dk tiles (bf16, 16 x 16 each, rows of 32 bytes) before their store
    static constexpr int SL = 16;
    static constexpr int NQW = DK / 16 * 4 / 8;           // c x d_k tiles per wave
    static constexpr int oStg = (oPart + partFloats * 4 + 15) / 16 * 16;
    static constexpr int stgHalfs = NQW * 2 * 16 * SL;    // per wave
    static_assert(oStg + 8 * stgHalfs * 2 <= blkEnd, "the after-pass data fits the pass region");
    static constexpr int total = blkEnd;
};

template <int DK, int DV>
__global__ __launch_bounds__(512) void bwd_chunk_kernel(BwdArgs a)
{
    using L = CkLds<DK>;
    constexpr int LK = L::LK;
    constexpr int KT = DK / 16;                 // 16-column tiles of d_k
    constexpr int NQ = 4 * KT / 8;              // c x d_k tiles per wave
    constexpr int KP = C * DK / 8;
    __shared__ __align__(16) unsigned char smem[L::total];
    uint16_t *sK = (uint16_t *)(smem + L::oK), *sT = (uint16_t *)(smem + L::oT);
    uint16_t *sP = (uint16_t *)(smem + L::oP), *sLt = (uint16_t *)(smem + L::oLt);
    float *g = (float *)(smem + L::oG), *gam = (float *)(smem + L::oGam);
    float *rat = (float *)(smem + L::oRat), *bet = (float *)(smem + L::oBet);
    float *dbp = (float *)(smem + L::oDbp);
    uint16_t *sS = (uint16_t *)(smem + L::oS), *sD = (uint16_t *)(smem + L::oD);
    uint16_t *sSl = (uint16_t *)(smem + L::oSl), *sDl = (uint16_t *)(smem + L::oDl);
    uint16_t *sRtl = (uint16_t *)(smem + L::oRtl), *sUtl = (uint16_t *)(smem + L::oUtl);
    uint16_t *sV = (uint16_t *)(smem + L::oV), *sY = (uint16_t *)(smem + L::oY);
    uint16_t *sRt = (uint16_t *)(smem + L::oRt), *sUt = (uint16_t *)(smem + L::oUt);
    uint16_t *sDUt = (uint16_t *)(smem + L::oDUt), *sZt = (uint16_t *)(smem + L::oZt);
    uint16_t *sEt = (uint16_t *)(smem + L::oEt);
    uint16_t *sQ = (uint16_t *)(smem + L::oQ), *sDPt = (uint16_t *)(smem + L::oDPt);
    uint16_t *sDLt = (uint16_t *)(smem + L::oDLt);

    const int H = a.H;
    const long long slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int n, c, nv;
    long long t0;
    if (!decode_slot(a, slot, n, c, t0, nv)) return;
    const uint16_t *rec = a.rec + (slot * H + h) * (long long)kRecHalfs;
    const float *hs = a.hs + (slot * H + h) * (long long)DK * DV;
    const float *dhs = a.dhs + (slot * H + h) * (long long)DK * DV;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q4 = (lane >> 4) * 4;

    // K, the record's T', P^T and g, and beta and alpha of the chunk's rows (clamped into the
    // chunk) go out at once; Q follows with the first pass's S and D and is held in
    // registers until the passes are done.
    constexpr int NP = (KP + 511) / 512;
    u32x4 qx[NP];
    float al;
    {
        u32x4 kx[NP];
#pragma unroll
        for (int u = 0; u < NP; ++u)
            kx[u] = piece_clamped<DK, DK>(a.k, t0, nv, H, h, 0, (tid + 512 * u) % KP);
        const u32x4 tx = rec_piece(rec, kRT, tid), px = rec_piece(rec, kRP, tid);
        const int tc = tid % C < nv ? tid % C : nv - 1;
        const float gt = ((const float *)(rec + kRG))[tid % C];
        const float gl = ((const float *)(rec + kRG))[C - 1];
        const float bt = a.beta[(t0 + tc) * H + h];
        al = a.alpha[(t0 + tc) * H + h];
#pragma unroll
        for (int u = 0; u < NP; ++u)
            if (KP % 512 == 0 || tid + 512 * u < KP)
                put_piece<DK>(sK, LK, tid + 512 * u, piece_keep<DK>(kx[u], nv, tid + 512 * u));
        put_rec_piece(sT, tid, tx);
        put_rec_piece(sP, tid, px);
        // every thread stores its row's gate values (the eight threads of a row store the same
        // values), so the gate loads are not held back behind a branch
        const int tr = tid % C;
        g[tr] = gt;
        gam[tr] = __expf(gt);
        rat[tr] = __expf(gl - gt);
        bet[tr] = tr < nv ? bt : 0.f;
        dbp[tr] = 0.f;
        dbp[C + tr] = 0.f;
    }
    __syncthreads();
    // L = strictlower(K K^T (.) Gamma), stored transposed: 16 tiles, two per wave
#pragma unroll
    for (int tile = wave; tile < 16; tile += 8) {
        const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
        f32x4 kk = zero4();
        mm<false, true>(kk, sK, LK, sK, LK, m0, n0, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = m0 + q4 + i, s = n0 + r;
            kk[i] = s < t ? kk[i] * decay(g, t, s) : 0.f;
        }
        put_t(sLt, L64, m0, n0, kk);
    }

    // accumulators over the passes (c x c tiles wave, wave + 8; c x d_k tiles wave + 8 j)
    f32x4 accM[2], accEu[2], accGq[NQ], accGa[NQ], accGb[NQ];
#pragma unroll
    for (int i = 0; i < 2; ++i) accM[i] = accEu[i] = zero4();
#pragma unroll
    for (int i = 0; i < NQ; ++i) accGq[i] = accGa[i] = accGb[i] = zero4();
    float sd = 0.f;                             // partial <S, D>
    const int mt = wave >> 1, nt = wave & 1;    // this wave's c x 32 tile of a pass

    // the next pass's S and D columns (fp32) and V or dY columns are fetched into registers
    // while the current pass computes
    constexpr int SP = DK * DVB / 4 / 512;
    f32x4 ps[SP], pd[SP];
    u32x4 pvy;
    auto fetch = [&](int col0) {
#pragma unroll
        for (int j = 0; j < SP; ++j) {
            const int i = tid + 512 * j;
            const int row = i / (DVB / 4), c4 = 4 * (i % (DVB / 4));
            ps[j] = *(const f32x4 *)(hs + row * DV + col0 + c4);
            pd[j] = *(const f32x4 *)(dhs + row * DV + col0 + c4);
        }
        // V for the first 256 threads, dY for the rest: one load on either side
        const uint16_t *src = tid < C * DVB / 8 ? a.v : a.dy;
        pvy = piece_clamped<DV, DVB>(src, t0, nv, H, h, col0, tid % (C * DVB / 8));
    };
    auto commit = [&]() {
#pragma unroll
        for (int j = 0; j < SP; ++j) {
            const int i = tid + 512 * j;
            const int row = i / (DVB / 4), c4 = 4 * (i % (DVB / 4));
            const f32x4 s4 = ps[j], d4 = pd[j];
            sd += s4[0] * d4[0] + s4[1] * d4[1] + s4[2] * d4[2] + s4[3] * d4[3];
            const bf16x4 sh = __builtin_convertvector(s4, bf16x4);
            const bf16x4 dh = __builtin_convertvector(d4, bf16x4);
            *(bf16x4 *)(sS + row * LVT + c4) = sh;
            *(bf16x4 *)(sD + row * LVT + c4) = dh;
            *(bf16x4 *)(sSl + row * LVT + c4) =
                __builtin_convertvector(s4 - __builtin_convertvector(sh, f32x4), bf16x4);
            *(bf16x4 *)(sDl + row * LVT + c4) =
                __builtin_convertvector(d4 - __builtin_convertvector(dh, f32x4), bf16x4);
        }
        const int iv = tid % (C * DVB / 8);
        put_piece<DVB>(tid < C * DVB / 8 ? sV : sY, LVT, iv, piece_keep<DVB>(pvy, nv, iv));
    };
    static_assert(2 * C * DVB / 8 == 512 && SP >= 1, "one V or dY piece per thread");

#pragma unroll
    for (int u = 0; u < NP; ++u)
        qx[u] = piece_clamped<DK, DK>(a.q, t0, nv, H, h, 0, (tid + 512 * u) % KP);
    fetch(0);
    for (int col0 = 0; col0 < DV; col0 += DVB) {
        __syncthreads();   // the previous pass is done (and L^T written before the first)
        commit();
        __syncthreads();
        fetch(col0 + DVB < DV ? col0 + DVB : col0);   // the last pass: its own columns again
        // phase 1: R = V - diag(gamma) K S;  diag(gamma_C / gamma) K D (kept in registers)
        f32x4 R = zero4(), kd = zero4();
        mm<false, false>(R, sK, LK, sS, LVT, 16 * mt, 16 * nt, DK);
        mm<false, false>(kd, sK, LK, sD, LVT, 16 * mt, 16 * nt, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * mt + q4 + i;
            R[i] = bf(sV + t * LVT + 16 * nt + r) - gam[t] * R[i];
            kd[i] *= rat[t];
        }
        put_t2(sRt, sRtl, L64, 16 * mt, 16 * nt, R);
        __syncthreads();
        // phase 2: U = T' R;  dU = P^T dY + diag(gamma_C / gamma) K D
        {
            f32x4 U = zero4();
            mm2<false, true>(U, sT, L64, sRt, sRtl, L64, 16 * mt, 16 * nt, C);
            put_t2(sUt, sUtl, L64, 16 * mt, 16 * nt, U);
        }
        f32x4 dU = kd;
        mm<false, false>(dU, sP, L64, sY, LVT, 16 * mt, 16 * nt, C);
        put_t(sDUt, L64, 16 * mt, 16 * nt, dU);
        __syncthreads();
        // phase 3: Z = T'^T dU (= dV)
        {
            f32x4 Z = zero4();
            mm<true, true>(Z, sT, L64, sDUt, L64, 16 * mt, 16 * nt, C);
            put_t(sZt, L64, 16 * mt, 16 * nt, Z);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + q4 + i;
                if (t < nv)
                    Elem<uint16_t>::store(a.dv + ((t0 + t) * H + h) * (long long)DV + col0 +
                                              16 * nt + r, Z[i]);
            }
        }
        __syncthreads();
        // phase 4: E = dU - L^T Z;  dbeta_t += sum_j E_tj R_tj
        {
            f32x4 lz = zero4();
            mm<false, true>(lz, sLt, L64, sZt, L64, 16 * mt, 16 * nt, C);
            const f32x4 E = dU - lz;
            put_t(sEt, L64, 16 * mt, 16 * nt, E);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = sum16(E[i] * R[i]);
                if (r == 0) dbp[nt * C + 16 * mt + q4 + i] += s;   // one writer per (nt, t)
            }
        }
        __syncthreads();
        // phase 5: M += dY U^T, Eu += E U^T (c x c);  Gq += dY S^T, Ga += Z S^T, Gb += U D^T
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + 8 * i;
            const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
            mm2<false, false>(accM[i], sY, LVT, sUt, sUtl, L64, m0, n0, DVB);
            mm<true, false>(accEu[i], sEt, L64, sUt, L64, m0, n0, DVB);
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int tile = wave + 8 * i;
            const int m0 = 16 * (tile / KT), n0 = 16 * (tile % KT);
            mm2<false, true>(accGq[i], sY, LVT, sS, sSl, LVT, m0, n0, DVB);
            mm2<true, true>(accGa[i], sZt, L64, sS, sSl, LVT, m0, n0, DVB);
            mm2<true, true>(accGb[i], sUt, L64, sD, sDl, LVT, m0, n0, DVB);
        }
    }
    __syncthreads();   // the pass region now takes Q, (dP (.) Gamma)^T, (dL (.) Gamma)^T, partials

#pragma unroll
    for (int u = 0; u < NP; ++u)
        if (KP % 512 == 0 || tid + 512 * u < KP)
            put_piece<DK>(sQ, LK, tid + 512 * u, piece_keep<DK>(qx[u], nv, tid + 512 * u));
    // Row sums are written per source tile and added in a fixed order afterwards, so every
    // output is bitwise repeatable.
    //   pG[kt][t]  row dot of the c x d_k accumulators, column tile kt
    //   pR[ct][t]  row sums of dP (.) P + dL (.) L over column tile ct
    //   pC[rt][s]  column sums of the same over row tile rt
    //   pB[ct][t]  row sums of L (.) Eu over column tile ct
    //   pX[...]    per-tile sums of K (.) Gb (up to 32) and per-wave partials of <S, D> (8)
    float *pG = (float *)(smem + L::oPart);
    float *pR = pG + 8 * C, *pC = pR + 4 * C, *pB = pC + 4 * C, *pX = pB + 4 * C;
    __syncthreads();
    // Every LDS operand of the sums below is read before any sum is stored, so the reads go
    // out together.
    float qv[NQ][4], kv[NQ][4], gm[NQ][4], rt[NQ][4];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile / KT), n0 = 16 * (tile % KT);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = m0 + q4 + ii, col = n0 + r;
            qv[i][ii] = bf(sQ + t * LK + col);
            kv[i][ii] = bf(sK + t * LK + col);
            gm[i][ii] = gam[t];
            rt[i][ii] = rat[t];
        }
    }
    float gt2[2][4], gs2[2][4], lv2[2][4], pv2[2][4], bt2[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = m0 + q4 + ii, s = n0 + r;
            gt2[i][ii] = g[t];
            gs2[i][ii] = g[s];
            bt2[i][ii] = bet[t];
        }
        // L^T and P^T hold the four rows t of a lane next to each other
        const bf16x4 l4 = *(const bf16x4 *)(sLt + (n0 + r) * L64 + m0 + q4);
        const bf16x4 p4 = *(const bf16x4 *)(sP + (n0 + r) * L64 + m0 + q4);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            lv2[i][ii] = (float)l4[ii];
            pv2[i][ii] = (float)p4[ii];
        }
    }
    // row dots of the c x d_k accumulators
    float dG[NQ][4], xs[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        xs[i] = 0.f;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            accGq[i][ii] *= gm[i][ii];
            accGa[i][ii] *= -gm[i][ii];
            accGb[i][ii] *= rt[i][ii];
            const float xb = kv[i][ii] * accGb[i][ii];
            dG[i][ii] = sum16(qv[i][ii] * accGq[i][ii] + kv[i][ii] * accGa[i][ii] - xb);
            xs[i] += xb;
        }
        xs[i] = sum64(xs[i]);
    }
    const float sdw = sum64(sd);
    // dP = lower_incl(M), dL = -diag(beta) strictlower(Eu) and their decayed forms;
    // dg from (dP (.) P + dL (.) L): + row sums, - column sums;  dbeta -= sum_i L (.) Eu
    f32x4 dpg[2], dlg[2];
    float rs[2][4], bs[2][4], cs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
        cs[i] = 0.f;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = m0 + q4 + ii, s = n0 + r;
            const float e = __expf(fminf(gt2[i][ii] - gs2[i][ii], 0.f));
            const float G = s <= t ? e : 0.f;
            const float dP = s <= t ? accM[i][ii] : 0.f;
            const float dL = s < t ? -bt2[i][ii] * accEu[i][ii] : 0.f;
            dpg[i][ii] = dP * G;
            dlg[i][ii] = dL * G;
            const float w = dP * pv2[i][ii] + dL * lv2[i][ii];
            rs[i][ii] = sum16(w);
            bs[i][ii] = sum16(s < t ? lv2[i][ii] * accEu[i][ii] : 0.f);
            cs[i] += w;
        }
        cs[i] = row_sum4(cs[i]);
    }
    // the sums and the decayed tiles to LDS
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile / KT), n0 = 16 * (tile % KT);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            if (r == 0) pG[(n0 / 16) * C + m0 + q4 + ii] = dG[i][ii];
        if (lane == 0) pX[tile] = xs[i];
    }
    if (lane == 0) pX[32 + wave] = sdw;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile >> 2), n0 = 16 * (tile & 3);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            if (r == 0) {
                pR[(n0 / 16) * C + m0 + q4 + ii] = rs[i][ii];
                pB[(n0 / 16) * C + m0 + q4 + ii] = bs[i][ii];
            }
        }
        put_t(sDPt, L64, m0, n0, dpg[i]);
        put_t(sDLt, L64, m0, n0, dlg[i]);
        if (lane < 16) pC[(m0 / 16) * C + n0 + r] = cs[i];
    }
    __syncthreads();
    // dQ = Gq + (dP (.) Gamma) K;  dK = Ga + Gb + (dP (.) Gamma)^T Q + (dL (.) Gamma) K
    //                                   + (dL (.) Gamma)^T K
    // The wave's tiles go to its own LDS block and from there to HBM in 16-byte pieces (one
    // wave's LDS accesses complete in order, so no barrier stands between the two).
    constexpr int SL = L::SL;
    static_assert(L::NQW == NQ, "tiles per wave");
    __bf16 *stg = (__bf16 *)(smem + L::oStg) + wave * L::stgHalfs;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int tile = wave + 8 * i;
        const int m0 = 16 * (tile / KT), n0 = 16 * (tile % KT);
        f32x4 aq = accGq[i];
        mm<true, false>(aq, sDPt, L64, sK, LK, m0, n0, C);
        f32x4 ak = accGa[i] + accGb[i];
        mm<false, false>(ak, sDPt, L64, sQ, LK, m0, n0, C);
        mm<true, false>(ak, sDLt, L64, sK, LK, m0, n0, C);
        mm<false, false>(ak, sDLt, L64, sK, LK, m0, n0, C);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            stg[((2 * i) * 16 + q4 + ii) * SL + r] = (__bf16)aq[ii];
            stg[((2 * i + 1) * 16 + q4 + ii) * SL + r] = (__bf16)ak[ii];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        // piece (tile i, dq or dk, row rr of the tile, half hf of its 16 columns)
        const int pc = lane + 64 * j;
        const int hf = pc & 1, rr = (pc >> 1) & 15, ten = (pc >> 5) & 1, i = pc >> 6;
        const int tile = wave + 8 * i;
        const int t = 16 * (tile / KT) + rr, n0 = 16 * (tile % KT);
        const u32x4 x = *(const u32x4 *)(stg + ((2 * i + ten) * 16 + rr) * SL + 8 * hf);
        if (t < nv)
            *(u32x4 *)((ten ? a.dk : a.dq) + ((t0 + t) * H + h) * (long long)DK + n0 + 8 * hf) = x;
    }
    // dlog alpha = reverse prefix of dg (the chunk-end terms land on the last slot)
    if (tid < C) {
        const int t = tid;
        float x = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) x += pG[kt * C + t];
        float bt = dbp[t] + dbp[C + t];
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
        x = suffix_sum64(x);
        if (t < nv) {
            const long long o = (t0 + t) * H + h;
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
                       dim3(kThreadsScan), 0, stream, a);
    hipLaunchKernelGGL((bwd_dstates_kernel<DK, DV>), dim3((unsigned)(units * (DV / DVT))),
                       dim3(kThreadsScan), 0, stream, a);
    hipLaunchKernelGGL((bwd_chunk_kernel<DK, DV>), dim3((unsigned)slots), dim3(512), 0, stream,
                       a);
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t backward_workspace_bytes(int num_seqs, long long total_T, int H, int dk, int dv)
{
    const long long nslots = total_T / kChunk + num_seqs;
    const size_t rec = align256((size_t)nslots * H * kRecHalfs * 2);
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
    const size_t rec = align256((size_t)a.nslots * p.H * kRecHalfs * 2);
    const size_t st = align256((size_t)a.nslots * p.H * p.dk * p.dv * 4);
    a.rec = (uint16_t *)workspace;
    a.hs = (float *)((unsigned char *)workspace + rec);
    a.dhs = (float *)((unsigned char *)workspace + rec + st);
    if (p.dk == 128 && p.dv == 128) return launch_bwd_dims<128, 128>(a, stream);
    if (p.dk == 128 && p.dv == 64) return launch_bwd_dims<128, 64>(a, stream);
    if (p.dk == 64 && p.dv == 128) return launch_bwd_dims<64, 128>(a, stream);
    return launch_bwd_dims<64, 64>(a, stream);
}

}  // namespace gdn
