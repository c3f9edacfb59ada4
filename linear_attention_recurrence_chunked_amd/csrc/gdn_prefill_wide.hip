// gdn_prefill_wide.hip -- bf16 prefill for d_k = d_v = 128 in one launch: one workgroup per
// (segment of a sequence, head) carries the whole 128 x 128 fp32 state and forms every
// chunk-local quantity itself, so nothing but the inputs, y and the states crosses HBM.
//
// The chunk algebra is the WY / UT form of the reading notes' transition-matrix recurrence
// (Gated DeltaNet, section 2.1), with g the in-chunk inclusive prefix of log2 alpha,
// gamma = 2^g, Gamma_ti = gamma_t / gamma_i, A = diag(beta) strictlower(K K^T (.) Gamma),
// T' = (I + A)^{-1} diag(beta), P = lower_incl(Q K^T (.) Gamma):
//
//     R = V - diag(gamma) K S,   U = T' R,   Y = diag(gamma) Q S + P U,
//     S <- gamma_C S + (diag(gamma_C / gamma) K)^T U.
//
// Twelve waves.  Waves 0-7 ("column waves") own 16 state columns each and run, for chunk j:
// K S, R, U = T' R, the state update, Shat^T Q^T of chunk j and Y of chunk j-1 (P of chunk
// j-1 arrives a step later).  Waves 8-11 ("prep waves") issue the direct-to-LDS copies of
// the chunks ahead and, for chunk j+1, form g, the Gram blocks, T' (blocked inversion, one
// 16 x 16 block row per wave) and the decay factors, and P of chunk j.  One workgroup barrier
// per chunk step; the prep waves meet once more inside a step through an LDS counter.
//
// Segments (long sequences, few chains).  A segment that does not start its sequence needs
// the state at its first token.  Its workgroup first scans, from a zero state and without
// writing y, the W chunks before it, where W is the least number of whole chunks over which
// the transition norm provably falls below 2^-48: per token
// ||alpha (I - beta k k^T)||_2 = alpha max(1, |1 - beta ||k||^2|), so the product of these
// over the window bounds how much of the true start state the warm-up omits (relative to the
// state at the window's start).  W is chosen from alpha alone and then verified with the
// keys; when no window within one segment reaches the bound (decay too slow), or the
// verification fails, the workgroup instead waits for the previous segment's workgroup to
// publish its exact end state (workgroups take their jobs in increasing order from an atomic
// counter, so the one waited for has already started and never waits on a later one).
#include <type_traits>

#include "gdn_prefill_ops.hpp"

namespace gdn {

constexpr int kWideCol = 8;                 // column waves, 16 state columns each
constexpr int kWidePrep = 4;                // prep waves
constexpr int kWideWaves = kWideCol + kWidePrep;
constexpr float kWarmBound = -48.f;         // log2 transition-norm bound a warm-up must reach
constexpr float kWarmAlpha = -50.f;         // the window choice on log2 alpha alone

template <int DK, int DV>
struct LdsWide {
    static constexpr int szK = kChunk * DK * 2;        // [64][DK] bf16 (K and Q tiles)
    static constexpr int szV = kChunk * DV * 2;        // [64][DV] bf16
    static constexpr int szT = kChunk * kChunk * 2;    // T' as a 64-wide swizzled tile
    static constexpr int szP = 6 * 1024;               // P as six operand fragments
    static constexpr int szF = 5 * kChunk * 4 + 16;    // gamma 2^ls, rho, g_C, g, 2^g, 2^-g
    static constexpr int szPG = 4 * kChunk * 4;        // a prep wave's g, beta, 2^g, 2^-g
    static constexpr int szY = kChunk * DV * 2;        // y of a chunk, bf16 rows (staging)
    static constexpr int LDB = 16;                     // fp32 rows of an A block
    static constexpr int LDX = 16;                     // rows of a diagonal X block
    static constexpr int sK = 0;                       // chunk j in stage j % 3
    static constexpr int sQ = sK + 3 * szK;            // chunk j in stage j % 2
    static constexpr int sV = sQ + 2 * szK;            // chunk j in stage j % 2
    static constexpr int sT = sV + 2 * szV;            // T' of the chunk being scanned, then of the next
    static constexpr int sP = sT + szT;                // P of the chunk whose y is formed next
    static constexpr int sY = sP + szP;                // y rows on their way to memory
    static constexpr int sAB = sY + szY;               // raw gates [alpha 64][beta 64], j % 2
    static constexpr int sF = sAB + 2 * 512;           // factors of chunk j in buffer j % 2
    static constexpr int sPG = sF + 2 * szF;           // [prep wave] g, beta, 2^g, 2^-g
    static constexpr int sA = sPG + kWidePrep * szPG;  // six strictly lower A blocks
    static constexpr int sX = sA + 6 * 16 * LDB * 4;        // four diagonal X blocks
    static constexpr int sMisc = sX + 4 * 16 * LDX * 4;
    static constexpr int total = sMisc + 256;
    static_assert(total <= 160 * 1024, "LDS");
};

// misc words (int or float)
enum {
    kMiscPbar = 0,       // prep-wave barrier counter
    kMiscJob = 1,        // job id
    kMiscLamWin = 2,     // running log2 bound over the warm-up chunks (float)
    kMiscLamPart = 4,    // [2][4] per-wave key terms of a chunk's bound (float)
    kMiscSums = 16,      // [12] window search: log2 alpha sums of chunks (float)
    kMiscCntT = 28,      // column waves that read the T' of their chunk (one count per step)
    kMiscCntP = 29,      // column waves that read the P of the previous chunk (one per step)
    kMiscCntY = 30,      // column waves that staged their y pieces
};

// The gate parameters of one head: alpha itself, or its pre-activation a with
// log2 alpha = -e^A softplus(a + b_alpha) / ln 2 (read once per workgroup).
struct GateHead {
    bool pre;        // gates given as pre-activations
    float scale;     // -e^A / ln 2
    float b_alpha;
};

// log2 alpha of one (token, head), clamped like the scan's decay prefix
__device__ __forceinline__ float wide_log2_alpha(const GateHead &g, float x)
{
    if (g.pre) {
        const float u = x + g.b_alpha;
        const float sp = u > 20.f ? u : log1pf(__expf(u));
        return fmaxf(g.scale * sp, kLog2AlphaFloor);
    }
    return fmaxf(__builtin_amdgcn_logf(x), kLog2AlphaFloor);
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += wave_xor(x, m);
    return x;
}

// V tile byte address: 256-byte rows, granule g of row r at slot g ^ 4 (r % 4), so the four
// rows a transposing read meets land on distinct slots.
template <int DV>
__device__ __forceinline__ int vswz(int row, int col)
{
    const int b = col * 2;
    return row * (DV * 2) + ((((b >> 4) ^ ((row & 3) << 2))) << 4) + (b & 15);
}

// Direct-to-LDS copies (lane l's 16 or 4 bytes land at lds + 16 l or lds + 4 l) from a
// wave-uniform base address plus a 32-bit per-lane byte offset, written in inline asm so
// that the compiler does not treat the wave's later LDS reads as waiting on them: the prep
// waves read other stages while these copies fly, and wait for them (s_waitcnt vmcnt(0))
// only before the step barrier that hands them to their readers.  The instruction has no
// register output; M0 carries the LDS address.  The compiler does not honour a clobber of M0
// (it warns so), which is safe here only because nothing else in this kernel uses M0: its
// AMD assembly holds no M0 access besides these copies' own "s_mov_b32 m0" (no indexed
// register moves, no messages, no compiler-emitted direct-to-LDS loads).
__device__ __forceinline__ unsigned lds_addr(const void *p)
{
    return (unsigned)(size_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void copy16_async(const void *base, unsigned off, unsigned lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
                 "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void copy4_async(const void *base, unsigned off, unsigned lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base),
                 "s"(lds)
                 : "memory", "m0");
}
// Output gate of eight elements of a 128-value row of y whose pieces are held by 16
// consecutive lanes (one DPP row): sigmoid(z) y / sqrt(mean(y^2) + eps) (1 + w), bf16 in and
// out, fp32 inside.  The row's sum of squares reaches every lane of the row identically.
__device__ __forceinline__ u32x4 out_gate8(u32x4 y, u32x4 z, const float *w, float eps)
{
    float yf[8], ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t u = y[e >> 1];
        yf[e] = __builtin_bit_cast(float, (e & 1) ? (u & 0xffff0000u) : (u << 16));
        ss += yf[e] * yf[e];
    }
    ss += dpp_f32<0xb1, 0xf>(ss);          // quad_perm [1, 0, 3, 2]
    ss += dpp_f32<0x4e, 0xf>(ss);          // quad_perm [2, 3, 0, 1]
    ss += dpp_f32<0x141, 0xf>(ss);         // row_half_mirror
    ss += dpp_f32<0x140, 0xf>(ss);         // row_mirror
    const float inv = __builtin_amdgcn_rsqf(ss * (1.f / 128.f) + eps);
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        float o[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t u = z[(e + d) >> 1];
            const float zf = __builtin_bit_cast(float, d ? (u & 0xffff0000u) : (u << 16));
            o[d] = yf[e + d] * inv * (1.f + w[e + d]) * __builtin_amdgcn_rcpf(1.f + __expf(-zf));
        }
        const bf16x2 h = bf16x2{(__bf16)o[0], (__bf16)o[1]};
        r[e >> 1] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
}

// A wave-uniform value as such (its lanes are known to agree).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ long long uni64(long long x)
{
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)x);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T *uptr(T *p)
{
    return (T *)uni64((long long)(size_t)p);
}
// Keeps a register value opaque to the optimizer from this point (no code).
__device__ __forceinline__ void opaque(unsigned &x) { asm volatile("" : "+v"(x)); }
// Granule permutation of the 256-byte K and Q rows (the slot before the row's XOR key).
__device__ __forceinline__ int kq_pi(int g) { return ((g & 1) << 3) | ((g >> 1) & 7); }

template <int DK, int DV>
__global__ __launch_bounds__(64 * kWideWaves) void wide_scan_kernel(WideArgs w)
{
    using L = LdsWide<DK, DV>;
    using OP = uint16_t;
    using M = Mma<OP>;
    constexpr int MBK = DK / 16;           // 16-row blocks of the state
    constexpr int KBD = DK / 32;           // K-blocks over the key dimension
    constexpr int KG = DK / 8;             // 16-byte granules per key row
    constexpr int CK = L::szK / 1024;      // 1 KiB copies per K or Q tile
    constexpr int CV = L::szV / 1024;      // ... per V tile
    static_assert(DV == 128 && DK == 128, "the wide scan is built for 128 x 128 states");
    static_assert(CK % kWidePrep == 0 && CV % kWidePrep == 0, "copy split");

    __shared__ __align__(16) unsigned char smem[L::total];
    const PrefillArgs &a = w.a;
    const int tid = threadIdx.x;
    int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int ln = lane & 15, lg = lane >> 4;
    // Called at the top of every chunk step: the lane index becomes opaque to the optimizer,
    // so the LDS addresses derived from it are formed inside the step instead of being hoisted
    // out of the loop (where they would outnumber the registers and spill).
    auto refresh_lane = [&]() {
        asm volatile("" : "+v"(lane));
        ln = lane & 15;
        lg = lane >> 4;
    };
    int *const misc = (int *)(smem + L::sMisc);
    float *const miscf = (float *)(smem + L::sMisc);
    typedef __attribute__((address_space(3))) int lint;
    lint *const misc_l = (lint *)(smem + L::sMisc);

    // ---- job ----
    typedef __attribute__((address_space(1))) int32_t gint;
    if (tid == 0)
        misc[kMiscJob] = w.counter ? __hip_atomic_fetch_add((gint *)w.counter, 1, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                   : (int)blockIdx.x;
    if (tid == 1) misc[kMiscPbar] = 0;
    if (tid == 2) miscf[kMiscLamWin] = 0.f;
    if (tid >= 3 && tid < 6) misc[kMiscCntT + tid - 3] = 0;
    __syncthreads();
    const int job = uni(misc[kMiscJob]);
    const int H = a.H;
    const long long njobs = (long long)(a.table ? *a.n_entries : a.num_seqs) * H;
    if (job >= njobs) return;
    const int e = job / H, h = job % H;
    int n, seg, nseg, len;
    long long tok0;
    if (a.table) {
        const SegEntry en = a.table[e];
        n = uni(en.n);
        tok0 = uni64(en.tok0);
        len = uni(en.len);
        seg = uni(en.seg);
        nseg = uni(en.nseg);
    } else {
        n = e;
        seq_bounds(a, n, tok0, len);
        seg = 0;
        nseg = 1;
    }
    long long srow0;
    int slen;
    seq_bounds(a, n, srow0, slen);
    srow0 = uni64(srow0);
    slen = uni(slen);
    GateHead gh;
    gh.pre = a.gate_A != nullptr;
    gh.scale = gh.pre ? -__expf(a.gate_A[h]) * 1.44269504088896341f : 0.f;
    gh.b_alpha = gh.pre ? a.gate_b_alpha[h] : 0.f;
    const int c0 = (int)((tok0 - srow0) / kChunk);      // first own chunk in the sequence
    const int nown = (len + kChunk - 1) / kChunk;

    // ---- warm-up window (segments after a sequence's first) ----
    // mode 0: start from S0 (or zero) at c0; 1: warm up from zero over [b, c0), verify;
    // 2: warm up from S0 over [0, c0) (exact); 3: wait for the previous segment's end state
    int b = c0, mode = 0;
    if (seg > 0) {
        const int R = c0 < w.wmax ? c0 : w.wmax;
        float cum = 0.f;
        int found = -1;
        float *const sums = miscf + kMiscSums;
        for (int r0 = 0; r0 < R && found < 0; r0 += kWideWaves) {
            const int i = r0 + wave;
            float s = 0.f;
            if (i < R) {
                const long long t = srow0 + (long long)(c0 - 1 - i) * kChunk + lane;
                s = wave_sum(wide_log2_alpha(gh, a.alpha[t * H + h]));
            }
            if (lane == 0) sums[wave] = s;
            __syncthreads();
            for (int q = 0; q < kWideWaves && r0 + q < R; ++q) {
                cum += sums[q];
                if (cum <= kWarmAlpha) {
                    found = r0 + q;
                    break;
                }
            }
            __syncthreads();
        }
        if (found >= 0) {
            b = c0 - 1 - found;
            mode = b == 0 ? 2 : 1;
        } else if (R == c0) {
            b = 0;
            mode = 2;
        } else {
            mode = 3;
        }
    }
    b = uni(b);
    mode = uni(mode);
    const int nwarm = c0 - b;
    const int nch = nwarm + nown;
    auto nvalid = [&](int j) {          // valid tokens of processed chunk j
        const int r = slen - (b + j) * kChunk;
        return r < kChunk ? r : kChunk;
    };
    auto row0_of = [&](int j) { return srow0 + (long long)(b + j) * kChunk; };
    auto lds_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    // LDS counters between waves of the workgroup: a wave adds one after its LDS operations
    // complete; a waiting wave spins until the count reaches its target (bounded: a count that
    // never arrives ends the wait, so no logic error can hang the device)
    auto lds_count = [&](int which) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0)      // one lane's LDS add (written out: no cross-lane bookkeeping needed)
            asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(misc + which)), "v"(1) : "memory");
    };
    auto lds_wait = [&](int which, int target) {
        for (int spin = 0; spin < (1 << 22); ++spin) {
            if (__hip_atomic_load(misc_l + which, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >=
                target)
                break;
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
    };

    // ================================================================ prep waves
    if (wave >= kWideCol) {
        const int pw = wave - kWideCol;
        // Gram fragment rows: see make_t
        unsigned o_g;
        {
            const int ln0 = lane & 15, lg0 = lane >> 4;
            const int rr = 16 * ((ln0 >> 2) & 1) + 4 * (ln0 >> 3) + (ln0 & 3);
            o_g = rr * 256 + ((kq_pi(lg0) ^ (rr & 7)) << 4);
        }
        const unsigned oab = (unsigned)lane * (unsigned)H * 4u;
        auto copy_chunk_gates = [&](int j) {
            if (pw < 2) {
                const long long t0 = row0_of(j);
                const int last = nvalid(j) - 1;
                const float *src = (pw == 0 ? a.alpha : a.beta) + t0 * H + h;
                const unsigned o = last == kChunk - 1 ? oab
                                                      : (unsigned)(lane < last ? lane : last) * (unsigned)H * 4u;
                copy4_async(src, o, lds_addr(smem + L::sAB + (j & 1) * 512 + pw * 256));
            }
        };
        // g, beta, 2^g and 2^-g of chunk j in this wave's own slot (no other wave reads it;
        // it is written and read within one step)
        auto gates = [&](int j) {
            const float *ab = (const float *)(smem + L::sAB + (j & 1) * 512);
            float *pg = (float *)(smem + L::sPG + pw * L::szPG);
            const int nv = nvalid(j);
            float x = 0.f, bt = 0.f;
            if (lane < nv) {
                x = wide_log2_alpha(gh, ab[lane]);
                const float rb = ab[64 + lane];
                bt = gh.pre ? __builtin_amdgcn_rcpf(1.f + __expf(-rb)) : rb;
            }
            x += dpp_f32<0x111, 0xf>(x);
            x += dpp_f32<0x112, 0xf>(x);
            x += dpp_f32<0x114, 0xf>(x);
            x += dpp_f32<0x118, 0xf>(x);
            x += dpp_f32<0x142, 0xa>(x);
            x += dpp_f32<0x143, 0xc>(x);
            pg[lane] = x;
            pg[64 + lane] = bt;
            pg[128 + lane] = __builtin_amdgcn_exp2f(x);
            pg[192 + lane] = __builtin_amdgcn_exp2f(-x);
        };
        // y of chunk jp, which the column waves stage in LDS as whole rows: this wave stores
        // rows 16 pw .. 16 pw + 15 (four passes of four rows, 16 lanes per row), through the
        // output gate when one is given
        // With the output gate, this lane's eight weights are read once, and the z pieces of the
        // rows a step stores are requested at the step's start (their latency then passes
        // while the step forms T').
        int ycount = 0;
        int ypending = -1;
        float wg[8];
        u32x4 zpre[4];
        if (a.og_z) {
            const float *wp = a.og_w + 8 * (lane & 15);
#pragma unroll
            for (int e = 0; e < 8; ++e) wg[e] = wp[e];
        }
        auto y_row0 = [&](int jp) { return ((row0_of(jp) + 16 * pw) * H + h) * (long long)(DV * 2); };
        auto y_off = [&](int q) {
            return (unsigned)((4 * q + (lane >> 4)) * H * DV * 2 + 16 * (lane & 15));
        };
        auto load_z = [&](int jp) {
            const long long yrow = y_row0(jp);
            const int nv = nvalid(jp);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                zpre[q] = u32x4{0u, 0u, 0u, 0u};
                if (16 * pw + 4 * q + (lane >> 4) < nv)
                    zpre[q] = *(const u32x4 *)((const unsigned char *)a.og_z + yrow + y_off(q));
            }
        };
        auto store_y = [&](int jp) {
            ycount += kWideCol;
            lds_wait(kMiscCntY, ycount);
            const long long yrow = y_row0(jp);
            const int nv = nvalid(jp);
            const unsigned char *bY = smem + L::sY;
            const int lgy = lane >> 4, g = lane & 15;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 16 * pw + 4 * q + lgy;
                const u32x4 v = *(const u32x4 *)(bY + t * (DV * 2) + ((g ^ (t & 15)) << 4));
                if (t < nv) {                       // whole rows (16 lanes) agree
                    u32x4 o = v;
                    if (a.og_z) o = out_gate8(v, zpre[q], wg, a.og_eps);
                    *(u32x4 *)((unsigned char *)a.y + yrow + y_off(q)) = o;
                }
            }
        };
        int pbar_target = 0;
        auto prep_barrier = [&]() {
            lds_count(kMiscPbar);
            pbar_target += kWidePrep;
            lds_wait(kMiscPbar, pbar_target);
        };
        // T' of chunk j (and its key terms of the transition bound).  Wave pw owns block row
        // and column pw of the 4 x 4 grid of 16 x 16 blocks.
        auto make_t = [&](int j) {
            const unsigned char *bK = smem + L::sK + (j % 3) * L::szK;
            unsigned char *bT = smem + L::sT;
            const float *sG = (const float *)(smem + L::sPG + pw * L::szPG);
            const float *sBeta = sG + 64;
            const float *sE = sG + 128;        // 2^g
            const float *sIE = sG + 192;       // 2^-g
            // g is non-increasing inside a chunk: while the chunk's total decay stays above -60,
            // 2^g_t and 2^-g_i are both normal and Gamma_ti is their product; below, every
            // element takes its own 2^(g_t - g_i)
            const bool factored = __builtin_amdgcn_readfirstlane((int)(sG[kChunk - 1] >= -60.f));
            float *sA = (float *)(smem + L::sA);
            float *sX = (float *)(smem + L::sX);
            const int d0 = pw * 16;
            const int np = pw < 2 ? 3 : 2;
            const int tb0 = pw == 0 ? 1 : (pw == 1 ? 2 : (pw == 2 ? 2 : 3));
            const int ib0 = pw == 0 ? 0 : (pw == 1 ? 0 : (pw == 2 ? 1 : 2));
            const int ib1 = pw == 0 ? 0 : 1;
            const int tbs[3] = {pw, tb0, 3};
            const int ibs[3] = {pw, ib0, ib1};
            f32x4 accG[3];
#pragma unroll
            for (int p = 0; p < 3; ++p) accG[p] = f32x4{0.f, 0.f, 0.f, 0.f};
            // fragment of tokens 16 ib + ln (tile rows split_pos(16 ib + ln) =
            // 32 (ib / 2) + 8 (ib % 2) + [16 (ln / 4 % 2) + 4 (ln / 8) + ln % 4]), granule 4 kb + lg
            auto rowoff = [](int ib) { return (32 * (ib >> 1) + 8 * (ib & 1)) * 256; };
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                const unsigned o = o_g ^ (32 * kb);
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    if (p < np) {
                        const auto ai = *(const bf16x8 *)(bK + rowoff(ibs[p]) + o);
                        const auto bt = *(const bf16x8 *)(bK + rowoff(tbs[p]) + o);
                        M::mma(accG[p], ai, bt);
                    }
                }
            }
            // accG[p][r] = k_i . k_t, i = ib 16 + 4 lg + r, t = tb 16 + ln
            // key terms of the bound: max(0, log2 |1 - beta_t ||k_t||^2|) over this block row
            // (warm-up chunks only)
            if (j < nwarm) {
                float term = 0.f;
                if (lg == (ln >> 2)) {
                    const float kk = accG[0][ln & 3];
                    const float bt = sBeta[d0 + ln];
                    term = fmaxf(__builtin_amdgcn_logf(fabsf(1.f - bt * kk)), 0.f);
                }
                term = wave_sum(term);
                if (lane == 0) miscf[kMiscLamPart + (j & 1) * 4 + pw] = term;
            }
            auto masked = [&](int tb, int ib, f32x4 g_, f32x4 &av) {
                const int t = tb * 16 + ln;
                const float bt_ = sBeta[t];
                if (factored) {
                    const float c = bt_ * sE[t];
                    const f32x4 ie = *(const f32x4 *)(sIE + ib * 16 + 4 * lg);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = ib * 16 + 4 * lg + r;
                        av[r] = (i < t) ? (c * ie[r]) * g_[r] : 0.f;
                    }
                } else {
                    const float gt = sG[t];
                    const f32x4 gi = *(const f32x4 *)(sG + ib * 16 + 4 * lg);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = ib * 16 + 4 * lg + r;
                        av[r] = (i < t) ? bt_ * g_[r] * __builtin_amdgcn_exp2f(gt - gi[r]) : 0.f;
                    }
                }
            };
            f32x4 nT, a1, a2;
            masked(pw, pw, accG[0], nT);
            masked(tb0, ib0, accG[1], a1);
            if (np == 3) masked(3, ib1, accG[2], a2);
            f32x4 nC;
            {
                const int t = d0 + ln;
                const f32x4 bi = *(const f32x4 *)(sBeta + d0 + 4 * lg);
                if (factored) {
                    const float iet = sIE[t];
                    const f32x4 ei = *(const f32x4 *)(sE + d0 + 4 * lg);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = d0 + 4 * lg + r;
                        nC[r] = (t < i) ? (bi[r] * (ei[r] * iet)) * accG[0][r] : 0.f;
                    }
                } else {
                    const float gt = sG[t];
                    const f32x4 gi = *(const f32x4 *)(sG + d0 + 4 * lg);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = d0 + 4 * lg + r;
                        nC[r] = (t < i) ? bi[r] * accG[0][r] * __builtin_amdgcn_exp2f(gi[r] - gt) : 0.f;
                    }
                }
            }
            // (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since N^16 = 0
            f32x4 eye;
#pragma unroll
            for (int r = 0; r < 4; ++r) eye[r] = (4 * lg + r == ln) ? 1.f : 0.f;
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
            auto ablk = [&](int i, int m) {
                return sA + ((i * (i - 1) / 2 + m) * 16 + ln) * L::LDB + 4 * lg;
            };
            *(f32x4 *)ablk(tb0, ib0) = a1;
            if (np == 3) *(f32x4 *)ablk(3, ib1) = a2;
            *(f32x4 *)(sX + (d0 + ln) * L::LDX + 4 * lg) = xT;
            // the rows of y staged in this step leave: waves 2 and 3 (two Gram blocks each) here,
            // while the column waves reach their T' read; waves 0 and 1 (three blocks, short
            // work after the barrier below) right after that barrier
            if (ypending >= 0 && pw >= 2) {
                store_y(ypending);
                ypending = -1;
            }
            // the tile still holds the T' the column waves read in this step until every one of
            // them has loaded it (chunk j's is written during step j - 1)
            lds_wait(kMiscCntT, kWideCol * j);
            // the blocks above the diagonal that the column waves read, (0, 1) and (2, 3), are zero
            if (pw == 0 || pw == 2)
                M::put4((OP *)(bT + swz<OP, kChunk>(split_pos(d0 + ln), d0 + 16 + 4 * lg)),
                        f32x4{0.f, 0.f, 0.f, 0.f});
            {
                const f32x4 bcol = *(const f32x4 *)(sBeta + d0 + 4 * lg);
                M::put4((OP *)(bT + swz<OP, kChunk>(split_pos(d0 + ln), d0 + 4 * lg)), xT * bcol);
            }
            prep_barrier();
            if (ypending >= 0) {
                store_y(ypending);
                ypending = -1;
            }
            // The tile holds T' within each 32-token half, T'_AA = X_A diag(beta_A) and
            // T'_BB = X_B diag(beta_B), and -W with W = X_B A_BA in place of T'_BA (the column
            // waves form U_B = T'_BB R_B - W U_A).  Blocks of 16: X_10 = -X_11 A_10 X_00 and
            // X_32 = -X_33 A_32 X_22 (waves 0 and 2), and W_2m = X_22 A_2m,
            // W_3m = X_33 (A_3m - A_32 W_2m) for m = 0 (wave 1) and m = 1 (wave 3), right to
            // left so that every product is in the accumulator layout.
            {
                auto arow = [&](int i, int m) { return split4(*(const f32x4 *)ablk(i, m)); };
                // block (i, m) of A in the accumulator layout (lane holds A_im[4 lg + r][ln])
                auto acol = [&](int i, int m) {
                    const float *b = sA + (i * (i - 1) / 2 + m) * 16 * L::LDB;
                    f32x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = b[(4 * lg + r) * L::LDB + ln];
                    return v;
                };
                auto xrow = [&](int i) {
                    return split4(*(const f32x4 *)(sX + (16 * i + ln) * L::LDX + 4 * lg));
                };
                // store a block given in the accumulator layout at block (i, jc) of the tile
                auto put_blk = [&](int i, int jc, f32x4 z, float scale) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Elem<OP>::store((OP *)(bT + swz<OP, kChunk>(split_pos(16 * i + 4 * lg + r), 16 * jc + ln)),
                                        z[r] * scale);
                };
                if (pw == 0 || pw == 2) {
                    // X_{pw+1, pw} = -X_{pw+1, pw+1} A_{pw+1, pw} X_{pw, pw}, times diag(beta_pw)
                    const f32x4 acc = mm3r(arow(pw + 1, pw), split4(xC));
                    const f32x4 x1 = -mm3r(xrow(pw + 1), split4(acc));
                    put_blk(pw + 1, pw, x1, sBeta[16 * pw + ln]);
                } else {
                    const int m = pw == 1 ? 0 : 1;
                    const f32x4 w2 = mm3r(xrow(2), split4(acol(2, m)));
                    const f32x4 u = acol(3, m) - mm3r(arow(3, 2), split4(w2));
                    const f32x4 w3 = mm3r(xrow(3), split4(u));
                    put_blk(2, m, -w2, 1.f);
                    put_blk(3, m, -w3, 1.f);
                }
            }
            // the bound of a warm-up chunk joins the window's sum (fixed order of terms)
            if (pw == 0 && j < nwarm && lane == 0) {
                const float *part = miscf + kMiscLamPart + (j & 1) * 4;
                const float lam = sG[kChunk - 1] + part[0] + part[1] + part[2] + part[3];
                miscf[kMiscLamWin] += lam;
            }
        };
        // Decay factors of chunk j (wave 2, whose work after the prep barrier is the shortest):
        // the scan holds S = 2^ls Shat; ls starts at 0 and
        // after each chunk becomes ls + g_C, or 0 when that would fall below -32 (the column
        // waves then rescale Shat by the same rule on the same g_C).
        //   F[t] = gamma_t 2^ls,  F[64 + t] = (gamma_C / gamma_t) / 2^ls',  F[128] = g_C,
        //   F[132 + t] = g_t,  F[196 + t] = 2^g_t,  F[260 + t] = 2^-g_t
        float lsl = 0.f;
        auto factors = [&](int j) {
            const float *gc = (const float *)(smem + L::sPG + pw * L::szPG);
            float *F = (float *)(smem + L::sF + (j & 1) * L::szF);
            const float gt = gc[lane], gC = gc[kChunk - 1];
            const float lsc = lsl;
            float lsn = lsc + gC;
            if (lsn < -32.f) lsn = 0.f;
            F[lane] = __builtin_amdgcn_exp2f(gt + lsc);
            F[64 + lane] = __builtin_amdgcn_exp2f((gC - gt) - lsn);
            if (lane == 0) F[128] = gC;
            F[132 + lane] = gt;
            F[196 + lane] = gc[128 + lane];
            F[260 + lane] = gc[192 + lane];
            lsl = lsn;
        };

        if (nch > 0) {
            copy_chunk_gates(0);
            if (nch > 1) copy_chunk_gates(1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();                                  // #0: chunk 0 (and K, gates of 1) staged
        if (nch > 0) {
            gates(0);
            make_t(0);
            if (pw == 2) factors(0);
        }
        lds_barrier();                                  // #1: T'(0), factors(0)
        // the prep waves' work is one long dependent chain per step that every step waits for:
        // the SIMDs issue their instructions first
        __builtin_amdgcn_s_setprio(3);
        for (int j = 0; j < nch; ++j) {
            refresh_lane();
            opaque(o_g);
            if (j + 2 < nch) copy_chunk_gates(j + 2);
            // the column waves stage the y of chunk j - 1 in this step
            if (j >= 1 && j - 1 >= nwarm) {
                ypending = j - 1;
                if (a.og_z) load_z(j - 1);
            }
            if (j + 1 < nch) {
                gates(j + 1);
                make_t(j + 1);
                if (pw == 2) factors(j + 1);
            }
            if (ypending >= 0) {
                store_y(ypending);
                ypending = -1;
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
        }
        // the last chunk's y, staged by the column waves after their loop
        if (nch > 0 && nch - 1 >= nwarm) {
            if (a.og_z) load_z(nch - 1);
            store_y(nch - 1);
        }
        return;
    }

    // ================================================================ column waves
    const int cw = wave;
    const int tile = cw >> 1, sw = cw & 1;
    // this lane's state column: the two waves of a 32-column tile interleave in runs of four,
    // so a lane of the output layout holds 4 columns that sit next to the other wave's 4
    const int col = 32 * tile + 8 * (ln >> 2) + 4 * sw + (ln & 3);
    const long long stride_s = (long long)DK * DV;
    // Byte offsets of this lane's per-step LDS and global accesses.  Every access adds to one
    // of them a uniform stage base and a constant, after at most an XOR with a constant on
    // bits 5-6 (where the swizzles depend on the contraction block); they are made opaque at
    // each step so that the optimizer forms these few operations there rather than keeping
    // every combination live across the loop.
    //   o_kq: K or Q fragment (row 16 tb + ln, granule 4 kb + lg): + 4096 tb, ^ 32 kb
    //   o_kt: transposing K^T read (rows 32 kt + 4 lg + ln / 4 (+ 16), granule
    //         4 (m / 2) + ln % 4, byte 8 (m % 2)): + 8192 kt + 4096 hi + 8 (m % 2), ^ 32 (m / 2)
    //   o_tt: T' fragment (row 16 mb + ln, granule lg): + 2048 mb, ^ 32 mb
    //   o_v:  transposing V read (rows 32 (tb / 2) + 8 lg + 4 (tb % 2) + ln / 4, this lane's
    //         four columns): + 8192 (tb / 2) + 1024 (tb % 2)
    //   o_ys: y staging write (row 16 tb + ln)
    unsigned o_kq = ln * 256 + ((kq_pi(lg) ^ (ln & 7)) << 4);
    unsigned o_kt = (4 * lg + (ln >> 2)) * 256 + ((kq_pi(ln & 3) ^ (4 * (lg & 1) + (ln >> 2))) << 4);
    unsigned o_tt = ln * 128 + ((lg ^ (ln & 7) ^ (ln >> 3)) << 4);
    unsigned o_v = (8 * lg + (ln >> 2)) * 256 + (((4 * tile + (ln & 3)) ^ ((ln >> 2) << 2)) << 4) + 8 * sw;
    unsigned o_ys = ln * 256 + (((4 * tile + lg) ^ ln) << 4) + 8 * sw;
    unsigned o_lane = lane;
    f32x4 S[MBK];
    auto load_state = [&](const float *src, float scale) {
#pragma unroll
        for (int m = 0; m < MBK; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[m][i] = src ? src[(long long)split_orig(16 * m + 4 * lg + i) * DV + col] * scale
                              : 0.f;
    };
    // the previous segment's published end state (exact chain)
    auto wait_previous = [&]() -> const float * {
        const int pj = (e - 1) * H + h;
        gint *flag = (gint *)(w.flags + pj);
        long long spins = 0;
        while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < kWideCol) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > (1ll << 26)) {          // a bounded wait: never expected to end here
                if (lane == 0)
                    __hip_atomic_fetch_or((gint *)w.error, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                return nullptr;
            }
        }
        return w.seg_state + (long long)pj * stride_s;
    };
    if (mode == 0 || mode == 2)
        load_state(a.s0 ? a.s0 + ((long long)n * H + h) * stride_s : nullptr, 1.f);
    else if (mode == 1)
        load_state(nullptr, 1.f);
    else
        load_state(wait_previous(), 1.f);

    bf16x8 Sb[KBD];
    auto pack_state = [&]() {
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) Sb[kb] = pack8s(S[2 * kb], S[2 * kb + 1]);
    };
    pack_state();
    float ls = 0.f;
    // carried from chunk j to step j + 1: gamma 2^ls (Shat^T Q^T) and bf16 U
    f32x4 yq[4];
    bf16x8 Uu0 = {}, Uu1 = {};
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) yq[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Y of chunk jp = carried gamma 2^ls (Shat^T Q^T) + U^T P^T.  Each wave holds 4 columns of
    // each of 64 tokens; the pieces meet in LDS (16-byte granules of a row XOR-swizzled by the
    // row), from where the prep waves store them as whole rows.
    auto finish = [&](int jp) {
        (void)jp;
        const unsigned char *bP = smem + L::sP + 16 * o_lane;
        unsigned char *bY = smem + L::sY;
        bf16x8 fp[6];
#pragma unroll
        for (int f = 0; f < 6; ++f) fp[f] = *(const bf16x8 *)(bP + f * 1024);
        f32x4 pu[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            pu[tb] = yq[tb];
            M::mma(pu[tb], Uu0, fp[tb]);
        }
        M::mma(pu[2], Uu1, fp[4]);
        M::mma(pu[3], Uu1, fp[5]);
        lds_count(kMiscCntP);              // P may now be overwritten by this step's
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            *(bf16x4 *)(bY + o_ys + 4096 * tb) = __builtin_convertvector(pu[tb], bf16x4);
        lds_count(kMiscCntY);              // the prep waves store the staged rows
    };

    // P = lower_incl(Q K^T (.) Gamma) of chunk j as the six operand fragments read a step
    // later (fragment f < 4: rows 16 f .. 16 f + 15, columns 0 .. 31; fragments 4, 5: rows
    // 32 .. 47 and 48 .. 63, columns 32 .. 63), one 16 x 16 block in each 8-byte half of a
    // lane's 16 bytes.  Column waves 0-3 form fragment cw, waves 4-7 one block of fragments 4
    // and 5.  The K operand takes the tile's rows as they lie (internal token order):
    // accumulator [r] of block (tb, ib) = k_i . q_t, t = 16 tb + ln,
    // i = 32 (ib / 2) + 8 lg + 4 (ib % 2) + r.
    auto make_p = [&](int j, const unsigned char *bK, const unsigned char *bQ, const float *F) {
        const float *gc = F + 132;
        unsigned char *bP = smem + L::sP + 16 * o_lane;
        constexpr int kTb[12] = {0, 0, 1, 1, 2, 2, 3, 3, 2, 2, 3, 3};
        constexpr int kIb[12] = {0, 1, 0, 1, 0, 1, 0, 1, 2, 3, 2, 3};
        // g is non-increasing inside a chunk: while the chunk's total decay stays above -60,
        // 2^g_t and 2^-g_i are both normal and Gamma_ti is their product; below, every element
        // takes its own 2^(g_t - g_i) (0 * inf otherwise)
        const bool factored = __builtin_amdgcn_readfirstlane((int)(F[128] >= -60.f));
        const int nb = cw < 4 ? 2 : 1;               // blocks of this wave
        const int p0 = cw < 4 ? 2 * cw : 8 + (cw - 4);
        const int tb = kTb[p0];
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            const unsigned o = o_kq ^ (32 * kb);
            const bf16x8 fq = *(const bf16x8 *)(bQ + 4096 * tb + o);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u < nb)
                    M::mma(acc[u], *(const bf16x8 *)(bK + 4096 * kIb[p0 + u] + o), fq);
            }
        }
        const int t = tb * 16 + ln;
        f32x4 pv[2];
        if (factored) {
            const float et = F[196 + t];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ib = kIb[p0 + u];
                const f32x4 ie = *(const f32x4 *)(F + 260 + 32 * (ib >> 1) + 8 * lg + 4 * (ib & 1));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 32 * (ib >> 1) + 8 * lg + 4 * (ib & 1) + r;
                    pv[u][r] = (i <= t) ? acc[u][r] * (et * ie[r]) : 0.f;
                }
            }
        } else {
            const float gt = gc[t];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ib = kIb[p0 + u];
                const f32x4 gi = *(const f32x4 *)(gc + 32 * (ib >> 1) + 8 * lg + 4 * (ib & 1));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 32 * (ib >> 1) + 8 * lg + 4 * (ib & 1) + r;
                    pv[u][r] = (i <= t) ? acc[u][r] * __builtin_amdgcn_exp2f(gt - gi[r]) : 0.f;
                }
            }
        }
        // every column wave has read the previous chunk's P (one count per step)
        lds_wait(kMiscCntP, kWideCol * (j + 1));
        if (cw < 4) {
            *(bf16x8 *)(bP + cw * 1024) = pack8s(pv[0], pv[1]);
        } else {
            const int f = 4 + ((cw - 4) >> 1), half = (cw - 4) & 1;
            *(bf16x4 *)(bP + f * 1024 + 8 * half) = __builtin_convertvector(pv[0], bf16x4);
        }
    };

    // The K, Q and V tiles of the chunks ahead (K two chunks ahead, Q and V one), copied by the
    // column waves: wave cw fills the 1 KiB pieces jj = 2 cw + q (q = 0, 1) of each tile, lane
    // (ln, lg) slot ln of tile row r = 8 cw + 4 q + lg.  In a K or Q tile that slot holds logical
    // granule kq_logical(r, ln), a function of r % 8 = 4 q + lg; the K tile's row r holds token
    // split_orig(r) = split_orig(8 cw + 4 q) + lg, the Q tile's token r.  In a V tile the slot
    // holds granule ln ^ 4 lg.  A full chunk's copies thus take a per-lane byte offset and a
    // uniform row; a sequence's last, partial chunk repeats its last row past the end.
    const unsigned rsK = (unsigned)(H * DK) * 2, rsV = (unsigned)(H * DV) * 2;   // bytes
    static_assert(CK == 2 * kWideCol && CV == 2 * kWideCol && KG == 16, "copy layout");
    auto copy_tiles = [&](int j, bool with_k, bool with_qv) {
        const long long t0 = row0_of(j);
        const int last = nvalid(j) - 1;
        const long long head = (t0 * H + h) * (long long)DK * 2;
        const unsigned char *ck = (const unsigned char *)a.k + head;
        const unsigned char *cq = (const unsigned char *)a.q + head;
        const unsigned char *cv = (const unsigned char *)a.v + (t0 * H + h) * (long long)DV * 2;
        unsigned char *dk = smem + L::sK + (j % 3) * L::szK;
        unsigned char *dq = smem + L::sQ + (j & 1) * L::szK;
        unsigned char *dv = smem + L::sV + (j & 1) * L::szV;
        const int lnc = (int)(o_lane & 15), lgc = (int)(o_lane >> 4);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int jj = 2 * cw + q;
            const int r0 = 8 * cw + 4 * q;                 // tile row of lane group 0
            const unsigned gk = 16 * kq_logical<DK>(4 * q + lgc, lnc);
            const unsigned gv = 16 * (lnc ^ (lgc << 2));
            if (last == kChunk - 1) {
                if (with_k)
                    copy16_async(ck + split_orig(r0) * rsK, lgc * rsK + gk, lds_addr(dk + 1024 * jj));
                if (with_qv) {
                    copy16_async(cq + r0 * rsK, lgc * rsK + gk, lds_addr(dq + 1024 * jj));
                    copy16_async(cv + r0 * rsV, lgc * rsV + gv, lds_addr(dv + 1024 * jj));
                }
            } else {
                const int r = r0 + lgc;
                if (with_k) {
                    const int rk = split_orig(r) < last ? split_orig(r) : last;
                    copy16_async(ck, (unsigned)rk * rsK + gk, lds_addr(dk + 1024 * jj));
                }
                if (with_qv) {
                    const int rq = r < last ? r : last;
                    copy16_async(cq, (unsigned)rq * rsK + gk, lds_addr(dq + 1024 * jj));
                    copy16_async(cv, (unsigned)rq * rsV + gv, lds_addr(dv + 1024 * jj));
                }
            }
        }
    };
    if (nch > 0) {
        copy_tiles(0, true, true);
        if (nch > 1) copy_tiles(1, true, false);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();            // #0: chunk 0 (and K of chunk 1) staged
    lds_barrier();            // #1
    for (int j = 0; j < nch; ++j) {
        opaque(o_kq);
        opaque(o_kt);
        opaque(o_tt);
        opaque(o_v);
        opaque(o_ys);
        opaque(o_lane);
        if (j + 2 < nch) copy_tiles(j + 2, true, false);
        if (j + 1 < nch) copy_tiles(j + 1, false, true);
        if (mode == 1 && j == nwarm) {
            // the warm-up reached the bound, or the exact chain takes over
            const float lw = __builtin_bit_cast(
                float, __hip_atomic_load(misc_l + kMiscLamWin, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP));
            if (!(lw <= kWarmBound)) {
                load_state(wait_previous(), __builtin_amdgcn_exp2f(-ls));
                pack_state();
            }
        }
        const unsigned char *bK = smem + L::sK + (j % 3) * L::szK;
        const unsigned char *bQ = smem + L::sQ + (j & 1) * L::szK;
        const unsigned char *bV = smem + L::sV + (j & 1) * L::szV;
        const unsigned char *bT = smem + L::sT;
        const float *F = (const float *)(smem + L::sF + (j & 1) * L::szF);
        const bool normal = j >= nwarm;

        // ---- Y of chunk j - 1 first (its P arrived with this step): the carries die early ----
        if (j >= 1 && j - 1 >= nwarm) finish(j - 1);
        else lds_count(kMiscCntP);
        __builtin_amdgcn_sched_barrier(0);

        // ---- K Shat (the head of the state chain) and, beside it, Shat^T Q^T: both read the
        // chunk-start state's operands ----
        f32x4 acc_ks[4], accQ[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            acc_ks[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            accQ[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // eight groups (contraction block kb, token blocks 2 h2 and 2 h2 + 1), software-pipelined:
        // the fragments of group g + 1 are requested before the products of group g issue
        auto ks_qs = [&](auto with_q) {
            constexpr bool WQ = decltype(with_q)::value;
            auto ld = [&](int g, bf16x8 *fk, bf16x8 *fq) {
                const unsigned o = o_kq ^ (32 * (g >> 1));
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    fk[u] = *(const bf16x8 *)(bK + 4096 * (2 * (g & 1) + u) + o);
                    if constexpr (WQ) fq[u] = *(const bf16x8 *)(bQ + 4096 * (2 * (g & 1) + u) + o);
                }
            };
            auto mm = [&](int g, const bf16x8 *fk, const bf16x8 *fq) {
#pragma unroll
                for (int u = 0; u < 2; ++u) M::mma(acc_ks[2 * (g & 1) + u], fk[u], Sb[g >> 1]);
                if constexpr (WQ) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) M::mma(accQ[2 * (g & 1) + u], Sb[g >> 1], fq[u]);
                }
            };
            bf16x8 fkA[2], fqA[2], fkB[2], fqB[2];
            ld(0, fkA, fqA);
#pragma unroll
            for (int g = 0; g < 2 * KBD; g += 2) {
                ld(g + 1, fkB, fqB);
                __builtin_amdgcn_sched_barrier(0);
                mm(g, fkA, fqA);
                __builtin_amdgcn_sched_barrier(0);
                if (g + 2 < 2 * KBD) ld(g + 2, fkA, fqA);
                __builtin_amdgcn_sched_barrier(0);
                mm(g + 1, fkB, fqB);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (normal) ks_qs(std::true_type{});
        else ks_qs(std::false_type{});
        if (normal) {
            const float *Fl = F + (o_lane & 15);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) yq[tb] = accQ[tb] * Fl[tb * 16];
        }
        // T' fragments: rows 16 mb + ln at granule lg (mb < 4), and rows 32 + ln, 48 + ln at
        // granule 4 + lg, which take the slots of granule lg in rows ln and 16 + ln
        bf16x8 ft[6];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) ft[mb] = *(const bf16x8 *)(bT + 2048 * mb + (o_tt ^ (32 * mb)));
        ft[4] = *(const bf16x8 *)(bT + 4096 + o_tt);
        ft[5] = *(const bf16x8 *)(bT + 6144 + (o_tt ^ 32));
        lds_count(kMiscCntT);              // the prep waves may now write the next chunk's T'

        // ---- R = V - diag(gamma 2^ls) K Shat;  U = T' R ----
        f32x4 U[4];
        {
            f32x4 R[4];
            const float *Fq = F + 8 * (o_lane >> 4);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                // V[o0 .. o0 + 3][column], o0 = split_orig(16 tb + 4 lg) = 32 (tb / 2) + 8 lg +
                // 4 (tb % 2), by one transposing read: lane j receives column
                // 32 tile + 8 (j / 4) + 4 sw + j % 4 of rows o0 .. o0 + 3
                const int c0 = 32 * (tb >> 1) + 4 * (tb & 1);
                const f32x4 gam = *(const f32x4 *)(Fq + c0);
                const bf16x4 v4 = ldtr(bV + 256 * c0 + o_v);
                R[tb] = __builtin_convertvector(v4, f32x4) - gam * acc_ks[tb];
            }
            const bf16x8 Rb0 = pack8s(R[0], R[1]);
            const bf16x8 Rb1 = pack8s(R[2], R[3]);
            // U_A = T'_AA R_A;  U_B = T'_BB R_B - W U_A (the tile holds -W in T'_BA's place)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) U[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
            M::mma(U[0], ft[0], Rb0);
            M::mma(U[1], ft[1], Rb0);
            M::mma(U[2], ft[4], Rb1);
            M::mma(U[3], ft[5], Rb1);
            const bf16x8 Ua = pack8s(U[0], U[1]);
            M::mma(U[2], ft[2], Ua);
            M::mma(U[3], ft[3], Ua);
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- chunk j's other carry: bf16 U ----
        if (normal) {
            Uu0 = pack8s(U[0], U[1]);
            Uu1 = pack8s(U[2], U[3]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (normal) make_p(j, bK, bQ, F);
        __builtin_amdgcn_sched_barrier(0);

        // ---- S = gamma_C S + K^T diag(gamma_C / gamma) U, as Shat += K^T diag(rho) U ----
        // K^T fragment: columns 32 (m / 2) + 8 (ln % 4) + 4 (m % 2) .. + 3 of the tokens
        // 32 kt + 8 lg + ln / 4 (+ 4), which sit at tile rows 32 kt + 4 lg + ln / 4 (+ 16)
        auto frag_kt = [&](int m, int kt) {
            const unsigned char *p = bK + 8192 * kt + 8 * (m & 1) + (o_kt ^ (32 * (m >> 1)));
            const bf16x4 lo = ldtr(p);
            const bf16x4 hi = ldtr(p + 4096);
            return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        {
            float ln_ = ls + F[128];
            ln_ = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ln_)));
            if (ln_ < -32.f) {                     // fold the scale into Shat (rare)
                const float f = __builtin_amdgcn_exp2f(ln_);
#pragma unroll
                for (int m = 0; m < MBK; ++m) S[m] *= f;
                ln_ = 0.f;
            }
            ls = ln_;
            bf16x8 Ub[2];
            {
                f32x4 Us[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const f32x4 rho = *(const f32x4 *)(F + 64 + 8 * (o_lane >> 4) + 32 * (mb >> 1) + 4 * (mb & 1));
                    Us[mb] = U[mb] * rho;
                }
                Ub[0] = pack8s(Us[0], Us[1]);
                Ub[1] = pack8s(Us[2], Us[3]);
            }
            // four groups (kt, half) of four K^T fragments, software-pipelined like K Shat
            auto ldt = [&](int g, bf16x8 *f) {
#pragma unroll
                for (int q = 0; q < MBK / 2; ++q) f[q] = frag_kt((g & 1) * (MBK / 2) + q, g >> 1);
            };
            auto mmt = [&](int g, const bf16x8 *f) {
#pragma unroll
                for (int q = 0; q < MBK / 2; ++q) M::mma(S[(g & 1) * (MBK / 2) + q], f[q], Ub[g >> 1]);
            };
            bf16x8 ftA[MBK / 2], ftB[MBK / 2];
            ldt(0, ftA);
#pragma unroll
            for (int g = 0; g < 4; g += 2) {
                ldt(g + 1, ftB);
                __builtin_amdgcn_sched_barrier(0);
                mmt(g, ftA);
                __builtin_amdgcn_sched_barrier(0);
                if (g + 2 < 4) ldt(g + 2, ftA);
                __builtin_amdgcn_sched_barrier(0);
                mmt(g + 1, ftB);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        pack_state();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
    }
    if (nch > 0 && nch - 1 >= nwarm) finish(nch - 1);

    // ---- state out: the final state of the sequence, or the segment's end state for the
    // next segment's workgroup ----
    const float sp = __builtin_amdgcn_exp2f(ls);
    float *dst = nullptr;
    const bool publish = a.table && seg < nseg - 1;
    if (publish) dst = w.seg_state + (long long)job * stride_s;
    else if (a.s_final) dst = a.s_final + ((long long)n * H + h) * stride_s;
    if (dst) {
#pragma unroll
        for (int m = 0; m < MBK; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[(long long)split_orig(16 * m + 4 * lg + i) * DV + col] = S[m][i] * sp;
    }
    if (publish) {
        // every lane's stores are ordered before its wave's release of the flag
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0)
            __hip_atomic_fetch_add((gint *)(w.flags + job), 1, __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

// =========================================================================================
// Host side
// =========================================================================================
hipError_t launch_wide_scan(const WideArgs &w, long long jobs, hipStream_t stream)
{
    if (jobs <= 0) return hipSuccess;
    hipLaunchKernelGGL((wide_scan_kernel<128, 128>), dim3((unsigned)jobs),
                       dim3(64 * kWideWaves), 0, stream, w);
    return hipGetLastError();
}

}  // namespace gdn
