// gdn_api.cpp -- the C ABI of libgdn (declared in include/gdn.h).
//
// Host-side argument validation and launch.  Nothing here allocates device memory,
// synchronises or keeps state between calls; every check that can be made from the host
// happens before the first HIP call, so invalid arguments never reach the runtime.
#include <stdint.h>
#include <string.h>

#include "../../include/gdn.h"
#include "gdn_internal.hpp"

namespace {

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool dim_ok(int32_t d) { return d == 64 || d == 128; }

// [a, a + na) and [b, b + nb) overlap (both non-empty)
bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

size_t esize(int32_t dtype) { return dtype == GDN_DTYPE_BF16 ? 2 : 4; }

gdn_status check_common(int64_t rows, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype)
{
    if (rows < 0 || H <= 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_INVALID_ARGUMENT;
    if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if (!dim_ok(d_k) || !dim_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_status_str(int32_t status)
{
    switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "GDN_ERR_WORKSPACE_TOO_SMALL";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    default: return "GDN_ERR_UNKNOWN";
    }
}

const char *gdn_version(void) { return "gdn-gfx950 0.1"; }

static bool plan_for(int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k, int32_t d_v,
                     int32_t dtype, int32_t dv_tile, int32_t seg, gdn::PrefillPlan *plan)
{
    if (num_seqs <= 0 || check_common(total_T, H, d_k, d_v, dtype) != GDN_OK) return false;
    return gdn::make_plan(num_seqs, total_T, H, d_k, d_v, dtype, dv_tile, seg, plan);
}

size_t gdn_prefill_workspace_bytes_ex(int32_t num_seqs, int64_t total_T, int32_t H,
                                      int32_t d_k, int32_t d_v, int32_t dtype,
                                      int32_t dv_tile, int32_t segment_chunks)
{
    gdn::PrefillPlan plan;
    if (!plan_for(num_seqs, total_T, H, d_k, d_v, dtype, dv_tile, segment_chunks, &plan))
        return 0;
    return plan.ws_table + plan.ws_seg + plan.ws_prep + plan.ws_wide;
}

size_t gdn_prefill_workspace_bytes(int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                                   int32_t d_v, int32_t dtype)
{
    return gdn_prefill_workspace_bytes_ex(num_seqs, total_T, H, d_k, d_v, dtype, 0, 0);
}

gdn_status gdn_prefill_plan(int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                            int32_t d_v, int32_t dtype, int32_t *dv_tile,
                            int32_t *segment_chunks)
{
    if (!dv_tile || !segment_chunks) return GDN_ERR_INVALID_ARGUMENT;
    gdn_status st = check_common(total_T, H, d_k, d_v, dtype);
    if (st != GDN_OK) return st;
    if (num_seqs <= 0) return GDN_ERR_INVALID_ARGUMENT;
    gdn::PrefillPlan plan;
    if (!gdn::make_plan(num_seqs, total_T, H, d_k, d_v, dtype, 0, 0, &plan))
        return GDN_ERR_UNSUPPORTED;
    *dv_tile = plan.dv_tile;
    *segment_chunks = plan.seg_chunks;
    return GDN_OK;
}

// The output gate that gdn_prefill_output_gated applies to y.
struct OutGate {
    const void *z;
    const float *w;
    float eps;
};

// gdn_prefill_ex, gdn_prefill_gated and gdn_prefill_output_gated: with gate_A non-null
// (gated), alpha and beta are the gate pre-activations a and b, and gate_A, gate_b_alpha [H]
// complete them; with og non-null, y receives the output gate's result.
static gdn_status prefill_impl(const void *q, const void *k, const void *v, const float *alpha,
                               const float *beta, const float *gate_A,
                               const float *gate_b_alpha, bool gated,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                               int32_t d_v, int32_t dtype, void *y, float *final_state,
                               void *workspace, size_t workspace_bytes, void *stream,
                               int32_t dv_tile, int32_t segment_chunks,
                               const OutGate *og = nullptr)
{
    gdn_status st = check_common(total_T, H, d_k, d_v, dtype);
    if (st != GDN_OK) return st;
    if (og) {
        if (!(og->eps >= 0.f) || !(og->eps <= 3.4e38f)) return GDN_ERR_INVALID_ARGUMENT;
        if (total_T > 0 && (!og->z || !og->w)) return GDN_ERR_INVALID_ARGUMENT;
        if ((og->z && !aligned(og->z, 16)) || (og->w && !aligned(og->w, 4)))
            return GDN_ERR_INVALID_ARGUMENT;
    }
    if (gated) {
        if (dtype != GDN_DTYPE_BF16 || dv_tile != 0 || segment_chunks != 0)
            return GDN_ERR_UNSUPPORTED;
        if (total_T > 0 && (!gate_A || !gate_b_alpha)) return GDN_ERR_INVALID_ARGUMENT;
        if ((gate_A && !aligned(gate_A, 4)) || (gate_b_alpha && !aligned(gate_b_alpha, 4)))
            return GDN_ERR_INVALID_ARGUMENT;
    }
    if (num_seqs <= 0) return GDN_ERR_INVALID_ARGUMENT;
    if (!cu_seqlens && total_T % num_seqs != 0) return GDN_ERR_INVALID_ARGUMENT;
    if (total_T > 0 && (!q || !k || !v || !alpha || !beta || !y))
        return GDN_ERR_INVALID_ARGUMENT;
    // q, k, v, y, states, workspace: 16 bytes; gates, cu_seqlens: 4 bytes
    const void *quads[] = {q, k, v, y};
    for (const void *p : quads)
        if (p && !aligned(p, 16)) return GDN_ERR_INVALID_ARGUMENT;
    const void *vec[] = {initial_state, final_state, workspace};
    for (const void *p : vec)
        if (p && !aligned(p, 16)) return GDN_ERR_INVALID_ARGUMENT;
    const void *words[] = {alpha, beta, cu_seqlens};
    for (const void *p : words)
        if (p && !aligned(p, 4)) return GDN_ERR_INVALID_ARGUMENT;
    if (dv_tile < 0 || segment_chunks < -1) return GDN_ERR_INVALID_ARGUMENT;

    // In-place resume (final_state == initial_state) never splits sequences: a later
    // segment would overwrite the state that the first segment of its sequence still reads.
    const bool in_place = final_state && final_state == initial_state;
    if (in_place && segment_chunks > 0) return GDN_ERR_INVALID_ARGUMENT;
    gdn::PrefillPlan plan;
    if (!gdn::make_plan(num_seqs, total_T, H, d_k, d_v, dtype, dv_tile,
                        in_place ? -1 : segment_chunks, &plan))
        return dv_tile != 0 ? GDN_ERR_UNSUPPORTED : GDN_ERR_INVALID_ARGUMENT;
    const size_t need = plan.ws_table + plan.ws_seg + plan.ws_prep + plan.ws_wide;
    if (workspace_bytes < need || (need > 0 && !workspace)) return GDN_ERR_WORKSPACE_TOO_SMALL;

    // aliasing: outputs may not overlap inputs (final_state == initial_state is allowed)
    const size_t e = esize(dtype);
    const size_t rows = (size_t)total_T;
    const size_t n_qk = rows * H * d_k * e, n_v = rows * H * d_v * e, n_g = rows * H * 4;
    const size_t n_s = (size_t)num_seqs * H * d_k * d_v * 4;
    const size_t n_cu = cu_seqlens ? (size_t)(num_seqs + 1) * 4 : 0;
    struct Span { const void *p; size_t n; };
    const size_t n_h = gated ? (size_t)H * 4 : 0;
    const Span inputs[] = {{q, n_qk}, {k, n_qk}, {v, n_v}, {alpha, n_g}, {beta, n_g},
                           {cu_seqlens, n_cu}, {gate_A, n_h}, {gate_b_alpha, n_h},
                           {og ? og->z : nullptr, og ? n_v : 0},
                           {og ? og->w : nullptr, og ? (size_t)d_v * 4 : 0}};
    const Span outs[] = {{y, n_v}, {final_state, final_state ? n_s : 0}, {workspace, need}};
    for (const Span &o : outs) {
        for (const Span &in : inputs)
            if (overlap(o.p, o.n, in.p, in.n)) return GDN_ERR_INVALID_ARGUMENT;
        if (o.p != final_state && overlap(o.p, o.n, initial_state, initial_state ? n_s : 0))
            return GDN_ERR_INVALID_ARGUMENT;
    }
    if (final_state && initial_state && final_state != initial_state &&
        overlap(final_state, n_s, initial_state, n_s))
        return GDN_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return GDN_ERR_INVALID_ARGUMENT;

    gdn::PrefillProblem p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.alpha = alpha;
    p.beta = beta;
    p.s0 = initial_state;
    p.cu = cu_seqlens;
    p.num_seqs = num_seqs;
    p.total_T = total_T;
    p.H = H;
    p.dk = d_k;
    p.dv = d_v;
    p.dtype = dtype;
    p.y = y;
    p.s_final = final_state;
    if (gated) {
        if (!plan.two_launch && !plan.wide) return GDN_ERR_UNSUPPORTED;
        p.gated = true;
        p.gate_A = gate_A;
        p.gate_b_alpha = gate_b_alpha;
    }
    // the one-launch scan gates each row of y as it leaves; other plans gate y in place after
    const bool fused_gate = og && plan.wide;
    if (fused_gate) {
        p.og_z = og->z;
        p.og_w = og->w;
        p.og_eps = og->eps;
    }
    hipError_t err = gdn::launch_prefill(p, plan, workspace, (hipStream_t)stream);
    if (err == hipSuccess && og && !fused_gate && total_T > 0)
        err = gdn::launch_output_gate(y, og->z, og->w, total_T * H, d_v, og->eps, dtype, y,
                                      (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_prefill_output_gated(const void *q, const void *k, const void *v,
                                    const float *alpha, const float *beta,
                                    const float *initial_state, const int32_t *cu_seqlens,
                                    int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                                    int32_t d_v, int32_t dtype, const void *z,
                                    const float *weight, float eps, void *out,
                                    float *final_state, void *workspace,
                                    size_t workspace_bytes, void *stream, int32_t dv_tile,
                                    int32_t segment_chunks)
{
    const OutGate og{z, weight, eps};
    return prefill_impl(q, k, v, alpha, beta, nullptr, nullptr, false, initial_state,
                        cu_seqlens, num_seqs, total_T, H, d_k, d_v, dtype, out, final_state,
                        workspace, workspace_bytes, stream, dv_tile, segment_chunks, &og);
}

gdn_status gdn_prefill_ex(const void *q, const void *k, const void *v, const float *alpha,
                          const float *beta, const float *initial_state,
                          const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_T,
                          int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, void *y,
                          float *final_state, void *workspace, size_t workspace_bytes,
                          void *stream, int32_t dv_tile, int32_t segment_chunks)
{
    return prefill_impl(q, k, v, alpha, beta, nullptr, nullptr, false, initial_state,
                        cu_seqlens, num_seqs, total_T, H, d_k, d_v, dtype, y, final_state,
                        workspace, workspace_bytes, stream, dv_tile, segment_chunks);
}

gdn_status gdn_prefill_gated(const void *q, const void *k, const void *v, const float *a,
                             const float *b, const float *A, const float *b_alpha,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                             int32_t d_v, int32_t dtype, void *y, float *final_state,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    return prefill_impl(q, k, v, a, b, A, b_alpha, true, initial_state, cu_seqlens, num_seqs,
                        total_T, H, d_k, d_v, dtype, y, final_state, workspace,
                        workspace_bytes, stream, 0, 0);
}

gdn_status gdn_prefill(const void *q, const void *k, const void *v, const float *alpha,
                       const float *beta, const float *initial_state,
                       const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_T,
                       int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, void *y,
                       float *final_state, void *workspace, size_t workspace_bytes,
                       void *stream)
{
    return gdn_prefill_ex(q, k, v, alpha, beta, initial_state, cu_seqlens, num_seqs, total_T,
                          H, d_k, d_v, dtype, y, final_state, workspace, workspace_bytes,
                          stream, 0, 0);
}

size_t gdn_prefill_backward_workspace_bytes(int32_t num_seqs, int64_t total_T, int32_t H,
                                            int32_t d_k, int32_t d_v, int32_t dtype)
{
    if (num_seqs <= 0 || check_common(total_T, H, d_k, d_v, dtype) != GDN_OK) return 0;
    if (dtype != GDN_DTYPE_BF16) return 0;
    return gdn::backward_workspace_bytes(num_seqs, total_T, H, d_k, d_v);
}

gdn_status gdn_prefill_backward(const void *q, const void *k, const void *v, const float *alpha,
                                const float *beta, const float *initial_state,
                                const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_T,
                                int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                                const void *dy, const float *d_final_state, void *dq, void *dk,
                                void *dv, float *dalpha, float *dbeta, float *d_initial_state,
                                void *workspace, size_t workspace_bytes, void *stream)
{
    gdn_status st = check_common(total_T, H, d_k, d_v, dtype);
    if (st != GDN_OK) return st;
    if (dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if (num_seqs <= 0) return GDN_ERR_INVALID_ARGUMENT;
    if (!cu_seqlens && total_T % num_seqs != 0) return GDN_ERR_INVALID_ARGUMENT;
    if (total_T > 0 && (!q || !k || !v || !alpha || !beta || !dy || !dq || !dk || !dv ||
                        !dalpha || !dbeta))
        return GDN_ERR_INVALID_ARGUMENT;
    const void *quads[] = {q, k, v, dy, dq, dk, dv, initial_state, d_final_state,
                           d_initial_state, workspace};
    for (const void *p : quads)
        if (p && !aligned(p, 16)) return GDN_ERR_INVALID_ARGUMENT;
    const void *words[] = {alpha, beta, dalpha, dbeta, cu_seqlens};
    for (const void *p : words)
        if (p && !aligned(p, 4)) return GDN_ERR_INVALID_ARGUMENT;
    const size_t need = gdn::backward_workspace_bytes(num_seqs, total_T, H, d_k, d_v);
    if (workspace_bytes < need || !workspace) return GDN_ERR_WORKSPACE_TOO_SMALL;

    // outputs overlap neither the inputs nor each other
    const size_t rows = (size_t)total_T;
    const size_t n_qk = rows * H * d_k * 2, n_v = rows * H * d_v * 2, n_g = rows * H * 4;
    const size_t n_s = (size_t)num_seqs * H * d_k * d_v * 4;
    const size_t n_cu = cu_seqlens ? (size_t)(num_seqs + 1) * 4 : 0;
    struct Span { const void *p; size_t n; };
    const Span inputs[] = {{q, n_qk}, {k, n_qk}, {v, n_v}, {alpha, n_g}, {beta, n_g},
                           {dy, n_v}, {cu_seqlens, n_cu},
                           {initial_state, initial_state ? n_s : 0},
                           {d_final_state, d_final_state ? n_s : 0}};
    const Span outs[] = {{dq, n_qk}, {dk, n_qk}, {dv, n_v}, {dalpha, n_g}, {dbeta, n_g},
                         {d_initial_state, d_initial_state ? n_s : 0}, {workspace, need}};
    constexpr int NO = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < NO; ++i) {
        for (const Span &in : inputs)
            if (overlap(outs[i].p, outs[i].n, in.p, in.n)) return GDN_ERR_INVALID_ARGUMENT;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return GDN_ERR_INVALID_ARGUMENT;
    }

    gdn::BackwardProblem p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.dy = dy;
    p.alpha = alpha;
    p.beta = beta;
    p.s0 = initial_state;
    p.ds_final = d_final_state;
    p.cu = cu_seqlens;
    p.num_seqs = num_seqs;
    p.total_T = total_T;
    p.H = H;
    p.dk = d_k;
    p.dv = d_v;
    p.dq = dq;
    p.dk_out = dk;
    p.dv_out = dv;
    p.dalpha = dalpha;
    p.dbeta = dbeta;
    p.ds0 = d_initial_state;
    hipError_t err = gdn::launch_backward(p, workspace, (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_channel_gated(const void *q, const void *k, const void *v, const float *decay,
                             const float *erase, const float *write,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                             int32_t d_v, int32_t dtype, void *y, float *final_state,
                             void *stream)
{
    gdn_status st = check_common(total_T, H, d_k, d_v, dtype);
    if (st != GDN_OK) return st;
    if (num_seqs <= 0) return GDN_ERR_INVALID_ARGUMENT;
    if (!cu_seqlens && total_T % num_seqs != 0) return GDN_ERR_INVALID_ARGUMENT;
    if (total_T > 0 && (!q || !k || !v || !decay || !erase || !write || !y))
        return GDN_ERR_INVALID_ARGUMENT;
    const void *quads[] = {q, k, v, y, decay, initial_state, final_state};
    for (const void *p : quads)
        if (p && !aligned(p, 16)) return GDN_ERR_INVALID_ARGUMENT;
    const void *words[] = {erase, write, cu_seqlens};
    for (const void *p : words)
        if (p && !aligned(p, 4)) return GDN_ERR_INVALID_ARGUMENT;
    const size_t e = esize(dtype);
    const size_t rows = (size_t)total_T;
    const size_t n_qk = rows * H * d_k * e, n_v = rows * H * d_v * e;
    const size_t n_a = rows * H * d_k * 4, n_g = rows * H * d_v * 4;
    const size_t n_s = (size_t)num_seqs * H * d_k * d_v * 4;
    const size_t n_cu = cu_seqlens ? (size_t)(num_seqs + 1) * 4 : 0;
    struct Span { const void *p; size_t n; };
    const Span inputs[] = {{q, n_qk}, {k, n_qk}, {v, n_v}, {decay, n_a}, {erase, n_g},
                           {write, n_g}, {cu_seqlens, n_cu}};
    const Span outs[] = {{y, n_v}, {final_state, final_state ? n_s : 0}};
    for (const Span &o : outs) {
        for (const Span &in : inputs)
            if (overlap(o.p, o.n, in.p, in.n)) return GDN_ERR_INVALID_ARGUMENT;
        if (o.p != final_state && overlap(o.p, o.n, initial_state, initial_state ? n_s : 0))
            return GDN_ERR_INVALID_ARGUMENT;
    }
    if (overlap(y, n_v, final_state, final_state ? n_s : 0)) return GDN_ERR_INVALID_ARGUMENT;
    // the state may be carried in place (final_state == initial_state exactly)
    if (final_state && initial_state && final_state != initial_state &&
        overlap(final_state, n_s, initial_state, n_s))
        return GDN_ERR_INVALID_ARGUMENT;

    gdn::ChannelProblem c;
    c.q = q;
    c.k = k;
    c.v = v;
    c.a = decay;
    c.b = erase;
    c.w = write;
    c.s0 = initial_state;
    c.cu = cu_seqlens;
    c.num_seqs = num_seqs;
    c.total_T = total_T;
    c.H = H;
    c.dk = d_k;
    c.dv = d_v;
    c.dtype = dtype;
    c.y = y;
    c.s_final = final_state;
    hipError_t err = gdn::launch_channel_gated(c, (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_qsa_workspace_bytes(int64_t n)
{
    if (n <= 0 || n > gdn::qsa_max_tokens()) return 0;
    return gdn::qsa_workspace_bytes(n);
}

gdn_status gdn_qsa_index(const void *q, const void *k, int64_t n, int32_t dtype,
                         int32_t block_budget, int32_t *blocks, int32_t *tokens,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if (n <= 0 || block_budget <= 0) return GDN_ERR_INVALID_ARGUMENT;
    if (n > gdn::qsa_max_tokens() || block_budget > (1 << 24) ||
        !gdn::qsa_budget_supported(n, block_budget))
        return GDN_ERR_UNSUPPORTED;
    if (!q || !k || !workspace || (!blocks && !tokens)) return GDN_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(workspace, 16) ||
        (blocks && !aligned(blocks, 4)) || (tokens && !aligned(tokens, 4)))
        return GDN_ERR_INVALID_ARGUMENT;
    const size_t need = gdn::qsa_workspace_bytes(n);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE_TOO_SMALL;
    const size_t e = esize(dtype);
    const size_t n_q = (size_t)n * 4 * 128 * e, n_k = (size_t)n * 128 * e;
    const size_t n_b = (size_t)n * block_budget * 4;
    const size_t n_t = (size_t)n * ((size_t)block_budget * 4 + 3) * 4;
    struct Span { const void *p; size_t n; };
    const Span ins[] = {{q, n_q}, {k, n_k}};
    const Span outs[] = {{blocks, blocks ? n_b : 0}, {tokens, tokens ? n_t : 0},
                         {workspace, need}};
    for (int i = 0; i < 3; ++i) {
        for (const Span &in : ins)
            if (overlap(outs[i].p, outs[i].n, in.p, in.n)) return GDN_ERR_INVALID_ARGUMENT;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return GDN_ERR_INVALID_ARGUMENT;
    }
    gdn::QsaProblem p;
    p.q = q;
    p.k = k;
    p.n = n;
    p.dtype = dtype;
    p.block_budget = block_budget;
    p.blocks = blocks;
    p.tokens = tokens;
    hipError_t err = gdn::launch_qsa(p, workspace, (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_decode_step(const void *q, const void *k, const void *v, const float *alpha,
                           const float *beta, float *state, void *y, int32_t B, int32_t H,
                           int32_t d_k, int32_t d_v, int32_t dtype, void *stream)
{
    gdn_status st = check_common(B, H, d_k, d_v, dtype);
    if (st != GDN_OK) return st;
    if (B == 0) return GDN_OK;
    if (!q || !k || !v || !alpha || !beta || !state || !y) return GDN_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(y, 16) ||
        !aligned(state, 16) || !aligned(alpha, 4) || !aligned(beta, 4))
        return GDN_ERR_INVALID_ARGUMENT;
    const size_t e = esize(dtype);
    const size_t n_s = (size_t)B * H * d_k * d_v * 4;
    const size_t n_qk = (size_t)B * H * d_k * e, n_v = (size_t)B * H * d_v * e;
    const size_t n_g = (size_t)B * H * 4;
    struct Span { const void *p; size_t n; };
    const Span others[] = {{q, n_qk}, {k, n_qk}, {v, n_v}, {alpha, n_g}, {beta, n_g}, {y, n_v}};
    for (const Span &o : others)
        if (overlap(state, n_s, o.p, o.n)) return GDN_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 5; ++i)
        if (overlap(y, n_v, others[i].p, others[i].n)) return GDN_ERR_INVALID_ARGUMENT;
    hipError_t err = gdn::launch_decode(q, k, v, alpha, beta, state, y, B, H, d_k, d_v, dtype,
                                        (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_short_conv(const void *x, const float *weight, const int32_t *cu_seqlens,
                          int32_t num_seqs, int64_t total_T, int32_t channels, int32_t width,
                          int32_t head_dim, int32_t dtype, void *out, const float *state_in,
                          float *state_out, void *stream)
{
    if (total_T < 0 || num_seqs <= 0 || channels <= 0 || channels % 64 != 0)
        return GDN_ERR_INVALID_ARGUMENT;
    if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if (width < 1 || width > 4) return GDN_ERR_UNSUPPORTED;
    if (head_dim != 0 && head_dim != 64 && head_dim != 128) return GDN_ERR_UNSUPPORTED;
    if (head_dim != 0 && channels % head_dim != 0) return GDN_ERR_INVALID_ARGUMENT;
    if (!cu_seqlens && total_T % num_seqs != 0) return GDN_ERR_INVALID_ARGUMENT;
    if (!weight || (total_T > 0 && (!x || !out))) return GDN_ERR_INVALID_ARGUMENT;
    if ((x && !aligned(x, 16)) || (out && !aligned(out, 16)) || !aligned(weight, 4) ||
        (state_in && !aligned(state_in, 4)) || (state_out && !aligned(state_out, 4)) ||
        (cu_seqlens && !aligned(cu_seqlens, 4)))
        return GDN_ERR_INVALID_ARGUMENT;
    const size_t n_x = (size_t)total_T * channels * esize(dtype);
    const size_t n_w = (size_t)channels * width * 4;
    const size_t n_s = (size_t)num_seqs * channels * (width - 1) * 4;
    const size_t n_cu = cu_seqlens ? (size_t)(num_seqs + 1) * 4 : 0;
    struct Span { const void *p; size_t n; };
    const Span ins[] = {{x, n_x}, {weight, n_w}, {state_in, n_s}, {cu_seqlens, n_cu}};
    for (const Span &i : ins) {
        if (overlap(out, n_x, i.p, i.n)) return GDN_ERR_INVALID_ARGUMENT;
        // the carried state may be updated in place (state_out == state_in exactly)
        if (i.p != state_in || state_out != state_in)
            if (overlap(state_out, n_s, i.p, i.n)) return GDN_ERR_INVALID_ARGUMENT;
    }
    if (overlap(state_out, n_s, out, n_x)) return GDN_ERR_INVALID_ARGUMENT;
    hipError_t err = gdn::launch_short_conv(x, weight, cu_seqlens, num_seqs, total_T, channels,
                                            width, head_dim, dtype, state_in, state_out, out,
                                            (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_gates(const float *a, const float *b, const float *A, const float *b_alpha,
                     int64_t total_T, int32_t H, float *alpha, float *beta, void *stream)
{
    if (total_T < 0 || H <= 0) return GDN_ERR_INVALID_ARGUMENT;
    if (total_T == 0) return GDN_OK;
    if (!a || !b || !A || !b_alpha || !alpha || !beta) return GDN_ERR_INVALID_ARGUMENT;
    const void *all[] = {a, b, A, b_alpha, alpha, beta};
    for (const void *p : all)
        if (!aligned(p, 4)) return GDN_ERR_INVALID_ARGUMENT;
    const size_t n = (size_t)total_T * H * 4, nh = (size_t)H * 4;
    struct Span { const void *p; size_t n; };
    const Span ins[] = {{a, n}, {b, n}, {A, nh}, {b_alpha, nh}};
    for (const Span &i : ins)
        if (overlap(alpha, n, i.p, i.n) || overlap(beta, n, i.p, i.n))
            return GDN_ERR_INVALID_ARGUMENT;
    if (overlap(alpha, n, beta, n)) return GDN_ERR_INVALID_ARGUMENT;
    hipError_t err = gdn::launch_gates(a, b, A, b_alpha, total_T, H, alpha, beta,
                                       (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_output_gate(const void *y, const void *z, const float *weight, int64_t rows,
                           int32_t d_v, float eps, int32_t dtype, void *out, void *stream)
{
    if (rows < 0 || !(eps >= 0.f)) return GDN_ERR_INVALID_ARGUMENT;
    if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if (!dim_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (rows == 0) return GDN_OK;
    if (!y || !z || !weight || !out) return GDN_ERR_INVALID_ARGUMENT;
    if (!aligned(y, 16) || !aligned(z, 16) || !aligned(out, 16) || !aligned(weight, 4))
        return GDN_ERR_INVALID_ARGUMENT;
    const size_t n = (size_t)rows * d_v * esize(dtype);
    // out may be y exactly (each row is read whole before it is written)
    if ((out != y && overlap(out, n, y, n)) || overlap(out, n, z, n) ||
        overlap(out, n, weight, (size_t)d_v * 4))
        return GDN_ERR_INVALID_ARGUMENT;
    hipError_t err = gdn::launch_output_gate(y, z, weight, rows, d_v, eps, dtype, out,
                                             (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
