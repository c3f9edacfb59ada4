// gdn_internal.hpp -- host-side declarations shared by the libgdn translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;
constexpr int kChunk = 64;    // tokens per chunk of the chunked prefill
// Workspace record per (chunk slot, head) of the two-launch bf16 prefill: T' ([64][64]
// bf16) and the 64 log2 decay prefixes (fp32).
constexpr int kPrepRecordBytes = kChunk * kChunk * 2 + kChunk * 4;

// Problem description handed from the C ABI to the prefill launchers.
struct PrefillProblem {
    const void *q, *k, *v;
    const float *alpha, *beta;
    const float *s0;            // [N, H, dk, dv] or null
    const int32_t *cu;          // [N+1] device or null (equal lengths)
    int num_seqs;
    long long total_T;
    int H, dk, dv, dtype;
    void *y;
    float *s_final;             // or null
    // gate pre-activations instead of alpha and beta (bf16 two-launch plans only): alpha and
    // beta then hold a and b [T, H]; gate_A and gate_b_alpha are [H]
    bool gated = false;
    const float *gate_A = nullptr, *gate_b_alpha = nullptr;
    // output gate on y (one-launch bf16 plans only): z [T, H, dv], weight [dv], eps
    const void *og_z = nullptr;
    const float *og_w = nullptr;
    float og_eps = 0.f;
};

// Launch plan: columns of the state per workgroup and chunks per segment (-1: no split).
struct PrefillPlan {
    int dv_tile;
    int seg_chunks;
    long long max_segments;     // upper bound on table entries (segments over all sequences)
    int two_launch;             // 1: chunk-parallel records, then the state scan (bf16)
    long long nslots;           // chunk slots of the records
    size_t ws_table, ws_seg;    // workspace bytes for the table and per-segment matrices
    size_t ws_prep;             // workspace bytes for the chunk records
    int wide = 0;               // 1: one-launch scan with the whole 128 x 128 state per workgroup
    size_t ws_wide = 0;         // its job counter, publication flags and segment end states
};

bool make_plan(int num_seqs, long long total_T, int H, int dk, int dv, int dtype,
               int dv_tile_req, int seg_chunks_req, PrefillPlan *plan);

hipError_t launch_prefill(const PrefillProblem &p, const PrefillPlan &plan, void *workspace,
                          hipStream_t stream);

// Problem description of the chunked backward (bf16 activations).
struct BackwardProblem {
    const void *q, *k, *v, *dy;
    const float *alpha, *beta;
    const float *s0, *ds_final;  // [N, H, dk, dv] or null (zeros)
    const int32_t *cu;
    int num_seqs;
    long long total_T;
    int H, dk, dv;
    void *dq, *dk_out, *dv_out;
    float *dalpha, *dbeta, *ds0;  // ds0 may be null
};

size_t backward_workspace_bytes(int num_seqs, long long total_T, int H, int dk, int dv);
hipError_t launch_backward(const BackwardProblem &p, void *workspace, hipStream_t stream);

// Channel-wise gated variants: decay per key channel, erase and write gates per value
// channel (token by token).
struct ChannelProblem {
    const void *q, *k, *v;
    const float *a, *b, *w;     // [T, H, dk], [T, H, dv], [T, H, dv]
    const float *s0;            // [N, H, dk, dv] or null
    const int32_t *cu;
    int num_seqs;
    long long total_T;
    int H, dk, dv, dtype;
    void *y;
    float *s_final;             // or null; may equal s0
};
hipError_t launch_channel_gated(const ChannelProblem &c, hipStream_t stream);

// Sparse-attention block indexer (4 query heads, one 128-dim key head, blocks of 4 tokens).
struct QsaProblem {
    const void *q, *k;          // [n, 4, 128], [n, 128] dtype
    long long n;
    int dtype, block_budget;
    int32_t *blocks, *tokens;   // [n, budget], [n, 4 budget + 3] or null
};
size_t qsa_workspace_bytes(long long n);
long long qsa_max_tokens();
bool qsa_budget_supported(long long n, int block_budget);
hipError_t launch_qsa(const QsaProblem &p, void *workspace, hipStream_t stream);

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *alpha,
                         const float *beta, float *state, void *y, int B, int H, int dk,
                         int dv, int dtype, hipStream_t stream);

hipError_t launch_short_conv(const void *x, const float *w, const int32_t *cu, int nseq,
                             long long total_T, int C, int W, int head_dim, int dtype,
                             const float *state_in, float *state_out, void *out,
                             hipStream_t stream);
hipError_t launch_gates(const float *a, const float *b, const float *A, const float *b_alpha,
                        long long total_T, int H, float *alpha, float *beta, hipStream_t stream);
hipError_t launch_output_gate(const void *y, const void *z, const float *w, long long rows,
                              int dv, float eps, int dtype, void *out, hipStream_t stream);

}  // namespace gdn
