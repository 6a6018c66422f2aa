// Internal launchers, one per kernel family (defined next to their kernels).
#pragma once

#include "common.h"

namespace attn {

struct Problem {
  int total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, window;
  float scale;
  float softcap;   // > 0: logits become softcap * tanh(logit / softcap); 0: no cap
  int band;        // 1: band-block key/query ranges (window > 0 only); 0: tight ranges
  int max_seqlen;  // the caller's bound on segment lengths (picks kernel variants only)
};

// Constants of the capped logit in the exp2 domain:
//   log2(e) * softcap * tanh(scale * qk / softcap) = cap_c2 * tanh(cap_a * qk).
struct CapConstants {
  float cap_a, cap_c2;
};
inline CapConstants cap_constants(const Problem& p) {
  return p.softcap > 0.f ? CapConstants{p.scale / p.softcap, p.softcap * LOG2E}
                         : CapConstants{0.f, 0.f};
}

// Builds the sorted tile lists in the workspace from cu_seqlens: the
// forward-order list always, the backward-order list only when need_bwd.
hipError_t launch_schedule(const int32_t* cu_seqlens, const Problem& p, bool need_bwd,
                           void* workspace, const WorkspaceLayout& w, hipStream_t stream);

hipError_t launch_forward(const void* q, const void* k, const void* v, const Problem& p,
                          void* out, float* lse, void* workspace, const WorkspaceLayout& w,
                          hipStream_t stream);

// dQ, and each row's lse * log2(e) and D = rowsum(dout * out) into the
// workspace; must precede launch_dkdv.
hipError_t launch_dq(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, const Problem& p, void* dq,
                     void* workspace, const WorkspaceLayout& w, hipStream_t stream);

hipError_t launch_dkdv(const void* q, const void* k, const void* v, const float* lse,
                       const void* dout, const Problem& p, void* dk, void* dv, void* workspace,
                       const WorkspaceLayout& w, hipStream_t stream);

// Gated delta-rule linear attention (delta.hip): chunks of DELTA_CHUNK
// tokens, head dim DELTA_DIM for keys and values.  Workspace: [header |
// per-segment chunk offsets | one fp32 record per (chunk, head)], and for the
// backward also [chunk-start states | end-state gradients | dU], one per
// (chunk, head).
constexpr int DELTA_CHUNK = 64;
constexpr int DELTA_DIM = 128;
// record: W, U0 [C][D]; P, T [C][C]; gamma, end decay and 4 C side values
constexpr size_t delta_record_floats() {
  return (size_t)2 * DELTA_CHUNK * DELTA_DIM + (size_t)2 * DELTA_CHUNK * DELTA_CHUNK +
         (size_t)6 * DELTA_CHUNK;
}
struct DeltaLayout {
  size_t header, seg_off, records, states, dstates, dubuf, dwbuf, pairbuf, total;
  size_t chunk_cap, record_bytes;
};
// Kimi Delta record: W, U0, q (x) gamma, k (x) end decay [C][D]; P, T and the
// decayed K K^T [C][C]; the chunk's total decay and a backward side value [D]
constexpr size_t kda_record_floats() {
  return (size_t)4 * DELTA_CHUNK * DELTA_DIM + (size_t)3 * DELTA_CHUNK * DELTA_CHUNK +
         (size_t)2 * DELTA_DIM;
}
// pair_area: the backward also keeps two C x C pair-gradient matrices per
// (chunk, head) (the per-channel gate's backward)
inline DeltaLayout delta_layout(int64_t total_tokens, int64_t num_seqs, int64_t num_heads,
                                bool backward = false,
                                size_t record_floats = delta_record_floats(),
                                bool pair_area = false) {
  DeltaLayout w;
  w.chunk_cap = (size_t)((total_tokens + DELTA_CHUNK - 1) / DELTA_CHUNK) + (size_t)num_seqs;
  w.record_bytes = record_floats * sizeof(float);
  const size_t units = w.chunk_cap * (size_t)num_heads;
  w.header = 0;
  w.seg_off = 256;
  w.records = w.seg_off + align256((size_t)(num_seqs + 1) * sizeof(int));
  w.states = w.records + units * w.record_bytes;
  w.dstates = w.states;
  w.dubuf = w.states;
  w.dwbuf = w.states;
  w.pairbuf = w.states;
  w.total = w.states;
  if (backward) {
    const size_t state_bytes = (size_t)DELTA_DIM * DELTA_DIM * sizeof(float);
    const size_t chunk_bytes = (size_t)DELTA_CHUNK * DELTA_DIM * sizeof(float);
    w.dstates = w.states + units * state_bytes;
    w.dubuf = w.dstates + units * state_bytes;
    w.dwbuf = w.dubuf + units * chunk_bytes;
    w.pairbuf = w.dwbuf + units * chunk_bytes;
    w.total = w.pairbuf + (pair_area ? units * (size_t)2 * DELTA_CHUNK * DELTA_CHUNK * sizeof(float) : 0);
  }
  return w;
}

hipError_t launch_delta_fwd(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens, int num_seqs,
                            int total_tokens, int num_heads, float scale, void* out,
                            void* workspace, const DeltaLayout& w, bool save,
                            hipStream_t stream);

// Kimi Delta Attention forward (delta.hip): the gate g is [T, H, DELTA_DIM],
// one log decay per key channel; workspace laid out with kda_record_floats().
hipError_t launch_kda_fwd(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* cu_seqlens, int num_seqs,
                          int total_tokens, int num_heads, float scale, void* out,
                          void* workspace, const DeltaLayout& w, bool save, hipStream_t stream);

// Kimi Delta Attention backward: dq, dk, dv bf16 [T, H, D], dg fp32
// [T, H, D], dbeta fp32 [T, H]; recomputes the forward's records and states
// (workspace laid out with backward = true, kda_record_floats() and the pair
// area), or with `reuse` takes those a saving forward left there.
hipError_t launch_kda_bwd(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const void* dout, const int32_t* cu_seqlens,
                          int num_seqs, int total_tokens, int num_heads, float scale, void* dq,
                          void* dk, void* dv, float* dg, float* dbeta, void* workspace,
                          const DeltaLayout& w, bool reuse, hipStream_t stream);

// Gradients of sum(dout * out) for the gated delta rule: dq, dk, dv bf16
// [T, H, D]; dg, dbeta fp32 [T, H].  Recomputes the forward's records and
// states in the workspace (laid out with backward = true), or with `reuse`
// takes those a saving forward left there.
hipError_t launch_delta_bwd(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const void* dout, const int32_t* cu_seqlens,
                            int num_seqs, int total_tokens, int num_heads, float scale, void* dq,
                            void* dk, void* dv, float* dg, float* dbeta, void* workspace,
                            const DeltaLayout& w, bool reuse, hipStream_t stream);

}  // namespace attn
