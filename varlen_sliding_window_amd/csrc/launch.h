// Internal launchers, one per kernel family (defined next to their kernels).
#pragma once

#include "common.h"

namespace attn {

struct Problem {
  int total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, window;
  float scale;
  float softcap;   // > 0: logits become softcap * tanh(logit / softcap); 0: no cap
  int band;        // 1: band-block key/query ranges (window > 0 only); 0: tight ranges
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

}  // namespace attn
