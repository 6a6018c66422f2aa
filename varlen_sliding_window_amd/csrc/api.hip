// C ABI of libattn_varlen.so (declared in include/attn_varlen.h).
//
// Host side only: argument checks that need no device read, the workspace
// layout, and kernel launches on the caller's stream.  Nothing here waits
// on the device or allocates memory.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "attn_varlen.h"
#include "common.h"
#include "launch.h"

namespace {

using attn::Problem;
using attn::WorkspaceLayout;

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

attn_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_EDEVICE;
  if (dev >= kMaxDevices) return ATTN_EDEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_EDEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? ATTN_OK : ATTN_EDEVICE;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape and scalar checks shared by every entry point.
attn_status check_shape(int32_t total_tokens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen) {
  if (total_tokens <= 0 || num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0)
    return ATTN_EINVAL;
  if (num_q_heads % num_kv_heads != 0) return ATTN_EINVAL;
  if (max_seqlen <= 0 || max_seqlen > total_tokens) return ATTN_EINVAL;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return ATTN_EUNSUPPORTED;
  // grid sizes must fit in 32 bits (a grid covers up to num_q_heads entries
  // per tile, in runs padded to 8 * LOCAL_RUN)
  const size_t cap = attn::tile_capacity(total_tokens, num_seqs);
  if ((cap + 8 * attn::LOCAL_RUN) * (size_t)num_q_heads >= (size_t)1 << 31) return ATTN_EUNSUPPORTED;
  // the kernels address k and v rows with 32-bit byte offsets from a
  // key-value head's first row
  if ((size_t)total_tokens * (size_t)num_kv_heads * (size_t)head_dim * 2 > (size_t)UINT32_MAX)
    return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

attn_status check_common(const void* q, const void* k, const void* v, const int32_t* cu,
                         int32_t total_tokens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen, float scale,
                         void* workspace, size_t workspace_bytes, WorkspaceLayout* w) {
  attn_status s = check_shape(total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                              max_seqlen);
  if (s != ATTN_OK) return s;
  if (!q || !k || !v || !cu) return ATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(cu, 4))
    return ATTN_EINVAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_EINVAL;
  *w = attn::workspace_layout(total_tokens, num_seqs, num_q_heads);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w->total) return ATTN_EWORKSPACE;
  return ATTN_OK;
}

// ---- optional kernel timing (attn_varlen_profile_start / _stop) ----------
enum KernelId {
  K_SCHEDULE = 0, K_FORWARD, K_DQ, K_DKDV, K_DELTA, K_DELTA_BWD, K_KDA, K_KDA_BWD, K_COUNT
};
const char* const kKernelNames[K_COUNT] = {"schedule",  "forward",   "dq",      "dkdv",
                                           "delta_fwd", "delta_bwd", "kda_fwd", "kda_bwd"};

struct ProfileRecord {
  int kernel;
  hipEvent_t start, stop;
};

std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfileRecord> g_prof;

// Launch f() on stream st; when profiling is on, bracket it with two events
// recorded on the same stream.
template <class F>
hipError_t timed_launch(int kernel, hipStream_t st, F&& f) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return f();
  ProfileRecord r{kernel, nullptr, nullptr};
  if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess)
    return f();
  (void)hipEventRecord(r.start, st);
  const hipError_t e = f();
  (void)hipEventRecord(r.stop, st);
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof.push_back(r);
  return e;
}

// A window of T or more keys can exclude nothing inside a segment, so it is
// the global (full causal) case; mapping it to 0 keeps index arithmetic far
// from int overflow.
int32_t effective_window(int32_t window, int32_t total_tokens) {
  return (window <= 0 || window >= total_tokens) ? 0 : window;
}

}  // namespace

namespace {

attn_status fwd_impl(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                     int32_t num_seqs, int32_t total_tokens, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen, int32_t window,
                     float scale, float softcap, uint32_t flags, bool band, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  WorkspaceLayout w;
  attn_status s = check_common(q, k, v, cu_seqlens, total_tokens, num_seqs, num_q_heads,
                               num_kv_heads, head_dim, max_seqlen, scale, workspace,
                               workspace_bytes, &w);
  if (s != ATTN_OK) return s;
  if (!out || !lse || !aligned(out, 16) || !aligned(lse, 4)) return ATTN_EINVAL;
  if (!std::isfinite(softcap) || softcap < 0.f) return ATTN_EINVAL;
  if (flags & ~(uint32_t)ATTN_FWD_REUSE_SCHEDULE) return ATTN_EINVAL;
  if (band && window <= 0) return ATTN_EINVAL;
  s = check_device();
  if (s != ATTN_OK) return s;
  const int32_t wnd = effective_window(window, total_tokens);
  const Problem p{total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, wnd, scale,
                  softcap, band && wnd > 0 ? 1 : 0, max_seqlen};
  hipStream_t st = static_cast<hipStream_t>(stream);
  // both lists, so that the matching backward call (and later layers) may
  // reuse them
  if (!(flags & ATTN_FWD_REUSE_SCHEDULE) && timed_launch(K_SCHEDULE, st, [&] {
        return attn::launch_schedule(cu_seqlens, p, true, workspace, w, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  if (timed_launch(K_FORWARD, st, [&] {
        return attn::launch_forward(q, k, v, p, out, lse, workspace, w, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  return ATTN_OK;
}

attn_status bwd_impl(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, const int32_t* cu_seqlens,
                     int32_t num_seqs, int32_t total_tokens, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen, int32_t window,
                     float scale, float softcap, uint32_t flags, bool band, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  WorkspaceLayout w;
  attn_status s = check_common(q, k, v, cu_seqlens, total_tokens, num_seqs, num_q_heads,
                               num_kv_heads, head_dim, max_seqlen, scale, workspace,
                               workspace_bytes, &w);
  if (s != ATTN_OK) return s;
  if (!out || !lse || !dout || !dq || !dk || !dv) return ATTN_EINVAL;
  if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(lse, 4) || !aligned(dq, 16) ||
      !aligned(dk, 16) || !aligned(dv, 16))
    return ATTN_EINVAL;
  if (!std::isfinite(softcap) || softcap < 0.f) return ATTN_EINVAL;
  if (flags & ~(uint32_t)ATTN_BWD_REUSE_SCHEDULE) return ATTN_EINVAL;
  if (band && window <= 0) return ATTN_EINVAL;
  s = check_device();
  if (s != ATTN_OK) return s;
  const int32_t wnd = effective_window(window, total_tokens);
  const Problem p{total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, wnd, scale,
                  softcap, band && wnd > 0 ? 1 : 0, max_seqlen};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!(flags & ATTN_BWD_REUSE_SCHEDULE) &&
      timed_launch(K_SCHEDULE, st, [&] {
        return attn::launch_schedule(cu_seqlens, p, true, workspace, w, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  if (timed_launch(K_DQ, st, [&] {
        return attn::launch_dq(q, k, v, out, lse, dout, p, dq, workspace, w, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  if (timed_launch(K_DKDV, st, [&] {
        return attn::launch_dkdv(q, k, v, lse, dout, p, dk, dv, workspace, w, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_varlen_workspace_size(int32_t total_tokens, int32_t num_seqs_cap,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seqlen, int32_t window) {
  (void)window;
  if (check_shape(total_tokens, num_seqs_cap, num_q_heads, num_kv_heads, head_dim,
                  max_seqlen) != ATTN_OK)
    return 0;
  return attn::workspace_layout(total_tokens, num_seqs_cap, num_q_heads).total;
}

attn_status attn_varlen_fwd_ex(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t max_seqlen, int32_t window, float scale, float softcap,
                               uint32_t flags, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, attn_stream_t stream) {
  return fwd_impl(q, k, v, cu_seqlens, num_seqs, total_tokens, num_q_heads, num_kv_heads,
                  head_dim, max_seqlen, window, scale, softcap, flags, false, out, lse, workspace,
                  workspace_bytes, stream);
}

attn_status attn_varlen_schedule(const int32_t* cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen,
                                 int32_t window, void* workspace, size_t workspace_bytes,
                                 attn_stream_t stream) {
  attn_status s = check_shape(total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                              max_seqlen);
  if (s != ATTN_OK) return s;
  if (!cu_seqlens || !aligned(cu_seqlens, 4)) return ATTN_EINVAL;
  const WorkspaceLayout w = attn::workspace_layout(total_tokens, num_seqs, num_q_heads);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w.total) return ATTN_EWORKSPACE;
  s = check_device();
  if (s != ATTN_OK) return s;
  const int32_t wnd = effective_window(window, total_tokens);
  const Problem p{total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, wnd, 1.f,
                  0.f, 0, max_seqlen};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (timed_launch(K_SCHEDULE, st, [&] {
        return attn::launch_schedule(cu_seqlens, p, true, workspace, w, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  return ATTN_OK;
}

attn_status attn_varlen_fwd(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_seqlen, int32_t window, float scale, void* out,
                            float* lse, void* workspace, size_t workspace_bytes,
                            attn_stream_t stream) {
  return attn_varlen_fwd_ex(q, k, v, cu_seqlens, num_seqs, total_tokens, num_q_heads,
                            num_kv_heads, head_dim, max_seqlen, window, scale, 0.f, 0u, out, lse,
                            workspace, workspace_bytes, stream);
}

attn_status attn_varlen_bwd_ex(const void* q, const void* k, const void* v, const void* out,
                               const float* lse, const void* dout, const int32_t* cu_seqlens,
                               int32_t num_seqs, int32_t total_tokens, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen,
                               int32_t window, float scale, float softcap, uint32_t flags,
                               void* dq, void* dk, void* dv, void* workspace,
                               size_t workspace_bytes, attn_stream_t stream) {
  return bwd_impl(q, k, v, out, lse, dout, cu_seqlens, num_seqs, total_tokens, num_q_heads,
                  num_kv_heads, head_dim, max_seqlen, window, scale, softcap, flags, false, dq,
                  dk, dv, workspace, workspace_bytes, stream);
}

attn_status attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t total_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen,
                            int32_t window, float scale, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  return attn_varlen_bwd_ex(q, k, v, out, lse, dout, cu_seqlens, num_seqs, total_tokens,
                            num_q_heads, num_kv_heads, head_dim, max_seqlen, window, scale, 0.f,
                            0u, dq, dk, dv, workspace, workspace_bytes, stream);
}

attn_status attn_varlen_band_fwd(const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seqlen, int32_t window,
                                 float scale, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, attn_stream_t stream) {
  return fwd_impl(q, k, v, cu_seqlens, num_seqs, total_tokens, num_q_heads, num_kv_heads,
                  head_dim, max_seqlen, window, scale, 0.f, 0u, true, out, lse, workspace,
                  workspace_bytes, stream);
}

attn_status attn_varlen_band_bwd(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, const void* dout, const int32_t* cu_seqlens,
                                 int32_t num_seqs, int32_t total_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen,
                                 int32_t window, float scale, void* dq, void* dk, void* dv,
                                 void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  return bwd_impl(q, k, v, out, lse, dout, cu_seqlens, num_seqs, total_tokens, num_q_heads,
                  num_kv_heads, head_dim, max_seqlen, window, scale, 0.f, 0u, true, dq, dk, dv,
                  workspace, workspace_bytes, stream);
}

namespace {
// Shape and pointer checks shared by the delta-rule calls.
attn_status check_delta(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                        int32_t total_tokens, int32_t num_heads, int32_t head_dim, float scale) {
  if (total_tokens <= 0 || num_seqs <= 0 || num_heads <= 0) return ATTN_EINVAL;
  if (head_dim != attn::DELTA_DIM) return ATTN_EUNSUPPORTED;
  if (!q || !k || !v || !g || !beta || !cu_seqlens) return ATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 4) ||
      !aligned(beta, 4) || !aligned(cu_seqlens, 4))
    return ATTN_EINVAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_EINVAL;
  const attn::DeltaLayout w = attn::delta_layout(total_tokens, num_seqs, num_heads);
  if (w.chunk_cap * (size_t)num_heads >= ((size_t)1 << 31) ||
      (size_t)num_seqs * num_heads * attn::DELTA_DIM >= ((size_t)1 << 31))
    return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

size_t delta_workspace(int32_t total_tokens, int32_t num_seqs_cap, int32_t num_heads,
                       int32_t head_dim, bool backward) {
  if (total_tokens <= 0 || num_seqs_cap <= 0 || num_heads <= 0 || head_dim != attn::DELTA_DIM)
    return 0;
  const attn::DeltaLayout w =
      attn::delta_layout(total_tokens, num_seqs_cap, num_heads, backward);
  if (w.chunk_cap * (size_t)num_heads >= ((size_t)1 << 31)) return 0;
  return w.total;
}
}  // namespace

size_t attn_delta_workspace_size(int32_t total_tokens, int32_t num_seqs_cap, int32_t num_heads,
                                 int32_t head_dim) {
  return delta_workspace(total_tokens, num_seqs_cap, num_heads, head_dim, false);
}

size_t attn_delta_bwd_workspace_size(int32_t total_tokens, int32_t num_seqs_cap,
                                     int32_t num_heads, int32_t head_dim) {
  return delta_workspace(total_tokens, num_seqs_cap, num_heads, head_dim, true);
}

attn_status attn_delta_fwd_ex(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                              float scale, uint32_t flags, void* out, void* workspace,
                              size_t workspace_bytes, attn_stream_t stream) {
  if (flags & ~(uint32_t)ATTN_DELTA_FWD_SAVE) return ATTN_EINVAL;
  const bool save = flags & ATTN_DELTA_FWD_SAVE;
  attn_status s = check_delta(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                              head_dim, scale);
  if (s != ATTN_OK) return s;
  if (!out || !aligned(out, 16)) return ATTN_EINVAL;
  const attn::DeltaLayout w = attn::delta_layout(total_tokens, num_seqs, num_heads, save);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w.total) return ATTN_EWORKSPACE;
  s = check_device();
  if (s != ATTN_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (timed_launch(K_DELTA, st, [&] {
        return attn::launch_delta_fwd(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens,
                                      num_heads, scale, out, workspace, w, save, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  return ATTN_OK;
}

attn_status attn_delta_fwd(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t total_tokens, int32_t num_heads, int32_t head_dim, float scale,
                           void* out, void* workspace, size_t workspace_bytes,
                           attn_stream_t stream) {
  return attn_delta_fwd_ex(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                           head_dim, scale, 0u, out, workspace, workspace_bytes, stream);
}

size_t attn_kda_workspace_size(int32_t total_tokens, int32_t num_seqs_cap, int32_t num_heads,
                               int32_t head_dim) {
  if (delta_workspace(total_tokens, num_seqs_cap, num_heads, head_dim, false) == 0) return 0;
  return attn::delta_layout(total_tokens, num_seqs_cap, num_heads, false, attn::kda_record_floats())
      .total;
}

attn_status attn_kda_fwd_ex(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                            float scale, uint32_t flags, void* out, void* workspace,
                            size_t workspace_bytes, attn_stream_t stream) {
  if (flags & ~(uint32_t)ATTN_DELTA_FWD_SAVE) return ATTN_EINVAL;
  const bool save = flags & ATTN_DELTA_FWD_SAVE;
  attn_status s = check_delta(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                              head_dim, scale);
  if (s != ATTN_OK) return s;
  if (!out || !aligned(out, 16) || !aligned(g, 16)) return ATTN_EINVAL;
  const attn::DeltaLayout w = attn::delta_layout(total_tokens, num_seqs, num_heads, save,
                                                 attn::kda_record_floats(), save);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w.total) return ATTN_EWORKSPACE;
  s = check_device();
  if (s != ATTN_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (timed_launch(K_KDA, st, [&] {
        return attn::launch_kda_fwd(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens,
                                    num_heads, scale, out, workspace, w, save, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  return ATTN_OK;
}

attn_status attn_kda_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                         int32_t total_tokens, int32_t num_heads, int32_t head_dim, float scale,
                         void* out, void* workspace, size_t workspace_bytes,
                         attn_stream_t stream) {
  return attn_kda_fwd_ex(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                         head_dim, scale, 0u, out, workspace, workspace_bytes, stream);
}

size_t attn_kda_bwd_workspace_size(int32_t total_tokens, int32_t num_seqs_cap,
                                   int32_t num_heads, int32_t head_dim) {
  if (delta_workspace(total_tokens, num_seqs_cap, num_heads, head_dim, false) == 0) return 0;
  return attn::delta_layout(total_tokens, num_seqs_cap, num_heads, true, attn::kda_record_floats(),
                           true)
      .total;
}

attn_status attn_kda_bwd_ex(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const void* dout, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                            int32_t head_dim, float scale, uint32_t flags, void* dq, void* dk,
                            void* dv, float* dg, float* dbeta, void* workspace,
                            size_t workspace_bytes, attn_stream_t stream) {
  if (flags & ~(uint32_t)ATTN_DELTA_BWD_REUSE) return ATTN_EINVAL;
  attn_status s = check_delta(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                              head_dim, scale);
  if (s != ATTN_OK) return s;
  if (!dout || !dq || !dk || !dv || !dg || !dbeta) return ATTN_EINVAL;
  if (!aligned(g, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
      !aligned(dv, 16) || !aligned(dg, 16) || !aligned(dbeta, 4))
    return ATTN_EINVAL;
  const attn::DeltaLayout w = attn::delta_layout(total_tokens, num_seqs, num_heads, true,
                                                 attn::kda_record_floats(), true);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w.total) return ATTN_EWORKSPACE;
  s = check_device();
  if (s != ATTN_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (timed_launch(K_KDA_BWD, st, [&] {
        return attn::launch_kda_bwd(q, k, v, g, beta, dout, cu_seqlens, num_seqs, total_tokens,
                                    num_heads, scale, dq, dk, dv, dg, dbeta, workspace, w,
                                    flags & ATTN_DELTA_BWD_REUSE, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  return ATTN_OK;
}

attn_status attn_kda_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const void* dout, const int32_t* cu_seqlens,
                         int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                         int32_t head_dim, float scale, void* dq, void* dk, void* dv, float* dg,
                         float* dbeta, void* workspace, size_t workspace_bytes,
                         attn_stream_t stream) {
  return attn_kda_bwd_ex(q, k, v, g, beta, dout, cu_seqlens, num_seqs, total_tokens, num_heads,
                         head_dim, scale, 0u, dq, dk, dv, dg, dbeta, workspace, workspace_bytes,
                         stream);
}

attn_status attn_delta_bwd_ex(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const void* dout, const int32_t* cu_seqlens,
                              int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                              int32_t head_dim, float scale, uint32_t flags, void* dq, void* dk,
                              void* dv, float* dg, float* dbeta, void* workspace,
                              size_t workspace_bytes, attn_stream_t stream) {
  if (flags & ~(uint32_t)ATTN_DELTA_BWD_REUSE) return ATTN_EINVAL;
  attn_status s = check_delta(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                              head_dim, scale);
  if (s != ATTN_OK) return s;
  if (!dout || !dq || !dk || !dv || !dg || !dbeta) return ATTN_EINVAL;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(dg, 4) || !aligned(dbeta, 4))
    return ATTN_EINVAL;
  const attn::DeltaLayout w = attn::delta_layout(total_tokens, num_seqs, num_heads, true);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w.total) return ATTN_EWORKSPACE;
  s = check_device();
  if (s != ATTN_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (timed_launch(K_DELTA_BWD, st, [&] {
        return attn::launch_delta_bwd(q, k, v, g, beta, dout, cu_seqlens, num_seqs, total_tokens,
                                      num_heads, scale, dq, dk, dv, dg, dbeta, workspace, w,
                                      flags & ATTN_DELTA_BWD_REUSE, st);
      }) != hipSuccess)
    return ATTN_ELAUNCH;
  return ATTN_OK;
}

attn_status attn_delta_bwd(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const void* dout, const int32_t* cu_seqlens,
                           int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                           int32_t head_dim, float scale, void* dq, void* dk, void* dv, float* dg,
                           float* dbeta, void* workspace, size_t workspace_bytes,
                           attn_stream_t stream) {
  return attn_delta_bwd_ex(q, k, v, g, beta, dout, cu_seqlens, num_seqs, total_tokens, num_heads,
                           head_dim, scale, 0u, dq, dk, dv, dg, dbeta, workspace, workspace_bytes,
                           stream);
}

}  // extern "C"

namespace {

// Device memory of attn_varlen_bwd_static: a file-scope array that every GPU
// the library runs on holds from module load until the process ends.  Host
// code never uses the array's name as an address (on the host it is only a
// stand-in symbol): the device address of each GPU's copy is looked up once
// per device with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = (size_t)ATTN_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call on
// that device, with the device current).
attn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_varlen_static_scratch_bytes(void) { return kScratchBytes; }

attn_status attn_varlen_bwd_static(const void* q, const void* k, const void* v, const void* out,
                                   const float* lse, const void* dout,
                                   const int32_t* cu_seqlens, int32_t num_seqs,
                                   int32_t total_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen,
                                   int32_t window, float scale, void* dq, void* dk, void* dv,
                                   attn_stream_t stream) {
  // The sizes are checked before the scratch is looked up, so a problem too
  // large for it is refused without touching the device.
  attn_status s = check_shape(total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                              max_seqlen);
  if (s != ATTN_OK) return s;
  if (attn::workspace_layout(total_tokens, num_seqs, num_q_heads).total > kScratchBytes)
    return ATTN_ESCRATCH;
  s = check_device();
  if (s != ATTN_OK) return s;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != ATTN_OK) return s;
  // Same kernels as attn_varlen_bwd, with the static scratch as workspace:
  // the schedule kernel rewrites the header and lists, and the dQ kernel
  // every row statistic the dK/dV kernel then reads, so nothing in the
  // scratch has to start at zero.
  return bwd_impl(q, k, v, out, lse, dout, cu_seqlens, num_seqs, total_tokens, num_q_heads,
                  num_kv_heads, head_dim, max_seqlen, window, scale, 0.f, 0u, false, dq, dk, dv,
                  ws, kScratchBytes, stream);
}

const char* attn_varlen_strerror(attn_status s) {
  switch (s) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument (null or misaligned pointer, bad size or scale)";
    case ATTN_EUNSUPPORTED: return "unsupported shape (head_dim must be 64, 128 or 256, k under 4 GiB)";
    case ATTN_EWORKSPACE: return "workspace missing, misaligned (256 B) or too small";
    case ATTN_EDEVICE: return "no usable gfx950 device";
    case ATTN_ELAUNCH: return "kernel launch failed";
    case ATTN_ESCRATCH: return "problem needs more workspace than the static scratch of attn_varlen_bwd_static";
  }
  return "unknown status";
}

int32_t attn_varlen_version(void) { return 30000; }

attn_status attn_varlen_profile_start(void) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  for (ProfileRecord& r : g_prof) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  g_prof_on.store(true);
  return ATTN_OK;
}

int32_t attn_varlen_profile_stop(attn_kernel_stats* stats, int32_t cap) {
  g_prof_on.store(false);
  std::lock_guard<std::mutex> lock(g_prof_mu);
  attn_kernel_stats acc[K_COUNT];
  std::memset(acc, 0, sizeof(acc));
  attn_status status = ATTN_OK;
  for (ProfileRecord& r : g_prof) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      status = ATTN_EDEVICE;
    attn_kernel_stats& a = acc[r.kernel];
    if (a.launches == 0 || ms < a.min_ms) a.min_ms = ms;
    if (ms > a.max_ms) a.max_ms = ms;
    a.total_ms += ms;
    a.launches += 1;
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  if (status != ATTN_OK) return status;
  int32_t n = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    if (acc[k].launches == 0) continue;
    if (stats && n < cap) {
      stats[n] = acc[k];
      std::snprintf(stats[n].name, sizeof(stats[n].name), "%s", kKernelNames[k]);
    }
    ++n;
  }
  return n;
}

}  // extern "C"
