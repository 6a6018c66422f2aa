/*
 * attn_varlen.h -- C ABI of libattn_varlen.so: document-masked (varlen)
 * causal grouped-query attention, forward and backward, for AMD Instinct
 * MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * A packed microbatch of T tokens is split into segments [cu[s], cu[s+1]).
 * Attention is confined to each segment and causal inside it
 * (research.dws.rip/llm/kernels, section 01 "How it was measured").  Local layers add a sliding window, global layers use full
 * causal context; query heads share key-value heads in groups (same page,
 * Fig. 2 "Benchmark setup": 8 query / 2 key-value heads of width 128,
 * 512-token window; section 02: the call is a varlen attention with sliding
 * windows and grouped-query attention).  With G = Hq / Hkv, query head h
 * reads key-value head floor(h / G), and for query i of segment [a, b):
 *
 *   visible keys  V(i) = { j : max(a, i - W + 1) <= j <= i }   (W <= 0: a <= j <= i)
 *   S_ij  = scale * q_{i,h} . k_{j,g}
 *   lse   = log sum_{j in V(i)} exp(S_ij)                       (natural log)
 *   out   = sum_j exp(S_ij - lse) v_{j,g}
 *
 * and the backward pass returns the gradients of sum(dout * out) with
 * respect to q, k and v (dk, dv summed over the G query heads of a group).
 *
 * Layouts (all row-major, head dim innermost, no strides):
 *   q, out, dout, dq : bf16 [T, Hq, D]
 *   k, v, dk, dv     : bf16 [T, Hkv, D]
 *   lse              : fp32 [Hq, T]
 *   cu_seqlens       : int32 [num_seqs + 1], on the device
 * Tensor pointers are device pointers, 16-byte aligned.  The caller owns
 * every buffer; the library never allocates, frees or keeps a pointer after
 * a call returns.
 *
 * Conventions where the pages are silent
 *   window <= 0      : full causal context inside each segment
 *   window W >= 1    : W keys counting the query itself (i - W < j <= i)
 *   cu_seqlens       : non-decreasing, cu[0] = 0, cu[num_seqs] = T; empty
 *                      segments are allowed (padding to a fixed count) and
 *                      change nothing, bit for bit
 *                      (research.dws.rip/llm/kernels, section 06 "CUDA
 *                      graphs work, with padding")
 *   max_seqlen       : >= the longest segment (used to bound the schedule)
 *   supported shapes : D in {64, 128, 256}, any Hq % Hkv == 0 (grouped,
 *                      multi-query or multi-head), and k (T x Hkv x D bf16)
 *                      under 4 GiB
 *
 * Execution
 *   Every call enqueues its kernels on `stream` and returns without waiting
 *   and without reading device memory on the host, so calls can be captured
 *   in a HIP graph.  The contents of cu_seqlens are checked on the device
 *   by the schedule kernel (cu[0] = 0, non-decreasing, cu[num_seqs] = T):
 *   malformed boundaries make every output of the call NaN (the kernels stay
 *   inside their buffers either way); the host cannot see them without a
 *   device read, so the call still returns ATTN_OK.  Calls are
 *   deterministic: the same inputs give bit-identical outputs (no
 *   floating-point atomics).
 *
 * Errors
 *   Host-checkable problems return a negative attn_status before anything is
 *   enqueued; outputs are then untouched.  ATTN_ELAUNCH reports a launch
 *   failure from the HIP runtime.  Nothing is thrown across the ABI.
 */
#ifndef ATTN_VARLEN_H
#define ATTN_VARLEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = -1,       /* null/misaligned pointer, bad size, bad scale, ... */
  ATTN_EUNSUPPORTED = -2, /* valid arguments this build does not implement (D, k >= 4 GiB) */
  ATTN_EWORKSPACE = -3,   /* workspace null or smaller than attn_varlen_workspace_size() */
  ATTN_EDEVICE = -4,      /* no usable gfx950 device / HIP runtime error before launch */
  ATTN_ELAUNCH = -5,      /* a kernel launch failed */
  ATTN_ESCRATCH = -6      /* attn_varlen_bwd_static: the problem needs more than its static scratch */
} attn_status;

/* opaque stream handle: a hipStream_t (0 = the legacy default stream) */
typedef void* attn_stream_t;

/*
 * Bytes of device workspace one fwd or bwd call needs.  It holds the tile
 * schedule (rebuilt on the device by every call) and, for the backward,
 * the per-row D = rowsum(dout * out) in fp32.  Returns 0 for arguments
 * the calls would reject.
 *   total_tokens  T > 0
 *   num_seqs_cap  the num_seqs the calls will pass (>= 1)
 */
size_t attn_varlen_workspace_size(int32_t total_tokens, int32_t num_seqs_cap,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seqlen, int32_t window);

/*
 * Forward pass: out and lse from q, k, v.
 *   q, k, v        bf16 inputs (layouts above), read only
 *   cu_seqlens     int32 device array of num_seqs + 1 segment boundaries
 *   scale          multiplies q.k before the softmax; finite and > 0
 *   out            bf16 [T, Hq, D], written fully
 *   lse            fp32 [Hq, T] natural-log normaliser, written fully
 *   workspace      device memory of at least attn_varlen_workspace_size()
 *                  bytes, 256-byte aligned; contents need not be initialised
 */
attn_status attn_varlen_fwd(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_seqlen, int32_t window, float scale,
                            void* out, float* lse,
                            void* workspace, size_t workspace_bytes, attn_stream_t stream);

/*
 * Backward pass: dq, dk, dv from q, k, v, the forward's out and lse, and
 * dout.  Same argument meanings as attn_varlen_fwd; out and lse must be the
 * forward's results for the same inputs.  dq, dk, dv are written fully
 * (rows of every segment; tokens outside all segments cannot exist since
 * cu[num_seqs] = T).
 */
attn_status attn_varlen_bwd(const void* q, const void* k, const void* v,
                            const void* out, const float* lse, const void* dout,
                            const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_seqlen, int32_t window, float scale,
                            void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes, attn_stream_t stream);

/*
 * Forward and backward with an optional logit soft-cap.  With softcap = c > 0
 * every scaled logit S = scale * q.k is replaced by c * tanh(S / c) before
 * the softmax (Gemma 2's attention soft-cap, which the performance reference
 * page dewml.dev/reference/performance lists, in its section on head
 * dimension 256 through tokamax's Triton flash attention, as a feature the
 * backward must support too), lse is taken over the capped logits, and the
 * backward carries the cap's derivative 1 - tanh^2(S / c) into dq and dk.
 * softcap = 0 is exactly attn_varlen_fwd / attn_varlen_bwd.  Other
 * arguments as there; the backward must get the same softcap as the forward
 * that produced out and lse.
 *   softcap   finite and >= 0; negative, NaN or infinite -> ATTN_EINVAL
 *   flags     forward: 0 or ATTN_FWD_REUSE_SCHEDULE; backward: 0 or
 *             ATTN_BWD_REUSE_SCHEDULE; other bits -> ATTN_EINVAL
 *
 * Schedule reuse: every forward call that builds a schedule leaves in its
 * workspace the tile lists of both passes (they depend only on cu_seqlens,
 * total_tokens, num_seqs and the window).  A later call on the same stream
 * with the same workspace and the same cu_seqlens contents, num_seqs,
 * total_tokens and window may skip rebuilding them: the backward of the same
 * layer (ATTN_BWD_REUSE_SCHEDULE), or the forward (ATTN_FWD_REUSE_SCHEDULE)
 * and backward of another layer of a stack that shares the boundaries and
 * the window.  The caller vouches for the cu_seqlens contents; the kernels
 * compare total_tokens, num_seqs and the window with the schedule's record
 * on the device and, if they differ (or the schedule's boundaries were
 * malformed), write NaN to every output of the call instead of computing
 * it.  Calls that share a workspace must not overlap in time (one stream).
 */
enum { ATTN_BWD_REUSE_SCHEDULE = 1, ATTN_FWD_REUSE_SCHEDULE = 1 };

/*
 * Builds only the tile schedule (the lists of both passes and their record,
 * as a forward call without ATTN_FWD_REUSE_SCHEDULE would) in workspace, so
 * that it can be made ahead of the calls that use it with the REUSE flags:
 * for instance on a second stream while the previous layer's kernels run,
 * the caller ordering the two streams (events) so that the schedule is done
 * before its first use and no call still using the workspace's previous
 * schedule overlaps it.  Arguments as for attn_varlen_fwd (the head counts
 * and head dim only size and validate the workspace).  Same error
 * behaviour; nothing but the workspace is written.
 */
attn_status attn_varlen_schedule(const int32_t* cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen,
                                 int32_t window, void* workspace, size_t workspace_bytes,
                                 attn_stream_t stream);

attn_status attn_varlen_fwd_ex(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens, int32_t num_seqs,
                               int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_seqlen, int32_t window, float scale,
                               float softcap, uint32_t flags, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, attn_stream_t stream);

attn_status attn_varlen_bwd_ex(const void* q, const void* k, const void* v,
                               const void* out, const float* lse, const void* dout,
                               const int32_t* cu_seqlens, int32_t num_seqs,
                               int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_seqlen, int32_t window, float scale,
                               float softcap, uint32_t flags, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, attn_stream_t stream);

/*
 * Band-block formulation of the windowed calls (the performance reference
 * page dewml.dev/reference/performance, section "Packed sliding-window
 * attention on GPU: local_attention": queries in blocks of W, each block
 * against a [W, 2W] band of keys, its own block and the one before it, with
 * the window, causal and document mask inside the band).  Blocks are aligned
 * to token 0 of the microbatch.  Same arguments, layouts, ownership and
 * errors as attn_varlen_fwd / attn_varlen_bwd, plus: window must be >= 1
 * (ATTN_EINVAL otherwise; a window >= total_tokens makes one band hold
 * everything, the global case).  Each q-tile loops over every key block of
 * its rows' bands (and each k-tile over every query block whose band holds
 * its keys) within the segment, with the same per-row mask, so the results
 * equal the plain calls' bit for bit while the kernels process the band's
 * masked blocks too: a cross-check of the window ranges and a measure of
 * the band's cost.  The backward always rebuilds its schedule.
 */
attn_status attn_varlen_band_fwd(const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seqlen, int32_t window,
                                 float scale, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, attn_stream_t stream);

attn_status attn_varlen_band_bwd(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, const void* dout, const int32_t* cu_seqlens,
                                 int32_t num_seqs, int32_t total_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen,
                                 int32_t window, float scale, void* dq, void* dk, void* dv,
                                 void* workspace, size_t workspace_bytes, attn_stream_t stream);

/*
 * Gated delta-rule linear attention (Gated DeltaNet), forward: the competing
 * local layer of the kernel benchmarks page (research.dws.rip/llm/kernels,
 * section 03 "What linear attention costs", Figs. 1 and 5), per the gated
 * delta rule it names.  Per head h and document of cu_seqlens (the state
 * starts at zero at every document start), with a d_v x d_k state S:
 *   S_t = exp(g_t) S_{t-1} + beta_t (v_t - exp(g_t) S_{t-1} k_t) k_t^T,
 *   out_t = scale S_t q_t.
 *   q, k, v     bf16 [T, H, D] (head dim D = d_k = d_v), contiguous, 16-byte aligned
 *   g           fp32 [T, H], log decay (<= 0 in use; not checked)
 *   beta        fp32 [T, H], write strength (in (0, 1) in use; not checked)
 *   out         bf16 [T, H, D], written fully for tokens inside documents
 *   scale       finite and > 0
 *   supported   D == 128 (ATTN_EUNSUPPORTED otherwise); any H >= 1
 *   workspace   >= attn_delta_workspace_size(T, num_seqs, H, D) bytes, 256-byte
 *               aligned: per (64-token chunk, head) fp32 records of the chunk's
 *               triangular-solve results, about 100 KB each
 * Enqueues three kernels on `stream` (chunk plan, per-chunk preparation,
 * per-document scan); same ownership and error conventions as the
 * attention calls.
 */
size_t attn_delta_workspace_size(int32_t total_tokens, int32_t num_seqs_cap, int32_t num_heads,
                                 int32_t head_dim);

attn_status attn_delta_fwd(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t total_tokens, int32_t num_heads, int32_t head_dim, float scale,
                           void* out, void* workspace, size_t workspace_bytes,
                           attn_stream_t stream);

/*
 * Gated delta-rule backward: the gradients of sum(dout * out) for the
 * forward above, with the same inputs and checks.
 *   dout        bf16 [T, H, D]
 *   dq, dk, dv  bf16 [T, H, D], written for tokens inside documents
 *   dg, dbeta   fp32 [T, H], written for tokens inside documents
 *   workspace   >= attn_delta_bwd_workspace_size(T, num_seqs, H, D) bytes,
 *               256-byte aligned: the forward's records (with the triangular
 *               inverse kept), each chunk's start state and end-state
 *               gradient (fp32 D x D), its dU and dW, about 297 KB per
 *               (64-token chunk, head)
 * Recomputes the forward's records and chunk states (three kernels), then
 * runs a reverse per-document scan and two per-chunk gradient kernels, all
 * on `stream`; nothing allocated.
 *
 * The _ex forms take flags (other bits -> ATTN_EINVAL):
 * ATTN_DELTA_FWD_SAVE (forward): the forward also keeps, in a workspace of
 * attn_delta_bwd_workspace_size bytes, everything its backward needs (the
 * records with the inverse, each chunk's start state and U).
 * ATTN_DELTA_BWD_REUSE (backward): skips recomputing them, taking those of
 * the last saving forward call in the same workspace on the same stream.
 * The caller vouches that it had the same q, k, v, g, beta and cu_seqlens
 * contents (the pair of calls of one layer in a training step); the kernels
 * check on the device that it was a saving forward with the same
 * total_tokens, heads and num_seqs, and otherwise do nothing (outputs
 * unwritten).  A reusing backward leaves the saved data intact, so it may
 * run more than once.
 */
enum { ATTN_DELTA_FWD_SAVE = 1, ATTN_DELTA_BWD_REUSE = 1 };

size_t attn_delta_bwd_workspace_size(int32_t total_tokens, int32_t num_seqs_cap,
                                     int32_t num_heads, int32_t head_dim);

attn_status attn_delta_bwd(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const void* dout, const int32_t* cu_seqlens,
                           int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                           int32_t head_dim, float scale, void* dq, void* dk, void* dv, float* dg,
                           float* dbeta, void* workspace, size_t workspace_bytes,
                           attn_stream_t stream);

attn_status attn_delta_fwd_ex(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                              float scale, uint32_t flags, void* out, void* workspace,
                              size_t workspace_bytes, attn_stream_t stream);

attn_status attn_delta_bwd_ex(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const void* dout, const int32_t* cu_seqlens,
                              int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                              int32_t head_dim, float scale, uint32_t flags, void* dq, void* dk,
                              void* dv, float* dg, float* dbeta, void* workspace,
                              size_t workspace_bytes, attn_stream_t stream);

/*
 * Kimi Delta Attention forward: the gated delta rule with one decay per key
 * channel, the second linear layer the kernel benchmarks page
 * (research.dws.rip/llm/kernels, section 03, Figs. 1 and 5) times, per the
 * published recurrence.  Per head and document (state reset to zero at
 * every document start), with alpha_t = exp(g_t) a vector over d_k:
 *   S'_t = S_{t-1} Diag(alpha_t),
 *   S_t = S'_t + beta_t (v_t - S'_t k_t) k_t^T,  out_t = scale S_t q_t.
 *   q, k, v, out  as attn_delta_fwd
 *   g             fp32 [T, H, D], per-channel log decay, 16-byte aligned
 *   beta          fp32 [T, H]
 *   workspace     >= attn_kda_workspace_size(T, num_seqs, H, D) bytes,
 *                 256-byte aligned: per (64-token chunk, head) an fp32 record
 *                 of about 181 KB (the backward's layout: its triangular
 *                 inverse and decayed K K^T are written only by the backward)
 * Enqueues three kernels (chunk plan, per-chunk preparation, per-document
 * scan) on `stream`; conventions as attn_delta_fwd.  The factors it forms
 * are decays over at most one chunk or, in the in-chunk products, over at
 * most three tokens, so any g <= 0 is safe.
 */
size_t attn_kda_workspace_size(int32_t total_tokens, int32_t num_seqs_cap, int32_t num_heads,
                               int32_t head_dim);

attn_status attn_kda_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                         int32_t total_tokens, int32_t num_heads, int32_t head_dim, float scale,
                         void* out, void* workspace, size_t workspace_bytes,
                         attn_stream_t stream);

/*
 * Kimi Delta Attention backward: the gradients of sum(dout * out) for
 * attn_kda_fwd with the same inputs and checks.
 *   dout          bf16 [T, H, D]
 *   dq, dk, dv    bf16 [T, H, D]; dg fp32 [T, H, D] (16-byte aligned);
 *                 dbeta fp32 [T, H]; written for tokens inside documents
 *   workspace     >= attn_kda_bwd_workspace_size(T, num_seqs, H, D) bytes,
 *                 256-byte aligned: the forward's records (with T and the
 *                 decayed K K^T), each chunk's start state and end-state
 *                 gradient, dU, dW and two pair-gradient matrices, about 410 KB per
 *                 (64-token chunk, head)
 * Recomputes the forward's records and chunk states, then runs a reverse
 * per-document scan and three per-chunk gradient kernels (state products,
 * triangular solve, decayed pair products): seven kernels on `stream`,
 * nothing allocated.  Every exponential it forms is a decay (at most 1).
 */
size_t attn_kda_bwd_workspace_size(int32_t total_tokens, int32_t num_seqs_cap,
                                   int32_t num_heads, int32_t head_dim);

/*
 * As the Gated DeltaNet _ex pair: attn_kda_fwd_ex(ATTN_DELTA_FWD_SAVE) keeps
 * the records and chunk states in a workspace of
 * attn_kda_bwd_workspace_size bytes, and attn_kda_bwd_ex(ATTN_DELTA_BWD_REUSE)
 * takes them instead of recomputing, under the same contract and device
 * check; the saved data stays intact, so a reusing backward may repeat.
 */
attn_status attn_kda_fwd_ex(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                            float scale, uint32_t flags, void* out, void* workspace,
                            size_t workspace_bytes, attn_stream_t stream);

attn_status attn_kda_bwd_ex(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const void* dout, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                            int32_t head_dim, float scale, uint32_t flags, void* dq, void* dk,
                            void* dv, float* dg, float* dbeta, void* workspace,
                            size_t workspace_bytes, attn_stream_t stream);

attn_status attn_kda_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const void* dout, const int32_t* cu_seqlens,
                         int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                         int32_t head_dim, float scale, void* dq, void* dk, void* dv, float* dg,
                         float* dbeta, void* workspace, size_t workspace_bytes,
                         attn_stream_t stream);

/*
 * Backward pass that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): attn_varlen_bwd with the same arguments minus
 * the workspace.  The schedule and the per-row statistics the kernels pass
 * between them live in a static device array of
 * ATTN_STATIC_SCRATCH_BYTES (16 MiB) that the library holds on every GPU it
 * runs on until the process ends; the call itself calls no allocator.
 *   - The problem's workspace (attn_varlen_workspace_size) must fit in it:
 *     otherwise ATTN_ESCRATCH, before anything is enqueued.  About 256 B per
 *     (32-token tile, query head) plus the tile lists: e.g. T = 16,384 with
 *     Hq = 8 needs 1.2 MB, and T = 65,536 with Hq = 16 about 8.6 MB.
 *   - Every call on a GPU shares that GPU's one scratch array and leaves its
 *     contents behind; the kernels rewrite everything they read, so nothing
 *     needs clearing, but calls that overlap in time on one GPU (other
 *     streams, other threads) race and give wrong results: serialise them.
 *   - No soft-cap and no schedule reuse; results equal attn_varlen_bwd's bit
 *     for bit (same kernels, same schedule).
 * attn_varlen_static_scratch_bytes() returns the array's size.
 */
#define ATTN_STATIC_SCRATCH_BYTES (16u << 20)

size_t attn_varlen_static_scratch_bytes(void);

attn_status attn_varlen_bwd_static(const void* q, const void* k, const void* v,
                                   const void* out, const float* lse, const void* dout,
                                   const int32_t* cu_seqlens, int32_t num_seqs,
                                   int32_t total_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen,
                                   int32_t window, float scale, void* dq, void* dk, void* dv,
                                   attn_stream_t stream);

/* Static description of a status code (never NULL). */
const char* attn_varlen_strerror(attn_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t attn_varlen_version(void);

/*
 * Kernel timing, a measurement aid (off by default; no cost when off).
 * attn_varlen_profile_start() clears earlier records and makes every later
 * fwd/bwd call bracket each of its kernel launches with a pair of HIP
 * events recorded on the call's stream.  attn_varlen_profile_stop() turns
 * recording off, waits for the recorded events, and writes up to `cap`
 * per-kernel summaries (kernels in launch-pipeline order: "schedule",
 * "forward", "dq", "dkdv", "delta_fwd", "delta_bwd", "kda_fwd", "kda_bwd"; only kernels that ran).  It returns the number of
 * kernels that ran (which may exceed cap), or a negative attn_status.  The
 * events add a few microseconds per launch, so time whole calls with
 * recording off.  Not for use while another thread is issuing calls.
 */
typedef struct {
  char name[32];
  int32_t launches;
  double total_ms;   /* sum of event-to-event durations */
  double min_ms;
  double max_ms;
} attn_kernel_stats;

attn_status attn_varlen_profile_start(void);
int32_t attn_varlen_profile_stop(attn_kernel_stats* stats, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_VARLEN_H */
