// Tile scheduler: turns cu_seqlens into the two work lists of one call.
//
// Segments are cut into tiles of TILE tokens starting at each segment start
// (the last tile of a segment may be short).  Because attention is confined
// to each document (research.dws.rip/llm/kernels, section 01 "How it was
// measured"), a tile only ever meets keys (forward, dQ) or
// queries (dK/dV) of its own segment, so fully masked tiles are never
// emitted.  The same tiles are sorted twice, longest first:
//   forward / dQ order : by the number of KBLK-key steps over the visible
//                        keys [max(a, t0 - W + 1), t1)
//   dK / dV order      : by the number of QBLK-query steps over the queries
//                        that see the tile, [t0, min(b, t1 - 1 + W))
// Without a window, the backward order sorts tiles by the cost of their
// chunk of GLOBAL_RUN neighbouring tiles instead (see run_length).  Work-groups are
// dispatched in list order, so the hardware's in-order dispatch gives a
// greedy longest-processing-time-first assignment.
//
// Everything runs on the device (one work-group), so nothing waits for the
// host and a call can be captured in a graph; the work lists live in the
// caller's workspace.  The kernel also checks the boundaries (cu[0] = 0,
// non-decreasing, cu[num_seqs] = T) and records the verdict in the
// workspace header: the attention kernels turn a malformed list into NaN
// outputs.  Segment bounds are clamped into [0, T] all the same, so that
// malformed cu_seqlens cannot send a kernel outside its buffers.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int SCHED_THREADS = 1024;
static_assert(SORT_BINS == SCHED_THREADS, "one sort bin per thread");

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// Inclusive block-wide scan (1024 threads = 16 waves): shuffles inside each
// wave, one wave scans the 16 wave totals.  *total receives the block sum.
__device__ int block_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  if (w == 0) {
    int x = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int t = __shfl_up(x, off);
      if (lane >= off) x += t;
    }
    if (lane < 16) wsum[lane] = x;
  }
  __syncthreads();
  const int r = v + (w > 0 ? wsum[w - 1] : 0);
  *total = wsum[15];
  __syncthreads();
  return r;
}

__device__ __forceinline__ Tile tile_at(int i, const int* __restrict__ seg_off,
                                        const int32_t* __restrict__ cu, int nseq, int T) {
  // largest s < nseq with seg_off[s] <= i (empty segments share an offset with the next)
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_off[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int a = clampi(cu[lo], 0, T);
  const int b = clampi(cu[lo + 1], a, T);
  // With valid boundaries t0 lies in [a, b).  Malformed ones (offsets that
  // overflowed) give an empty tile at b, which every kernel skips (and the
  // header marks the call's boundaries as malformed).
  long long t0 = (long long)a + ((long long)i - seg_off[lo]) * TILE;
  if (t0 < a || t0 > b) t0 = b;
  Tile t;
  t.t0 = (int)t0;
  t.t1 = (int)min(t0 + TILE, (long long)b);
  t.seg_a = a;
  t.seg_b = b;
  t.idx = i;
  t.total = t.window = t.stamp = 0;   // stamped when written
  return t;
}

__device__ __forceinline__ Tile stamped(Tile t, int T, int window, int stamp) {
  t.total = T;
  t.window = window;
  t.stamp = stamp;
  return t;
}

__device__ __forceinline__ int fwd_cost(int t0, int t1, int a, int window, int band) {
  const int klo = tile_key_lo(t0, a, window, band);
  return (t1 - klo + KBLK - 1) / KBLK;
}

__device__ __forceinline__ int bwd_cost(int t0, int t1, int b, int window, int band) {
  const int qhi = tile_query_hi(t1, b, window, band);
  return (qhi - t0 + QBLK - 1) / QBLK;
}

// Sort keys: the tile's own cost, except in the backward order without a
// window, where it is the cost of the tile's chunk of GLOBAL_RUN tiles (that
// of its first tile: costs fall along a document).
__device__ __forceinline__ int fwd_bin(const Tile& t, int window, int band) {
  return min(fwd_cost(t.t0, t.t1, t.seg_a, window, band), SORT_BINS - 1);
}

__device__ __forceinline__ int bwd_bin(const Tile& t, int window, int band) {
  int c = bwd_cost(t.t0, t.t1, t.seg_b, window, band);
  if (window <= 0) {
    const int span = TILE * GLOBAL_RUN;
    const int c0 = t.seg_a + ((t.t0 - t.seg_a) / span) * span;
    c = bwd_cost(c0, min(c0 + TILE, t.seg_b), t.seg_b, window, band);
  }
  return min(c, SORT_BINS - 1);
}

// Slot of this lane's tile in bucket `bin` (hist holds the next free slot of
// every bucket).  Called by whole waves; lanes with valid == false take none.
// Lanes sharing the bucket of the lowest unplaced lane get consecutive
// slots in lane order, for up to four buckets per wave.
__device__ int ordered_slot(int* hist, int bin, bool valid) {
  const int lane = threadIdx.x & 63;
  unsigned long long active = __ballot(valid);
  int slot = 0;
  for (int round = 0; round < 4 && active != 0ull; ++round) {
    const int leader = __ffsll((long long)active) - 1;
    const int b = __builtin_amdgcn_readlane(bin, leader);
    const unsigned long long m = __ballot(valid && bin == b) & active;
    int base = 0;
    if (lane == leader) base = atomicAdd(&hist[b], __popcll(m));
    base = __builtin_amdgcn_readlane(base, leader);
    if ((m >> lane) & 1ull) slot = base + __popcll(m & ((1ull << lane) - 1ull));
    active &= ~m;
  }
  if ((active >> lane) & 1ull) slot = atomicAdd(&hist[bin], 1);
  return slot;
}

// Segments whose boundaries and offsets fit here are scheduled from LDS;
// larger counts fall back to the workspace copy in global memory.
constexpr int SCHED_LDS_SEGS = 4096;

__global__ __launch_bounds__(SCHED_THREADS) void schedule_kernel(
    const int32_t* __restrict__ cu_g, int nseq, int T, int window, int band, int tile_cap,
    int need_bwd, int* __restrict__ header, Tile* __restrict__ fwd_list, Tile* __restrict__ bwd_list,
    int* __restrict__ seg_off_g) {
  __shared__ int buf[SCHED_THREADS / 64];
  __shared__ int hist_f[SORT_BINS];
  __shared__ int hist_b[SORT_BINS];
  __shared__ int lds_cu[SCHED_LDS_SEGS + 1];
  __shared__ int lds_off[SCHED_LDS_SEGS + 1];
  __shared__ int malformed;
  const int tid = threadIdx.x;
  if (tid == 0) malformed = (cu_g[0] != 0 || cu_g[nseq] != T) ? 1 : 0;
  const int32_t* cu = cu_g;
  int* seg_off = seg_off_g;
  if (nseq <= SCHED_LDS_SEGS) {
    for (int i = tid; i <= nseq; i += SCHED_THREADS) lds_cu[i] = cu_g[i];
    cu = lds_cu;
    seg_off = lds_off;
  }
  __syncthreads();

  // 1. tiles per segment -> exclusive offsets
  int carry = 0;
  for (int base = 0; base < nseq; base += SCHED_THREADS) {
    const int s = base + tid;
    int n = 0;
    if (s < nseq) {
      if (cu[s + 1] < cu[s]) malformed = 1;
      const int a = clampi(cu[s], 0, T);
      const int b = clampi(cu[s + 1], a, T);
      n = (b - a + TILE - 1) / TILE;
    }
    int total;
    const int incl = block_scan(n, buf, &total);
    if (s < nseq) seg_off[s] = carry + incl - n;
    carry += total;
  }
  // Valid boundaries give at most tile_cap tiles; malformed (overlapping) ones
  // are cut there so the lists never overflow the workspace.
  const int ntiles = min(carry, tile_cap);
  hist_f[tid] = 0;
  hist_b[tid] = 0;
  if (tid == 0) seg_off[nseq] = ntiles;
  __syncthreads();

  // 2. histogram of costs.  When every tile has a thread of its own (the
  // usual case: T / TILE + nseq <= 1024) it is built once and kept in
  // registers for the scatter.
  const bool one_pass = ntiles <= SCHED_THREADS;
  Tile mine;
  int my_bf = 0, my_bb = 0;
  const bool my_valid = one_pass && tid < ntiles;
  if (my_valid) {
    mine = tile_at(tid, seg_off, cu, nseq, T);
    my_bf = fwd_bin(mine, window, band);
    my_bb = bwd_bin(mine, window, band);
  }
  if (one_pass) {
    if (my_valid) {
      atomicAdd(&hist_f[my_bf], 1);
      if (need_bwd) atomicAdd(&hist_b[my_bb], 1);
    }
  } else {
    for (int i = tid; i < ntiles; i += SCHED_THREADS) {
      const Tile t = tile_at(i, seg_off, cu, nseq, T);
      atomicAdd(&hist_f[fwd_bin(t, window, band)], 1);
      if (need_bwd) atomicAdd(&hist_b[bwd_bin(t, window, band)], 1);
    }
  }
  __syncthreads();

  // 3. bucket start offsets, most expensive bucket first (both lists in one
  // scan, 16 bits each, while the counts fit)
  {
    const int c = SORT_BINS - 1 - tid;
    const int vf = hist_f[c];
    const int vb = hist_b[c];
    int total;
    if (ntiles < (1 << 15)) {
      const int inc = block_scan(vf | (vb << 16), buf, &total);
      hist_f[c] = (inc & 0xffff) - vf;
      hist_b[c] = (inc >> 16) - vb;
    } else {
      const int incf = block_scan(vf, buf, &total);
      const int incb = block_scan(vb, buf, &total);
      hist_f[c] = incf - vf;
      hist_b[c] = incb - vb;
    }
  }
  __syncthreads();

  // Every record carries this call's stamp; entries past the last tile are
  // written empty, so that no kernel takes a stale record for a tile.
  const int stamp = malformed ? -1 : tile_cap;
  {
    Tile e;
    e.t0 = e.t1 = e.seg_a = e.seg_b = e.idx = 0;
    e = stamped(e, T, window, stamp);
    for (int i = ntiles + tid; i < tile_cap; i += SCHED_THREADS) {
      fwd_list[i] = e;
      if (need_bwd) bwd_list[i] = e;
    }
  }

  // 4. scatter (results do not depend on the order inside a bucket).  In the
  // backward list each wave places its 64 consecutive tiles so that tiles of
  // one bucket from one wave keep their token order (a few ballot rounds,
  // then single atomics for what is left): runs of equal cost stay runs of
  // neighbouring tiles, which the dK/dV kernel maps onto one XCD, whose L2
  // then serves the rows that neighbouring tiles share.
  if (one_pass) {
    if (my_valid) fwd_list[atomicAdd(&hist_f[my_bf], 1)] = stamped(mine, T, window, stamp);
    if (need_bwd) {
      const int pb = ordered_slot(hist_b, my_bb, my_valid);
      if (my_valid) bwd_list[pb] = stamped(mine, T, window, stamp);
    }
  } else {
    for (int i0 = 0; i0 < ntiles; i0 += SCHED_THREADS) {
      const int i = i0 + tid;
      const bool valid = i < ntiles;
      Tile t;
      int bf = 0, bb = 0;
      if (valid) {
        t = tile_at(i, seg_off, cu, nseq, T);
        bf = fwd_bin(t, window, band);
        bb = bwd_bin(t, window, band);
      }
      if (valid) fwd_list[atomicAdd(&hist_f[bf], 1)] = stamped(t, T, window, stamp);
      if (need_bwd) {
        const int pb = ordered_slot(hist_b, bb, valid);
        if (valid) bwd_list[pb] = stamped(t, T, window, stamp);
      }
    }
  }
  if (tid == 0) {
    header[0] = ntiles;
    header[1] = T;
    header[2] = tile_cap;
    header[3] = window;
    header[4] = malformed ? 0 : 1;
  }
}

}  // namespace

hipError_t launch_schedule(const int32_t* cu_seqlens, const Problem& p, bool need_bwd,
                           void* workspace, const WorkspaceLayout& w, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(SCHED_THREADS), 0, stream, cu_seqlens,
                     p.num_seqs, p.total_tokens, p.window, p.band, (int)w.tile_cap,
                     need_bwd ? 1 : 0,
                     reinterpret_cast<int*>(ws + w.header),
                     reinterpret_cast<Tile*>(ws + w.tiles_fwd),
                     reinterpret_cast<Tile*>(ws + w.tiles_bwd),
                     reinterpret_cast<int*>(ws + w.seg_offsets));
  return hipGetLastError();
}

}  // namespace attn
