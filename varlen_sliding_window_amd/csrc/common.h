// Shared definitions of the gfx950 attention kernels: fragment types, tile
// geometry, the schedule's tile record and the workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Rows of one tile: a q-tile (forward, dQ) or a k-tile (dK/dV) is at most
// TILE consecutive tokens of one segment, starting at the segment start.
constexpr int TILE = 32;
// Keys per inner step of the forward and dQ kernels (the unit of the
// schedule's cost sort; head dim 256 runs 32-key steps, which sort the same).
constexpr int KBLK = 64;
// Queries per inner step of the dK/dV kernel.
constexpr int QBLK = 32;
// Cost buckets of the longest-first sort.
constexpr int SORT_BINS = 1024;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// One tile of one segment: tokens [t0, t1) of segment [seg_a, seg_b).
// idx numbers the tiles in token order; the tiles of one segment have
// consecutive indices, so tile idx + i starts TILE * i tokens later.  Every
// record also carries the call it was built for: the total tokens, the
// window and a stamp (the tile capacity, or -1 when the boundaries were
// malformed), so that a kernel checks its schedule with the one load that
// brings its tile.  Entries past the last tile are written empty (t0 = t1).
struct __attribute__((aligned(16))) Tile {
  int t0, t1, seg_a, seg_b;
  int idx, total, window, stamp;
};

// Per-row values the backward passes from the dQ kernel to the dK/dV kernel,
// stored per (query head, q-tile): the starting values of the S and dP
// accumulators of each row, -lse / scale and -D with D = rowsum(dout * out).
// Seeded with them, the dK/dV kernel's products give P = exp2(scale log2(e)
// acc_S) and dP - D = acc_dP directly.  With a logit soft-cap, s0 holds
// -lse log2(e) instead (added after the cap).  256 bytes per tile.
struct TileStats {
  float s0[TILE];
  float dp0[TILE];
};

// Workspace: [header | forward-order tiles | backward-order tiles |
//             per-segment tile offsets | TileStats [Hq][tile_cap]]
struct WorkspaceLayout {
  size_t header, tiles_fwd, tiles_bwd, seg_offsets, rowstats, total;
  size_t tile_cap;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline size_t tile_capacity(int64_t total_tokens, int64_t num_seqs) {
  // sum over segments of ceil(L / TILE) <= T / TILE + num_seqs
  return (size_t)((total_tokens + TILE - 1) / TILE) + (size_t)num_seqs;
}

inline WorkspaceLayout workspace_layout(int64_t total_tokens, int64_t num_seqs,
                                        int64_t num_q_heads) {
  WorkspaceLayout w;
  w.tile_cap = tile_capacity(total_tokens, num_seqs);
  w.header = 0;
  w.tiles_fwd = 256;
  w.tiles_bwd = w.tiles_fwd + align256(w.tile_cap * sizeof(Tile));
  w.seg_offsets = w.tiles_bwd + align256(w.tile_cap * sizeof(Tile));
  w.rowstats = w.seg_offsets + align256((size_t)(num_seqs + 1) * sizeof(int));
  w.total = w.rowstats + align256((size_t)num_q_heads * w.tile_cap * sizeof(TileStats));
  return w;
}

// Workspace header: [0] number of tiles, [1] the total tokens, [2] tile
// capacity and [3] window the schedule was built for, [4] 1 if cu_seqlens
// was well formed (cu[0] = 0, non-decreasing, cu[num_seqs] = T), else 0.
// (The kernels check the same facts in their tile records.)  A call whose
// schedule does not match its own arguments (a reused schedule built for
// another call) or whose boundaries were malformed writes NaN to all of its
// outputs instead of computing them, so that misuse cannot pass unnoticed;
// the schedule's clamping keeps every kernel inside its buffers either way.
constexpr int HEADER_WORDS = 5;

// A work-group's tile record and the check of its schedule, in one load.
// item may lie past the list (an idle work-group): the record then read
// (clamped to the list's capacity) is not used.  ok is false when the
// schedule was built for another call or from malformed boundaries.
struct ScheduleView {
  Tile tile;
  bool ok, valid;   // valid: a tile to compute
};
__device__ __forceinline__ ScheduleView read_schedule(const Tile* __restrict__ tiles, int item,
                                                      int tile_cap, int T, int window) {
  ScheduleView v;
  v.tile = tiles[min(item, tile_cap - 1)];
  // all fields at once (else the compiler loads the check's fields first and
  // the tile's after the check, a second round trip)
  asm volatile("" ::"s"(v.tile.t0), "s"(v.tile.t1), "s"(v.tile.seg_a), "s"(v.tile.seg_b),
               "s"(v.tile.idx), "s"(v.tile.total), "s"(v.tile.window), "s"(v.tile.stamp));
  v.ok = (v.tile.total == T) & (v.tile.window == window) & (v.tile.stamp == tile_cap);
  v.valid = item < tile_cap && v.tile.t0 < v.tile.t1;
  return v;
}

// Query heads per work-group of the forward and dQ kernels: 4 heads of one
// key-value group, one per wave.  A group of G query heads takes
// ceil(G / 4) work-groups per q-tile; waves past the group's last head
// stage the shared key/value blocks but compute nothing.
constexpr int HEADS_PER_WG = 4;
__host__ __device__ __forceinline__ int head_chunks(int Hq, int Hkv) {
  return Hkv * ((Hq / Hkv + HEADS_PER_WG - 1) / HEADS_PER_WG);
}

// Work-groups in runs per XCD.  Work-groups are dealt to the 8 XCDs
// round-robin, and each XCD has its own L2, so a kernel maps its blocks so
// that runs of run_len consecutive list entries, all with one head index
// (nh of them per entry), land on one XCD: neighbouring tiles of a document
// read mostly the same rows, which that XCD's L2 then serves.  Rounds of 8
// runs go to the XCDs in alternating directions, so that no XCD always gets
// a round's most expensive run.  Returns the list entry; *h the head index.
// The grid is run_grid(nh, tile_cap, run_len) blocks; entries at or past the
// list length are idle.
__device__ __forceinline__ int xcd_run_item(int bid, int run_len, int nh, int* h) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int round = slot / run_len;
  const int rx = (round & 1) ? 7 - xcd : xcd;
  const int pos = (round * 8 + rx) * run_len + (slot - round * run_len);
  const int run = pos / (run_len * nh), within = pos - run * run_len * nh;
  *h = within / run_len;
  return run * run_len + (within - *h * run_len);
}
inline unsigned run_grid(int nh, size_t tile_cap, int run_len) {
  const size_t items = (size_t)nh * (tile_cap + run_len - 1);
  const size_t round = 8 * (size_t)run_len;
  return (unsigned)((items + round - 1) / round * round);
}

// Run lengths and sort chunks.  Local layers: most tiles cost the same, the
// sorted lists keep equal-cost neighbours in token order, and long runs give
// the most L2 reuse.  Global layers: costs change along each document, so a
// plain longest-first sort interleaves documents.  The backward list (whose
// work-groups each stream a long run of Q/dO rows) is instead sorted by the
// cost of each tile's chunk (GLOBAL_RUN consecutive tiles of one document,
// ranked by its most expensive tile), so that a run is mostly one chunk, at
// some cost in balance; the forward list keeps the plain order, which
// balanced better there.
constexpr int LOCAL_RUN = 32;
constexpr int GLOBAL_RUN = 16;
__host__ __device__ __forceinline__ int run_length(int window) {
  return window > 0 ? LOCAL_RUN : GLOBAL_RUN;
}

// Visible key range of query i in segment starting at a (inclusive bounds).
__device__ __forceinline__ int first_visible_key(int i, int a, int window) {
  return window > 0 ? max(a, i - window + 1) : a;
}

// Key range a q-tile [q0, ...) of segment [a, ...) loops over: from its
// first visible key or, in the band-block formulation (the performance
// reference page, section "Packed sliding-window attention on GPU:
// local_attention"), from the start of the W-token block before the block
// of q0 (blocks aligned to token 0), cut to the segment.  The per-row mask is
// the same either way, so the band only adds fully masked key blocks.
__device__ __forceinline__ int tile_key_lo(int q0, int a, int window, int band) {
  return band ? max(a, (q0 / window - 1) * window) : first_visible_key(q0, a, window);
}

// Query range end (exclusive) that a k-tile [.., k1) of segment [.., b) meets:
// the queries that see its last key or, in the band-block formulation, every
// query of the W-token block after the block of key k1 - 1.
__device__ __forceinline__ int tile_query_hi(int k1, int b, int window, int band) {
  if (window <= 0) return b;
  return band ? min(b, ((k1 - 1) / window + 2) * window) : min(b, k1 - 1 + window);
}

}  // namespace attn
