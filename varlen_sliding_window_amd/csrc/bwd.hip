// Backward kernels: dQ (which also produces D) and dK/dV.
//
// The gradients follow from out = softmax(scale q k^T) v per segment:
//   P = exp(S - lse), dP = dO V^T, D = rowsum(dO * O), dS = P (dP - D),
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO,
// with dK and dV summed over the query heads that share a key-value head
// (research.dws.rip/llm/kernels, Fig. 2 "Benchmark setup": 8 query heads
// over 2 key-value heads).  P is rebuilt from the forward's lse, so no
// score matrix is ever stored.
//
// dQ kernel: one work-group per (q-tile, group of 4 query heads), one head
//   per wave, exactly like the forward: S^T and dP^T are computed with the
//   query in the lane, so per-row lse and D are one register each, and
//   dQ^T = K^T dS^T takes dS^T straight from registers.  Each wave also
//   forms D = rowsum(dO * O) for its rows (fp32) and writes -lse/scale and
//   -D per row to the workspace for the dK/dV kernel, which runs next on the
//   same stream and seeds its S and dP accumulators with them.
// dK/dV kernels: one work-group per (k-tile of 32 keys, key-value head); its
//   waves take the group's query heads and stream each head's Q/dO rows
//   through LDS in QBLK = 32-row steps (direct global-to-LDS loads), keeping
//   dK/dV partial sums in fp32 registers; the partials are added in a fixed
//   order through LDS at the end, so the head-group reduction needs no
//   atomics and is bit-for-bit reproducible.  Three variants by head dim:
//   D = 64, dkdv_kernel: 4 waves (wave w: heads w, w + 4, ...), K and V in
//     registers, each wave's Q/dO double-buffered and loaded one step ahead,
//     software-pipelined (the softmax of one step runs between the S/dP
//     products of the next);
//   D = 128, dkdv_occ_kernel: 8 waves, two per SIMD (a wave per head and
//     q-block parity), K and V shared in LDS, one Q/dO buffer per wave;
//   D = 256, dkdv_split_kernel: pairs of waves split the head dim.
//
// Logit soft-cap (the CAP instantiations): with t = tanh(scale qk / c) the
// softmax sees c t, so P = exp2(c log2(e) t - lse log2(e)), and dS picks up
// the cap's derivative, dS = P (dP - D)(1 - t^2), before the products that
// carry it to dQ and dK.  The tanh cannot take the lse seed inside, so the
// dK/dV kernel then starts S at zero and keeps -lse log2(e) per row beside it.
#include "device.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BWD_THREADS = 256;

template <int D, bool CAP>
__global__ __launch_bounds__(BWD_THREADS, BlockGeom<D>::MIN_WG) void dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ out, const bf16* __restrict__ dout, const float* __restrict__ lse,
    const Tile* __restrict__ tiles, int T, int Hq, int Hkv,
    int window, int band, float scale_log2, float scale, float cap_a, float cap_c2, int tile_cap,
    bf16* __restrict__ dq, TileStats* __restrict__ stats) {
  using Geo = BlockGeom<D>;
  constexpr int KB = Geo::KB, H2 = Geo::H2, KS = Geo::KS, DB = Geo::DB;
  __shared__ __attribute__((aligned(16))) char smem[2 * Geo::BUF_BYTES];

  // work-group -> (tile, key-value head g, chunk of 4 of its G query heads),
  // in runs of neighbouring tiles per XCD, whose key/value blocks meet in
  // that XCD's L2 (xcd_run_item)
  const int G = Hq / Hkv;
  const int cpg = (G + HEADS_PER_WG - 1) / HEADS_PER_WG;
  const int chunks = Hkv * cpg;
  int hc;
  const int item = xcd_run_item(blockIdx.x, run_length(window), chunks, &hc);
  const ScheduleView sv = read_schedule(tiles, item, tile_cap, T, window);
  const Tile tl = sv.tile;
  if (!sv.ok) {
    poison_words(dq, (size_t)T * Hq * (D / 2), NAN_BF16X2);
    return;
  }
  if (!sv.valid) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lh = lane >> 5, lq = lane & 31;
  const int g = hc / cpg;
  const int hrel = (hc - g * cpg) * HEADS_PER_WG + wave;
  const bool active = hrel < G;   // else: stages K/V only
  const int head = g * G + min(hrel, G - 1);
  const int q0 = tl.t0, q1 = tl.t1, a = tl.seg_a;
  const int klo = tile_key_lo(q0, a, window, band);
  const int nblk = (q1 - klo + KB - 1) / KB;
  const int qrow = q0 + lq;
  const size_t qstride = (size_t)Hq * D;
  const uint32_t kstride_b = (uint32_t)(Hkv * D * sizeof(bf16));

  // Block loads, as in the forward: wave w fills rows ROWS_PER_WAVE * w + [0,
  // ROWS_PER_WAVE) of the swizzled K and V tiles; keys before 0 re-read key 0
  // (always masked).
  const bf16* kbase = k + (size_t)g * D;
  const bf16* vbase = v + (size_t)g * D;
  const uint32_t lds0 = lds_address(smem) + (uint32_t)(wave * Geo::ROWS_PER_WAVE * D * sizeof(bf16));
  uint32_t coff[Geo::LOADS];
  int lrow[Geo::LOADS];
#pragma unroll
  for (int j = 0; j < Geo::LOADS; ++j) {
    lrow[j] = Geo::ROWS_PER_WAVE * wave + TileLoad<D>::RPD * j + lane / TileLoad<D>::CPR;
    coff[j] = TileLoad<D>::chunk_offset(lane, lrow[j]);
  }
  auto issue = [&](int n, int buf) {
    const int kb = q1 - KB * (n + 1);
    const uint32_t l = lds0 + (uint32_t)(buf * Geo::BUF_BYTES);
#pragma unroll
    for (int j = 0; j < Geo::LOADS; ++j) {
      const int key = max(kb + lrow[j], 0);
      const uint32_t off = (uint32_t)key * kstride_b + coff[j];
      dma16(kbase, off, l + j * 1024);
      dma16(vbase, off, l + Geo::TILE_BYTES + j * 1024);
    }
  };
  // Q^T and dO^T as B operands; D from dO and O at the same positions.  Up
  // to D = 128 a wave's 32 rows of Q fit in its quarter of the second K/V
  // buffer: Q arrives there as whole-row direct loads (with the first
  // block's and the lanes' loads of O) and is read out as fragments, then dO
  // takes its place the same way.  The second round trip costs less than
  // lanes loading dO row by row.  At D = 256 lanes load all three.
  constexpr bool STAGE = RowTile<D>::BYTES * 4 <= Geo::BUF_BYTES;
  auto wave_tile = [&](int b) {
    return reinterpret_cast<bf16*>(smem + b * Geo::BUF_BYTES + wave * RowTile<D>::BYTES);
  };
  const size_t tile_off = (size_t)q0 * qstride + (size_t)head * D;
  const uint32_t row_bytes = (uint32_t)(qstride * sizeof(bf16));
  const int rows = min(TILE, T - q0);
  // The row's lse, in the first round trip (rows past T read row T - 1, as
  // the staged tiles do; their results are never stored)
  const int qrow_c = min(qrow, T - 1);
  const float lse_row = lse[(size_t)head * T + qrow_c];
  if constexpr (STAGE) dma_tile_rows<D>(q + tile_off, row_bytes, rows, lds_address(wave_tile(1)), lane);
  issue(0, 0);
  bf16x8 qf[KS], df[KS];
  float dpart = 0.f;
  const size_t off = (size_t)qrow * qstride + (size_t)head * D + lh * 8;
  if constexpr (STAGE) {
    // O with the row clamped like the staged Q and dO rows: unconditional
    // loads, all in flight together
    const size_t off_c = (size_t)qrow_c * qstride + (size_t)head * D + lh * 8;
    bf16x8 ov[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ov[ks] = as_bf16x8(ldg16(out + off_c + ks * 16));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = swz_frag_cols<D>(wave_tile(1), ks, lane);
    // the Q reads are done before dO overwrites the tile
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    dma_tile_rows<D>(dout + tile_off, row_bytes, rows, lds_address(wave_tile(1)), lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      df[ks] = swz_frag_cols<D>(wave_tile(1), ks, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart += (float)df[ks][e] * (float)ov[ks][e];
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (qrow < T) {
        qf[ks] = as_bf16x8(ldg16(q + off + ks * 16));
        df[ks] = as_bf16x8(ldg16(dout + off + ks * 16));
        const bf16x8 ov = as_bf16x8(ldg16(out + off + ks * 16));
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart += (float)df[ks][e] * (float)ov[e];
      } else {
        qf[ks] = zero_bf16x8();
        df[ks] = zero_bf16x8();
      }
    }
  }
  // Make the compiler wait for these loads here, not inside the loop where
  // the wait would also cover the block loads in flight.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]), "v"(df[ks]));
  const float Dv = dpart + __shfl_xor(dpart, 32);
  const float lsev = qrow < T ? lse_row : 0.f;
  const float lse2 = lsev * LOG2E;
  if (active && lh == 0) {
    // Rows past the tile get seeds that make them vanish (P = 0, dP - D = 0),
    // so every value the dK/dV kernel reads is finite.
    TileStats* ts = stats + (size_t)head * tile_cap + tl.idx;
    ts->s0[lq] = qrow < q1 ? (CAP ? -lse2 : -lsev / scale) : -INFINITY;
    ts->dp0[lq] = qrow < q1 ? -Dv : 0.f;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();
  const int full_lo = first_visible_key(q0 + TILE - 1, a, window);
  const int my_lo = first_visible_key(qrow, a, window);

  for (int n = 0; n < nblk; ++n) {
    const int kb = q1 - KB * (n + 1);
    const int buf = n & 1;
    // This wave's loads of block n have landed; after the barrier so have
    // everyone's, and every wave is done with block n - 1, whose buffer the
    // loads of block n + 1 now overwrite.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (n + 1 < nblk) issue(n + 1, buf ^ 1);
    if (!active) continue;
    const bf16* Ks = reinterpret_cast<const bf16*>(smem + buf * Geo::BUF_BYTES);
    const bf16* Vs = Ks + KB * D;

    // One 32-key half of the block at a time: its S/dP products, dS, then its
    // share of dQ (fewer live registers, so the operand reads can run
    // further ahead of the products).
    const bool full = (kb + KB - 1 <= q0) && (kb >= full_lo);
    // S^T and dP^T of half h2
    auto sdp = [&](int h2, f32x16& s, f32x16& dp) {
      constexpr int NP = 2 * KS, AHEAD = 4;
      bf16x8 ring[AHEAD + 1];
      auto load = [&](int m) {
        return swz_frag_cols<D>(((m & 1) ? Vs : Ks) + h2 * 32 * D, m >> 1, lane);
      };
#pragma unroll
      for (int m = 0; m < AHEAD; ++m) ring[m] = load(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        if (m + AHEAD < NP) ring[(m + AHEAD) % (AHEAD + 1)] = load(m + AHEAD);
        if (m & 1)
          dp = mfma32(ring[m % (AHEAD + 1)], df[m >> 1], dp);
        else
          s = mfma32(ring[m % (AHEAD + 1)], qf[m >> 1], s);
        __builtin_amdgcn_sched_barrier(0);
      }
      // With a cap, s becomes tanh(S / c).  On blocks that cross the
      // diagonal, the window edge or the segment start, invisible elements
      // get dP = D and a logit whose P is finite (-inf without a cap, t = 0
      // with one), so their dS below is exactly zero.
      if constexpr (CAP) tanh_fragments<1>(&s, cap_a, TANH_NARROW / cap_a);
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + h2 * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
          const bool vis = (key >= my_lo) & (key <= qrow);
          s[r] = vis ? s[r] : (CAP ? 0.f : -INFINITY);
          dp[r] = vis ? dp[r] : Dv;
        }
      }
    };
    // dS^T = P^T (dP^T - D), elements r and r + 1
    auto ds_pair = [&](int r, const f32x16& s, const f32x16& dp, bf16x8* dsf) {
      float v[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if constexpr (CAP) {
          // An invisible element has dP - D = 0 exactly; its P may overflow
          // (exp2(-lse log2 e) for a very negative lse), so it is zeroed by
          // a select rather than a product.
          const float t = s[r + e];
          const float p = exp2_fast(cap_c2 * t - lse2);
          const float dd = dp[r + e] - Dv;
          v[e] = dd == 0.f ? 0.f : p * dd * (1.f - t * t);
        } else {
          const float p = exp2_fast(s[r + e] * scale_log2 - lse2);
          v[e] = p * (dp[r + e] - Dv);
        }
      }
      dsf[r >> 3][r & 7] = (bf16)v[0];
      dsf[r >> 3][(r & 7) + 1] = (bf16)v[1];
    };
    // dQ^T[d][q] += sum_key K^T[d][key] dS^T[key][q] over half h2's keys
    auto dqp = [&](int h2, const bf16x8* dsf) {
      constexpr int NP = 2 * DB, AHEAD = 3;
      bf16x8 ring[AHEAD + 1];
      auto load = [&](int m) { return swz_frag_rows<D>(Ks, (m % DB) * 32, 2 * h2 + m / DB, lane); };
#pragma unroll
      for (int m = 0; m < AHEAD; ++m) ring[m] = load(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        if (m + AHEAD < NP) ring[(m + AHEAD) % (AHEAD + 1)] = load(m + AHEAD);
        acc[m % DB] = mfma32(ring[m % (AHEAD + 1)], dsf[m / DB], acc[m % DB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
#pragma unroll
    for (int h2 = 0; h2 < H2; ++h2) {
      f32x16 s = zero_f32x16(), dp = zero_f32x16();
      sdp(h2, s, dp);
      bf16x8 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) ds_pair(r, s, dp, dsf);
      dqp(h2, dsf);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (!active) return;

  if constexpr (STAGE) {
    // Through the K/V buffer the last block did not use (idle since the
    // last barrier): whole-row stores.
    bf16* ot = wave_tile(nblk & 1);
    stage_acc_rows<D>(ot, acc, scale, lane);
    store_tile_rows<D>(dq + (size_t)q0 * qstride + (size_t)head * D, qstride, q1 - q0, ot, lane);
  } else if (qrow < q1) {
    bf16* op = dq + (size_t)qrow * qstride + (size_t)head * D + lh * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_bf16x4(op + db * 32 + j * 8, acc[db][4 * j] * scale, acc[db][4 * j + 1] * scale,
                     acc[db][4 * j + 2] * scale, acc[db][4 * j + 3] * scale);
  }
}

constexpr int DKDV_WAVES = 4;
static_assert(QBLK == TILE, "a dK/dV q-block is exactly one q-tile");

// Per-head-dim geometry of the dK/dV kernel.  Per wave and buffer: Q tile,
// dO tile (32 x D bf16 each, swizzled), then the q-tile's TileStats.
template <int D>
struct DkdvGeom {
  static constexpr int KS = D / 16;                     // k-steps of a D-long product
  static constexpr int DB = D / 32;                     // 32-column blocks of D
  static constexpr int RED_PITCH = D + 4;               // fp32 pitch of the reduction buffer
  static constexpr int TILE_BYTES = QBLK * D * (int)sizeof(bf16);
  static constexpr int BUF_BYTES = 2 * TILE_BYTES + (int)sizeof(TileStats);
  static constexpr size_t LDS_BYTES = (size_t)DKDV_WAVES * 2 * BUF_BYTES;
  static constexpr int LOADS = QBLK / TileLoad<D>::RPD;   // 1 KB loads per tile
  static_assert(LDS_BYTES <= 160 * 1024, "staging buffers must fit in LDS");
  static_assert((size_t)DKDV_WAVES * TILE * RED_PITCH * sizeof(float) <= LDS_BYTES,
                "reduction buffer must fit in the staging buffers");
};

// Used at D = 64 (at D = 128 its software pipeline needs 447 registers per
// wave, one wave per SIMD; dkdv_occ_kernel below runs two).  At D = 64 the
// uncapped kernel fits 256 registers, so two work-groups share a CU and each
// hides the other's start-up and load latency.
template <int D, bool CAP>
__global__ __launch_bounds__(BWD_THREADS, (D == 64 && !CAP) ? 2 : 1) void dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const TileStats* __restrict__ stats, int tile_cap,
    const Tile* __restrict__ tiles, int T, int Hq, int Hkv,
    int window, int band, float scale_log2, float scale, float cap_a, float cap_c2, int run_len,
    bf16* __restrict__ dk, bf16* __restrict__ dv) {
  using Geo = DkdvGeom<D>;
  constexpr int KS = Geo::KS, DB = Geo::DB, RED_PITCH = Geo::RED_PITCH;
  constexpr int DKDV_TILE_BYTES = Geo::TILE_BYTES, DKDV_BUF_BYTES = Geo::BUF_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[Geo::LDS_BYTES];

  // work-group -> (key tile, key-value head), in runs of neighbouring key
  // tiles per XCD, whose Q/dO rows meet in that XCD's L2 (xcd_run_item)
  int g;
  const int item = xcd_run_item(blockIdx.x, run_len, Hkv, &g);
  const ScheduleView sv = read_schedule(tiles, item, tile_cap, T, window);
  const Tile tl = sv.tile;
  if (!sv.ok) {
    poison_words(dk, (size_t)T * Hkv * (D / 2), NAN_BF16X2);
    poison_words(dv, (size_t)T * Hkv * (D / 2), NAN_BF16X2);
    return;
  }
  if (!sv.valid) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lh = lane >> 5, lq = lane & 31;
  const int G = Hq / Hkv;
  const int k0 = tl.t0, k1 = tl.t1, b = tl.seg_b;
  const int qhi = tile_query_hi(k1, b, window, band);
  const int nqb = (qhi - k0 + QBLK - 1) / QBLK;
  // (head, q-block) pairs of this wave: heads wave, wave + 4, ... of the group
  const int nheads = wave < G ? (G - wave + DKDV_WAVES - 1) / DKDV_WAVES : 0;
  const int steps = nheads * nqb;
  const size_t qstride = (size_t)Hq * D;
  const size_t kstride = (size_t)Hkv * D;

  char* wbase = smem + (size_t)wave * 2 * DKDV_BUF_BYTES;
  auto q_tile = [&](int buf) {
    return reinterpret_cast<const bf16*>(wbase + buf * DKDV_BUF_BYTES);
  };
  auto do_tile = [&](int buf) {
    return reinterpret_cast<const bf16*>(wbase + buf * DKDV_BUF_BYTES + DKDV_TILE_BYTES);
  };
  auto st_tile = [&](int buf) {
    return reinterpret_cast<const float*>(wbase + buf * DKDV_BUF_BYTES + 2 * DKDV_TILE_BYTES);
  };
  const uint32_t lds_wave = lds_address(wbase);

  // Lane part of the tile loads: load j (1 KB) fills rows RPD j + lane / CPR
  // of the swizzled tile; the lane fetches the 16-byte chunk that lands at
  // physical chunk lane % CPR of its row.
  const uint32_t rstride = (uint32_t)(qstride * sizeof(bf16));
  uint32_t dma_off[Geo::LOADS];
#pragma unroll
  for (int j = 0; j < Geo::LOADS; ++j) {
    const int r = TileLoad<D>::RPD * j + lane / TileLoad<D>::CPR;
    dma_off[j] = (uint32_t)r * rstride + TileLoad<D>::chunk_offset(lane, r);
  }

  // Loads of one step into buffer `buf`: Q and dO rows of q-block i (the
  // q-tile idx + i of this segment) of query head `head`, then that tile's
  // TileStats (lanes 0-15, 16 bytes each).  Rows past T re-read row T - 1;
  // rows past the segment hold other values.  Both are masked with selects,
  // so even NaNs there cannot leak.
  auto issue = [&](int head, int i, int buf) {
    const int qb = k0 + i * QBLK;
    const size_t hoff = (size_t)qb * qstride + (size_t)head * D;
    const bf16* qsrc = q + hoff;
    const bf16* dsrc = dout + hoff;
    const uint32_t l = lds_wave + (uint32_t)(buf * DKDV_BUF_BYTES);
    const int rmax = T - 1 - qb;
    if (rmax >= QBLK - 1) {
#pragma unroll
      for (int j = 0; j < Geo::LOADS; ++j) {
        dma16(qsrc, dma_off[j], l + j * 1024);
        dma16(dsrc, dma_off[j], l + DKDV_TILE_BYTES + j * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < Geo::LOADS; ++j) {
        const int r = TileLoad<D>::RPD * j + lane / TileLoad<D>::CPR;
        const uint32_t off = (uint32_t)min(r, rmax) * rstride + TileLoad<D>::chunk_offset(lane, r);
        dma16(qsrc, off, l + j * 1024);
        dma16(dsrc, off, l + DKDV_TILE_BYTES + j * 1024);
      }
    }
    if (lane < 16)
      dma16(stats + (size_t)head * tile_cap + tl.idx + i, (uint32_t)lane * 16,
            l + 2 * DKDV_TILE_BYTES);
  };
  // Steps run over (head, q-block) pairs: heads wave, wave + 4, ..., and for
  // each head q-blocks 0 .. nqb - 1.  (ld_head, ld_i) is the next step to load.
  int ld_head = g * G + wave, ld_i = 0;
  auto issue_next = [&](int buf) {
    issue(ld_head, ld_i, buf);
    if (++ld_i == nqb) {
      ld_i = 0;
      ld_head += DKDV_WAVES;
    }
  };
  if (steps > 0) issue_next(0);

  // K^T and V^T as B operands: lane holds k[k0 + lq][16 ks + 8 lh + 0..7]
  const int krow = k0 + lq;
  bf16x8 kf[KS], vf[KS];
  {
    const size_t off = (size_t)min(krow, T - 1) * kstride + (size_t)g * D + lh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = as_bf16x8(ldg16(k + off + ks * 16));
      vf[ks] = as_bf16x8(ldg16(v + off + ks * 16));
    }
    // Make the compiler wait for these loads here: a wait inside the loop
    // would also wait for the step's own prefetch.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(kf[ks]), "v"(vf[ks]));
  }

  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = zero_f32x16();
    dva[db] = zero_f32x16();
  }

  // Visibility of element r of a step at q-block qb: its query
  // qi = qb + 4 lh + 8(r/4) + r%4 sees this lane's key iff
  // 0 <= qi - krow <= vis_hi - krow.  Keys past the tile see nothing: their
  // offset is pushed far below zero.
  const bool kvalid = krow < k1;
  const int vis_hi = window > 0 ? min(b - 1, krow + window - 1) : b - 1;
  const int mbias = (kvalid ? 0 : -(1 << 30)) + 4 * lh - krow;
  const uint32_t mspan = kvalid ? (uint32_t)(vis_hi - krow) : 0u;

  // S = Q K^T and dP = dO V^T of the step held in buffer `buf` (two
  // independent chains), seeded with -lse/scale and -D: s[r] = S - lse/scale
  // and dp[r] = dP - D of query qb + 8(r/4) + 4 lh + r%4 and key k0 + lq.
  // With a cap, S starts at zero and ls[r] = -lse log2(e) of the same query.
  // Also reads the step's transposed dO and Q fragments (B operands of dV
  // and dK), so that the buffer is done with once this returns.
  auto s_dp = [&](int buf, f32x16& s, f32x16& dp, bf16x8* dof, bf16x8* qtf, f32x16& ls) {
    const float* st = st_tile(buf);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a4 = *reinterpret_cast<const float4*>(st + 8 * j + 4 * lh);
      const float4 b4 = *reinterpret_cast<const float4*>(st + TILE + 8 * j + 4 * lh);
      if constexpr (CAP) {
        ls[4 * j + 0] = a4.x; ls[4 * j + 1] = a4.y; ls[4 * j + 2] = a4.z; ls[4 * j + 3] = a4.w;
      } else {
        s[4 * j + 0] = a4.x; s[4 * j + 1] = a4.y; s[4 * j + 2] = a4.z; s[4 * j + 3] = a4.w;
      }
      dp[4 * j + 0] = b4.x; dp[4 * j + 1] = b4.y; dp[4 * j + 2] = b4.z; dp[4 * j + 3] = b4.w;
    }
    if constexpr (CAP) s = zero_f32x16();
    const bf16* Qs = q_tile(buf);
    const bf16* Ds = do_tile(buf);
    bf16x8 qa[KS], da[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[ks] = swz_frag_cols<D>(Qs, ks, lane);
      da[ks] = swz_frag_cols<D>(Ds, ks, lane);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32(qa[ks], kf[ks], s);
      dp = mfma32(da[ks], vf[ks], dp);
    }
#pragma unroll
    for (int x = 0; x < 2 * DB; ++x) {
      dof[x] = swz_frag_rows<D>(Ds, (x % DB) * 32, x / DB, lane);
      qtf[x] = swz_frag_rows<D>(Qs, (x % DB) * 32, x / DB, lane);
    }
  };
  // Half t of P and dS (queries 16t .. 16t + 15 of the step at qb) as bf16
  // A fragments (rows = keys, k = queries); invisible elements become 0.
  // With a cap, s already holds tanh(scale qk / c).
  auto p_ds = [&](const f32x16& s, const f32x16& dp, const f32x16& ls, int qb, int t,
                  bf16x8& pf, bf16x8& dsf) {
    const int x = qb + mbias;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 8 * t + e;
      if constexpr (CAP) {
        const float th = s[r];   // tanh(scale qk / c), see body
        float p = exp2_fast(cap_c2 * th + ls[r]);
        p = (uint32_t)(x + 8 * (r >> 2) + (r & 3)) <= mspan ? p : 0.f;
        pf[e] = (bf16)p;
        dsf[e] = (bf16)(p * dp[r] * (1.f - th * th));
      } else {
        float p = exp2_fast(s[r] * scale_log2);
        p = (uint32_t)(x + 8 * (r >> 2) + (r & 3)) <= mspan ? p : 0.f;
        pf[e] = (bf16)p;
        dsf[e] = (bf16)(p * dp[r]);
      }
    }
  };
  // Half t of dV[key][d] += P^T dO and dK[key][d] += dS^T Q (scale applied
  // at the end).
  auto dv_dk = [&](int t, const bf16x8& pf, const bf16x8& dsf, const bf16x8* dof,
                   const bf16x8* qtf) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dva[db] = mfma32(pf, dof[t * DB + db], dva[db]);
      dka[db] = mfma32(dsf, qtf[t * DB + db], dka[db]);
    }
  };

  // Software pipeline over the steps.  Iteration `it` finishes step it (its
  // S/dP products were computed one iteration earlier) while computing the
  // S/dP products of step it + 1: the softmax of step it runs between the
  // matrix products of step it + 1, then the dV/dK products of step it run.
  // Buffer it % 2 holds step it; every read of it happens in iteration
  // it - 1, so at the top of iteration it the loads of step it + 2 can go
  // there, with a whole iteration to land.  On the last iteration the S/dP
  // products of the step after are computed from stale data and discarded.
  auto body = [&](int it, int qb, f32x16& s_c, f32x16& dp_c, bf16x8* dof_c, bf16x8* qtf_c,
                  f32x16& ls_c, f32x16& s_n, f32x16& dp_n, bf16x8* dof_n, bf16x8* qtf_n,
                  f32x16& ls_n) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    if (it + 2 < steps) issue_next(it & 1);
    s_dp((it + 1) & 1, s_n, dp_n, dof_n, qtf_n, ls_n);
    if constexpr (CAP) tanh_fragments<1>(&s_c, cap_a, TANH_NARROW / cap_a);
    bf16x8 pf0, ds0, pf1, ds1;
    p_ds(s_c, dp_c, ls_c, qb, 0, pf0, ds0);
    p_ds(s_c, dp_c, ls_c, qb, 1, pf1, ds1);
    // The S/dP products (2 KS of them) interleaved with the step's LDS reads
    // (8 row-stat reads, 2 KS row reads, 8 DB transposing reads: 3 per
    // product after the first 8) and the softmax arithmetic (about 112 VALU).
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);    // 8 LDS reads
#pragma unroll
    for (int x = 0; x < 2 * KS; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // 3 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 112 / (2 * KS), 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    dv_dk(0, pf0, ds0, dof_c, qtf_c);
    dv_dk(1, pf1, ds1, dof_c, qtf_c);
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16 sA, dpA, sB, dpB, lsA, lsB;   // lsA, lsB: only with a cap
  bf16x8 dofA[2 * DB], qtfA[2 * DB], dofB[2 * DB], qtfB[2 * DB];
  if (steps > 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (steps > 1) issue_next(1);
    s_dp(0, sA, dpA, dofA, qtfA, lsA);
  }
  int qb = k0;
  auto next_qb = [&](int x) { return x + QBLK < k0 + nqb * QBLK ? x + QBLK : k0; };
  int it = 0;
  for (; it + 1 < steps; it += 2) {
    body(it, qb, sA, dpA, dofA, qtfA, lsA, sB, dpB, dofB, qtfB, lsB);
    qb = next_qb(qb);
    body(it + 1, qb, sB, dpB, dofB, qtfB, lsB, sA, dpA, dofA, qtfA, lsA);
    qb = next_qb(qb);
  }
  if (it < steps) body(it, qb, sA, dpA, dofA, qtfA, lsA, sB, dpB, dofB, qtfB, lsB);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

  // Head-group reduction in a fixed order (wave 0 + 1 + 2 + 3), then store.
  float* red = reinterpret_cast<float*>(smem);
  constexpr int OCOLS = D / 8;   // output columns per thread (32 keys x 8 threads)
  const int okey = tid >> 3, od = (tid & 7) * OCOLS;
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    float* mine = red + (size_t)wave * TILE * RED_PITCH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
        mine[key * RED_PITCH + db * 32 + lq] = pass == 0 ? dka[db][r] : dva[db][r];
      }
    __syncthreads();
    if (k0 + okey < k1) {
      const float mul = pass == 0 ? scale : 1.f;
      bf16* dst = (pass == 0 ? dk : dv) + (size_t)(k0 + okey) * kstride + (size_t)g * D + od;
#pragma unroll
      for (int e = 0; e < OCOLS; e += 4) {
        float acc4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < DKDV_WAVES; ++w)
            sum += red[(size_t)w * TILE * RED_PITCH + okey * RED_PITCH + od + e + x];
          acc4[x] = sum * mul;
        }
        store_bf16x4(dst + e, acc4[0], acc4[1], acc4[2], acc4[3]);
      }
    }
  }
}

// dK/dV at head dim 256.  At D = 256 one wave's share of the kernel above
// would not fit (the dK/dV accumulators of 32 keys alone fill a SIMD's
// registers, and double-buffered 256-wide Q/dO rows fill the LDS twice
// over), so each (key tile, query head) goes to a pair of waves that split
// the head dim: wave w takes columns 128 (w & 1) + [0, 128) of Q, dO, K, V,
// dK and dV, and query heads w / 2, w / 2 + 2, ... of the group.  Each wave
// forms its half of the S and dP contractions; the pair adds the two halves
// through LDS, after which both hold the step's whole S and dP and go on
// exactly as above on their own 128 columns.  One step at a time (no
// software pipeline), with the next step's Q/dO loads in flight; two
// barriers per step order the exchange.
template <bool CAP>
__global__ __launch_bounds__(BWD_THREADS, 1) void dkdv_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const TileStats* __restrict__ stats, int tile_cap,
    const Tile* __restrict__ tiles, int T, int Hq, int Hkv,
    int window, int band, float scale_log2, float scale, float cap_a, float cap_c2, int run_len,
    bf16* __restrict__ dk, bf16* __restrict__ dv) {
  constexpr int D = 256, DH = 128;      // head dim, columns per wave
  using Geo = DkdvGeom<DH>;             // staging of 128-wide half rows
  constexpr int KS = Geo::KS, DB = Geo::DB, RED_PITCH = Geo::RED_PITCH;
  constexpr int TILE_BYTES = Geo::TILE_BYTES, BUF_BYTES = Geo::BUF_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[Geo::LDS_BYTES];

  // work-group -> (key tile, key-value head): as in dkdv_kernel
  int g;
  const int item = xcd_run_item(blockIdx.x, run_len, Hkv, &g);
  const ScheduleView sv = read_schedule(tiles, item, tile_cap, T, window);
  const Tile tl = sv.tile;
  if (!sv.ok) {
    poison_words(dk, (size_t)T * Hkv * (D / 2), NAN_BF16X2);
    poison_words(dv, (size_t)T * Hkv * (D / 2), NAN_BF16X2);
    return;
  }
  if (!sv.valid) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lh = lane >> 5, lq = lane & 31;
  const int half = wave & 1, pair = wave >> 1;
  const int G = Hq / Hkv;
  const int k0 = tl.t0, k1 = tl.t1, b = tl.seg_b;
  const int qhi = tile_query_hi(k1, b, window, band);
  const int nqb = (qhi - k0 + QBLK - 1) / QBLK;
  // (head, q-block) pairs: pair p takes heads p, p + 2, ... of the group.
  // Both pairs run the same number of steps (the loop's barriers are shared);
  // when G is odd, pair 1's last head's steps are dummies that re-read a
  // valid head and add nothing.
  const int steps = ((G + 1) / 2) * nqb;
  const int live_steps = pair < G ? ((G - pair + 1) / 2) * nqb : 0;
  const size_t qstride = (size_t)Hq * D;
  const size_t kstride = (size_t)Hkv * D;

  char* wbase = smem + (size_t)wave * 2 * BUF_BYTES;
  const uint32_t lds_wave = lds_address(wbase);
  const uint32_t rstride = (uint32_t)(qstride * sizeof(bf16));
  uint32_t dma_off[Geo::LOADS];
#pragma unroll
  for (int j = 0; j < Geo::LOADS; ++j) {
    const int r = TileLoad<DH>::RPD * j + lane / TileLoad<DH>::CPR;
    dma_off[j] = (uint32_t)r * rstride + TileLoad<DH>::chunk_offset(lane, r);
  }
  // Loads of one step into buffer `buf`: this wave's 128 columns of the Q
  // and dO rows of q-block i of query head `head`, then the q-tile's
  // TileStats.  Rows past T re-read row T - 1 (masked later).
  auto issue = [&](int head, int i, int buf) {
    const int qb = k0 + i * QBLK;
    const size_t hoff = (size_t)qb * qstride + (size_t)head * D + (size_t)half * DH;
    const bf16* qsrc = q + hoff;
    const bf16* dsrc = dout + hoff;
    const uint32_t l = lds_wave + (uint32_t)(buf * BUF_BYTES);
    const int rmax = T - 1 - qb;
#pragma unroll
    for (int j = 0; j < Geo::LOADS; ++j) {
      const int r = TileLoad<DH>::RPD * j + lane / TileLoad<DH>::CPR;
      const uint32_t off = rmax >= QBLK - 1
                               ? dma_off[j]
                               : (uint32_t)min(r, rmax) * rstride + TileLoad<DH>::chunk_offset(lane, r);
      dma16(qsrc, off, l + j * 1024);
      dma16(dsrc, off, l + TILE_BYTES + j * 1024);
    }
    if (lane < 16)
      dma16(stats + (size_t)head * tile_cap + tl.idx + i, (uint32_t)lane * 16, l + 2 * TILE_BYTES);
  };
  int ld_head = g * G + pair, ld_i = 0;
  auto issue_next = [&](int buf) {
    issue(min(ld_head, g * G + G - 1), ld_i, buf);
    if (++ld_i == nqb) {
      ld_i = 0;
      ld_head += 2;
    }
  };
  if (steps > 0) issue_next(0);

  // this wave's 128 columns of K^T and V^T as B operands
  const int krow = k0 + lq;
  bf16x8 kf[KS], vf[KS];
  {
    const size_t off = (size_t)min(krow, T - 1) * kstride + (size_t)g * D + (size_t)half * DH + lh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = as_bf16x8(ldg16(k + off + ks * 16));
      vf[ks] = as_bf16x8(ldg16(v + off + ks * 16));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(kf[ks]), "v"(vf[ks]));
  }

  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = zero_f32x16();
    dva[db] = zero_f32x16();
  }
  const bool kvalid = krow < k1;
  const int vis_hi = window > 0 ? min(b - 1, krow + window - 1) : b - 1;
  const int mbias = (kvalid ? 0 : -(1 << 30)) + 4 * lh - krow;
  const uint32_t mspan = kvalid ? (uint32_t)(vis_hi - krow) : 0u;

  int qb = k0;
  for (int it = 0; it < steps; ++it) {
    const int buf = it & 1;
    // This wave's loads of step it have landed; after the barrier the partner
    // is done reading this wave's other buffer (last step's exchange), which
    // the loads of step it + 1 now overwrite.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < steps) issue_next(buf ^ 1);
    char* bb = wbase + buf * BUF_BYTES;
    const bf16* Qs = reinterpret_cast<const bf16*>(bb);
    const bf16* Ds = reinterpret_cast<const bf16*>(bb + TILE_BYTES);
    const float* st = reinterpret_cast<const float*>(bb + 2 * TILE_BYTES);

    // Half contractions, seeded (-lse/scale, -D) in the half-0 wave only.
    f32x16 s, dp, ls;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a4 = *reinterpret_cast<const float4*>(st + 8 * j + 4 * lh);
      const float4 b4 = *reinterpret_cast<const float4*>(st + TILE + 8 * j + 4 * lh);
      const float sa[4] = {a4.x, a4.y, a4.z, a4.w}, sb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (CAP) {
          ls[4 * j + e] = sa[e];
          s[4 * j + e] = 0.f;
        } else {
          s[4 * j + e] = half == 0 ? sa[e] : 0.f;
        }
        dp[4 * j + e] = half == 0 ? sb[e] : 0.f;
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32(swz_frag_cols<DH>(Qs, ks, lane), kf[ks], s);
      dp = mfma32(swz_frag_cols<DH>(Ds, ks, lane), vf[ks], dp);
    }
    bf16x8 dof[2 * DB], qtf[2 * DB];
#pragma unroll
    for (int x = 0; x < 2 * DB; ++x) {
      dof[x] = swz_frag_rows<DH>(Ds, (x % DB) * 32, x / DB, lane);
      qtf[x] = swz_frag_rows<DH>(Qs, (x % DB) * 32, x / DB, lane);
    }
    // Exchange: every read of this buffer has returned, so its Q region
    // takes this wave's halves (lane-contiguous float4s); after the barrier
    // each wave adds its partner's.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    float4* xs = reinterpret_cast<float4*>(bb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[j * 64 + lane] = make_float4(s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]);
      xs[(4 + j) * 64 + lane] = make_float4(dp[4 * j], dp[4 * j + 1], dp[4 * j + 2], dp[4 * j + 3]);
    }
    __syncthreads();
    const float4* px = reinterpret_cast<const float4*>(smem + (size_t)(wave ^ 1) * 2 * BUF_BYTES +
                                                       buf * BUF_BYTES);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 ps = px[j * 64 + lane];
      const float4 pd = px[(4 + j) * 64 + lane];
      s[4 * j] += ps.x; s[4 * j + 1] += ps.y; s[4 * j + 2] += ps.z; s[4 * j + 3] += ps.w;
      dp[4 * j] += pd.x; dp[4 * j + 1] += pd.y; dp[4 * j + 2] += pd.z; dp[4 * j + 3] += pd.w;
    }

    // P and dS (rows = this lane's key, k = the step's queries), then this
    // wave's 128 columns of dV += P^T dO and dK += dS^T Q.  A dummy step
    // (it >= live_steps) sees nothing.
    if constexpr (CAP) tanh_fragments<1>(&s, cap_a, TANH_NARROW / cap_a);
    const int x0 = it < live_steps ? qb + mbias : -(1 << 30);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 pf, dsf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * t + e;
        const bool vis = (uint32_t)(x0 + 8 * (r >> 2) + (r & 3)) <= mspan;
        if constexpr (CAP) {
          const float th = s[r];
          float p = exp2_fast(cap_c2 * th + ls[r]);
          p = vis ? p : 0.f;
          pf[e] = (bf16)p;
          dsf[e] = (bf16)(p * dp[r] * (1.f - th * th));
        } else {
          float p = exp2_fast(s[r] * scale_log2);
          p = vis ? p : 0.f;
          pf[e] = (bf16)p;
          dsf[e] = (bf16)(p * dp[r]);
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dva[db] = mfma32(pf, dof[t * DB + db], dva[db]);
        dka[db] = mfma32(dsf, qtf[t * DB + db], dka[db]);
      }
    }
    qb = qb + QBLK < k0 + nqb * QBLK ? qb + QBLK : k0;
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

  // Reduction over the two head sets in a fixed order (column half h is
  // wave h + wave h + 2), then store.
  float* red = reinterpret_cast<float*>(smem);
  constexpr int OCOLS = D / 8;   // output columns per thread (32 keys x 8 threads)
  const int okey = tid >> 3, od = (tid & 7) * OCOLS;
  const int oh = od / DH, oc = od - oh * DH;
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    float* mine = red + (size_t)wave * TILE * RED_PITCH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
        mine[key * RED_PITCH + db * 32 + lq] = pass == 0 ? dka[db][r] : dva[db][r];
      }
    __syncthreads();
    if (k0 + okey < k1) {
      const float mul = pass == 0 ? scale : 1.f;
      bf16* dst = (pass == 0 ? dk : dv) + (size_t)(k0 + okey) * kstride + (size_t)g * D + od;
      const float* r0 = red + (size_t)oh * TILE * RED_PITCH + okey * RED_PITCH + oc;
      const float* r1 = red + (size_t)(oh + 2) * TILE * RED_PITCH + okey * RED_PITCH + oc;
#pragma unroll
      for (int e = 0; e < OCOLS; e += 4)
        store_bf16x4(dst + e, (r0[e] + r1[e]) * mul, (r0[e + 1] + r1[e + 1]) * mul,
                     (r0[e + 2] + r1[e + 2]) * mul, (r0[e + 3] + r1[e + 3]) * mul);
    }
  }
}

// dK/dV at head dim 128 with two waves per SIMD: 8 waves per work-group,
// wave w taking query head w % 4 (+ 4 j) and the q-blocks of parity w / 4.
// The kernel above would need 447 registers per wave at this head dim for
// its software pipeline; this one fits 256 by giving that up: the key tile's K
// and V rows are staged once per work-group in LDS and shared by the 8
// waves, and each wave's Q/dO block has a single LDS buffer, so while one
// wave waits for its next block the other wave on its SIMD computes.  Inside
// a step the LDS operand reads run ahead of the products in small register
// rings (two k-steps for S/dP, four products for dV/dK), fenced so that the
// compiler keeps that distance.  The 8 partial sums are added in a fixed
// order at the end.
constexpr int OCC_WAVES = 8;
constexpr int OCC_THREADS = 64 * OCC_WAVES;

template <bool CAP>
__global__ __launch_bounds__(OCC_THREADS, 1) void dkdv_occ_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const TileStats* __restrict__ stats, int tile_cap,
    const Tile* __restrict__ tiles, int T, int Hq, int Hkv,
    int window, int band, float scale_log2, float scale, float cap_a, float cap_c2, int run_len,
    bf16* __restrict__ dk, bf16* __restrict__ dv) {
  constexpr int D = 128;
  using Geo = DkdvGeom<D>;
  constexpr int KS = Geo::KS, DB = Geo::DB, RED_PITCH = Geo::RED_PITCH;
  constexpr int TILE_BYTES = Geo::TILE_BYTES, BUF_BYTES = Geo::BUF_BYTES;
  constexpr int VT_BYTES = 2 * TILE * D * (int)sizeof(bf16);   // K and V tiles
  constexpr size_t LDS_BYTES = (size_t)VT_BYTES + (size_t)OCC_WAVES * BUF_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "staging must fit in LDS");
  static_assert((size_t)OCC_WAVES * TILE * RED_PITCH * sizeof(float) <= LDS_BYTES,
                "reduction buffer must fit in the staging buffers");
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

  int g;
  const int item = xcd_run_item(blockIdx.x, run_len, Hkv, &g);
  const ScheduleView sv = read_schedule(tiles, item, tile_cap, T, window);
  const Tile tl = sv.tile;
  if (!sv.ok) {
    poison_words(dk, (size_t)T * Hkv * (D / 2), NAN_BF16X2);
    poison_words(dv, (size_t)T * Hkv * (D / 2), NAN_BF16X2);
    return;
  }
  if (!sv.valid) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lh = lane >> 5, lq = lane & 31;
  const int hs = wave & 3, par = wave >> 2;
  const int G = Hq / Hkv;
  const int k0 = tl.t0, k1 = tl.t1, b = tl.seg_b;
  const int qhi = tile_query_hi(k1, b, window, band);
  const int nqb = (qhi - k0 + QBLK - 1) / QBLK;
  const int nmine = (nqb - par + 1) / 2;       // q-blocks of this parity
  const int nheads = hs < G ? (G - hs + 3) / 4 : 0;   // heads hs, hs + 4, ... of the group
  const int steps = nheads * nmine;
  const size_t qstride = (size_t)Hq * D;
  const size_t kstride = (size_t)Hkv * D;

  const bf16* Kt = reinterpret_cast<const bf16*>(smem);
  const bf16* Vt = Kt + TILE * D;
  char* wb = smem + VT_BYTES + (size_t)wave * BUF_BYTES;
  const bf16* Qs = reinterpret_cast<const bf16*>(wb);
  const bf16* Ds = reinterpret_cast<const bf16*>(wb + TILE_BYTES);
  const float* st = reinterpret_cast<const float*>(wb + 2 * TILE_BYTES);
  const uint32_t lds_wb = lds_address(wb);

  // K and V rows of the key tile: wave w loads rows 4w .. 4w + 3 (1 KB each)
  {
    const int r = TileLoad<D>::RPD * wave + lane / TileLoad<D>::CPR;
    const uint32_t off = (uint32_t)min(k0 + r, T - 1) * (uint32_t)(kstride * sizeof(bf16)) +
                         TileLoad<D>::chunk_offset(lane, r);
    dma16(k + (size_t)g * D, off, lds_address(smem) + (uint32_t)(wave * 1024));
    dma16(v + (size_t)g * D, off, lds_address(smem) + (uint32_t)(TILE * D * sizeof(bf16) + wave * 1024));
  }

  const uint32_t rstride = (uint32_t)(qstride * sizeof(bf16));
  auto issue = [&](int head, int i) {
    const int qb = k0 + i * QBLK;
    const size_t hoff = (size_t)qb * qstride + (size_t)head * D;
    const bf16* qsrc = q + hoff;
    const bf16* dsrc = dout + hoff;
    const int rmax = T - 1 - qb;
#pragma unroll
    for (int j = 0; j < Geo::LOADS; ++j) {
      const int r = TileLoad<D>::RPD * j + lane / TileLoad<D>::CPR;
      const uint32_t off = (uint32_t)min(r, rmax) * rstride + TileLoad<D>::chunk_offset(lane, r);
      dma16(qsrc, off, lds_wb + j * 1024);
      dma16(dsrc, off, lds_wb + TILE_BYTES + j * 1024);
    }
    if (lane < 16)
      dma16(stats + (size_t)head * tile_cap + tl.idx + i, (uint32_t)lane * 16,
            lds_wb + 2 * TILE_BYTES);
  };
  int ld_head = g * G + hs, ld_i = par;
  auto issue_next = [&]() {
    issue(ld_head, ld_i);
    ld_i += 2;
    if (ld_i >= nqb) {
      ld_i = par;
      ld_head += 4;
    }
  };
  if (steps > 0) issue_next();

  // K^T as the B operand of S: lane holds k[k0 + lq][16 ks + 8 lh + 0..7]
  const int krow = k0 + lq;
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = zero_f32x16();
    dva[db] = zero_f32x16();
  }
  const bool kvalid = krow < k1;
  const int vis_hi = window > 0 ? min(b - 1, krow + window - 1) : b - 1;
  const int mbias = (kvalid ? 0 : -(1 << 30)) + 4 * lh - krow;
  const uint32_t mspan = kvalid ? (uint32_t)(vis_hi - krow) : 0u;
  // the K and V tiles (every wave's rows) are in LDS after the barrier
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  int ci = par;   // q-block of the current step
  for (int it = 0; it < steps; ++it) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // S and dP seeded with -lse/scale and -D of the step's rows (with a cap,
    // S starts at zero and -lse log2(e) is read back from LDS for P below)
    f32x16 s, dp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 b4 = *reinterpret_cast<const float4*>(st + TILE + 8 * j + 4 * lh);
      if constexpr (CAP) {
        s[4 * j + 0] = 0.f; s[4 * j + 1] = 0.f; s[4 * j + 2] = 0.f; s[4 * j + 3] = 0.f;
      } else {
        const float4 a4 = *reinterpret_cast<const float4*>(st + 8 * j + 4 * lh);
        s[4 * j + 0] = a4.x; s[4 * j + 1] = a4.y; s[4 * j + 2] = a4.z; s[4 * j + 3] = a4.w;
      }
      dp[4 * j + 0] = b4.x; dp[4 * j + 1] = b4.y; dp[4 * j + 2] = b4.z; dp[4 * j + 3] = b4.w;
    }
    {
      // operand reads run two k-steps ahead of the products (ring of 3)
      bf16x8 ring[3][4];
      auto load = [&](int ks, bf16x8* r) {
        r[0] = swz_frag_cols<D>(Qs, ks, lane);
        r[1] = swz_frag_cols<D>(Kt, ks, lane);
        r[2] = swz_frag_cols<D>(Ds, ks, lane);
        r[3] = swz_frag_cols<D>(Vt, ks, lane);
      };
      load(0, ring[0]);
      load(1, ring[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) load(ks + 2, ring[(ks + 2) % 3]);
        s = mfma32(ring[ks % 3][0], ring[ks % 3][1], s);
        dp = mfma32(ring[ks % 3][2], ring[ks % 3][3], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (CAP) tanh_fragments<1>(&s, cap_a, TANH_NARROW / cap_a);
    const int x0 = k0 + ci * QBLK + mbias;
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * t + e;
        const bool vis = (uint32_t)(x0 + 8 * (r >> 2) + (r & 3)) <= mspan;
        if constexpr (CAP) {
          const float th = s[r];
          const float ls = st[8 * (r >> 2) + 4 * lh + (r & 3)];   // -lse log2(e)
          float p = exp2_fast(cap_c2 * th + ls);
          p = vis ? p : 0.f;
          pf[t][e] = (bf16)p;
          dsf[t][e] = (bf16)(p * dp[r] * (1.f - th * th));
        } else {
          float p = exp2_fast(s[r] * scale_log2);
          p = vis ? p : 0.f;
          pf[t][e] = (bf16)p;
          dsf[t][e] = (bf16)(p * dp[r]);
        }
      }
    {
      // the 16 dV/dK products, their transposing reads four products ahead
      constexpr int NP = 4 * DB;   // products: (t, db, dV or dK)
      constexpr int AHEAD = 4;
      bf16x8 ring[AHEAD + 1];
      auto load = [&](int m) {
        const int t = m / (2 * DB), db = (m >> 1) % DB;
        return swz_frag_rows<D>((m & 1) ? Qs : Ds, db * 32, t, lane);
      };
#pragma unroll
      for (int m = 0; m < AHEAD; ++m) ring[m] = load(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        if (m + AHEAD < NP) ring[(m + AHEAD) % (AHEAD + 1)] = load(m + AHEAD);
        const int t = m / (2 * DB), db = (m >> 1) % DB;
        if (m & 1)
          dka[db] = mfma32(dsf[t], ring[m % (AHEAD + 1)], dka[db]);
        else
          dva[db] = mfma32(pf[t], ring[m % (AHEAD + 1)], dva[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // every read of this wave's buffer has returned (the products above
    // consumed them), so the next step's loads may overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (it + 1 < steps) issue_next();
    ci += 2;
    if (ci >= nqb) ci = par;
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

  // Reduction over the 8 waves in a fixed order, then store.
  float* red = reinterpret_cast<float*>(smem);
  constexpr int OCOLS = D / 16;   // output columns per thread (32 keys x 16 threads)
  const int okey = tid >> 4, od = (tid & 15) * OCOLS;
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    float* mine = red + (size_t)wave * TILE * RED_PITCH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
        mine[key * RED_PITCH + db * 32 + lq] = pass == 0 ? dka[db][r] : dva[db][r];
      }
    __syncthreads();
    if (k0 + okey < k1) {
      const float mul = pass == 0 ? scale : 1.f;
      bf16* dst = (pass == 0 ? dk : dv) + (size_t)(k0 + okey) * kstride + (size_t)g * D + od;
#pragma unroll
      for (int e = 0; e < OCOLS; e += 4) {
        float acc4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < OCC_WAVES; ++w)
            sum += red[(size_t)w * TILE * RED_PITCH + okey * RED_PITCH + od + e + x];
          acc4[x] = sum * mul;
        }
        store_bf16x4(dst + e, acc4[0], acc4[1], acc4[2], acc4[3]);
      }
    }
  }
}

// dK/dV at head dim 128 without a cap, two work-groups per CU: 4 waves per
// work-group (wave w takes query heads w, w + 4, ... of the group and all of
// their q-blocks), one work-group per (32-key tile, kv head).  LDS holds the
// tile's K and V rows (16 KB) and one Q/dO buffer per wave (16 KB): 80 KB, so
// that two work-groups share a CU and each one's start (boundaries, tile
// record, K/V rows, first block) and end (the reduction over its waves and
// the stores) overlap the other's products.  The TileStats seeds of a step
// go straight from global memory into the registers that become its S and
// dP accumulators; they are loaded during the previous step's dV/dK
// products, when those registers are free.  Otherwise each step is that of
// dkdv_occ_kernel; the 4 partial sums are added in a fixed order at the end.
constexpr int TWIN_WAVES = 4;
constexpr int TWIN_MAX_SPAN = 1024;   // queries per key tile, see launch_dkdv_kernel
constexpr int TWIN_THREADS = 64 * TWIN_WAVES;

__global__ __launch_bounds__(TWIN_THREADS, 2) void dkdv_twin_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const TileStats* __restrict__ stats, int tile_cap,
    const Tile* __restrict__ tiles, int T, int Hq, int Hkv,
    int window, int band, float scale_log2, float scale, int run_len, bf16* __restrict__ dk,
    bf16* __restrict__ dv) {
  constexpr int D = 128;
  using Geo = DkdvGeom<D>;
  constexpr int KS = Geo::KS, DB = Geo::DB, RED_PITCH = Geo::RED_PITCH;
  constexpr int TILE_BYTES = Geo::TILE_BYTES;                  // 32 x 128 bf16
  constexpr int KV_BYTES = 2 * TILE_BYTES;                     // K and V tiles
  constexpr int WBUF_BYTES = 2 * TILE_BYTES;                   // a wave's Q and dO
  constexpr size_t LDS_BYTES = (size_t)KV_BYTES + (size_t)TWIN_WAVES * WBUF_BYTES;
  static_assert(2 * LDS_BYTES <= 160 * 1024, "two work-groups per CU");
  static_assert((size_t)TWIN_WAVES * TILE * RED_PITCH * sizeof(float) <= LDS_BYTES,
                "reduction buffer must fit in the staging buffers");
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

  // work-group -> (key tile, key-value head), in runs of neighbouring key
  // tiles per XCD (xcd_run_item)
  int g;
  const int item = xcd_run_item(blockIdx.x, run_len, Hkv, &g);
  const ScheduleView sv = read_schedule(tiles, item, tile_cap, T, window);
  const Tile tl = sv.tile;
  if (!sv.ok) {
    poison_words(dk, (size_t)T * Hkv * (D / 2), NAN_BF16X2);
    poison_words(dv, (size_t)T * Hkv * (D / 2), NAN_BF16X2);
    return;
  }
  if (!sv.valid) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lh = lane >> 5, lq = lane & 31;
  const int G = Hq / Hkv;
  const int k0 = tl.t0, k1 = tl.t1, b = tl.seg_b;
  const int qhi = tile_query_hi(k1, b, window, band);
  const int nqb = (qhi - k0 + QBLK - 1) / QBLK;
  const int nheads = wave < G ? (G - wave + 3) / 4 : 0;   // heads wave, wave + 4, ...
  const int steps = nheads * nqb;
  const size_t qstride = (size_t)Hq * D;
  const size_t kstride = (size_t)Hkv * D;

  const bf16* Kt = reinterpret_cast<const bf16*>(smem);
  const bf16* Vt = Kt + TILE * D;
  char* wb = smem + KV_BYTES + (size_t)wave * WBUF_BYTES;
  const bf16* Qs = reinterpret_cast<const bf16*>(wb);
  const bf16* Ds = reinterpret_cast<const bf16*>(wb + TILE_BYTES);
  const uint32_t lds_wb = lds_address(wb);

  // K and V rows of the key tile: wave w loads rows 8w .. 8w + 7 (rows past
  // T re-read row T - 1; they are masked)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * wave + TileLoad<D>::RPD * j + lane / TileLoad<D>::CPR;
    const uint32_t off = (uint32_t)min(k0 + r, T - 1) * (uint32_t)(kstride * sizeof(bf16)) +
                         TileLoad<D>::chunk_offset(lane, r);
    dma16(k + (size_t)g * D, off, lds_address(smem) + (uint32_t)(wave * 2048 + j * 1024));
    dma16(v + (size_t)g * D, off, lds_address(smem) + (uint32_t)(TILE_BYTES + wave * 2048 + j * 1024));
  }

  // Step s: head g G + wave + 4 (s / nqb), q-block s % nqb.  Rows past T
  // re-read row T - 1 (masked later).
  const uint32_t rstride = (uint32_t)(qstride * sizeof(bf16));
  auto issue = [&](int s) {
    const int j = s / nqb, i = s - j * nqb;
    const int qb = k0 + i * QBLK;
    const size_t hoff = (size_t)qb * qstride + (size_t)(g * G + wave + 4 * j) * D;
    const int rmax = T - 1 - qb;
#pragma unroll
    for (int x = 0; x < Geo::LOADS; ++x) {
      const int r = TileLoad<D>::RPD * x + lane / TileLoad<D>::CPR;
      const uint32_t off = (uint32_t)min(r, rmax) * rstride + TileLoad<D>::chunk_offset(lane, r);
      dma16(q + hoff, off, lds_wb + x * 1024);
      dma16(dout + hoff, off, lds_wb + TILE_BYTES + x * 1024);
    }
  };
  // Seeds of step s (-lse / scale and -D of its rows, in accumulator order)
  auto seeds = [&](int s, f32x16& s0, f32x16& d0) {
    const int j = s / nqb, i = s - j * nqb;
    const TileStats* st = stats + (size_t)(g * G + wave + 4 * j) * tile_cap + tl.idx + i;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float4 a4 = *reinterpret_cast<const float4*>(st->s0 + 8 * x + 4 * lh);
      const float4 b4 = *reinterpret_cast<const float4*>(st->dp0 + 8 * x + 4 * lh);
      s0[4 * x + 0] = a4.x; s0[4 * x + 1] = a4.y; s0[4 * x + 2] = a4.z; s0[4 * x + 3] = a4.w;
      d0[4 * x + 0] = b4.x; d0[4 * x + 1] = b4.y; d0[4 * x + 2] = b4.z; d0[4 * x + 3] = b4.w;
    }
  };

  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = zero_f32x16();
    dva[db] = zero_f32x16();
  }
  const int krow = k0 + lq;
  const bool kvalid = krow < k1;
  const int vis_hi = window > 0 ? min(b - 1, krow + window - 1) : b - 1;
  const int mbias = (kvalid ? 0 : -(1 << 30)) + 4 * lh - krow;
  const uint32_t mspan = kvalid ? (uint32_t)(vis_hi - krow) : 0u;

  f32x16 seed_s = zero_f32x16(), seed_d = zero_f32x16();
  if (steps > 0) {
    seeds(0, seed_s, seed_d);
    issue(0);
  }
  // the K and V tiles (every wave's rows) are in LDS after the barrier
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int s = 0; s < steps; ++s) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int i = s % nqb;
    f32x16 sacc = seed_s, dpacc = seed_d;
    {
      // operand reads run two k-steps ahead of the products (ring of 3)
      bf16x8 ring[3][4];
      auto load = [&](int ks, bf16x8* r) {
        r[0] = swz_frag_cols<D>(Qs, ks, lane);
        r[1] = swz_frag_cols<D>(Kt, ks, lane);
        r[2] = swz_frag_cols<D>(Ds, ks, lane);
        r[3] = swz_frag_cols<D>(Vt, ks, lane);
      };
      load(0, ring[0]);
      load(1, ring[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) load(ks + 2, ring[(ks + 2) % 3]);
        sacc = mfma32(ring[ks % 3][0], ring[ks % 3][1], sacc);
        dpacc = mfma32(ring[ks % 3][2], ring[ks % 3][3], dpacc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int x0 = k0 + i * QBLK + mbias;
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * t + e;
        const bool vis = (uint32_t)(x0 + 8 * (r >> 2) + (r & 3)) <= mspan;
        float p = exp2_fast(sacc[r] * scale_log2);
        p = vis ? p : 0.f;
        pf[t][e] = (bf16)p;
        dsf[t][e] = (bf16)(p * dpacc[r]);
      }
    // the next step's seeds (this step's again after the last, so that the
    // seed registers are rewritten on every path and free during S/dP)
    seeds(s + 1 < steps ? s + 1 : s, seed_s, seed_d);
    {
      // the 16 dV/dK products, their transposing reads four products ahead
      constexpr int NP = 4 * DB;
      constexpr int AHEAD = 4;
      bf16x8 ring[AHEAD + 1];
      auto load = [&](int m) {
        const int t = m / (2 * DB), db = (m >> 1) % DB;
        return swz_frag_rows<D>((m & 1) ? Qs : Ds, db * 32, t, lane);
      };
#pragma unroll
      for (int m = 0; m < AHEAD; ++m) ring[m] = load(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        if (m + AHEAD < NP) ring[(m + AHEAD) % (AHEAD + 1)] = load(m + AHEAD);
        const int t = m / (2 * DB), db = (m >> 1) % DB;
        if (m & 1)
          dka[db] = mfma32(dsf[t], ring[m % (AHEAD + 1)], dka[db]);
        else
          dva[db] = mfma32(pf[t], ring[m % (AHEAD + 1)], dva[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // every read of this wave's buffer has returned (the products above
    // consumed them), so the next step's loads may overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (s + 1 < steps) issue(s + 1);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

  // Reduction over the 4 waves in a fixed order, then store: thread t sums
  // 16 columns of key t / 8.
  float* red = reinterpret_cast<float*>(smem);
  constexpr int OCOLS = D / 8;
  const int okey = tid >> 3, od = (tid & 7) * OCOLS;
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    float* mine = red + (size_t)wave * TILE * RED_PITCH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
        mine[key * RED_PITCH + db * 32 + lq] = pass == 0 ? dka[db][r] : dva[db][r];
      }
    __syncthreads();
    if (k0 + okey < k1) {
      const float mul = pass == 0 ? scale : 1.f;
      bf16* dst = (pass == 0 ? dk : dv) + (size_t)(k0 + okey) * kstride + (size_t)g * D + od;
#pragma unroll
      for (int e = 0; e < OCOLS; e += 4) {
        float acc4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < TWIN_WAVES; ++w)
            sum += red[(size_t)w * TILE * RED_PITCH + okey * RED_PITCH + od + e + x];
          acc4[x] = sum * mul;
        }
        store_bf16x4(dst + e, acc4[0], acc4[1], acc4[2], acc4[3]);
      }
    }
  }
}

template <int D, bool CAP>
void launch_dq_kernel(const void* q, const void* k, const void* v, const void* out,
                      const float* lse, const void* dout, const Problem& p, void* dq, char* ws,
                      const WorkspaceLayout& w, hipStream_t stream) {
  const unsigned grid = run_grid(head_chunks(p.num_q_heads, p.num_kv_heads), w.tile_cap,
                                 run_length(p.window));
  const CapConstants cc = cap_constants(p);
  hipLaunchKernelGGL((dq_kernel<D, CAP>), dim3(grid), dim3(BWD_THREADS), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(out),
                     static_cast<const bf16*>(dout), lse,
                     reinterpret_cast<const Tile*>(ws + w.tiles_fwd), p.total_tokens,
                     p.num_q_heads, p.num_kv_heads, p.window, p.band, p.scale * LOG2E, p.scale,
                     cc.cap_a, cc.cap_c2, (int)w.tile_cap, static_cast<bf16*>(dq),
                     reinterpret_cast<TileStats*>(ws + w.rowstats));
}

template <int D, bool CAP>
void launch_dkdv_kernel(const void* q, const void* k, const void* v, const void* dout,
                        const Problem& p, void* dk, void* dv, const char* ws,
                        const WorkspaceLayout& w, hipStream_t stream) {
  // Runs of run_length(window) list entries per key-value head, dealt to the
  // XCDs in rounds of 8 runs; the grid covers every (tile, head) pair.
  const int run_len = run_length(p.window);
  const unsigned grid = run_grid(p.num_kv_heads, w.tile_cap, run_len);
  const CapConstants cc = cap_constants(p);
  // When no tile meets more than TWIN_MAX_SPAN queries (a window, or short
  // documents) the two-work-groups-per-CU kernel runs; otherwise the 8-wave
  // one: a twin work-group streams all of a tile's q-blocks through each
  // wave, twice as long as an 8-wave one, and a long document's first tiles
  // then outlast the average work per CU (A/B at context 4,096: window-512
  // dK/dV 83.0 -> 79.7 us, global 180 -> 204 us).  The choice depends only on
  // the call's window and max_seqlen (not the band formulation), so a window
  // at least as long as every segment still gives the same bits as no
  // window, and a band call the same bits as a plain one.
  const int reach = p.window > 0 ? p.window : p.max_seqlen;
  if (D == 128 && !CAP && std::min(reach, p.max_seqlen) <= TWIN_MAX_SPAN) {
    hipLaunchKernelGGL(dkdv_twin_kernel, dim3(grid), dim3(TWIN_THREADS), 0, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), static_cast<const bf16*>(dout),
                       reinterpret_cast<const TileStats*>(ws + w.rowstats), (int)w.tile_cap,
                       reinterpret_cast<const Tile*>(ws + w.tiles_bwd), p.total_tokens,
                       p.num_q_heads, p.num_kv_heads, p.window, p.band, p.scale * LOG2E,
                       p.scale, run_len, static_cast<bf16*>(dk), static_cast<bf16*>(dv));
    return;
  }
  // head dim 256: pairs of waves split the head dim; 128: two waves per
  // SIMD; 64: the software-pipelined kernel
  constexpr bool occ = D == 128;
  void (*kernel)(const bf16*, const bf16*, const bf16*, const bf16*, const TileStats*, int,
                 const Tile*, int, int, int, int, int, float, float, float, float, int, bf16*,
                 bf16*);
  if constexpr (D == 256)
    kernel = dkdv_split_kernel<CAP>;
  else if constexpr (D == 128)
    kernel = dkdv_occ_kernel<CAP>;
  else
    kernel = dkdv_kernel<D, CAP>;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(occ ? OCC_THREADS : BWD_THREADS), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(dout),
                     reinterpret_cast<const TileStats*>(ws + w.rowstats), (int)w.tile_cap,
                     reinterpret_cast<const Tile*>(ws + w.tiles_bwd), p.total_tokens,
                     p.num_q_heads, p.num_kv_heads, p.window, p.band, p.scale * LOG2E, p.scale,
                     cc.cap_a, cc.cap_c2, run_len, static_cast<bf16*>(dk),
                     static_cast<bf16*>(dv));
}

}  // namespace

hipError_t launch_dq(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, const Problem& p, void* dq,
                     void* workspace, const WorkspaceLayout& w, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  const bool cap = p.softcap > 0.f;
#define ATTN_DQ(D)                                                                    \
  (cap ? launch_dq_kernel<D, true>(q, k, v, out, lse, dout, p, dq, ws, w, stream)     \
       : launch_dq_kernel<D, false>(q, k, v, out, lse, dout, p, dq, ws, w, stream))
  switch (p.head_dim) {
    case 64: ATTN_DQ(64); break;
    case 128: ATTN_DQ(128); break;
    case 256: ATTN_DQ(256); break;
    default: return hipErrorInvalidValue;
  }
#undef ATTN_DQ
  return hipGetLastError();
}

hipError_t launch_dkdv(const void* q, const void* k, const void* v, const float* lse,
                       const void* dout, const Problem& p, void* dk, void* dv, void* workspace,
                       const WorkspaceLayout& w, hipStream_t stream) {
  (void)lse;
  const char* ws = static_cast<const char*>(workspace);
  const bool cap = p.softcap > 0.f;
#define ATTN_DKDV(D)                                                                \
  (cap ? launch_dkdv_kernel<D, true>(q, k, v, dout, p, dk, dv, ws, w, stream)       \
       : launch_dkdv_kernel<D, false>(q, k, v, dout, p, dk, dv, ws, w, stream))
  switch (p.head_dim) {
    case 64: ATTN_DKDV(64); break;
    case 128: ATTN_DKDV(128); break;
    case 256: ATTN_DKDV(256); break;
    default: return hipErrorInvalidValue;
  }
#undef ATTN_DKDV
  return hipGetLastError();
}

}  // namespace attn
