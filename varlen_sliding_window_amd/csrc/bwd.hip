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
//   forms D = rowsum(dO * O) for its rows (fp32) and writes it to the
//   workspace for the dK/dV kernel, which runs next on the same stream.
// dK/dV kernel: one work-group per (k-tile of 32 keys, key-value head); its
//   4 waves take the group's query heads (wave w: heads w, w + 4, ...).  K
//   and V stay in registers; each wave streams its head's Q/dO rows through
//   its own LDS slice in QBLK = 32-row steps and keeps dK/dV partial sums in
//   fp32 registers.  The 4 partials are added in a fixed order through LDS
//   at the end, so the head-group reduction needs no atomics and is
//   bit-for-bit reproducible.
#include "device.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BWD_THREADS = 256;

__global__ __launch_bounds__(BWD_THREADS, 2) void dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ out, const bf16* __restrict__ dout, const float* __restrict__ lse,
    const int* __restrict__ header, const Tile* __restrict__ tiles, int T, int Hq, int Hkv,
    int window, float scale_log2, float scale, int tile_cap, bf16* __restrict__ dq,
    RowStats* __restrict__ rowstats) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[KBLK * LDS_PITCH];
  __shared__ __attribute__((aligned(16))) bf16 Vs[KBLK * LDS_PITCH];

  const int chunks = Hq >> 2;
  const int item = blockIdx.x / chunks;
  const int hc = blockIdx.x - item * chunks;
  if (item >= header[0]) return;
  const Tile tl = tiles[item];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lh = lane >> 5, lq = lane & 31;
  const int head = hc * 4 + wave;
  const int g = (hc * 4) / (Hq / Hkv);
  const int q0 = tl.t0, q1 = tl.t1, a = tl.seg_a;
  const int klo = first_visible_key(q0, a, window);
  const int nblk = (q1 - klo + KBLK - 1) / KBLK;
  const int qrow = q0 + lq;
  const size_t qstride = (size_t)Hq * HEAD_DIM;
  const size_t kstride = (size_t)Hkv * HEAD_DIM;

  // Q^T and dO^T as B operands; D from dO and O at the same positions
  bf16x8 qf[8], df[8];
  float dpart = 0.f;
  {
    const size_t off = (size_t)qrow * qstride + (size_t)head * HEAD_DIM + lh * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
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
  const float Dv = dpart + __shfl_xor(dpart, 32);
  const float lse2 = qrow < T ? lse[(size_t)head * T + qrow] * LOG2E : 0.f;
  if (qrow < q1 && lh == 0) {
    RowStats rs;
    rs.lse2 = lse2;
    rs.d = Dv;
    rowstats[((size_t)head * tile_cap + tl.idx) * TILE + lq] = rs;
  }

  const int srow = tid >> 4, scol = (tid & 15) * 8;
  uint4 kr[4], vr[4];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kb + srow + 16 * i;
      if (key >= 0) {
        const size_t off = (size_t)key * kstride + (size_t)g * HEAD_DIM + scol;
        kr[i] = ldg16(k + off);
        vr[i] = ldg16(v + off);
      } else {
        kr[i] = make_uint4(0u, 0u, 0u, 0u);
        vr[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = zero_f32x16();
  const int full_lo = first_visible_key(q0 + TILE - 1, a, window);
  const int my_lo = first_visible_key(qrow, a, window);

  gload(q1 - KBLK);
  for (int n = 0; n < nblk; ++n) {
    const int kb = q1 - KBLK * (n + 1);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(Ks + (srow + 16 * i) * LDS_PITCH + scol) = kr[i];
      *reinterpret_cast<uint4*>(Vs + (srow + 16 * i) * LDS_PITCH + scol) = vr[i];
    }
    __syncthreads();
    if (n + 1 < nblk) gload(kb - KBLK);

    f32x16 s[2], dp[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      s[h2] = zero_f32x16();
      dp[h2] = zero_f32x16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s[h2] = mfma32(lds_frag_cols(Ks + h2 * 32 * LDS_PITCH, ks, lane), qf[ks], s[h2]);
        dp[h2] = mfma32(lds_frag_cols(Vs + h2 * 32 * LDS_PITCH, ks, lane), df[ks], dp[h2]);
      }
    }
    const bool full = (kb + KBLK - 1 <= q0) && (kb >= full_lo);
    bf16x8 dsf[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + h2 * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
        const bool vis = full || (key >= my_lo && key <= qrow);
        const float p = vis ? exp2_fast(s[h2][r] * scale_log2 - lse2) : 0.f;
        dsf[h2 * 2 + (r >> 3)][r & 7] = (bf16)(p * (dp[h2][r] - Dv));
      }
    // dQ^T[d][q] += sum_key K^T[d][key] dS^T[key][q]
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc[db] = mfma32(lds_frag_rows(Ks + db * 32, t, lane), dsf[t], acc[db]);
  }

  if (qrow < q1) {
    bf16* op = dq + (size_t)qrow * qstride + (size_t)head * HEAD_DIM + lh * 4;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_bf16x4(op + db * 32 + j * 8, acc[db][4 * j] * scale, acc[db][4 * j + 1] * scale,
                     acc[db][4 * j + 2] * scale, acc[db][4 * j + 3] * scale);
  }
}

constexpr int DKDV_WAVES = 4;
constexpr int RED_PITCH = HEAD_DIM + 4;   // fp32 pitch of the reduction buffer
// Per wave and buffer: Q tile, dO tile (32 x 128 bf16 each, swizzled), then
// the 32 rows' RowStats.
static_assert(QBLK == TILE, "a dK/dV q-block is exactly one q-tile");
constexpr int DKDV_TILE_ELEMS = QBLK * HEAD_DIM;
constexpr size_t DKDV_BUF_BYTES = 2 * DKDV_TILE_ELEMS * sizeof(bf16) + QBLK * sizeof(RowStats);
constexpr size_t DKDV_LDS_BYTES = (size_t)DKDV_WAVES * 2 * DKDV_BUF_BYTES;
static_assert((size_t)DKDV_WAVES * TILE * RED_PITCH * sizeof(float) <= DKDV_LDS_BYTES,
              "reduction buffer must fit in the staging buffers");

__global__ __launch_bounds__(BWD_THREADS, 1) void dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const RowStats* __restrict__ rowstats, int tile_cap,
    const int* __restrict__ header, const Tile* __restrict__ tiles, int T, int Hq, int Hkv,
    int window, float scale_log2, float scale, bf16* __restrict__ dk, bf16* __restrict__ dv) {
  __shared__ __attribute__((aligned(16))) char smem[DKDV_LDS_BYTES];

  const int item = blockIdx.x / Hkv;
  const int g = blockIdx.x - item * Hkv;
  if (item >= header[0]) return;
  const Tile tl = tiles[item];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lh = lane >> 5, lq = lane & 31;
  const int G = Hq / Hkv;
  const int k0 = tl.t0, k1 = tl.t1, b = tl.seg_b;
  const int qhi = window > 0 ? min(b, k1 - 1 + window) : b;
  const int nqb = (qhi - k0 + QBLK - 1) / QBLK;
  const int steps = (G / DKDV_WAVES) * nqb;   // (head, q-block) pairs of this wave
  const size_t qstride = (size_t)Hq * HEAD_DIM;
  const size_t kstride = (size_t)Hkv * HEAD_DIM;

  char* wbase = smem + (size_t)wave * 2 * DKDV_BUF_BYTES;
  auto q_tile = [&](int buf) { return reinterpret_cast<bf16*>(wbase + buf * DKDV_BUF_BYTES); };
  auto do_tile = [&](int buf) { return q_tile(buf) + DKDV_TILE_ELEMS; };
  auto ld_vals = [&](int buf) {
    return reinterpret_cast<float*>(wbase + buf * DKDV_BUF_BYTES +
                                    2 * DKDV_TILE_ELEMS * sizeof(bf16));
  };

  // Prefetch of step `it` into buffer `buf`: Q and dO rows of q-block i (the
  // q-tile idx + i of this segment), then that tile's 32 RowStats (lanes 0-15,
  // 16 bytes each).  Rows past the segment hold stale values; they are
  // masked with selects, so even NaNs there cannot leak.
  auto issue = [&](int it, int buf) {
    const int head = g * G + wave + DKDV_WAVES * (it / nqb);
    const int i = it % nqb;
    const int qb = k0 + i * QBLK;
    swz_tile32_load_async(q_tile(buf), q + (size_t)head * HEAD_DIM, qstride, qb, T, lane);
    swz_tile32_load_async(do_tile(buf), dout + (size_t)head * HEAD_DIM, qstride, qb, T, lane);
    if (lane < 16) {
      const RowStats* src = rowstats + ((size_t)head * tile_cap + tl.idx + i) * TILE + 2 * lane;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)ld_vals(buf), 16, 0, 0);
    }
  };
  if (steps > 0) issue(0, 0);

  // K^T and V^T as B operands: lane holds k[k0 + lq][16 ks + 8 lh + 0..7]
  const int krow = k0 + lq;
  bf16x8 kf[8], vf[8];
  {
    const size_t off = (size_t)min(krow, T - 1) * kstride + (size_t)g * HEAD_DIM + lh * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kf[ks] = as_bf16x8(ldg16(k + off + ks * 16));
      vf[ks] = as_bf16x8(ldg16(v + off + ks * 16));
    }
  }

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dka[db] = zero_f32x16();
    dva[db] = zero_f32x16();
  }
  const bool keys_full = (k1 - k0) == TILE;

  for (int it = 0; it < steps; ++it) {
    const int buf = it & 1;
    // The only loads in flight are this step's; wait for them, take this
    // step's row statistics into registers, then start the next step's
    // loads so they overlap this step's math.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const float* LD = ld_vals(buf);   // (lse2, D) pairs of rows qb + 0..31
    float lv[16], dd[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a4 = *reinterpret_cast<const float4*>(LD + 2 * (8 * j + 4 * lh));
      const float4 b4 = *reinterpret_cast<const float4*>(LD + 2 * (8 * j + 4 * lh) + 4);
      lv[4 * j + 0] = a4.x; dd[4 * j + 0] = a4.y;
      lv[4 * j + 1] = a4.z; dd[4 * j + 1] = a4.w;
      lv[4 * j + 2] = b4.x; dd[4 * j + 2] = b4.y;
      lv[4 * j + 3] = b4.z; dd[4 * j + 3] = b4.w;
    }
    if (it + 1 < steps) issue(it + 1, buf ^ 1);
    const int qb = k0 + (it % nqb) * QBLK;
    const bf16* Qs = q_tile(buf);
    const bf16* Ds = do_tile(buf);

    // S[q][key] = Q K^T and dP = dO V^T: s[r] holds query qb + 8(r/4) + 4 lh + r%4, key k0 + lq
    f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s = mfma32(swz_frag_cols(Qs, ks, lane), kf[ks], s);
      dp = mfma32(swz_frag_cols(Ds, ks, lane), vf[ks], dp);
    }
    const bool full = keys_full && (qb + QBLK - 1 < b) && (qb >= k0 + TILE - 1) &&
                      (window <= 0 || qb + QBLK - 1 < k0 + window);
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * j + e;
        const int qi = qb + 8 * j + 4 * lh + e;
        const bool vis = full || (krow < k1 && qi < b && krow <= qi &&
                                  (window <= 0 || krow > qi - window));
        const float p = vis ? exp2_fast(s[r] * scale_log2 - lv[r]) : 0.f;
        const float ds = vis ? p * (dp[r] - dd[r]) : 0.f;
        pf[r >> 3][r & 7] = (bf16)p;
        dsf[r >> 3][r & 7] = (bf16)ds;
      }
    }
    // dV[key][d] += P^T dO ; dK[key][d] += dS^T Q  (scale applied at the end)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dva[db] = mfma32(pf[t], swz_frag_rows(Ds, db * 32, t, lane), dva[db]);
        dka[db] = mfma32(dsf[t], swz_frag_rows(Qs, db * 32, t, lane), dka[db]);
      }
  }

  // Head-group reduction in a fixed order (wave 0 + 1 + 2 + 3), then store.
  float* red = reinterpret_cast<float*>(smem);
  const int okey = tid >> 3, od = (tid & 7) * 16;
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    float* mine = red + (size_t)wave * TILE * RED_PITCH;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
        mine[key * RED_PITCH + db * 32 + lq] = pass == 0 ? dka[db][r] : dva[db][r];
      }
    __syncthreads();
    if (k0 + okey < k1) {
      const float mul = pass == 0 ? scale : 1.f;
      bf16* dst = (pass == 0 ? dk : dv) + (size_t)(k0 + okey) * kstride +
                  (size_t)g * HEAD_DIM + od;
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
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

}  // namespace

hipError_t launch_dq(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, const Problem& p, void* dq,
                     void* workspace, const WorkspaceLayout& w, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  const unsigned grid = (unsigned)(w.tile_cap * (size_t)(p.num_q_heads / 4));
  hipLaunchKernelGGL(dq_kernel, dim3(grid), dim3(BWD_THREADS), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(out),
                     static_cast<const bf16*>(dout), lse, reinterpret_cast<const int*>(ws + w.header),
                     reinterpret_cast<const Tile*>(ws + w.tiles_fwd), p.total_tokens,
                     p.num_q_heads, p.num_kv_heads, p.window, p.scale * LOG2E, p.scale,
                     (int)w.tile_cap, static_cast<bf16*>(dq),
                     reinterpret_cast<RowStats*>(ws + w.rowstats));
  return hipGetLastError();
}

hipError_t launch_dkdv(const void* q, const void* k, const void* v, const float* lse,
                       const void* dout, const Problem& p, void* dk, void* dv, void* workspace,
                       const WorkspaceLayout& w, hipStream_t stream) {
  const char* ws = static_cast<const char*>(workspace);
  const unsigned grid = (unsigned)(w.tile_cap * (size_t)p.num_kv_heads);
  hipLaunchKernelGGL(dkdv_kernel, dim3(grid), dim3(BWD_THREADS), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(dout),
                     reinterpret_cast<const RowStats*>(ws + w.rowstats), (int)w.tile_cap,
                     reinterpret_cast<const int*>(ws + w.header),
                     reinterpret_cast<const Tile*>(ws + w.tiles_bwd), p.total_tokens,
                     p.num_q_heads, p.num_kv_heads, p.window, p.scale * LOG2E, p.scale,
                     static_cast<bf16*>(dk), static_cast<bf16*>(dv));
  return hipGetLastError();
}

}  // namespace attn
