// Forward kernel: out and lse of document-masked causal GQA attention.
//
// One work-group (4 waves) takes one q-tile of TILE = 32 rows and 4 query
// heads of one key-value head group (research.dws.rip/llm/kernels, Fig. 2
// "Benchmark setup": 8 query heads share 2 key-value heads, so 4 query heads
// read the same K/V; a group of G heads takes ceil(G / 4) work-groups, and
// waves past its last head only help stage K/V).  Each wave owns one head: its 32 q rows stay in
// registers as MFMA operands, while the work-group streams the visible keys
// through LDS in blocks shared by the 4 heads (64 keys for head dims 64 and
// 128, 32 for 256, so that two double-buffered K/V blocks stay at 64 KB).  The blocks
// arrive by direct global-to-LDS loads, double-buffered: the loads of the
// next block go out as soon as every wave is done with the buffer they
// overwrite, one barrier per block.
//
// The wave computes S^T = K Q^T (keys x queries), so each lane holds one
// query's scores in registers: the row max needs one cross-half exchange,
// the row sum is kept per lane and combined once at the end, and P^T feeds
// the O^T = V^T P^T product straight from registers (V^T read from the
// natural-layout V tile with transposing LDS reads).  Softmax runs in the
// exp2 domain with scale * log2(e) folded into one multiply, and the
// running maximum is only moved (and O rescaled) when a block raises it by
// more than RESCALE_LOG2: in between, probabilities may exceed 1 by up to
// 2^RESCALE_LOG2, which bf16 and the fp32 sums carry exactly as well.  Key
// blocks are aligned to the tile end and walked from the diagonal backwards,
// so the first block sets a good maximum and only the diagonal block and the
// blocks at the segment start or window edge need the mask.
//
// With a logit soft-cap (the CAP instantiation) each score becomes
// softcap * tanh(scale * qk / softcap) right after its product, already in
// log2 units, and the rest of the kernel runs unchanged with a unit scale.
#include "device.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int FWD_THREADS = 256;
constexpr float RESCALE_LOG2 = 8.f;

template <int D, bool CAP>
__global__ __launch_bounds__(FWD_THREADS, BlockGeom<D>::MIN_WG) void fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const Tile* __restrict__ tiles, int tile_cap, int T, int Hq,
    int Hkv, int window, int band, float scale_log2, float cap_a, float cap_c2,
    bf16* __restrict__ out, float* __restrict__ lse) {
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
    poison_words(out, (size_t)T * Hq * (D / 2), NAN_BF16X2);
    poison_words(lse, (size_t)Hq * T, NAN_F32);
    return;
  }
  if (!sv.valid) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lh = lane >> 5, lq = lane & 31;
  const int g = hc / cpg;
  const int hrel = (hc - g * cpg) * HEADS_PER_WG + wave;   // head within the group
  // A wave past the group's last head (G not a multiple of 4) still stages
  // its share of every key/value block but computes and stores nothing.
  const bool active = hrel < G;
  const int head = g * G + min(hrel, G - 1);
  const int q0 = tl.t0, q1 = tl.t1, a = tl.seg_a;
  const int klo = tile_key_lo(q0, a, window, band);
  const int nblk = (q1 - klo + KB - 1) / KB;
  const int qrow = q0 + lq;
  const size_t qstride = (size_t)Hq * D;
  const uint32_t kstride_b = (uint32_t)(Hkv * D * sizeof(bf16));

  // Block loads: wave w fills rows ROWS_PER_WAVE * w + [0, ROWS_PER_WAVE) of
  // the K and V tiles, RPD rows (1 KB) per load.  Keys before 0 re-read key
  // 0; they are always masked.
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
  // Q^T as the B operand: lane holds q[qrow][16 ks + 8 lh + 0..7].  Up to
  // D = 128 a wave's 32 q rows fit in its quarter of the second K/V buffer,
  // so they arrive there as whole-row direct loads (ahead of the first
  // block's) and are read out as fragments; at D = 256 lanes load them.
  constexpr bool STAGE = RowTile<D>::BYTES * 4 <= Geo::BUF_BYTES;
  auto wave_tile = [&](int b) {
    return reinterpret_cast<bf16*>(smem + b * Geo::BUF_BYTES + wave * RowTile<D>::BYTES);
  };
  bf16x8 qf[KS];
  if constexpr (STAGE) {
    dma_tile_rows<D>(q + (size_t)q0 * qstride + (size_t)head * D, (uint32_t)(qstride * sizeof(bf16)),
                     min(TILE, T - q0), lds_address(wave_tile(1)), lane);
    issue(0, 0);
    // the Q rows have landed (the block's 2 * LOADS loads may still be in flight)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * Geo::LOADS) : "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = swz_frag_cols<D>(wave_tile(1), ks, lane);
  } else {
    issue(0, 0);
    const bf16* qp = q + (size_t)qrow * qstride + (size_t)head * D + lh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qrow < T ? as_bf16x8(ldg16(qp + ks * 16)) : zero_bf16x8();
    // Make the compiler wait for these loads here, not inside the loop where
    // the wait would also cover the block loads in flight.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero_f32x16();
  float m = -INFINITY, lsum = 0.f;
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

    // S^T for keys kb + 32 h2 + [0, 32): s[h2][r] = q[qrow] . k[kb + 32 h2 + 8(r/4) + 4 lh + r%4]
    f32x16 s[H2];
#pragma unroll
    for (int h2 = 0; h2 < H2; ++h2) s[h2] = zero_f32x16();
    {
      // K fragment reads run AHEAD products ahead of the products that use
      // them (a register ring; the fences keep the compiler from sinking them)
      constexpr int NP = H2 * KS, AHEAD = 6;
      bf16x8 ring[AHEAD + 1];
      auto load = [&](int m) {
        const int ks = m / H2, h2 = m % H2;
        return swz_frag_cols<D>(Ks + h2 * 32 * D, ks, lane);
      };
#pragma unroll
      for (int m = 0; m < AHEAD; ++m) ring[m] = load(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        if (m + AHEAD < NP) ring[(m + AHEAD) % (AHEAD + 1)] = load(m + AHEAD);
        const int ks = m / H2, h2 = m % H2;
        s[h2] = mfma32(ring[m % (AHEAD + 1)], qf[ks], s[h2]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (CAP) {
      tanh_fragments<H2>(s, cap_a, TANH_NARROW / cap_a);
#pragma unroll
      for (int h2 = 0; h2 < H2; ++h2)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[h2][r] *= cap_c2;
    }
    const bool full = (kb + KB - 1 <= q0) && (kb >= full_lo);
    if (!full) {
#pragma unroll
      for (int h2 = 0; h2 < H2; ++h2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + h2 * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
          if (key < my_lo || key > qrow) s[h2][r] = -INFINITY;
        }
    }

    // online softmax (log2 domain) for this lane's query, lazy rescaling
    float mx = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < H2; ++h2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[h2][r]);
    mx = row_halves_max(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m + RESCALE_LOG2)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = mnew == -INFINITY ? 1.f : exp2_fast(m - mnew);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      lsum *= alpha;
      m = mnew;
    }
    const float mref = m == -INFINITY ? 0.f : m;
    bf16x8 pf[2 * H2];
    float rs = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < H2; ++h2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(s[h2][r] * scale_log2 - mref);
        rs += p;
        pf[h2 * 2 + (r >> 3)][r & 7] = (bf16)p;
      }
    lsum += rs;

    // O^T[d][q] += sum_key V^T[d][key] P^T[key][q]
#pragma unroll
    for (int t = 0; t < 2 * H2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = mfma32(swz_frag_rows<D>(Vs, db * 32, t, lane), pf[t], o[db]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (!active) return;

  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / lt;
  if constexpr (STAGE) {
    // Through the K/V buffer the last block did not use (idle since the
    // last barrier): whole-row stores.
    bf16* ot = wave_tile(nblk & 1);
    stage_acc_rows<D>(ot, o, inv, lane);
    store_tile_rows<D>(out + (size_t)q0 * qstride + (size_t)head * D, qstride, q1 - q0, ot, lane);
  } else if (qrow < q1) {
    bf16* op = out + (size_t)qrow * qstride + (size_t)head * D + lh * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_bf16x4(op + db * 32 + j * 8, o[db][4 * j] * inv, o[db][4 * j + 1] * inv,
                     o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv);
  }
  if (lh == 0 && qrow < q1) lse[(size_t)head * T + qrow] = (m + log2_fast(lt)) * LN2;
}

template <int D, bool CAP>
void launch_fwd_kernel(unsigned grid, hipStream_t stream, const void* q, const void* k,
                       const void* v, const char* ws, const WorkspaceLayout& w, const Problem& p,
                       void* out, float* lse) {
  const CapConstants cc = cap_constants(p);
  // capped scores arrive in log2 units already: unit scale
  hipLaunchKernelGGL((fwd_kernel<D, CAP>), dim3(grid), dim3(FWD_THREADS), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), reinterpret_cast<const Tile*>(ws + w.tiles_fwd), (int)w.tile_cap,
                     p.total_tokens, p.num_q_heads, p.num_kv_heads, p.window, p.band,
                     CAP ? 1.f : p.scale * LOG2E,
                     cc.cap_a, cc.cap_c2, static_cast<bf16*>(out), lse);
}

template <int D>
void launch_fwd_dim(unsigned grid, hipStream_t stream, const void* q, const void* k,
                    const void* v, const char* ws, const WorkspaceLayout& w, const Problem& p,
                    void* out, float* lse) {
  if (p.softcap > 0.f)
    launch_fwd_kernel<D, true>(grid, stream, q, k, v, ws, w, p, out, lse);
  else
    launch_fwd_kernel<D, false>(grid, stream, q, k, v, ws, w, p, out, lse);
}

}  // namespace

hipError_t launch_forward(const void* q, const void* k, const void* v, const Problem& p,
                          void* out, float* lse, void* workspace, const WorkspaceLayout& w,
                          hipStream_t stream) {
  const char* ws = static_cast<const char*>(workspace);
  const unsigned grid = run_grid(head_chunks(p.num_q_heads, p.num_kv_heads), w.tile_cap,
                                 run_length(p.window));
  switch (p.head_dim) {
    case 64: launch_fwd_dim<64>(grid, stream, q, k, v, ws, w, p, out, lse); break;
    case 128: launch_fwd_dim<128>(grid, stream, q, k, v, ws, w, p, out, lse); break;
    case 256: launch_fwd_dim<256>(grid, stream, q, k, v, ws, w, p, out, lse); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
