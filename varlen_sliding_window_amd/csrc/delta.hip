// Gated delta-rule linear attention (Gated DeltaNet), forward, chunked.
//
// The kernel benchmarks page (research.dws.rip/llm/kernels, section 03 "What
// linear attention costs") times Gated DeltaNet as the competing local
// layer.  Per head, a d_v x d_k state S, reset at every document start:
//   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
//   o_t = scale S_t q_t,  alpha_t = exp(g_t).
// Over a chunk of C tokens with in-chunk cumulative log decay G_i (gamma_i =
// exp(G_i)), the state is S_i = gamma_i S_0 + sum_{j <= i} exp(G_i - G_j)
// u_j k_j^T with pseudo-values u solving the unit lower-triangular system
//   (I + A) U = diag(beta) V - diag(beta gamma) K S_0^T,
//   A_ij = beta_i exp(G_i - G_j) (k_i . k_j)  (j < i),
// so U = U0 - W S_0^T with W and U0 the solutions for the right-hand sides
// diag(beta gamma) K and diag(beta) V, which do not depend on S_0.  Then
//   O = scale (diag(gamma) Q S_0^T + (Gamma o Q K^T)_{j <= i} U)
//   S_C = gamma_C S_0 + U^T diag(exp(G_C - G)) K.
// delta_prep_kernel forms W, U0, the masked decayed scores P and the decays
// of every (chunk, head) in parallel; delta_scan_kernel then walks each
// document's chunks in order carrying S, one work-group per (document, head,
// slice of d_v): the rows of S, the columns of U and of O of different d_v
// indices never mix.  Everything is fp32 arithmetic on the vector ALU.
#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int DC = DELTA_CHUNK;       // tokens per chunk
constexpr int DD = DELTA_DIM;         // d_k = d_v
constexpr int PLAN_THREADS = 1024;
constexpr int PREP_THREADS = 256;
constexpr int SCAN_THREADS = 512;
constexpr int SLICE = 32;             // d_v columns per scan work-group
constexpr int LP = DD + 1;            // LDS pitch of DD-wide fp32 rows

__device__ __forceinline__ float bf(const bf16 x) { return (float)x; }

// Chunks per segment -> exclusive offsets; header[0] = chunk count.
__global__ __launch_bounds__(PLAN_THREADS) void delta_plan_kernel(const int32_t* __restrict__ cu,
                                                                   int nseq, int T, int chunk_cap,
                                                                   int* __restrict__ header,
                                                                   int* __restrict__ seg_off) {
  __shared__ int part[PLAN_THREADS];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nseq; base += PLAN_THREADS) {
    const int s = base + (int)threadIdx.x;
    int n = 0;
    if (s < nseq) {
      const int a = min(max(cu[s], 0), T);
      const int b = min(max(cu[s + 1], a), T);
      n = (b - a + DC - 1) / DC;
    }
    part[threadIdx.x] = n;
    __syncthreads();
    // Hillis-Steele inclusive scan over the block
    for (int off = 1; off < PLAN_THREADS; off <<= 1) {
      const int add = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (s < nseq) seg_off[s] = carry + part[threadIdx.x] - n;
    __syncthreads();
    if (threadIdx.x == PLAN_THREADS - 1) carry += part[PLAN_THREADS - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int total = min(carry, chunk_cap);
    seg_off[nseq] = total;
    header[0] = total;
    header[1] = T;
  }
}

// One record per (chunk, head): W [DC][DD], U0 [DC][DD], P [DC][DC], gamma
// [DC], decay to the chunk end [DC], fp32.
struct DeltaRecord {
  static constexpr size_t W = 0;
  static constexpr size_t U0 = W + (size_t)DC * DD;
  static constexpr size_t P = U0 + (size_t)DC * DD;
  static constexpr size_t GAM = P + (size_t)DC * DC;
  static constexpr size_t END = GAM + DC;
  static constexpr size_t FLOATS = END + DC;
};

__global__ __launch_bounds__(PREP_THREADS) void delta_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int nseq, int T, int H, const int* __restrict__ header, const int* __restrict__ seg_off,
    float* __restrict__ records) {
  constexpr int BP = DD + 8;   // bf16 row pitch (16 bytes of padding)
  __shared__ __attribute__((aligned(16))) bf16 Ks[DC * BP];
  __shared__ __attribute__((aligned(16))) bf16 Qs[DC * BP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[DC * BP];
  __shared__ float As[DC * (DC + 1)];   // A, then T = (I + A)^-1 in place
  __shared__ float Gs[DC], Bs[DC];
  const int chunk = blockIdx.x / H, h = blockIdx.x - chunk * H;
  if (chunk >= header[0]) return;
  // segment of this chunk: largest s with seg_off[s] <= chunk
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_off[mid] <= chunk) lo = mid; else hi = mid - 1;
  }
  const int a = min(max(cu[lo], 0), T);
  const int b = min(max(cu[lo + 1], a), T);
  const int c0 = a + (chunk - seg_off[lo]) * DC;
  const int n = max(0, min(DC, b - c0));
  const int tid = threadIdx.x;
  const size_t rs = (size_t)H * DD;   // token stride of q, k, v

  // q and k rows, 16 bytes per lane (rows past the chunk are zero)
#pragma unroll
  for (int r = 0; r < DC * DD / 8 / PREP_THREADS; ++r) {
    const int f = tid + PREP_THREADS * r, i = f / (DD / 8), ch = f % (DD / 8);
    const size_t off = (size_t)(c0 + i) * rs + (size_t)h * DD + ch * 8;
    const uint4 z = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(Ks + i * BP + ch * 8) = i < n ? *reinterpret_cast<const uint4*>(k + off) : z;
    *reinterpret_cast<uint4*>(Qs + i * BP + ch * 8) = i < n ? *reinterpret_cast<const uint4*>(q + off) : z;
    *reinterpret_cast<uint4*>(Vs + i * BP + ch * 8) = i < n ? *reinterpret_cast<const uint4*>(v + off) : z;
  }
  if (tid < DC) {
    const bool in = tid < n;
    Gs[tid] = in ? g[(size_t)(c0 + tid) * H + h] : 0.f;
    Bs[tid] = in ? beta[(size_t)(c0 + tid) * H + h] : 0.f;
  }
  __syncthreads();
  if (tid == 0) {   // in-chunk cumulative log decay
    float acc = 0.f;
    for (int i = 0; i < DC; ++i) {
      acc += Gs[i];
      Gs[i] = acc;
    }
  }
  __syncthreads();
  float* rec = records + (size_t)blockIdx.x * DeltaRecord::FLOATS;
  // Gram products, a 4 x 4 block of (row, column) pairs per thread: A from
  // K K^T (strictly below the diagonal), P from Q K^T (on and below it).
  {
    const int i0 = (tid / 16) * 4, j0 = (tid % 16) * 4;
    float kk[4][4] = {}, qk[4][4] = {};
    for (int d = 0; d < DD; d += 8) {
      bf16x8 ki[4], qi[4], kj[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        ki[x] = *reinterpret_cast<const bf16x8*>(Ks + (i0 + x) * BP + d);
        qi[x] = *reinterpret_cast<const bf16x8*>(Qs + (i0 + x) * BP + d);
        kj[x] = *reinterpret_cast<const bf16x8*>(Ks + (j0 + x) * BP + d);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            kk[x][y] += (float)ki[x][e] * (float)kj[y][e];
            qk[x][y] += (float)qi[x][e] * (float)kj[y][e];
          }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = i0 + x, j = j0 + y;
        const float dec = j <= i ? __expf(Gs[i] - Gs[j]) : 0.f;
        As[i * (DC + 1) + j] = j < i ? Bs[i] * dec * kk[x][y] : 0.f;
        rec[DeltaRecord::P + i * DC + j] = j <= i ? dec * qk[x][y] : 0.f;
      }
  }
  if (tid < DC) {
    rec[DeltaRecord::GAM + tid] = __expf(Gs[tid]);
    const int last = n > 0 ? n - 1 : 0;
    rec[DeltaRecord::END + tid] = tid < n ? __expf(Gs[last] - Gs[tid]) : 0.f;
  }
  __syncthreads();
  // T = (I + A)^-1, unit lower triangular, row by row in place of A: for
  // c < i, T_ic = -A_ic - sum_{c < j < i} A_ij T_jc (thread c).  Row i reads
  // its own A entries and the finished rows j < i, and is written only after
  // every thread of the row has read it.
  for (int i = 1; i < DC; ++i) {
    float acc = 0.f;
    if (tid < i) {
      const int c = tid;
      // four interleaved partial sums shorten the dependent chain
      float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
      int j = c + 1;
      for (; j + 3 < i; j += 4) {
        p0 += As[i * (DC + 1) + j] * As[j * (DC + 1) + c];
        p1 += As[i * (DC + 1) + j + 1] * As[(j + 1) * (DC + 1) + c];
        p2 += As[i * (DC + 1) + j + 2] * As[(j + 2) * (DC + 1) + c];
        p3 += As[i * (DC + 1) + j + 3] * As[(j + 3) * (DC + 1) + c];
      }
      for (; j < i; ++j) p0 += As[i * (DC + 1) + j] * As[j * (DC + 1) + c];
      acc = -As[i * (DC + 1) + c] - ((p0 + p1) + (p2 + p3));
    }
    __syncthreads();
    if (tid < i) As[i * (DC + 1) + tid] = acc;
    __syncthreads();
  }
  // W = T diag(beta gamma) K and U0 = T diag(beta) V: thread (4 rows, 8
  // columns) of each, T's diagonal being 1.
  {
    const int i0 = (tid / 16) * 4, d8 = (tid % 16) * 8;
    float w[4][8] = {}, u[4][8] = {};
    for (int j = 0; j < DC; ++j) {
      const float sw = Bs[j] * __expf(Gs[j]), su = Bs[j];
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(Ks + j * BP + d8);
      const bf16x8 vv = *reinterpret_cast<const bf16x8*>(Vs + j * BP + d8);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int i = i0 + x;
        const float t = j < i ? As[i * (DC + 1) + j] : (j == i ? 1.f : 0.f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          w[x][e] += t * sw * (float)kv[e];
          u[x][e] += t * su * (float)vv[e];
        }
      }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      float4* dw = reinterpret_cast<float4*>(rec + DeltaRecord::W + (i0 + x) * DD + d8);
      float4* du = reinterpret_cast<float4*>(rec + DeltaRecord::U0 + (i0 + x) * DD + d8);
      dw[0] = make_float4(w[x][0], w[x][1], w[x][2], w[x][3]);
      dw[1] = make_float4(w[x][4], w[x][5], w[x][6], w[x][7]);
      du[0] = make_float4(u[x][0], u[x][1], u[x][2], u[x][3]);
      du[1] = make_float4(u[x][4], u[x][5], u[x][6], u[x][7]);
    }
  }
}

// Walks a document's chunks in order for one head and a slice of SLICE d_v
// columns, carrying those rows of S in LDS.  The next chunk's record and q/k
// rows are loaded into registers while the current chunk computes.
__global__ __launch_bounds__(SCAN_THREADS) void delta_scan_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const int32_t* __restrict__ cu,
    int nseq, int T, int H, float scale, const int* __restrict__ seg_off,
    const float* __restrict__ records, bf16* __restrict__ out) {
  constexpr int SL = DD / SLICE;       // slices per head
  constexpr int BP = DD + 8;           // bf16 row pitch (16 bytes of padding)
  __shared__ float Ss[SLICE * LP];     // S rows c0 .. c0 + SLICE - 1, all d_k
  __shared__ float Ws[DC * LP];
  __shared__ __attribute__((aligned(16))) bf16 Qs[DC * BP];
  __shared__ __attribute__((aligned(16))) bf16 Ks[DC * BP];
  __shared__ float Ps[DC * (DC + 1)];
  __shared__ float U0s[DC * (SLICE + 1)];
  __shared__ float Us[DC * (SLICE + 1)];
  __shared__ float QSs[DC * (SLICE + 1)];
  __shared__ float Gm[DC], En[DC];
  const int sl = blockIdx.x % SL;
  const int h = (blockIdx.x / SL) % H;
  const int s = blockIdx.x / (SL * H);
  if (s >= nseq) return;
  const int a = min(max(cu[s], 0), T);
  const int b = min(max(cu[s + 1], a), T);
  // seg_off[nseq] holds the chunk total, cut to the workspace's capacity
  const int total = seg_off[nseq];
  const int first = min(seg_off[s], total);
  const int count = max(0, min(seg_off[s + 1], total) - first);
  const int tid = threadIdx.x;
  const int cbase = sl * SLICE;
  const size_t rs = (size_t)H * DD;
  for (int e = tid; e < SLICE * LP; e += SCAN_THREADS) Ss[e] = 0.f;

  // register staging of one chunk: W, P, q and k rows, the slice of U0 and
  // gamma / end decay, spread over the work-group's threads
  constexpr int NT = SCAN_THREADS;
  constexpr int WR = DC * DD / 4 / NT, PR = DC * DC / 4 / NT, QR = DC * DD / 8 / NT;
  float4 wr[WR], pr[PR], ur = make_float4(0.f, 0.f, 0.f, 0.f);
  uint4 qr[QR], kr[QR];
  float gr = 0.f;
  auto fetch = [&](int ci) {
    const int c0 = a + ci * DC;
    const int n = min(DC, b - c0);
    const float* rec = records + ((size_t)(first + ci) * H + h) * DeltaRecord::FLOATS;
    const float4* r4 = reinterpret_cast<const float4*>(rec);
#pragma unroll
    for (int r = 0; r < WR; ++r) wr[r] = r4[DeltaRecord::W / 4 + tid + NT * r];
#pragma unroll
    for (int r = 0; r < PR; ++r) pr[r] = r4[DeltaRecord::P / 4 + tid + NT * r];
#pragma unroll
    for (int r = 0; r < QR; ++r) {
      const int f = tid + NT * r, i = f / (DD / 8), ch = f % (DD / 8);
      const size_t off = (size_t)(c0 + i) * rs + (size_t)h * DD + ch * 8;
      qr[r] = i < n ? *reinterpret_cast<const uint4*>(q + off) : make_uint4(0, 0, 0, 0);
      kr[r] = i < n ? *reinterpret_cast<const uint4*>(k + off) : make_uint4(0, 0, 0, 0);
    }
    if (tid < DC * SLICE / 4)
      ur = r4[(DeltaRecord::U0 + (size_t)(tid / (SLICE / 4)) * DD + cbase) / 4 + (tid % (SLICE / 4))];
    gr = tid < DC ? rec[DeltaRecord::GAM + tid] : (tid < 2 * DC ? rec[DeltaRecord::END + tid - DC] : 0.f);
  };
  if (count > 0) fetch(0);

  for (int ci = 0; ci < count; ++ci) {
    const int c0 = a + ci * DC;
    const int n = min(DC, b - c0);
    __syncthreads();   // every read of the previous chunk's LDS data is done
#pragma unroll
    for (int r = 0; r < WR; ++r) {
      const int f = tid + NT * r, i = f / (DD / 4), c4 = (f % (DD / 4)) * 4;
      Ws[i * LP + c4] = wr[r].x;
      Ws[i * LP + c4 + 1] = wr[r].y;
      Ws[i * LP + c4 + 2] = wr[r].z;
      Ws[i * LP + c4 + 3] = wr[r].w;
    }
#pragma unroll
    for (int r = 0; r < PR; ++r) {
      const int f = tid + NT * r, pi = f / (DC / 4), pj = (f % (DC / 4)) * 4;
      Ps[pi * (DC + 1) + pj] = pr[r].x;
      Ps[pi * (DC + 1) + pj + 1] = pr[r].y;
      Ps[pi * (DC + 1) + pj + 2] = pr[r].z;
      Ps[pi * (DC + 1) + pj + 3] = pr[r].w;
    }
#pragma unroll
    for (int r = 0; r < QR; ++r) {
      const int f = tid + NT * r, i = f / (DD / 8), ch = f % (DD / 8);
      *reinterpret_cast<uint4*>(Qs + i * BP + ch * 8) = qr[r];
      *reinterpret_cast<uint4*>(Ks + i * BP + ch * 8) = kr[r];
    }
    if (tid < DC * SLICE / 4) {
      const int i = tid / (SLICE / 4), c4 = (tid % (SLICE / 4)) * 4;
      U0s[i * (SLICE + 1) + c4] = ur.x;
      U0s[i * (SLICE + 1) + c4 + 1] = ur.y;
      U0s[i * (SLICE + 1) + c4 + 2] = ur.z;
      U0s[i * (SLICE + 1) + c4 + 3] = ur.w;
    }
    if (tid < DC) Gm[tid] = gr;
    else if (tid < 2 * DC) En[tid - DC] = gr;
    __syncthreads();
    if (ci + 1 < count) fetch(ci + 1);

    // U = U0 - W S^T and Q S^T: thread (row i, CPT slice columns)
    constexpr int CPT = DC * SLICE / NT;          // columns per thread
    const int i = tid / (SLICE / CPT), cc = (tid % (SLICE / CPT)) * CPT;
    {
      float ws[CPT] = {}, qs[CPT] = {};
      for (int d = 0; d < DD; ++d) {
        const float w = Ws[i * LP + d];
        const float qv = (float)Qs[i * BP + d];
#pragma unroll
        for (int x = 0; x < CPT; ++x) {
          const float sv = Ss[(cc + x) * LP + d];
          ws[x] += w * sv;
          qs[x] += qv * sv;
        }
      }
#pragma unroll
      for (int x = 0; x < CPT; ++x) {
        Us[i * (SLICE + 1) + cc + x] = U0s[i * (SLICE + 1) + cc + x] - ws[x];
        QSs[i * (SLICE + 1) + cc + x] = qs[x];
      }
    }
    __syncthreads();
    // O = scale (gamma Q S^T + P U) for the chunk's rows inside the document
    if (i < n) {
      float acc[CPT];
#pragma unroll
      for (int x = 0; x < CPT; ++x) acc[x] = Gm[i] * QSs[i * (SLICE + 1) + cc + x];
      for (int j = 0; j <= i; ++j) {
        const float p = Ps[i * (DC + 1) + j];
#pragma unroll
        for (int x = 0; x < CPT; ++x) acc[x] += p * Us[j * (SLICE + 1) + cc + x];
      }
      bf16* op = out + (size_t)(c0 + i) * rs + (size_t)h * DD + cbase + cc;
#pragma unroll
      for (int x = 0; x < CPT; ++x) op[x] = (bf16)(scale * acc[x]);
    }
    // S_C = gamma_C S + U^T diag(end decay) K: thread (row c, DPT columns of d)
    {
      constexpr int DPT = SLICE * DD / NT;
      const int c = tid / (DD / DPT), d0 = (tid % (DD / DPT)) * DPT;
      float acc[DPT] = {};
      for (int j = 0; j < n; ++j) {
        const float u = Us[j * (SLICE + 1) + c] * En[j];
#pragma unroll
        for (int y = 0; y < DPT; ++y) acc[y] += u * (float)Ks[j * BP + d0 + y];
      }
      const float gc = Gm[n - 1];
      // each thread updates only its own entries of S, and every read of S
      // in this chunk came before the last barrier
#pragma unroll
      for (int y = 0; y < DPT; ++y) Ss[c * LP + d0 + y] = gc * Ss[c * LP + d0 + y] + acc[y];
    }
  }
}

}  // namespace

hipError_t launch_delta_fwd(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens, int num_seqs,
                            int total_tokens, int num_heads, float scale, void* out,
                            void* workspace, const DeltaLayout& w, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  int* header = reinterpret_cast<int*>(ws + w.header);
  int* seg_off = reinterpret_cast<int*>(ws + w.seg_off);
  float* records = reinterpret_cast<float*>(ws + w.records);
  hipLaunchKernelGGL(delta_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, cu_seqlens,
                     num_seqs, total_tokens, (int)w.chunk_cap, header, seg_off);
  hipLaunchKernelGGL(delta_prep_kernel, dim3((unsigned)(w.chunk_cap * (size_t)num_heads)),
                     dim3(PREP_THREADS), 0, stream, static_cast<const bf16*>(q),
                     static_cast<const bf16*>(k), static_cast<const bf16*>(v), g, beta,
                     cu_seqlens, num_seqs, total_tokens, num_heads, header, seg_off, records);
  hipLaunchKernelGGL(delta_scan_kernel,
                     dim3((unsigned)((size_t)num_seqs * num_heads * (DD / SLICE))),
                     dim3(SCAN_THREADS), 0, stream, static_cast<const bf16*>(q),
                     static_cast<const bf16*>(k), cu_seqlens, num_seqs, total_tokens, num_heads,
                     scale, seg_off, records, static_cast<bf16*>(out));
  return hipGetLastError();
}

}  // namespace attn
