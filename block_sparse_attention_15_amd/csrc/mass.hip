// Token-exact attention mass per candidate block.
//
// The abstract of Sparse Forcing has the persistent memory keep the blocks
// that matter most to the current queries; besides the pooled-score mass of
// the selection step, the library offers the mass taken from the attention
// itself: block j receives, from every query token t of the chunk, the
// probability that t's softmax (persistent rows plus its query block's
// selected local blocks) puts on j's rows.
//
// The forward leaves, for every query t and every block j it attends, the
// log-sum-exp of t's scores over j's rows (blse, base 2); with t's full
// log-sum-exp (lse, natural log) that probability is 2^(blse - lse*log2 e).
// Three small HBM-bound kernels reduce it, in a fixed order (no atomics, so
// the result is deterministic):
//   * tmass_pers: one workgroup per (slot, head, batch) sums over the chunk's
//     queries;
//   * tmass_part: one workgroup per (query block, head, batch) sums over the
//     block's queries for each of its K selections, then scatters the K sums
//     to a dense row part[i][p] (zeros elsewhere);
//   * tmass_local: one thread per (local block, head, batch) adds its column
//     of part over the query blocks, ascending (loads issued eight at a time).
#include "common.h"

namespace pbsa {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void tmass_pers_kernel(Geo g, const int32_t* __restrict__ plen,
                                                              const float* __restrict__ lse,
                                                              const float* __restrict__ blse_p,
                                                              float* __restrict__ mass) {
  __shared__ float red[kThreads / 64];
  const int s = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * g.H + blockIdx.y;
  const float* bl = blse_p + (bh * g.S + s) * g.ct;
  const float* ls = lse + bh * g.ct;
  float acc = 0.f;
  if (plen[bh * g.S + s] > 0)
    for (int t = threadIdx.x; t < g.ct; t += kThreads) acc += exp2f(bl[t] - ls[t] * kLog2e);
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
    mass[bh * (g.S + g.nl) + s] = tot;
  }
}

constexpr int kMaxBlocks = 2048;  // plan limit on K and on local blocks

__global__ __launch_bounds__(kThreads) void tmass_part_kernel(Geo g, const int32_t* __restrict__ topk,
                                                              const float* __restrict__ lse,
                                                              const float* __restrict__ blse_l,
                                                              float* __restrict__ part) {
  __shared__ float sums[kMaxBlocks];
  __shared__ float row[kMaxBlocks];
  const int i = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * g.H + blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int x = threadIdx.x; x < g.nl; x += kThreads) row[x] = 0.f;
  const BlockExt e = block_ext(g, i);
  const float* ls = lse + bh * g.ct;
  for (int k = wave; k < g.K; k += kThreads / 64) {
    const float* bl = blse_l + (bh * g.K + k) * g.ct;
    float acc = 0.f;
    for (int r = lane; r < e.len; r += 64) {
      const int t = block_token(g, e, r);
      acc += exp2f(bl[t] - ls[t] * kLog2e);
    }
    acc = wave_sum(acc);
    if (lane == 0) sums[k] = acc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // sequential: a block listed twice accumulates both parts
    const int32_t* sel = topk + (bh * g.nq + i) * g.K;
    for (int k = 0; k < g.K; ++k) {
      const int p = sel[k];
      if ((unsigned)p < (unsigned)g.nl) row[p] += sums[k];
    }
  }
  __syncthreads();
  float* out = part + (bh * g.nq + i) * g.nl;
  for (int x = threadIdx.x; x < g.nl; x += kThreads) out[x] = row[x];
}

constexpr int kLocalThreads = 64;

__global__ __launch_bounds__(kLocalThreads) void tmass_local_kernel(Geo g, const float* __restrict__ part,
                                                                    float* __restrict__ mass) {
  const int p = blockIdx.x * kLocalThreads + threadIdx.x;
  const size_t bh = blockIdx.y;
  if (p >= g.nl) return;
  const float* col = part + bh * g.nq * (size_t)g.nl + p;
  float acc = 0.f;
  int i = 0;
  for (; i + 8 <= g.nq; i += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = col[(size_t)(i + u) * g.nl];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; i < g.nq; ++i) acc += col[(size_t)i * g.nl];
  mass[bh * (g.S + g.nl) + g.S + p] = acc;
}

}  // namespace

hipError_t launch_token_mass(const Geo& g, const int32_t* plen, const int32_t* topk, const float* lse,
                             const float* blse_p, const float* blse_l, float* part, float* mass, hipStream_t s) {
  if (g.K > kMaxBlocks || g.nl > kMaxBlocks) return hipErrorInvalidValue;
  if (g.S > 0) {
    tmass_pers_kernel<<<dim3(g.S, g.H, g.B), kThreads, 0, s>>>(g, plen, lse, blse_p, mass);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  tmass_part_kernel<<<dim3(g.nq, g.H, g.B), kThreads, 0, s>>>(g, topk, lse, blse_l, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tmass_local_kernel<<<dim3((g.nl + kLocalThreads - 1) / kLocalThreads, g.B * g.H), kLocalThreads, 0, s>>>(g, part,
                                                                                                         mass);
  return hipGetLastError();
}

}  // namespace pbsa
