// Block pooling, pooled block scores, per-query-block top-k selection and
// pooled attention masses.
//
// Scoring follows the project page's "learned top-k selection" and the
// abstract's "dynamically selected local neighborhood", read as: score of
// local block l for query block i = softmax_scale * mean(q over i) . mean(k
// over l); the K best local blocks (exact ties to the lower logical index,
// oldest chunk first) are attended.  The masses feed the persistent update:
// for each query block a softmax of the same pooled scores over valid
// persistent slots and all local blocks, summed over query blocks.
//
// Memory-bound: pooling reads Q and the local K once (coalesced row
// segments); scoring works on the pooled fp32 vectors, which stay in L2.
#include "common.h"

namespace pbsa {
namespace {

constexpr int kThreads = 256;

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  __device__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <> struct Vec4<bf16_t> {
  __device__ static float4 load(const bf16_t* p) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
};

// Mean of `len` rows (row(i) gives the row index) of a [*, D] tensor, written
// to out[D].  Fixed summation order: each thread sums rows rg, rg+nrg, ...;
// the row groups are then added in order 0..nrg-1; the sum is divided by len
// (0 rows give 0).
template <typename T, typename RowFn>
__device__ void pool_rows(const T* base, int D, int len, RowFn row, float* red /* [nrg][D] */,
                          float* out) {
  const int ncg = D / 4;              // column groups of 4 elements
  const int nrg = kThreads / ncg;     // row groups
  const int cg = threadIdx.x % ncg, rg = threadIdx.x / ncg;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = rg; i < len; i += nrg) {
    float4 v = Vec4<T>::load(base + (size_t)row(i) * D + cg * 4);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  float* r = red + rg * D + cg * 4;
  r[0] = acc.x;
  r[1] = acc.y;
  r[2] = acc.z;
  r[3] = acc.w;
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float s = 0.f;
    for (int k = 0; k < nrg; ++k) s += red[k * D + d];
    out[d] = len > 0 ? s / (float)len : 0.f;
  }
}

// grid (nq + nl, H, B): query block means -> qbar, local block means -> kbar_l.
template <typename T>
__global__ __launch_bounds__(kThreads) void pool_blocks_kernel(Geo g, const T* __restrict__ q,
                                                               const T* __restrict__ kl, float* __restrict__ qbar,
                                                               float* __restrict__ kbar_l) {
  __shared__ float red[kThreads * 4];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  const bool is_q = j < g.nq;
  const int p = is_q ? j : j - g.nq;
  const int off = is_q ? 0 : (p / g.nq) * g.ct;
  const BlockExt e = block_ext(g, p % g.nq);
  const T* base = is_q ? q + bh * g.ct * g.D : kl + bh * (size_t)g.NL * g.D;
  float* out = is_q ? qbar + (bh * g.nq + p) * g.D : kbar_l + (bh * g.nl + p) * g.D;
  pool_rows<T>(base, g.D, e.len, [&](int i) { return off + block_token(g, e, i); }, red, out);
}

// grid (S, H, B): mean of each slot's first len rows (0 for empty slots).
template <typename T>
__global__ __launch_bounds__(kThreads) void pool_slots_kernel(Geo g, const T* __restrict__ kp,
                                                              const int32_t* __restrict__ plen,
                                                              float* __restrict__ kbar) {
  __shared__ float red[kThreads * 4];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bhs = ((size_t)b * g.H + h) * g.S + s;
  const int len = min(max(plen[bhs], 0), g.C);
  pool_rows<T>(kp + bhs * g.C * g.D, g.D, len, [](int i) { return i; }, red, kbar + bhs * g.D);
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ float block_reduce(float v, float* sh, bool is_max) {
  // fixed-order tree within each wave, then waves 0..3 in order
  for (int o = 32; o > 0; o >>= 1) {
    float w = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  const int wid = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[wid] = v;
  __syncthreads();
  float r = sh[0];
  for (int k = 1; k < kThreads / 64; ++k) r = is_max ? fmaxf(r, sh[k]) : r + sh[k];
  return r;
}

// grid (nq, H, B): scores of one query block against every local block and
// every valid persistent slot; top-k selection; one pooled softmax row.
__global__ __launch_bounds__(kThreads) void score_topk_kernel(Geo g, const int32_t* __restrict__ ring_head,
                                                              const float* __restrict__ qbar,
                                                              const float* __restrict__ kbar_l,
                                                              const float* __restrict__ kbar_p,
                                                              const int32_t* __restrict__ plen,
                                                              int32_t* __restrict__ topk,
                                                              float* __restrict__ prow) {
  extern __shared__ float smem[];
  float* qb = smem;                 // [D]
  float* sl = qb + g.D;             // [nl]   local scores
  float* sp = sl + g.nl;            // [S]    persistent scores (-inf if empty)
  int* sel = (int*)(sp + g.S);      // [nl]   selected flags
  __shared__ float red[kThreads / 64];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = kThreads / 64;
  for (int d = threadIdx.x; d < g.D; d += kThreads) qb[d] = qbar[(bh * g.nq + i) * g.D + d];
  __syncthreads();
  const int rh = *ring_head;
  // dot products: one wave per candidate, lanes split the head dimension
  for (int c = wid; c < g.nl + g.S; c += nw) {
    const bool loc = c < g.nl;
    const int idx = loc ? c : c - g.nl;
    if (!loc && plen[bh * g.S + idx] <= 0) {
      if (lane == 0) sp[idx] = -INFINITY;
      continue;
    }
    const float* kv = loc ? kbar_l + (bh * g.nl + idx) * g.D : kbar_p + (bh * g.S + idx) * g.D;
    float part = 0.f;
    for (int d = lane; d < g.D; d += 64) part = fmaf(qb[d], kv[d], part);
    part = wave_sum(part) * g.scale;
    if (lane == 0) (loc ? sl : sp)[idx] = part;
  }
  __syncthreads();
  // top-k by rank: rank(p) = #candidates strictly better (higher score, or
  // equal score and lower logical index)
  for (int p = threadIdx.x; p < g.nl; p += kThreads) {
    const float mine = sl[p];
    const int cp = p / g.nq;
    const int lp = ((cp - rh) % g.R + g.R) % g.R * g.nq + (p - cp * g.nq);
    int rank = 0;
    for (int o = 0; o < g.nl; ++o) {
      const float x = sl[o];
      const int co = o / g.nq;
      const int lo = ((co - rh) % g.R + g.R) % g.R * g.nq + (o - co * g.nq);
      rank += (x > mine) || (x == mine && lo < lp);
    }
    sel[p] = rank < g.K;
  }
  __syncthreads();
  int32_t* out = topk + (bh * g.nq + i) * g.K;
  for (int p = threadIdx.x; p < g.nl; p += kThreads) {
    if (!sel[p]) continue;
    int pos = 0;
    for (int o = 0; o < p; ++o) pos += sel[o];
    out[pos] = p;
  }
  // pooled softmax over valid slots and all local blocks
  float mx = -INFINITY;
  for (int c = threadIdx.x; c < g.nl + g.S; c += kThreads) mx = fmaxf(mx, c < g.nl ? sl[c] : sp[c - g.nl]);
  mx = block_reduce(mx, red, true);
  float sum = 0.f;
  for (int c = threadIdx.x; c < g.nl + g.S; c += kThreads) {
    const float x = c < g.nl ? sl[c] : sp[c - g.nl];
    sum += x == -INFINITY ? 0.f : expf(x - mx);
  }
  sum = block_reduce(sum, red, false);
  float* row = prow + (bh * g.nq + i) * (size_t)(g.S + g.nl);
  for (int c = threadIdx.x; c < g.nl + g.S; c += kThreads) {
    const float x = c < g.nl ? sl[c] : sp[c - g.nl];
    const float pv = x == -INFINITY ? 0.f : expf(x - mx) / sum;
    row[c < g.nl ? g.S + c : c - g.nl] = pv;
  }
}

// grid (ceil((S+nl)/256), H, B): mass[j] = sum over query blocks, in order.
__global__ __launch_bounds__(kThreads) void mass_kernel(Geo g, const float* __restrict__ prow,
                                                        float* __restrict__ mass) {
  const int j = blockIdx.x * kThreads + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int W = g.S + g.nl;
  if (j >= W) return;
  const size_t bh = (size_t)b * g.H + h;
  const float* r = prow + bh * g.nq * (size_t)W + j;
  float s = 0.f;
  for (int i = 0; i < g.nq; ++i) s += r[(size_t)i * W];
  mass[bh * W + j] = s;
}

}  // namespace

hipError_t launch_pool_slots(const Geo& g, const void* k_p, const int32_t* plen, float* kbar, hipStream_t s) {
  dim3 grid(g.S, g.H, g.B);
  if (g.dtype == PBSA_BF16)
    pool_slots_kernel<bf16_t><<<grid, kThreads, 0, s>>>(g, (const bf16_t*)k_p, plen, kbar);
  else
    pool_slots_kernel<float><<<grid, kThreads, 0, s>>>(g, (const float*)k_p, plen, kbar);
  return hipGetLastError();
}

hipError_t launch_score_select(const Geo& g, const void* q, const void* k_l, const int32_t* ring_head,
                               const float* kbar_p, const int32_t* plen, int32_t* topk, float* mass,
                               float* kbar_l, WsScore ws, hipStream_t s) {
  dim3 g1(g.nq + g.nl, g.H, g.B);
  if (g.dtype == PBSA_BF16)
    pool_blocks_kernel<bf16_t><<<g1, kThreads, 0, s>>>(g, (const bf16_t*)q, (const bf16_t*)k_l, ws.qbar, kbar_l);
  else
    pool_blocks_kernel<float><<<g1, kThreads, 0, s>>>(g, (const float*)q, (const float*)k_l, ws.qbar, kbar_l);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  size_t shm = (size_t)(g.D + g.nl + g.S) * 4 + (size_t)g.nl * 4;
  score_topk_kernel<<<dim3(g.nq, g.H, g.B), kThreads, shm, s>>>(g, ring_head, ws.qbar, kbar_l, kbar_p, plen, topk,
                                                               ws.prow);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mass_kernel<<<dim3((g.S + g.nl + kThreads - 1) / kThreads, g.H, g.B), kThreads, 0, s>>>(g, ws.prow, mass);
  return hipGetLastError();
}

}  // namespace pbsa
