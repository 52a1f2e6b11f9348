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

// Mean of `len` (<= 64) rows (row(i) gives the row index) of a [*, D]
// tensor, written to out[D].  Fixed summation order: each thread sums rows
// rg, rg+nrg, ...; the row groups are then added in order 0..nrg-1; the sum
// is divided by len (0 rows give 0).  All of a thread's row loads are issued
// before the first add.
template <int D, typename T, typename RowFn>
__device__ void pool_rows(const T* base, int len, RowFn row, float* red /* [nrg][D] */, float* out) {
  constexpr int ncg = D / 4;              // column groups of 4 elements
  constexpr int nrg = kThreads / ncg;     // row groups
  constexpr int kIt = 64 / nrg;           // rows per thread at most
  const int cg = threadIdx.x % ncg, rg = threadIdx.x / ncg;
  float4 v[kIt];
#pragma unroll
  for (int u = 0; u < kIt; ++u) {
    const int i = rg + nrg * u;
    v[u] = i < len ? Vec4<T>::load(base + (size_t)row(i) * D + cg * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kIt; ++u) {
    if (rg + nrg * u < len) {
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
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
template <int D, typename T>
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
  pool_rows<D, T>(base, e.len, [&](int i) { return off + block_token(g, e, i); }, red, out);
}

// grid (S, H, B): mean of each slot's first len rows (0 for empty slots).
template <int D, typename T>
__global__ __launch_bounds__(kThreads) void pool_slots_kernel(Geo g, const T* __restrict__ kp,
                                                              const int32_t* __restrict__ plen,
                                                              float* __restrict__ kbar) {
  __shared__ float red[kThreads * 4];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bhs = ((size_t)b * g.H + h) * g.S + s;
  const int len = min(max(plen[bhs], 0), g.C);
  pool_rows<D, T>(kp + bhs * g.C * D, len, [](int i) { return i; }, red, kbar + bhs * D);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

constexpr int kRadixSlots = 4;  // keys per lane for the radix select (local blocks <= 256)

// grid (ceil(nq/QPW), H, B): pooled scores of QPW (<= 4) query blocks against
// every local block and every valid persistent slot (each candidate's pooled
// key is read once for the QPW query blocks), then per query block (one wave)
// the top-k (a wavefront radix select up to 256 local blocks, ranks by
// counting beyond) and one pooled softmax row.  QPW is the largest of 4, 2,
// 1 whose LDS (scores, sort keys and flags of every candidate) fits.
template <int D, int kQPerWg>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(Geo g, const int32_t* __restrict__ ring_head,
                                                              const float* __restrict__ qbar,
                                                              const float* __restrict__ kbar_l,
                                                              const float* __restrict__ kbar_p,
                                                              const int32_t* __restrict__ plen,
                                                              int32_t* __restrict__ topk,
                                                              float* __restrict__ prow,
                                                              uint32_t* __restrict__ status) {
  extern __shared__ float smem[];
  const int W = g.nl + g.S;        // candidates: local blocks, then slots
  float* qb = smem;                // [4][D]
  float* sc = qb + kQPerWg * g.D;  // [4][W] scores (-inf for empty slots)
  int* sel = (int*)(sc + kQPerWg * W);  // [4][nl] 64-bit sort keys, then [4][nl] flags
  const int i0 = blockIdx.x * kQPerWg, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int x = threadIdx.x; x < kQPerWg * g.D; x += kThreads) {
    const int qi = i0 + x / g.D;
    qb[x] = qi < g.nq ? qbar[(bh * g.nq + qi) * g.D + x % g.D] : 0.f;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < W; c += kThreads) {
    const bool loc = c < g.nl;
    const int idx = loc ? c : c - g.nl;
    if (!loc && plen[bh * g.S + idx] <= 0) {
      for (int k = 0; k < kQPerWg; ++k) sc[k * W + c] = -INFINITY;
      continue;
    }
    const float4* kv = reinterpret_cast<const float4*>(loc ? kbar_l + (bh * g.nl + idx) * D
                                                           : kbar_p + (bh * g.S + idx) * D);
    float4 kr[D / 4];  // the candidate's pooled key, all loads in flight together
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4) kr[d4] = kv[d4];
    float acc[kQPerWg] = {};
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const float4 k4 = kr[d4];
#pragma unroll
      for (int k = 0; k < kQPerWg; ++k) {
        const float4 q4 = reinterpret_cast<const float4*>(qb + k * D)[d4];
        acc[k] = fmaf(q4.x, k4.x, acc[k]);
        acc[k] = fmaf(q4.y, k4.y, acc[k]);
        acc[k] = fmaf(q4.z, k4.z, acc[k]);
        acc[k] = fmaf(q4.w, k4.w, acc[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kQPerWg; ++k) sc[k * W + c] = acc[k] * g.scale;
  }
  __syncthreads();
  const int i = i0 + w;
  const bool has = w < kQPerWg && i < g.nq;
  const float* row = sc + w * W;
  unsigned long long* key = reinterpret_cast<unsigned long long*>(sel) + w * g.nl;
  const int rh = read_ring_head(ring_head, g.R, status);
  // composite key: descending score, then ascending logical index (oldest
  // chunk first); rank(p) = #local blocks with a larger key
  if (has) {
    for (int p = lane; p < g.nl; p += 64) {
      const int cp = p / g.nq;
      const unsigned lg = (unsigned)(((cp - rh) % g.R + g.R) % g.R * g.nq + (p - cp * g.nq));
      unsigned u = row[p] == 0.f ? 0u : __float_as_uint(row[p]);  // -0 ties +0
      u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // order-preserving map to unsigned
      key[p] = ((unsigned long long)u << 32) | (0xffffffffu - lg);
    }
  }
  __syncthreads();
  if (!has) return;
  int32_t* out = topk + (bh * g.nq + i) * g.K;
  if (g.nl <= 64 * kRadixSlots) {
    // wavefront radix select: the K-th largest key T, one bit at a time from
    // the top (keep the bit when at least K keys are >= the candidate), with
    // the keys in registers and the counts by ballot; the keys are distinct,
    // so exactly K are >= T
    unsigned long long kr[kRadixSlots];
#pragma unroll
    for (int u = 0; u < kRadixSlots; ++u) {
      const int p = lane + 64 * u;
      kr[u] = p < g.nl ? key[p] : 0ull;  // 0 is below every key
    }
    unsigned long long thr = 0ull;
    for (int b = 63; b >= 0; --b) {
      const unsigned long long cand = thr | (1ull << b);
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < kRadixSlots; ++u) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(kr[u] >= cand));
      if (cnt >= g.K) thr = cand;
    }
#pragma unroll
    for (int u = 0; u < kRadixSlots; ++u) {
      const int p = lane + 64 * u;
      if (p < g.nl) sel[g.nl * 2 * kQPerWg + w * g.nl + p] = kr[u] >= thr;
    }
  } else {
    // every lane ranks its own candidates against all keys (LDS broadcast reads)
    for (int p = lane; p < g.nl; p += 64) {
      const unsigned long long kp = key[p];
      int rank = 0;
      for (int o = 0; o < g.nl; ++o) rank += key[o] > kp;
      sel[g.nl * 2 * kQPerWg + w * g.nl + p] = rank < g.K;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int* sl = sel + g.nl * 2 * kQPerWg + w * g.nl;
  // ascending physical ids: position = selected count below p (ballot prefix)
  int running = 0;
  for (int p0 = 0; p0 < g.nl; p0 += 64) {
    const int p = p0 + lane;
    const bool on = p < g.nl && sl[p];
    const unsigned long long m = __builtin_amdgcn_ballot_w64(on);
    if (on) out[running + __builtin_popcountll(m & ((1ull << lane) - 1))] = p;
    running += __builtin_popcountll(m);
  }
  // pooled softmax over valid slots and all local blocks
  float mx = -INFINITY;
  for (int c = lane; c < W; c += 64) mx = fmaxf(mx, row[c]);
  mx = wave_max(mx);
  float sum = 0.f;
  for (int c = lane; c < W; c += 64) sum += row[c] == -INFINITY ? 0.f : expf(row[c] - mx);
  sum = wave_sum(sum);
  float* pr = prow + (bh * g.nq + i) * (size_t)W;
  for (int c = lane; c < W; c += 64) {
    const float x = row[c];
    pr[c < g.nl ? g.S + c : c - g.nl] = x == -INFINITY ? 0.f : expf(x - mx) / sum;
  }
}

// grid (ceil((S+nl)/64), H, B), 256 threads = 64 columns x 4 row groups:
// mass[j] = sum over query blocks; partial sums over rows rg, rg+4, ... are
// added in row-group order (fixed, deterministic).
__global__ __launch_bounds__(kThreads) void mass_kernel(Geo g, const float* __restrict__ prow,
                                                        float* __restrict__ mass) {
  __shared__ float red[4][64];
  const int W = g.S + g.nl;
  const int col = blockIdx.x * 64 + (threadIdx.x & 63), rg = threadIdx.x >> 6;
  const size_t bh = (size_t)blockIdx.z * g.H + blockIdx.y;
  float s = 0.f;
  if (col < W) {
    const float* r = prow + bh * g.nq * (size_t)W + col;
    for (int i = rg; i < g.nq; i += 4) s += r[(size_t)i * W];
  }
  red[rg][threadIdx.x & 63] = s;
  __syncthreads();
  if (rg == 0 && col < W) mass[bh * W + col] = ((red[0][col & 63] + red[1][col & 63]) + red[2][col & 63]) + red[3][col & 63];
}

}  // namespace

constexpr int kScoreLdsMax = 160 * 1024;

size_t score_lds(const Geo& g, int qpw) { return (size_t)qpw * (g.D + g.nl + g.S + 3 * g.nl) * 4; }

int score_qpw(const Geo& g) {
  for (int q = 4; q > 1; q /= 2)
    if (score_lds(g, q) <= (size_t)kScoreLdsMax) return q;
  return 1;
}

template <int D>
void pool_slots_d(const Geo& g, const void* k_p, const int32_t* plen, float* kbar, hipStream_t s) {
  dim3 grid(g.S, g.H, g.B);
  if (g.dtype == PBSA_BF16)
    pool_slots_kernel<D, bf16_t><<<grid, kThreads, 0, s>>>(g, (const bf16_t*)k_p, plen, kbar);
  else
    pool_slots_kernel<D, float><<<grid, kThreads, 0, s>>>(g, (const float*)k_p, plen, kbar);
}

hipError_t launch_pool_slots(const Geo& g, const void* k_p, const int32_t* plen, float* kbar, hipStream_t s) {
  if (g.D == 128)
    pool_slots_d<128>(g, k_p, plen, kbar, s);
  else
    pool_slots_d<64>(g, k_p, plen, kbar, s);
  return hipGetLastError();
}

template <int D>
hipError_t score_select_d(const Geo& g, const void* q, const void* k_l, const int32_t* ring_head,
                          const float* kbar_p, const int32_t* plen, int32_t* topk, float* mass, float* kbar_l,
                          WsScore ws, uint32_t* status, hipStream_t s) {
  dim3 g1(g.nq + g.nl, g.H, g.B);
  if (g.dtype == PBSA_BF16)
    pool_blocks_kernel<D, bf16_t><<<g1, kThreads, 0, s>>>(g, (const bf16_t*)q, (const bf16_t*)k_l, ws.qbar, kbar_l);
  else
    pool_blocks_kernel<D, float><<<g1, kThreads, 0, s>>>(g, (const float*)q, (const float*)k_l, ws.qbar, kbar_l);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static PerDeviceOnce attr;
  e = attr.run([] {
    for (const void* f : {(const void*)score_topk_kernel<D, 4>, (const void*)score_topk_kernel<D, 2>,
                          (const void*)score_topk_kernel<D, 1>}) {
      const hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kScoreLdsMax);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  });
  if (e != hipSuccess) return e;
  const int qpw = score_qpw(g);
  const size_t shm = score_lds(g, qpw);
  const dim3 grid((g.nq + qpw - 1) / qpw, g.H, g.B);
  if (qpw == 4)
    score_topk_kernel<D, 4><<<grid, kThreads, shm, s>>>(g, ring_head, ws.qbar, kbar_l, kbar_p, plen, topk, ws.prow, status);
  else if (qpw == 2)
    score_topk_kernel<D, 2><<<grid, kThreads, shm, s>>>(g, ring_head, ws.qbar, kbar_l, kbar_p, plen, topk, ws.prow, status);
  else
    score_topk_kernel<D, 1><<<grid, kThreads, shm, s>>>(g, ring_head, ws.qbar, kbar_l, kbar_p, plen, topk, ws.prow, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mass_kernel<<<dim3((g.S + g.nl + 63) / 64, g.H, g.B), kThreads, 0, s>>>(g, ws.prow, mass);
  return hipGetLastError();
}

hipError_t launch_score_select(const Geo& g, const void* q, const void* k_l, const int32_t* ring_head,
                               const float* kbar_p, const int32_t* plen, int32_t* topk, float* mass,
                               float* kbar_l, WsScore ws, uint32_t* status, hipStream_t s) {
  return g.D == 128 ? score_select_d<128>(g, q, k_l, ring_head, kbar_p, plen, topk, mass, kbar_l, ws, status, s)
                    : score_select_d<64>(g, q, k_l, ring_head, kbar_p, plen, topk, mass, kbar_l, ws, status, s);
}

}  // namespace pbsa
