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
// Pooled keys are cache metadata: a persistent slot's mean key is carried
// with the slot, and a local block's mean key is computed when its chunk is
// written into the ring (pbsa_ring_append pools while it copies; a ring
// filled from outside is pooled once by pbsa_pool_local).  Scoring therefore
// reads only the queries and the pooled keys.  Two launches, no
// synchronisation between workgroups:
//  1. per workgroup QPW query blocks of one head (512 threads; 1024 for eight): pool them
//     (16-byte row loads, fixed-order reduction), score them against every
//     candidate (the candidates' pooled keys loaded coalesced, all loads of
//     the first chunks issued with the query rows, and staged through LDS a
//     chunk at a time; one thread per (candidate, query block)), per query
//     block a two-phase radix select of the top K (one wave) and, beside it
//     on another wave, one softmax row, and the column sums of those rows
//     (ascending rows);
//  2. the masses: per (head, candidate) the sum of the workgroups' column
//     sums in ascending workgroup order -- deterministic.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace pbsa {

// Scratch of pbsa_score_select_noalloc: one array per device, held by the
// library until the process ends.  Host code never uses this name as an
// address (it is a host-side stand-in there); it takes the device address
// from hipGetSymbolAddress, once per device, in score_static_scratch().
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

hipError_t score_static_scratch(void** out, size_t* bytes) {
  static std::mutex mu;
  static void* addr[PerDeviceOnce::kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= PerDeviceOnce::kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;
constexpr int kPartBatch = 16;  // partial-sum loads in flight per thread in the last workgroup

template <int D, typename T> struct Rows {
  static constexpr int VEC = 16 / sizeof(T);        // elements per 16-byte chunk
  static constexpr int CPR = D / VEC;               // chunks per row
  static constexpr int NRG = kThreads / CPR;        // row groups
  static constexpr int RPT = (64 + NRG - 1) / NRG;  // rows per thread at most (blocks <= 64 rows)
};

__device__ __forceinline__ void add_chunk(float* acc, uint4 v, bf16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[2 * k] += __uint_as_float(w[k] << 16);
    acc[2 * k + 1] += __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void add_chunk(float* acc, uint4 v, float) {
  acc[0] += __uint_as_float(v.x);
  acc[1] += __uint_as_float(v.y);
  acc[2] += __uint_as_float(v.z);
  acc[3] += __uint_as_float(v.w);
}

// Mean of the `len` (<= 64) rows src_row(i) of a [*, D] tensor into out[D],
// fixed summation order (each thread sums its row group's rows in order, the
// row groups are added in order 0..NRG-1, then divided by len; 0 rows give
// 0).  With COPY the rows are also written to dst_row(i) (the same loads).
// All of a thread's loads are issued before the first add.
template <int D, typename T, bool COPY, typename SrcFn, typename DstFn>
__device__ __forceinline__ void pool_rows(const T* src, T* dst, int len, SrcFn src_row, DstFn dst_row,
                                          float* red /* [NRG][D] */, float* out) {
  using R = Rows<D, T>;
  const int c = threadIdx.x % R::CPR, rg = threadIdx.x / R::CPR;
  uint4 v[R::RPT];
#pragma unroll
  for (int u = 0; u < R::RPT; ++u) {
    const int i = rg + R::NRG * u;
    v[u] = i < len ? *reinterpret_cast<const uint4*>(src + (size_t)src_row(i) * D + c * R::VEC)
                   : make_uint4(0, 0, 0, 0);
  }
  if (COPY) {
#pragma unroll
    for (int u = 0; u < R::RPT; ++u) {
      const int i = rg + R::NRG * u;
      if (i < len) *reinterpret_cast<uint4*>(dst + (size_t)dst_row(i) * D + c * R::VEC) = v[u];
    }
  }
  float acc[R::VEC] = {};
#pragma unroll
  for (int u = 0; u < R::RPT; ++u) add_chunk(acc, v[u], T{});  // rows past len were loaded as zero
#pragma unroll
  for (int k = 0; k < R::VEC; ++k) red[rg * D + c * R::VEC + k] = acc[k];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float s = 0.f;
    for (int k = 0; k < R::NRG; ++k) s += red[k * D + d];
    out[d] = len > 0 ? s / (float)len : 0.f;
  }
}

// grid (nq, H, B): write block j of a new chunk (k_new / v_new, [B,H,ct,D])
// into the newest ring slot, (ring_head + R - 1) mod R, and its mean key into
// kbar_local.  APPEND = false (pbsa_pool_local): grid (nl, H, B), only pool
// physical local block j of the ring.
template <int D, typename T, bool APPEND>
__global__ __launch_bounds__(kThreads) void local_pool_kernel(Geo g, const T* __restrict__ k_new,
                                                              const T* __restrict__ v_new,
                                                              const int32_t* __restrict__ ring_head,
                                                              T* __restrict__ kl, T* __restrict__ vl,
                                                              float* __restrict__ kbar_l,
                                                              uint32_t* __restrict__ status) {
  __shared__ float red[Rows<D, T>::NRG * D];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  const BlockExt e = block_ext(g, j % g.nq);
  T* kb = kl + bh * (size_t)g.NL * D;
  if (APPEND) {
    const int slot = (read_ring_head(ring_head, g.R, status) + g.R - 1) % g.R;
    const int off = slot * g.ct;
    // every K and V row load of the thread is issued before the first store
    using R = Rows<D, T>;
    const int c = threadIdx.x % R::CPR, rg = threadIdx.x / R::CPR;
    const T* ks = k_new + bh * g.ct * D;
    const T* vs = v_new + bh * g.ct * D;
    T* vb = vl + bh * (size_t)g.NL * D;
    int tk[R::RPT];
    uint4 kv[R::RPT], vv[R::RPT];
#pragma unroll
    for (int u = 0; u < R::RPT; ++u) {
      const int i = rg + R::NRG * u;
      tk[u] = i < e.len ? block_token(g, e, i) : -1;
      kv[u] = tk[u] >= 0 ? *reinterpret_cast<const uint4*>(ks + (size_t)tk[u] * D + c * R::VEC) : make_uint4(0, 0, 0, 0);
      vv[u] = tk[u] >= 0 ? *reinterpret_cast<const uint4*>(vs + (size_t)tk[u] * D + c * R::VEC) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < R::RPT; ++u) {
      if (tk[u] >= 0) {
        const size_t d = (size_t)(off + tk[u]) * D + c * R::VEC;
        *reinterpret_cast<uint4*>(kb + d) = kv[u];
        *reinterpret_cast<uint4*>(vb + d) = vv[u];
      }
    }
    float acc[R::VEC] = {};
#pragma unroll
    for (int u = 0; u < R::RPT; ++u) add_chunk(acc, kv[u], T{});  // rows past the block were loaded as zero
#pragma unroll
    for (int k = 0; k < R::VEC; ++k) red[rg * D + c * R::VEC + k] = acc[k];
    __syncthreads();
    float* out = kbar_l + (bh * g.nl + slot * g.nq + j) * D;
    for (int d = threadIdx.x; d < D; d += kThreads) {
      float sum = 0.f;
      for (int k = 0; k < R::NRG; ++k) sum += red[k * D + d];
      out[d] = e.len > 0 ? sum / (float)e.len : 0.f;
    }
  } else {
    const int off = (j / g.nq) * g.ct;
    pool_rows<D, T, false>(kb, (T*)nullptr, e.len, [&](int i) { return off + block_token(g, e, i); },
                           [](int i) { return i; }, red, kbar_l + (bh * g.nl + j) * D);
  }
}

// grid (S, H, B): mean of each slot's first len rows (0 for empty slots).
template <int D, typename T>
__global__ __launch_bounds__(kThreads) void pool_slots_kernel(Geo g, const T* __restrict__ kp,
                                                              const int32_t* __restrict__ plen,
                                                              float* __restrict__ kbar) {
  __shared__ float red[Rows<D, T>::NRG * D];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bhs = ((size_t)b * g.H + h) * g.S + s;
  const int len = min(max(plen[bhs], 0), g.C);
  pool_rows<D, T, false>(kp + bhs * g.C * D, (T*)nullptr, len, [](int i) { return i; }, [](int i) { return i; },
                         red, kbar + bhs * D);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int wave_count(bool p) { return __builtin_popcountll(__builtin_amdgcn_ballot_w64(p)); }

// Order-preserving map of a float to an unsigned key (-0 taken as +0).
__device__ __forceinline__ unsigned float_key(float x) {
  unsigned u = x == 0.f ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wavefront selection of the K largest of n distinct 64-bit keys (hi, lo),
// lane l holding keys l, l+64, ... (KPL per lane; hi = 0 marks no key).
// Two radix passes, one bit per ballot round: the K-th largest hi value T,
// then -- only when several keys share T and not all of them fit -- the
// largest lo among those.  Returns, per held key, whether it is selected.
template <int KPL>
__device__ __forceinline__ void select_top(const unsigned (&hi)[KPL], const unsigned (&lo)[KPL], int K,
                                           bool (&sel)[KPL]) {
  unsigned thr = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < KPL; ++u) cnt += wave_count(hi[u] >= cand);
    if (cnt >= K) thr = cand;
  }
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    n_gt += wave_count(hi[u] > thr);
    n_eq += wave_count(hi[u] == thr);
  }
  const int need = K - n_gt;  // >= 1 keys with hi == thr are taken
  unsigned thr2 = 0u;
  if (n_eq > need) {
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned cand = thr2 | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < KPL; ++u) cnt += wave_count(hi[u] == thr && lo[u] >= cand);
      if (cnt >= need) thr2 = cand;
    }
  }
#pragma unroll
  for (int u = 0; u < KPL; ++u) sel[u] = hi[u] > thr || (hi[u] == thr && lo[u] >= thr2);
}

// XCD-aware remap of a 1-D grid: hardware places workgroup i on XCD i % 8, so
// each XCD gets a contiguous range of the linear work index (a head's
// workgroups then share one L2).
__device__ __forceinline__ int xcd_remap(int total) {
  const int per_xcd = (total + 7) / 8;
  return (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
}

constexpr int kScoreThreads = 512;  // up to four query blocks per workgroup
// Threads of a scoring workgroup: one selecting and one softmax wave per
// query block, at least 512 (eight query blocks: 1024).
constexpr int score_threads(int qpw) { return qpw > 4 ? 128 * qpw : kScoreThreads; }
constexpr int kScoreChunk = 128;      // candidate keys staged in LDS at a time
constexpr int kScoreChunksHeld = 3;   // chunks whose loads are issued up front (registers)

// Pooling of QPW query blocks by one workgroup: score_threads(QPW) / QPW threads
// per block, each summing its row group's rows in order; row groups are then
// added in order (fixed order, deterministic).
template <int D, typename T, int QPW> struct QPool {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int CPR = D / VEC;             // 16-byte chunks per row
  static constexpr int TPB = score_threads(QPW) / QPW; // threads per query block
  static constexpr int NRG = TPB / CPR;           // row groups per block
  static constexpr int RPT = (64 + NRG - 1) / NRG;
  static_assert(NRG >= 1 && TPB % CPR == 0, "pooling layout");
};

// 1-D grid over (B, H, group of QPW query blocks).  qbar is pooled here; the
// scores, top-K ids, softmax rows and the workgroup's column sums follow.
template <int D, typename T, int QPW, int KPL>
__global__ __launch_bounds__(score_threads(QPW)) void score_topk_kernel(Geo g, const T* __restrict__ q,
                                                                   const int32_t* __restrict__ ring_head,
                                                                   const float* __restrict__ kbar_l,
                                                                   const float* __restrict__ kbar_p,
                                                                   const int32_t* __restrict__ plen,
                                                                   int32_t* __restrict__ topk,
                                                                   float* __restrict__ part,
                                                                   uint32_t* __restrict__ status) {
  using P = QPool<D, T, QPW>;
  extern __shared__ float smem[];
  const int W = g.nl + g.S;        // candidates: local blocks, then slots
  const int ngrp = (g.nq + QPW - 1) / QPW;
  const int total = g.B * g.H * ngrp;
  const int lin = xcd_remap(total);
  if (lin >= total) return;
  const int grp = lin % ngrp;
  const size_t bh = lin / ngrp;
  constexpr int QST = D + 4;                // LDS row stride (floats) of pooled queries and keys:
                                            // consecutive rows start in different banks
  float* qb = smem;                         // [QPW][QST]
  float* sc = qb + QPW * QST;               // [QPW][W] scores, then softmax rows (-inf / 0 for empty slots)
  int* flag = (int*)(sc + QPW * W);         // [QPW][nl] selected flags
  float* red = (float*)(flag + QPW * g.nl); // [QPW][NRG][D] pooling partial sums, then:
  float* kch = red;                         // [kScoreChunk][QST] a chunk of the candidates' pooled keys
  int* clen = (int*)(kch + kScoreChunk * QST);  // [kScoreChunk] their slot lengths (1: local block)
  const int i0 = grp * QPW;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // Candidates' pooled keys reach LDS kScoreChunk rows at a time, loaded
  // coalesced (consecutive lanes read consecutive 16-byte pieces of a row).
  // The loads of the first kScoreChunksHeld chunks are all issued up front,
  // into registers, together with the query rows: one round of global loads
  // for up to kScoreChunksHeld * kScoreChunk candidates; later chunks (larger
  // local windows) are loaded when their turn comes.
  constexpr int PPR = D / 4;                  // float4 pieces per row
  constexpr int TH = score_threads(QPW);
  constexpr int RPP = TH / PPR;               // rows per pass
  constexpr int NP = kScoreChunk / RPP;       // float4 loads per thread per chunk
  static_assert(NP * RPP == kScoreChunk, "chunk layout");
  const int pc = threadIdx.x % PPR, pr = threadIdx.x / PPR;
  float4 kreg[kScoreChunksHeld][NP];
  int lreg[kScoreChunksHeld];
  auto load_chunk = [&](int cb, float4 (&kr)[NP], int& lr) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int c = cb + pr + RPP * u;
      kr[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < W) {
        const float* src = c < g.nl ? kbar_l + (bh * g.nl + c) * D : kbar_p + (bh * g.S + (c - g.nl)) * D;
        kr[u] = reinterpret_cast<const float4*>(src)[pc];
      }
    }
    const int c = cb + (int)threadIdx.x;
    lr = 0;
    if (threadIdx.x < kScoreChunk) lr = c < g.nl ? 1 : (c < W ? plen[bh * g.S + (c - g.nl)] : 0);
  };
  auto store_chunk = [&](const float4 (&kr)[NP], int lr) {
#pragma unroll
    for (int u = 0; u < NP; ++u) reinterpret_cast<float4*>(kch + (pr + RPP * u) * QST)[pc] = kr[u];
    if (threadIdx.x < kScoreChunk) clen[threadIdx.x] = lr;
  };
#pragma unroll
  for (int h = 0; h < kScoreChunksHeld; ++h)
    if (h * kScoreChunk < W) load_chunk(h * kScoreChunk, kreg[h], lreg[h]);
  const int rh_raw = *ring_head;  // in flight with the other loads, checked after the pooling
  // pool the query blocks: every row load of the thread in flight together
  {
    const int blk = threadIdx.x / P::TPB, t = threadIdx.x % P::TPB;
    const int c = t % P::CPR, rg = t / P::CPR;
    const int qi = i0 + blk;
    const BlockExt e = block_ext(g, qi < g.nq ? qi : 0);
    const int len = qi < g.nq ? e.len : 0;
    const T* qh = q + bh * g.ct * D;
    uint4 v[P::RPT];
#pragma unroll
    for (int u = 0; u < P::RPT; ++u) {
      const int r = rg + P::NRG * u;
      v[u] = r < len ? *reinterpret_cast<const uint4*>(qh + (size_t)block_token(g, e, r) * D + c * P::VEC)
                     : make_uint4(0, 0, 0, 0);
    }
    float acc[P::VEC] = {};
#pragma unroll
    for (int u = 0; u < P::RPT; ++u) add_chunk(acc, v[u], T{});
#pragma unroll
    for (int k = 0; k < P::VEC; ++k) red[(blk * P::NRG + rg) * D + c * P::VEC + k] = acc[k];
    __syncthreads();
    for (int x = threadIdx.x; x < QPW * D; x += TH) {
      const int b2 = x / D, d = x % D;
      float s = 0.f;
      for (int k = 0; k < P::NRG; ++k) s += red[(b2 * P::NRG + k) * D + d];
      const int l2 = i0 + b2 < g.nq ? block_ext(g, i0 + b2).len : 0;
      qb[b2 * QST + d] = l2 > 0 ? s / (float)l2 : 0.f;
    }
  }
  if ((unsigned)rh_raw >= (unsigned)g.R) atomicOr(status, kStatusRingHead);
  const int rh = ring_wrap(rh_raw, g.R);
  __syncthreads();  // the pooling sums are read: their LDS takes the key chunks
  // scores: one thread per (candidate, query block), d in ascending order
  auto score_chunk = [&](int cb) {
    for (int x = threadIdx.x; x < kScoreChunk * QPW; x += TH) {
      const int r = x / QPW, k = x - r * QPW, c = cb + r;
      if (c >= W) break;
      float sv = -INFINITY;  // empty slot
      if (c < g.nl || clen[r] > 0) {
        const float4* kr = reinterpret_cast<const float4*>(kch + r * QST);
        const float4* qr = reinterpret_cast<const float4*>(qb + k * QST);
        float acc = 0.f;
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 k4 = kr[d4], q4 = qr[d4];
          acc = fmaf(q4.x, k4.x, acc);
          acc = fmaf(q4.y, k4.y, acc);
          acc = fmaf(q4.z, k4.z, acc);
          acc = fmaf(q4.w, k4.w, acc);
        }
        sv = acc * g.scale;
      }
      sc[k * W + c] = sv;
    }
  };
#pragma unroll
  for (int h = 0; h < kScoreChunksHeld; ++h) {
    if (h * kScoreChunk >= W) break;
    if (h > 0) __syncthreads();  // the previous chunk is scored
    store_chunk(kreg[h], lreg[h]);
    __syncthreads();
    score_chunk(h * kScoreChunk);
  }
  for (int cb = kScoreChunksHeld * kScoreChunk; cb < W; cb += kScoreChunk) {
    load_chunk(cb, kreg[0], lreg[0]);
    __syncthreads();
    store_chunk(kreg[0], lreg[0]);
    __syncthreads();
    score_chunk(cb);
  }
  __syncthreads();
  // waves 0..QPW-1 select the top K of their query block's local scores,
  // waves SW..SW+QPW-1 (SW = max(4, QPW)) turn the same rows into softmax
  // rows: the selecting
  // waves take their keys into registers first, then both run side by side
  constexpr int SW = QPW > 4 ? QPW : 4;  // first softmax wave
  static_assert(TH / 64 >= SW + QPW, "selecting and softmax waves");
  const int i = i0 + w;
  float* row = sc + w * W;
  const bool selects = w < QPW && i < g.nq;
  // keys: descending score, then ascending logical index (oldest chunk first)
  unsigned hi[KPL], lo[KPL];
  if (selects) {
#pragma unroll
    for (int u = 0; u < KPL; ++u) {
      const int p = lane + 64 * u;
      hi[u] = 0u;
      lo[u] = 0u;
      if (p < g.nl) {
        const int cp = p / g.nq;
        hi[u] = float_key(row[p]);
        lo[u] = 0xffffffffu - (unsigned)(ring_wrap(cp - rh, g.R) * g.nq + (p - cp * g.nq));
      }
    }
  }
  __syncthreads();  // the keys are in registers: the rows may be overwritten
  if (selects) {
    bool on[KPL];
    select_top<KPL>(hi, lo, g.K, on);
    int* fl = flag + w * g.nl;
#pragma unroll
    for (int u = 0; u < KPL; ++u) {
      const int p = lane + 64 * u;
      if (p < g.nl) fl[p] = on[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ascending physical ids: position = selected count below p (ballot prefix)
    int32_t* out = topk + (bh * g.nq + i) * g.K;
    int running = 0;
    for (int p0 = 0; p0 < g.nl; p0 += 64) {
      const int p = p0 + lane;
      const bool sp = p < g.nl && fl[p];
      const unsigned long long m = __builtin_amdgcn_ballot_w64(sp);
      if (sp) out[running + __builtin_popcountll(m & ((1ull << lane) - 1))] = p;
      running += __builtin_popcountll(m);
    }
  }
  const int wsm = w - SW;  // softmax wave of query block i0 + wsm
  if (wsm >= 0 && wsm < QPW && i0 + wsm < g.nq) {
    // pooled softmax over valid slots and all local blocks, in place of the scores
    float* srow = sc + wsm * W;
    float mx = -INFINITY;
    for (int c = lane; c < W; c += 64) mx = fmaxf(mx, srow[c]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int c = lane; c < W; c += 64) {  // each exponential once, kept in the row
      const float x = srow[c], e = x == -INFINITY ? 0.f : expf(x - mx);
      srow[c] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    for (int c = lane; c < W; c += 64) srow[c] = srow[c] / sum;
  }
  __syncthreads();
  // this workgroup's column sums (rows in ascending order), in the masses'
  // layout (column c is local block c or slot c - nl)
  const int nrows = min(QPW, g.nq - i0);
  float* mypart = part + (bh * ngrp + grp) * (size_t)W;
  for (int c = threadIdx.x; c < W; c += TH) {
    float v = 0.f;
    for (int k = 0; k < nrows; ++k) v += sc[k * W + c];
    mypart[c < g.nl ? g.S + c : c - g.nl] = v;
  }
}

// grid over (B, H, candidate): mass = the score workgroups' column sums added
// in ascending workgroup order, kPartBatch loads in flight per thread.
__global__ __launch_bounds__(kThreads) void mass_kernel(Geo g, int ngrp, const float* __restrict__ part,
                                                        float* __restrict__ mass) {
  const int W = g.S + g.nl;
  const size_t x = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (x >= (size_t)g.B * g.H * W) return;
  const size_t bh = x / W;
  const int c = (int)(x - bh * W);
  const float* hp = part + bh * ngrp * (size_t)W + c;
  float s = 0.f;
  for (int g0 = 0; g0 < ngrp; g0 += kPartBatch) {
    float v[kPartBatch];
#pragma unroll
    for (int u = 0; u < kPartBatch; ++u) v[u] = g0 + u < ngrp ? hp[(size_t)(g0 + u) * W] : 0.f;
#pragma unroll
    for (int u = 0; u < kPartBatch; ++u) s += v[u];
  }
  mass[x] = s;
}

}  // namespace

constexpr int kScoreLdsMax = 159 * 1024;  // dynamic LDS

// LDS of the score kernel at QPW query blocks per workgroup: pooled queries,
// scores, flags, then the larger of the pooling scratch (sized for the
// largest layout: fp32 rows, score_threads(QPW) / QPW threads per block) and one chunk of
// candidate keys with their lengths.
size_t score_lds(const Geo& g, int qpw) {
  const int vec = g.dtype == PBSA_BF16 ? 8 : 4;
  const int nrg = (score_threads(qpw) / qpw) / (g.D / vec);
  const size_t pool = (size_t)qpw * nrg * g.D, chunk = (size_t)kScoreChunk * (g.D + 4 + 1);
  return ((size_t)qpw * (g.D + 4 + g.nl + g.S + g.nl) + std::max(pool, chunk)) * 4;
}

int score_qpw(const Geo& g) {
  // eight query blocks per workgroup (1024 threads) when four would need
  // more workgroups than the GPU has compute units: each workgroup loads every
  // candidate's pooled key, so fewer, fuller workgroups cost less
  const long long wg4 = (long long)g.B * g.H * ((g.nq + 3) / 4);
  // (bf16 inputs: the fp32 rows need more registers than 1024 threads leave)
  if (g.dtype == PBSA_BF16 && wg4 > 256 && score_lds(g, 8) <= (size_t)kScoreLdsMax) return 8;
  for (int q = 4; q > 1; q /= 2)
    if (score_lds(g, q) <= (size_t)kScoreLdsMax) return q;
  return 1;
}

size_t score_workspace(const Geo& g) {
  const size_t BH = (size_t)g.B * g.H;
  const size_t ngrp = (g.nq + score_qpw(g) - 1) / score_qpw(g);
  return ((BH * ngrp * (g.S + g.nl) * 4) + 255) & ~size_t(255);
}

template <int D, typename T>
void pool_slots_t(const Geo& g, const void* k_p, const int32_t* plen, float* kbar, hipStream_t s) {
  pool_slots_kernel<D, T><<<dim3(g.S, g.H, g.B), kThreads, 0, s>>>(g, (const T*)k_p, plen, kbar);
}

hipError_t launch_pool_slots(const Geo& g, const void* k_p, const int32_t* plen, float* kbar, hipStream_t s) {
  if (g.D == 128)
    g.dtype == PBSA_BF16 ? pool_slots_t<128, bf16_t>(g, k_p, plen, kbar, s) : pool_slots_t<128, float>(g, k_p, plen, kbar, s);
  else
    g.dtype == PBSA_BF16 ? pool_slots_t<64, bf16_t>(g, k_p, plen, kbar, s) : pool_slots_t<64, float>(g, k_p, plen, kbar, s);
  return hipGetLastError();
}

template <int D, typename T, bool APPEND>
void local_pool_t(const Geo& g, const void* k_new, const void* v_new, const int32_t* ring_head, void* k_l, void* v_l,
                  float* kbar_l, uint32_t* status, hipStream_t s) {
  local_pool_kernel<D, T, APPEND><<<dim3(APPEND ? g.nq : g.nl, g.H, g.B), kThreads, 0, s>>>(
      g, (const T*)k_new, (const T*)v_new, ring_head, (T*)k_l, (T*)v_l, kbar_l, status);
}

template <bool APPEND>
hipError_t local_pool(const Geo& g, const void* k_new, const void* v_new, const int32_t* ring_head, void* k_l,
                      void* v_l, float* kbar_l, uint32_t* status, hipStream_t s) {
  const bool bf = g.dtype == PBSA_BF16;
  if (g.D == 128)
    bf ? local_pool_t<128, bf16_t, APPEND>(g, k_new, v_new, ring_head, k_l, v_l, kbar_l, status, s)
       : local_pool_t<128, float, APPEND>(g, k_new, v_new, ring_head, k_l, v_l, kbar_l, status, s);
  else
    bf ? local_pool_t<64, bf16_t, APPEND>(g, k_new, v_new, ring_head, k_l, v_l, kbar_l, status, s)
       : local_pool_t<64, float, APPEND>(g, k_new, v_new, ring_head, k_l, v_l, kbar_l, status, s);
  return hipGetLastError();
}

hipError_t launch_ring_append(const Geo& g, const void* k_new, const void* v_new, const int32_t* ring_head,
                              void* k_l, void* v_l, float* kbar_l, uint32_t* status, hipStream_t s) {
  return local_pool<true>(g, k_new, v_new, ring_head, k_l, v_l, kbar_l, status, s);
}

hipError_t launch_pool_local(const Geo& g, const void* k_l, float* kbar_l, hipStream_t s) {
  return local_pool<false>(g, nullptr, nullptr, nullptr, const_cast<void*>(k_l), nullptr, kbar_l, nullptr, s);
}

template <int D, typename T, int QPW, int KPL>
hipError_t score_launch(const Geo& g, const void* q, const int32_t* ring_head, const float* kbar_l,
                        const float* kbar_p, const int32_t* plen, int32_t* topk, float* part, uint32_t* status,
                        hipStream_t s) {
  static PerDeviceOnce attr;
  hipError_t e = attr.run([] {
    return hipFuncSetAttribute((const void*)score_topk_kernel<D, T, QPW, KPL>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, kScoreLdsMax);
  });
  if (e != hipSuccess) return e;
  const int ngrp = (g.nq + QPW - 1) / QPW;
  const int total = g.B * g.H * ngrp;
  score_topk_kernel<D, T, QPW, KPL><<<(total + 7) / 8 * 8, score_threads(QPW), score_lds(g, QPW), s>>>(
      g, (const T*)q, ring_head, kbar_l, kbar_p, plen, topk, part, status);
  return hipGetLastError();
}

template <int D, typename T, int KPL>
hipError_t score_qpw_launch(const Geo& g, const void* q, const int32_t* ring_head, const float* kbar_l,
                            const float* kbar_p, const int32_t* plen, int32_t* topk, float* part, uint32_t* status,
                            hipStream_t s) {
  switch (score_qpw(g)) {
    case 8: return score_launch<D, T, 8, KPL>(g, q, ring_head, kbar_l, kbar_p, plen, topk, part, status, s);
    case 4: return score_launch<D, T, 4, KPL>(g, q, ring_head, kbar_l, kbar_p, plen, topk, part, status, s);
    case 2: return score_launch<D, T, 2, KPL>(g, q, ring_head, kbar_l, kbar_p, plen, topk, part, status, s);
    default: return score_launch<D, T, 1, KPL>(g, q, ring_head, kbar_l, kbar_p, plen, topk, part, status, s);
  }
}

template <int D, typename T>
hipError_t score_select_t(const Geo& g, const void* q, const float* kbar_l, const int32_t* ring_head,
                          const float* kbar_p, const int32_t* plen, int32_t* topk, float* mass, WsScore ws,
                          uint32_t* status, hipStream_t s) {
  hipError_t e = g.nl <= 256
                     ? score_qpw_launch<D, T, 4>(g, q, ring_head, kbar_l, kbar_p, plen, topk, ws.part, status, s)
                     : score_qpw_launch<D, T, 32>(g, q, ring_head, kbar_l, kbar_p, plen, topk, ws.part, status, s);
  if (e != hipSuccess) return e;
  const int ngrp = (g.nq + score_qpw(g) - 1) / score_qpw(g);
  const size_t n = (size_t)g.B * g.H * (g.S + g.nl);
  mass_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(g, ngrp, ws.part, mass);
  return hipGetLastError();
}

hipError_t launch_score_select(const Geo& g, const void* q, const float* kbar_l, const int32_t* ring_head,
                               const float* kbar_p, const int32_t* plen, int32_t* topk, float* mass, WsScore ws,
                               uint32_t* status, hipStream_t s) {
  const bool bf = g.dtype == PBSA_BF16;
  if (g.D == 128)
    return bf ? score_select_t<128, bf16_t>(g, q, kbar_l, ring_head, kbar_p, plen, topk, mass, ws, status, s)
              : score_select_t<128, float>(g, q, kbar_l, ring_head, kbar_p, plen, topk, mass, ws, status, s);
  return bf ? score_select_t<64, bf16_t>(g, q, kbar_l, ring_head, kbar_p, plen, topk, mass, ws, status, s)
            : score_select_t<64, float>(g, q, kbar_l, ring_head, kbar_p, plen, topk, mass, ws, status, s);
}

}  // namespace pbsa
