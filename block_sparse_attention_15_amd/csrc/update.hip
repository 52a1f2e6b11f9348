// Persistent-cache update and local-ring maintenance.
//
// The abstract describes a memory that learns to "compress, preserve, and
// update" persistent blocks; the training algorithm's cache pass updates the
// persistent (P) and local (L) caches after attention.  Reading used here:
// the candidates are the valid persistent slots and the blocks of the oldest
// local chunk (the ones leaving the sliding window); the S candidates with the
// largest pooled attention mass stay (ties: incumbents first, then lower slot
// or block index); vacated slots, ascending, receive the admitted blocks,
// ascending, and slots left over are emptied.
//
// Two launches: a per-(batch, head) decision kernel that ranks candidates and
// rewrites slot metadata, then a data-movement kernel with one workgroup per
// slot that copies admitted rows with 16-byte coalesced loads/stores, zero-fills
// padding and emptied slots, and advances the ring head.
#include "common.h"

namespace pbsa {
namespace {

constexpr int kThreads = 256;

// plan[b,h,s]: -2 keep, -1 empty the slot, p >= 0 fill from physical local block p.
__global__ __launch_bounds__(kThreads) void update_decide_kernel(Geo g, const float* __restrict__ mass,
                                                                 const float* __restrict__ kbar_l,
                                                                 const int32_t* __restrict__ ring_head,
                                                                 int32_t step_id, int32_t* __restrict__ plen,
                                                                 int32_t* __restrict__ psrc,
                                                                 float* __restrict__ pkbar,
                                                                 int32_t* __restrict__ n_rep,
                                                                 int32_t* __restrict__ plan) {
  extern __shared__ int sm[];
  const int NC = g.S + g.nq;
  float* cm = (float*)sm;        // [NC] candidate mass
  int* valid = sm + NC;          // [NC]
  int* kept = valid + NC;        // [NC]
  int* alist = kept + NC;        // [nq] admitted entrants in order
  __shared__ int n_adm;
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = (size_t)b * g.H + h;
  const int old = *ring_head;
  const float* mrow = mass + bh * (g.S + g.nl);
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    if (c < g.S) {
      valid[c] = plen[bh * g.S + c] > 0;
      cm[c] = mrow[c];
    } else {
      valid[c] = 1;
      cm[c] = mrow[g.S + old * g.nq + (c - g.S)];
    }
  }
  __syncthreads();
  // rank among valid candidates; candidate order (slots, then entrants, each
  // by index) is the tie-break order
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    int k = 0;
    if (valid[c]) {
      const float mc = cm[c];
      int rank = 0;
      for (int o = 0; o < NC; ++o) rank += valid[o] && (cm[o] > mc || (cm[o] == mc && o < c));
      k = rank < g.S;
    }
    kept[c] = k;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < g.nq; e += kThreads) {
    if (!kept[g.S + e]) continue;
    int pos = 0;
    for (int o = 0; o < e; ++o) pos += kept[g.S + o];
    alist[pos] = e;
  }
  if (threadIdx.x == 0) {
    int n = 0;
    for (int e = 0; e < g.nq; ++e) n += kept[g.S + e];
    n_adm = n;
    n_rep[bh] = n;
  }
  __syncthreads();
  for (int s = threadIdx.x; s < g.S; s += kThreads) {
    const size_t bs = bh * g.S + s;
    if (valid[s] && kept[s]) {
      plan[bs] = -2;
      continue;
    }
    int j = 0;  // rank of this slot among vacated slots
    for (int o = 0; o < s; ++o) j += !(valid[o] && kept[o]);
    if (j < n_adm) {
      const int e = alist[j];
      const int p = old * g.nq + e;
      plan[bs] = p;
      plen[bs] = block_ext(g, e).len;
      psrc[bs] = step_id * g.nq + e;
      for (int d = 0; d < g.D; ++d) pkbar[bs * g.D + d] = kbar_l[(bh * g.nl + p) * g.D + d];
    } else {
      plan[bs] = -1;
      plen[bs] = 0;
      psrc[bs] = kEmptySrc;
      for (int d = 0; d < g.D; ++d) pkbar[bs * g.D + d] = 0.f;
    }
  }
}

// grid (S, H, B): move rows according to the plan; block (0,0,0) advances the ring head.
template <typename T>
__global__ __launch_bounds__(kThreads) void update_copy_kernel(Geo g, const int32_t* __restrict__ plan,
                                                               const T* __restrict__ kl, const T* __restrict__ vl,
                                                               T* __restrict__ kp, T* __restrict__ vp,
                                                               int32_t* __restrict__ ring_head) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  if (s == 0 && h == 0 && b == 0 && threadIdx.x == 0) *ring_head = (*ring_head + 1) % g.R;
  const int p = plan[bh * g.S + s];
  if (p == -2) return;
  constexpr int kVec = 16 / sizeof(T);           // elements per 16-byte chunk
  const int cpr = g.D / kVec;                      // chunks per row
  int len = 0, off = 0;
  BlockExt e;
  if (p >= 0) {
    e = block_ext(g, p % g.nq);
    len = e.len;
    off = (p / g.nq) * g.ct;
  }
  const size_t dst = (bh * g.S + s) * (size_t)g.C * g.D;
  for (int c = threadIdx.x; c < g.C * cpr; c += kThreads) {
    const int r = c / cpr, k = c - r * cpr;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (r < len) {
      const size_t src = (bh * g.NL + off + block_token(g, e, r)) * (size_t)g.D + k * kVec;
      kv = *reinterpret_cast<const uint4*>(kl + src);
      vv = *reinterpret_cast<const uint4*>(vl + src);
    }
    *reinterpret_cast<uint4*>(kp + dst + (size_t)r * g.D + k * kVec) = kv;
    *reinterpret_cast<uint4*>(vp + dst + (size_t)r * g.D + k * kVec) = vv;
  }
}

__global__ void ring_advance_kernel(int32_t* ring_head, int R) { *ring_head = (*ring_head + 1) % R; }

// grid-stride copy of a [B,H,Nq,D] chunk into the newest ring slot.
template <typename T>
__global__ __launch_bounds__(kThreads) void ring_append_kernel(Geo g, const T* __restrict__ kn,
                                                               const T* __restrict__ vn,
                                                               const int32_t* __restrict__ ring_head,
                                                               T* __restrict__ kl, T* __restrict__ vl) {
  constexpr int kVec = 16 / sizeof(T);
  const int slot = (*ring_head + g.R - 1) % g.R;
  const size_t per_bh = (size_t)g.ct * g.D / kVec;   // 16-byte chunks per (b,h)
  const size_t total = per_bh * g.B * g.H;
  for (size_t c = (size_t)blockIdx.x * kThreads + threadIdx.x; c < total; c += (size_t)gridDim.x * kThreads) {
    const size_t bh = c / per_bh, w = c - bh * per_bh;
    const size_t dst = (bh * g.NL + (size_t)slot * g.ct) * g.D + w * kVec;
    *reinterpret_cast<uint4*>(kl + dst) = *reinterpret_cast<const uint4*>(kn + c * kVec);
    *reinterpret_cast<uint4*>(vl + dst) = *reinterpret_cast<const uint4*>(vn + c * kVec);
  }
}

}  // namespace

hipError_t launch_persist_update(const Geo& g, const float* mass, const void* k_l, const void* v_l,
                                 const float* kbar_l, int32_t* ring_head, int32_t step_id, void* k_p,
                                 void* v_p, int32_t* plen, int32_t* psrc, float* pkbar, int32_t* n_rep,
                                 int32_t* plan, hipStream_t s) {
  const int NC = g.S + g.nq;
  const size_t shm = (size_t)NC * 3 * 4 + (size_t)g.nq * 4;
  update_decide_kernel<<<dim3(g.H, g.B), kThreads, shm, s>>>(g, mass, kbar_l, ring_head, step_id, plen, psrc, pkbar,
                                                              n_rep, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.S == 0) {
    ring_advance_kernel<<<1, 1, 0, s>>>(ring_head, g.R);
    return hipGetLastError();
  }
  dim3 grid(g.S, g.H, g.B);
  if (g.dtype == PBSA_BF16)
    update_copy_kernel<bf16_t><<<grid, kThreads, 0, s>>>(g, plan, (const bf16_t*)k_l, (const bf16_t*)v_l,
                                                        (bf16_t*)k_p, (bf16_t*)v_p, ring_head);
  else
    update_copy_kernel<float><<<grid, kThreads, 0, s>>>(g, plan, (const float*)k_l, (const float*)v_l,
                                                       (float*)k_p, (float*)v_p, ring_head);
  return hipGetLastError();
}

hipError_t launch_ring_append(const Geo& g, const void* k_new, const void* v_new, const int32_t* ring_head,
                              void* k_l, void* v_l, hipStream_t s) {
  const size_t chunks = (size_t)g.B * g.H * g.ct * g.D * (g.dtype == PBSA_BF16 ? 2 : 4) / 16;
  const int blocks = (int)((chunks + kThreads - 1) / kThreads < 2048 ? (chunks + kThreads - 1) / kThreads : 2048);
  if (g.dtype == PBSA_BF16)
    ring_append_kernel<bf16_t><<<blocks, kThreads, 0, s>>>(g, (const bf16_t*)k_new, (const bf16_t*)v_new, ring_head,
                                                          (bf16_t*)k_l, (bf16_t*)v_l);
  else
    ring_append_kernel<float><<<blocks, kThreads, 0, s>>>(g, (const float*)k_new, (const float*)v_new, ring_head,
                                                         (float*)k_l, (float*)v_l);
  return hipGetLastError();
}

}  // namespace pbsa
