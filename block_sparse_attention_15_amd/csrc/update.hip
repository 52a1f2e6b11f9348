// Persistent-cache update and local-ring maintenance.
//
// The abstract describes a memory that learns to "compress, preserve, and
// update" persistent blocks; the training algorithm's cache pass updates the
// persistent (P) and local (L) caches after attention.  Reading used here:
// the candidates are the valid persistent slots and the blocks of the oldest
// local chunk (the ones leaving the sliding window); the S candidates with the
// largest pooled attention mass stay (ties: incumbents first, then lower slot
// or block index); vacated slots, ascending, receive the admitted blocks,
// ascending, and slots left over are emptied.  With Z pinned sink slots
// (the project page's "sink" pattern) the first Z slots are not candidates: a
// valid one stays, an empty one takes the evicted block of its own index, and
// the other candidates compete for the remaining S - Z slots.
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
// Candidates carry a 64-bit key (mass, then the tie order: slots before
// entrants, lower index first); a candidate is kept when fewer than S - Z
// valid candidates have a larger key.  Wave 0 then pairs vacated slots with
// admitted entrants by ballot prefix counts.
__global__ __launch_bounds__(kThreads) void update_decide_kernel(Geo g, const float* __restrict__ mass,
                                                                 const int32_t* __restrict__ ring_head,
                                                                 const int32_t* __restrict__ step_counter,
                                                                 int32_t* __restrict__ plen,
                                                                 int32_t* __restrict__ psrc,
                                                                 int32_t* __restrict__ n_rep,
                                                                 int32_t* __restrict__ plan,
                                                                 uint32_t* __restrict__ status) {
  extern __shared__ unsigned long long sk[];
  const int NC = g.S + g.nq;
  unsigned long long* key = sk;            // [NC], 0 for empty slots
  int* kept = (int*)(sk + NC);             // [NC]
  int* alist = kept + NC;                  // [nq] admitted entrants in order
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = (size_t)b * g.H + h;
  const int old = read_ring_head(ring_head, g.R, status);
  const int step_id = read_step(step_counter, g.nq, status);
  const float* mrow = mass + bh * (g.S + g.nl);
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    // sink slots, and evicted blocks reserved for an empty sink slot, are not candidates
    const bool valid = c < g.S ? (c >= g.Z && plen[bh * g.S + c] > 0)
                               : !(c - g.S < g.Z && plen[bh * g.S + (c - g.S)] == 0);
    const float m = c < g.S ? mrow[c] : mrow[g.S + old * g.nq + (c - g.S)];
    unsigned u = m == 0.f ? 0u : __float_as_uint(m);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    key[c] = valid ? ((unsigned long long)u << 32) | (0xffffffffu - (unsigned)c) : 0ull;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    const unsigned long long kc = key[c];
    int rank = 0;
    for (int o = 0; o < NC; ++o) rank += key[o] > kc;
    kept[c] = kc != 0ull && rank < g.S - g.Z;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int n_sink_fill = 0;  // empty sink slots, each filled with the evicted block of its index
  for (int s0 = 0; s0 < g.Z; s0 += 64) {
    const int s = s0 + lane;
    const bool fill = s < g.Z && plen[bh * g.S + s] == 0;
    n_sink_fill += __builtin_popcountll(__builtin_amdgcn_ballot_w64(fill));
    if (s < g.Z) {
      const size_t bs = bh * g.S + s;
      if (fill) {
        plan[bs] = old * g.nq + s;
        plen[bs] = block_ext(g, s).len;
        psrc[bs] = step_id * g.nq + s;
      } else {
        plan[bs] = -2;
      }
    }
  }
  const unsigned long long below = (1ull << lane) - 1;
  int n_adm = 0;
  for (int e0 = 0; e0 < g.nq; e0 += 64) {
    const int e = e0 + lane;
    const bool on = e < g.nq && kept[g.S + e];
    const unsigned long long m = __builtin_amdgcn_ballot_w64(on);
    if (on) alist[n_adm + __builtin_popcountll(m & below)] = e;
    n_adm += __builtin_popcountll(m);
  }
  if (lane == 0) n_rep[bh] = n_adm + n_sink_fill;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int nvac = 0;
  for (int s0 = g.Z; s0 < g.S; s0 += 64) {
    const int s = s0 + lane;
    const bool in = s < g.S;
    const bool vac = in && !(key[s] != 0ull && kept[s]);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(vac);
    if (in) {
      const size_t bs = bh * g.S + s;
      if (!vac) {
        plan[bs] = -2;
      } else {
        const int j = nvac + __builtin_popcountll(m & below);  // rank among vacated slots
        if (j < n_adm) {
          const int e = alist[j];
          plan[bs] = old * g.nq + e;
          plen[bs] = block_ext(g, e).len;
          psrc[bs] = step_id * g.nq + e;
        } else {
          plan[bs] = -1;
          plen[bs] = 0;
          psrc[bs] = kEmptySrc;
        }
      }
    }
    nvac += __builtin_popcountll(m);
  }
}

// grid (S, H, B): move rows and pooled keys according to the plan; block
// (0,0,0) advances the ring head and the step counter.
template <typename T>
__global__ __launch_bounds__(kThreads) void update_copy_kernel(Geo g, const int32_t* __restrict__ plan,
                                                               const T* __restrict__ kl, const T* __restrict__ vl,
                                                               const float* __restrict__ kbar_l,
                                                               T* __restrict__ kp, T* __restrict__ vp,
                                                               float* __restrict__ pkbar,
                                                               int32_t* __restrict__ ring_head,
                                                               int32_t* __restrict__ step_counter) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  if (s == 0 && h == 0 && b == 0 && threadIdx.x == 0) {
    *ring_head = (ring_wrap(*ring_head, g.R) + 1) % g.R;
    *step_counter += 1;
  }
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
  for (int d = threadIdx.x; d < g.D; d += kThreads)
    pkbar[(bh * g.S + s) * g.D + d] = p >= 0 ? kbar_l[(bh * g.nl + p) * g.D + d] : 0.f;
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

__global__ void ring_advance_kernel(int32_t* ring_head, int32_t* step_counter, int R) {
  *ring_head = (ring_wrap(*ring_head, R) + 1) % R;
  *step_counter += 1;
}

// grid-stride copy of a [B,H,Nq,D] chunk into the newest ring slot.
template <typename T>
__global__ __launch_bounds__(kThreads) void ring_append_kernel(Geo g, const T* __restrict__ kn,
                                                               const T* __restrict__ vn,
                                                               const int32_t* __restrict__ ring_head,
                                                               T* __restrict__ kl, T* __restrict__ vl,
                                                               uint32_t* __restrict__ status) {
  constexpr int kVec = 16 / sizeof(T);
  const int slot = (read_ring_head(ring_head, g.R, status) + g.R - 1) % g.R;
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
                                 const float* kbar_l, int32_t* ring_head, int32_t* step_counter, void* k_p,
                                 void* v_p, int32_t* plen, int32_t* psrc, float* pkbar, int32_t* n_rep,
                                 int32_t* plan, uint32_t* status, hipStream_t s) {
  const int NC = g.S + g.nq;
  const size_t shm = (size_t)NC * 8 + (size_t)NC * 4 + (size_t)g.nq * 4;
  update_decide_kernel<<<dim3(g.H, g.B), kThreads, shm, s>>>(g, mass, ring_head, step_counter, plen, psrc, n_rep,
                                                              plan, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.S == 0) {
    ring_advance_kernel<<<1, 1, 0, s>>>(ring_head, step_counter, g.R);
    return hipGetLastError();
  }
  dim3 grid(g.S, g.H, g.B);
  if (g.dtype == PBSA_BF16)
    update_copy_kernel<bf16_t><<<grid, kThreads, 0, s>>>(g, plan, (const bf16_t*)k_l, (const bf16_t*)v_l, kbar_l,
                                                        (bf16_t*)k_p, (bf16_t*)v_p, pkbar, ring_head,
                                                        step_counter);
  else
    update_copy_kernel<float><<<grid, kThreads, 0, s>>>(g, plan, (const float*)k_l, (const float*)v_l, kbar_l,
                                                       (float*)k_p, (float*)v_p, pkbar, ring_head,
                                                       step_counter);
  return hipGetLastError();
}

hipError_t launch_ring_append(const Geo& g, const void* k_new, const void* v_new, const int32_t* ring_head,
                              void* k_l, void* v_l, uint32_t* status, hipStream_t s) {
  const size_t chunks = (size_t)g.B * g.H * g.ct * g.D * (g.dtype == PBSA_BF16 ? 2 : 4) / 16;
  const int blocks = (int)((chunks + kThreads - 1) / kThreads < 2048 ? (chunks + kThreads - 1) / kThreads : 2048);
  if (g.dtype == PBSA_BF16)
    ring_append_kernel<bf16_t><<<blocks, kThreads, 0, s>>>(g, (const bf16_t*)k_new, (const bf16_t*)v_new, ring_head,
                                                          (bf16_t*)k_l, (bf16_t*)v_l, status);
  else
    ring_append_kernel<float><<<blocks, kThreads, 0, s>>>(g, (const float*)k_new, (const float*)v_new, ring_head,
                                                         (float*)k_l, (float*)v_l, status);
  return hipGetLastError();
}

}  // namespace pbsa
