// Persistent-cache update.
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
// Two launches:
//  1. one workgroup per (batch, head) takes the head's decision once from the
//     masses (about 1 KB): a two-phase wavefront radix select of the
//     (S - Z)-th largest candidate key from registers, then ballot prefix
//     counts that pair vacated slots with admitted blocks; it writes the plan
//     of every slot to the workspace;
//  2. one workgroup per (batch, head, group of kSlotsPerWg slots) carries out
//     the plan of its slots (16-byte coalesced row copies, zero padding,
//     pooled keys, new lengths and source ids), and workgroup 0 advances the
//     ring head and the step counter.  Workgroups of the second launch read
//     only the plan, never the lengths another one writes.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace pbsa {
namespace {

constexpr int kThreads = 256;
constexpr int kSlotsPerWg = 2;

__device__ __forceinline__ int wave_count(bool p) { return __builtin_popcountll(__builtin_amdgcn_ballot_w64(p)); }

__device__ __forceinline__ unsigned mass_key(float m) {
  unsigned u = m == 0.f ? 0u : __float_as_uint(m);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Thresholds of the K largest of the keys (hi, lo) held in registers, lane l
// holding keys l, l+64, ... (hi = 0: not a candidate): the K-th largest hi
// value thr and, when several keys share it and not all fit, the smallest lo
// taken among those (thr2; 0 when every key with hi == thr is taken).  A key
// is among the K largest iff hi > thr || (hi == thr && lo >= thr2).  Two radix
// passes, one bit per ballot round (see select_top in score.hip).
template <int KPL>
__device__ __forceinline__ void radix_threshold(const unsigned (&hi)[KPL], const unsigned (&lo)[KPL], int K,
                                                unsigned& thr, unsigned& thr2) {
  thr = 0u;
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
  const int need = K - n_gt;
  thr2 = 0u;
  if (n_eq > need) {
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned cand = thr2 | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < KPL; ++u) cnt += wave_count(hi[u] == thr && lo[u] >= cand);
      if (cnt >= need) thr2 = cand;
    }
  }
}

// One workgroup per (batch, head): the head's whole decision, taken once.
// Loads the head's masses, slot lengths, ring head and step counter in one
// round, forms the candidate keys in LDS, and in one wavefront from
// registers selects the (S - Z) largest, lists the admitted entrants
// ascending, ranks the vacated slots ascending and writes the plan of every
// slot: -2 keep, -1 empty, e >= 0 fill from evicted block e.  meta[0] and
// meta[1] (written by head 0): the ring position of the evicted chunk and
// the step id, for the copy kernel, which reads neither ring head nor step
// counter.
template <int KPL>
__global__ __launch_bounds__(kThreads) void update_decide_kernel(Geo g, const float* __restrict__ mass,
                                                                 const int32_t* __restrict__ ring_head,
                                                                 const int32_t* __restrict__ step_counter,
                                                                 const int32_t* __restrict__ plen,
                                                                 int32_t* __restrict__ plan, int32_t* __restrict__ meta,
                                                                 int32_t* __restrict__ n_rep,
                                                                 uint32_t* __restrict__ status) {
  extern __shared__ unsigned sk[];
  if (g.S == 0) {  // no persistent memory: nothing is admitted
    if (threadIdx.x == 0) n_rep[blockIdx.x] = 0;
    return;
  }
  const int NC = g.S + g.nq;
  unsigned* hi = sk;                      // [NC] candidate keys (0: not a candidate)
  unsigned* lo = hi + NC;                 // [NC]
  int* alist = (int*)(lo + NC);           // [nq] admitted entrants, ascending
  float* mall = (float*)(alist + g.nq);   // [S + nl]
  int* lall = (int*)(mall + g.S + g.nl);  // [S]
  const size_t bh = blockIdx.x;
  const float* mrow = mass + bh * (g.S + g.nl);
  const int32_t* prow = plen + bh * g.S;
  // every mass and length of the head is loaded while the ring head is: the
  // evicted chunk's masses are picked from LDS once it is known
  for (int c = threadIdx.x; c < g.S + g.nl; c += kThreads) mall[c] = mrow[c];
  for (int c = threadIdx.x; c < g.S; c += kThreads) lall[c] = prow[c];
  const int old = read_ring_head(ring_head, g.R, status);
  const int step_id = read_step(step_counter, g.nq, status);
  __syncthreads();
  // sink slots, and evicted blocks reserved for an empty sink slot, are not candidates
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    const bool slot = c < g.S;
    const bool valid = slot ? (c >= g.Z && lall[c] > 0) : !(c - g.S < g.Z && lall[c - g.S] == 0);
    const float m = slot ? mall[c] : mall[g.S + old * g.nq + (c - g.S)];
    hi[c] = valid ? mass_key(m) : 0u;
    lo[c] = 0xffffffffu - (unsigned)c;  // ties: slots before entrants, lower index first
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  // one wavefront decides from registers: candidate c = lane + 64 u
  const int lane = threadIdx.x;
  const unsigned long long below = (1ull << lane) - 1;
  unsigned hr[KPL], lr[KPL];
  int nvalid = 0;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int c = lane + 64 * u;
    hr[u] = c < NC ? hi[c] : 0u;
    lr[u] = c < NC ? lo[c] : 0u;
    nvalid += wave_count(hr[u] != 0u);
  }
  unsigned thr = 1u, thr2 = 0u;  // every candidate stays when they all fit
  if (nvalid > g.S - g.Z) radix_threshold<KPL>(hr, lr, g.S - g.Z, thr, thr2);
  // admitted entrants (kept, and not a sink fill) listed ascending; the rank
  // of a vacated slot among the vacated slots (ascending) picks its entrant
  int n_adm = 0, nvac = 0, vrank[KPL];
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int c = lane + 64 * u;
    const bool kept = hr[u] != 0u && (hr[u] > thr || (hr[u] == thr && lr[u] >= thr2));
    const bool adm = c >= g.S && c < NC && kept;
    const bool vac = c >= g.Z && c < g.S && !kept;
    const unsigned long long ma = __builtin_amdgcn_ballot_w64(adm), mv = __builtin_amdgcn_ballot_w64(vac);
    if (adm) alist[n_adm + __builtin_popcountll(ma & below)] = c - g.S;
    vrank[u] = vac ? nvac + __builtin_popcountll(mv & below) : -1;
    n_adm += __builtin_popcountll(ma);
    nvac += __builtin_popcountll(mv);
  }
  int n_sink_fill = 0;
  for (int s0 = 0; s0 < g.Z; s0 += 64) n_sink_fill += wave_count(s0 + lane < g.Z && lall[s0 + lane] == 0);
  __builtin_amdgcn_wave_barrier();  // alist entries of every lane written before they are read
  int32_t* prow_plan = plan + bh * g.S;
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int c = lane + 64 * u;
    if (c < g.S) {
      int e;
      if (c < g.Z)  // sink slot: a valid one stays, an empty one takes the evicted block of its index
        e = lall[c] > 0 ? -2 : c;
      else
        e = vrank[u] < 0 ? -2 : (vrank[u] < n_adm ? alist[vrank[u]] : -1);
      prow_plan[c] = e;
    }
  }
  if (lane == 0) {
    n_rep[bh] = n_adm + n_sink_fill;
    if (bh == 0) {
      meta[0] = old;
      meta[1] = step_id;
    }
  }
}

// 1-D grid over (B, H, group of kSlotsPerWg slots): carries out the plan of
// its slots -- rows of each filled slot copied from the evicted chunk (the
// ring token of each row computed once, into LDS; every load issued before the
// first store; zero padding), pooled keys copied, emptied slots zeroed, new
// lengths and source ids written -- and workgroup 0 advances the ring head
// and the step counter (no workgroup of this launch reads them: the evicted
// chunk's position and the step id come from meta).
template <typename T>
__global__ __launch_bounds__(kThreads) void update_copy_kernel(Geo g, const int32_t* __restrict__ plan,
                                                               const int32_t* __restrict__ meta,
                                                               const T* __restrict__ kl, const T* __restrict__ vl,
                                                               const float* __restrict__ kbar_l,
                                                               T* __restrict__ kp, T* __restrict__ vp,
                                                               float* __restrict__ pkbar, int32_t* __restrict__ plen,
                                                               int32_t* __restrict__ psrc,
                                                               int32_t* __restrict__ ring_head,
                                                               int32_t* __restrict__ step_counter) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *ring_head = (ring_wrap(*ring_head, g.R) + 1) % g.R;
    *step_counter += 1;
  }
  if (g.S == 0) return;
  __shared__ int s_plan[kSlotsPerWg];
  __shared__ int s_tok[kSlotsPerWg][64];  // ring token of each row of each filled slot's block
  const int ngrp = (g.S + kSlotsPerWg - 1) / kSlotsPerWg;
  const int grp = blockIdx.x % ngrp;
  const size_t bh = blockIdx.x / ngrp;
  const int old = meta[0], step_id = meta[1];
  if ((int)threadIdx.x < kSlotsPerWg) {
    const int s = grp * kSlotsPerWg + threadIdx.x;
    s_plan[threadIdx.x] = s < g.S ? plan[bh * g.S + s] : -2;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < kSlotsPerWg * 64; x += kThreads) {
    const int k = x >> 6, r = x & 63;
    const int e = s_plan[k];
    int tok = -1;
    if (e >= 0) {
      const BlockExt be = block_ext(g, e);
      if (r < be.len) tok = block_token(g, be, r);
    }
    s_tok[k][r] = tok;
  }
  __syncthreads();
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kCopyIt = 64 * (128 / kVec) / kThreads;  // 16-byte chunks per thread of a 64-row, d<=128 slot
  const int cpr = g.D / kVec;
  uint4 kv[kSlotsPerWg][kCopyIt], vv[kSlotsPerWg][kCopyIt];
  float kb[kSlotsPerWg];
  const size_t ring0 = bh * g.NL + (size_t)old * g.ct;  // first token of the evicted chunk
#pragma unroll
  for (int k = 0; k < kSlotsPerWg; ++k) {
    const int e = s_plan[k];
    kb[k] = 0.f;
#pragma unroll
    for (int u = 0; u < kCopyIt; ++u) kv[k][u] = vv[k][u] = make_uint4(0, 0, 0, 0);
    if (e < 0) continue;  // uniform: kept or emptied slots load nothing
    if ((int)threadIdx.x < g.D) kb[k] = kbar_l[(bh * g.nl + old * g.nq + e) * g.D + threadIdx.x];
    const int tok0 = s_tok[k][0];  // rows past the block's length load its first row (discarded)
#pragma unroll
    for (int u = 0; u < kCopyIt; ++u) {
      const int c = threadIdx.x + kThreads * u, r = c / cpr, q = c - r * cpr;
      const int tok = r < 64 ? s_tok[k][r] : -1;
      const bool on = tok >= 0;
      const size_t src = (ring0 + (on ? tok : tok0)) * (size_t)g.D + q * kVec;
      const uint4 kx = *reinterpret_cast<const uint4*>(kl + src);
      const uint4 vx = *reinterpret_cast<const uint4*>(vl + src);
      if (on) {
        kv[k][u] = kx;
        vv[k][u] = vx;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kSlotsPerWg; ++k) {
    const int s = grp * kSlotsPerWg + k;
    if (s >= g.S) break;
    const int e = s_plan[k];
    if (e == -2) continue;
    const size_t bs = bh * g.S + s;
    if (threadIdx.x == 0) {
      plen[bs] = e >= 0 ? block_ext(g, e).len : 0;
      psrc[bs] = e >= 0 ? step_id * g.nq + e : kEmptySrc;
    }
    if ((int)threadIdx.x < g.D) pkbar[bs * g.D + threadIdx.x] = kb[k];
    const size_t dst = bs * (size_t)g.C * g.D;
#pragma unroll
    for (int u = 0; u < kCopyIt; ++u) {
      const int c = threadIdx.x + kThreads * u, r = c / cpr, q = c - r * cpr;
      if (c < g.C * cpr) {
        *reinterpret_cast<uint4*>(kp + dst + (size_t)r * g.D + q * kVec) = kv[k][u];
        *reinterpret_cast<uint4*>(vp + dst + (size_t)r * g.D + q * kVec) = vv[k][u];
      }
    }
  }
}

}  // namespace

size_t update_workspace(const Geo& g) {
  const size_t n = (size_t)g.B * g.H * g.S * 4;
  return ((n + 255) & ~size_t(255)) + 256;  // plan, then meta
}

hipError_t launch_persist_update(const Geo& g, const float* mass, const void* k_l, const void* v_l,
                                 const float* kbar_l, int32_t* ring_head, int32_t* step_counter, void* k_p,
                                 void* v_p, int32_t* plen, int32_t* psrc, float* pkbar, int32_t* n_rep,
                                 void* ws, uint32_t* status, hipStream_t s) {
  const size_t n = (size_t)g.B * g.H * g.S * 4;
  int32_t* plan = (int32_t*)ws;
  int32_t* meta = (int32_t*)((char*)ws + ((n + 255) & ~size_t(255)));
  const int NC = g.S + g.nq;
  const size_t shm = (size_t)NC * 8 + (size_t)g.nq * 4 + (size_t)(g.S + g.nl) * 4 + (size_t)g.S * 4;
  auto go = [&](auto kpl) {
    constexpr int KPL = decltype(kpl)::value;
    static PerDeviceOnce attr;
    const hipError_t ea = attr.run([] {
      return hipFuncSetAttribute((const void*)update_decide_kernel<KPL>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 128 * 1024);
    });
    if (ea != hipSuccess) return ea;
    update_decide_kernel<KPL><<<g.B * g.H, kThreads, shm, s>>>(g, mass, ring_head, step_counter, plen, plan, meta,
                                                               n_rep, status);
    return hipGetLastError();
  };
  // candidates per lane: each radix round of the decision costs one ballot per key a lane holds
  hipError_t e = NC <= 256    ? go(std::integral_constant<int, 4>{})
                 : NC <= 512  ? go(std::integral_constant<int, 8>{})
                 : NC <= 1024 ? go(std::integral_constant<int, 16>{})
                              : go(std::integral_constant<int, 64>{});
  if (e != hipSuccess) return e;
  const int grid = std::max(1, g.B * g.H * ((g.S + kSlotsPerWg - 1) / kSlotsPerWg));
  if (g.dtype == PBSA_BF16)
    update_copy_kernel<bf16_t><<<grid, kThreads, 0, s>>>(g, plan, meta, (const bf16_t*)k_l, (const bf16_t*)v_l, kbar_l,
                                                         (bf16_t*)k_p, (bf16_t*)v_p, pkbar, plen, psrc, ring_head,
                                                         step_counter);
  else
    update_copy_kernel<float><<<grid, kThreads, 0, s>>>(g, plan, meta, (const float*)k_l, (const float*)v_l, kbar_l,
                                                        (float*)k_p, (float*)v_p, pkbar, plen, psrc, ring_head,
                                                        step_counter);
  return hipGetLastError();
}

}  // namespace pbsa
