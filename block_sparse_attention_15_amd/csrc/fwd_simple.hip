// Sparse attention forward, plain VALU version (fp32 inputs, and any shape the
// matrix-core kernel does not cover).
//
// Every query token of query block i attends all valid rows of all persistent
// slots plus every token of its K selected local blocks, with one softmax over
// that union (abstract: persistent salient blocks plus a selected local
// neighbourhood; project page: local block-sparse attention with persistent
// blocks).  One workgroup per (query block, head, batch); one lane per query
// token; key/value tiles of up to 64 rows are staged through LDS and read as
// broadcasts.  Online softmax in fp32.  Optionally (blse_p non-null) writes
// each query's log-sum-exp over every slot and selected block, in base 2, the
// input of the token-exact attention mass.
#include "common.h"

namespace pbsa {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(64) void fwd_simple_kernel(Geo g, const T* __restrict__ q, const T* __restrict__ kp,
                                                        const T* __restrict__ vp, const int32_t* __restrict__ plen,
                                                        const T* __restrict__ kl, const T* __restrict__ vl,
                                                        const int32_t* __restrict__ topk, T* __restrict__ o,
                                                        float* __restrict__ lse, float* __restrict__ blse_p,
                                                        float* __restrict__ blse_l) {
  constexpr int kRows = 32;  // rows staged per sub-tile (all lanes read the same row: broadcast)
  __shared__ float ks[kRows][D];
  __shared__ float vs[kRows][D];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  const int lane = threadIdx.x;
  const BlockExt e = block_ext(g, i);
  const bool active = lane < e.len;
  const int tok = active ? block_token(g, e, lane) : 0;
  float qr[D], acc[D];
  const T* qrow = q + (bh * g.ct + tok) * D;
  for (int d = 0; d < D; ++d) {
    qr[d] = active ? to_f<T>(qrow[d]) * g.scale : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int ntiles = g.S + g.K;
  for (int t = 0; t < ntiles; ++t) {
    // rows of this tile: a persistent slot or a selected local block
    int n;
    const T *kb, *vb;
    BlockExt le;
    int loff = 0;
    bool pers = t < g.S;
    float* blse = nullptr;  // where this query's log-sum-exp over the tile's rows goes
    if (blse_p && active)
      blse = pers ? blse_p + (bh * g.S + t) * g.ct + tok : blse_l + (bh * g.K + (t - g.S)) * g.ct + tok;
    if (pers) {
      n = min(plen[bh * g.S + t], g.C);
      kb = kp + (bh * g.S + t) * g.C * D;
      vb = vp + (bh * g.S + t) * g.C * D;
    } else {
      const int p = topk[(bh * g.nq + i) * g.K + (t - g.S)];
      if ((unsigned)p >= (unsigned)g.nl) {  // ids outside the cache are ignored
        if (blse) *blse = -INFINITY;
        continue;
      }
      le = block_ext(g, p % g.nq);
      loff = (p / g.nq) * g.ct;
      n = le.len;
      kb = kl + bh * (size_t)g.NL * D;
      vb = vl + bh * (size_t)g.NL * D;
    }
    float bsum = 0.f;  // probability sum over this tile's rows, relative to m
    for (int r0 = 0; r0 < n; r0 += kRows) {
      const int nr = min(kRows, n - r0);
      __syncthreads();
      for (int r = 0; r < nr; ++r) {
        const size_t row = pers ? (size_t)(r0 + r) : (size_t)(loff + block_token(g, le, r0 + r));
        for (int d = lane; d < D; d += 64) {
          ks[r][d] = to_f<T>(kb[row * D + d]);
          vs[r][d] = to_f<T>(vb[row * D + d]);
        }
      }
      __syncthreads();
      float s[kRows];
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        float a = 0.f;
        if (r < nr) {
          for (int d = 0; d < D; ++d) a = fmaf(qr[d], ks[r][d], a);
          tmax = fmaxf(tmax, a);
        }
        s[r] = a;
      }
      const float mn = fmaxf(m, tmax);
      const float corr = expf(m - mn);
      l *= corr;
      bsum *= corr;
      for (int d = 0; d < D; ++d) acc[d] *= corr;
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        if (r < nr) {
          const float p = expf(s[r] - mn);
          l += p;
          bsum += p;
          for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[r][d], acc[d]);
        }
      }
      m = mn;
    }
    if (blse) *blse = bsum > 0.f ? (m + logf(bsum)) * 1.4426950408889634f : -INFINITY;  // log2 units
  }
  if (!active) return;
  const float inv = 1.0f / l;
  T* orow = o + (bh * g.ct + tok) * D;
  for (int d = 0; d < D; ++d) orow[d] = from_f<T>(acc[d] * inv);
  lse[bh * g.ct + tok] = m + logf(l);
}

}  // namespace

hipError_t launch_fwd_simple(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                             const void* k_l, const void* v_l, const int32_t* topk, void* o, float* lse,
                             float* blse_p, float* blse_l, hipStream_t s) {
  dim3 grid(g.nq, g.H, g.B);
#define PBSA_LAUNCH(T, D)                                                                                   \
  fwd_simple_kernel<T, D><<<grid, 64, 0, s>>>(g, (const T*)q, (const T*)k_p, (const T*)v_p, plen, (const T*)k_l, \
                                              (const T*)v_l, topk, (T*)o, lse, blse_p, blse_l)
  if (g.dtype == PBSA_BF16) {
    if (g.D == 64) PBSA_LAUNCH(bf16_t, 64); else PBSA_LAUNCH(bf16_t, 128);
  } else {
    if (g.D == 64) PBSA_LAUNCH(float, 64); else PBSA_LAUNCH(float, 128);
  }
#undef PBSA_LAUNCH
  return hipGetLastError();
}

}  // namespace pbsa
