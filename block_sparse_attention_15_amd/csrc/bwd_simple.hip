// Sparse attention backward, plain VALU version (fp32 inputs, and any shape
// the matrix-core kernels do not cover) plus the shared preparation kernels.
//
// The project page lists full gradient support for training.  For a fixed
// block mask (persistent slots plus the selected local blocks), the gradients
// are those of softmax attention: P = exp(scale*q.k - lse), dV = P^T dO,
// dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D), dQ = scale * dS K,
// dK = scale * dS^T Q.  Deterministic: dQ is computed query-outer and dK/dV
// key-outer, each with a fixed loop order; no floating-point atomics.
#include "common.h"

namespace pbsa {

namespace {

// grid (ceil(ct/RPW), H, B), 256 threads: each lane loads 16 bytes of a
// query row of O and of dO (EPT elements), TPR = D/EPT lanes share a row
// (RPW = 256/TPR rows per workgroup).  D = rowsum(dO * O): every lane sums
// its EPT products in order, then the row's lanes are combined by a fixed
// xor tree, so the result is the same on every run.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(Geo g, const T* __restrict__ o, const T* __restrict__ dout,
                                                        const float* __restrict__ lse, float* __restrict__ delta,
                                                        float* __restrict__ lse2, float* __restrict__ zrow) {
  constexpr int EPT = 16 / sizeof(T), TPR = D / EPT, RPW = 256 / TPR;
  static_assert(TPR <= 64 && (TPR & (TPR - 1)) == 0, "row lanes");
  const size_t bh = (size_t)blockIdx.z * g.H + blockIdx.y;
  // sentinel row after the last head: rows that do not exist read lse2 = +inf
  // (probability 0) and D = 0; and a zero row that gathers read for key rows
  // that do not exist
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
    if (threadIdx.x == 0) {
      const size_t end = (size_t)g.B * g.H * g.ct;
      lse2[end] = INFINITY;
      delta[end] = 0.f;
    }
    if (threadIdx.x < 16) reinterpret_cast<float4*>(zrow)[threadIdx.x] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int t = blockIdx.x * RPW + threadIdx.x / TPR, c = threadIdx.x % TPR;
  const bool ok = t < g.ct;
  const size_t row = bh * g.ct + (ok ? t : 0);
  const uint4 ov = *reinterpret_cast<const uint4*>(o + row * D + c * EPT);
  const uint4 dv = *reinterpret_cast<const uint4*>(dout + row * D + c * EPT);
  const T* op = reinterpret_cast<const T*>(&ov);
  const T* dp = reinterpret_cast<const T*>(&dv);
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) a = fmaf(to_f<T>(op[e]), to_f<T>(dp[e]), a);
#pragma unroll
  for (int k = TPR / 2; k > 0; k >>= 1) a += __shfl_xor(a, k, TPR);
  if (ok && c == 0) {
    delta[row] = a;
    lse2[row] = lse[row] * 1.4426950408889634f;
  }
}

// grid (H, B): for each local block, the query blocks that selected it, ascending.
// When the (local block x query block) incidence fits in LDS it is built there
// as a byte matrix from the top-k lists, then each thread scans one row.
constexpr int kTindexLds = 48 * 1024;

__global__ __launch_bounds__(256) void bwd_tindex_kernel(Geo g, const int32_t* __restrict__ topk,
                                                         int32_t* __restrict__ tcount, int32_t* __restrict__ tlist) {
  // Incidence of (local block, query block) marked in LDS for as many query
  // blocks at a time as fit, then appended to each local block's list in
  // ascending query-block order; thread t owns local blocks t, t+256, ...
  extern __shared__ unsigned char mark[];
  constexpr int kOwn = 2048 / 256;  // local blocks per thread at most (plan limit)
  const size_t bh = (size_t)blockIdx.y * g.H + blockIdx.x;
  const int32_t* tk = topk + bh * g.nq * g.K;
  const int chunk = max(1, min(g.nq, kTindexLds / g.nl));
  int n[kOwn];
#pragma unroll
  for (int u = 0; u < kOwn; ++u) n[u] = 0;
  for (int i0 = 0; i0 < g.nq; i0 += chunk) {
    const int ni = min(chunk, g.nq - i0);
    __syncthreads();
    for (int x = threadIdx.x; x < g.nl * ni; x += 256) mark[x] = 0;
    __syncthreads();
    for (int x = threadIdx.x; x < ni * g.K; x += 256) {
      const int p = tk[(size_t)i0 * g.K + x];
      if ((unsigned)p < (unsigned)g.nl) mark[p * ni + x / g.K] = 1;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kOwn; ++u) {
      const int p = threadIdx.x + 256 * u;
      if (p < g.nl) {
        int32_t* out = tlist + (bh * g.nl + p) * g.nq;
        for (int i = 0; i < ni; ++i)
          if (mark[p * ni + i]) out[n[u]++] = i0 + i;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kOwn; ++u) {
    const int p = threadIdx.x + 256 * u;
    if (p < g.nl) tcount[bh * g.nl + p] = n[u];
  }
}

// grid 8: the launch order of the key-outer local workgroups.  Workgroup
// b of that kernel runs on XCD b%8 and takes index (b%8)*per + b/8 of the
// (B,H,local block) list (per = ceil(total/8)), so each XCD works through one
// contiguous range of it; here each range is ordered by descending number of
// selecting query blocks (a counting sort over that number, ties in any
// order), so that the longest workgroups start first and the short ones fill
// in behind them.  korder[lo + i] = the list index the i-th workgroup of the
// range takes.
__global__ __launch_bounds__(256) void bwd_korder_kernel(Geo g, const int32_t* __restrict__ tcount,
                                                         int32_t* __restrict__ korder) {
  extern __shared__ int hist[];  // [nq + 1] buckets (bucket nq - count), then [256] partial sums
  int* part = hist + g.nq + 1;
  const int total = g.B * g.H * g.nl, per = (total + 7) / 8;
  const int lo = blockIdx.x * per, hi = min(total, lo + per);
  const int nb = g.nq + 1, cb = (nb + 255) / 256, t = threadIdx.x;
  for (int k = t; k < nb; k += 256) hist[k] = 0;
  __syncthreads();
  for (int e = lo + t; e < hi; e += 256) atomicAdd(&hist[g.nq - min(max(tcount[e], 0), g.nq)], 1);
  __syncthreads();
  // exclusive scan over the buckets: thread t owns buckets [t*cb, t*cb + cb)
  int sum = 0;
  for (int k = t * cb; k < min(nb, t * cb + cb); ++k) sum += hist[k];
  part[t] = sum;
  __syncthreads();
  int base = 0;
  for (int j = 0; j < t; ++j) base += part[j];
  for (int k = t * cb; k < min(nb, t * cb + cb); ++k) {
    const int v = hist[k];
    hist[k] = base;
    base += v;
  }
  __syncthreads();
  for (int e = lo + t; e < hi; e += 256) {
    const int pos = atomicAdd(&hist[g.nq - min(max(tcount[e], 0), g.nq)], 1);
    korder[lo + pos] = e;
  }
}

// dQ, query-outer.  grid (nq, H, B), 64 lanes = query tokens of one block.
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_dq_simple_kernel(Geo g, const T* __restrict__ q, const T* __restrict__ kp,
                                                           const T* __restrict__ vp, const int32_t* __restrict__ plen,
                                                           const T* __restrict__ kl, const T* __restrict__ vl,
                                                           const int32_t* __restrict__ topk,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ delta, const T* __restrict__ dout,
                                                           float* __restrict__ dq) {
  constexpr int kRows = 32;
  __shared__ float ks[kRows][D];
  __shared__ float vs[kRows][D];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  const int lane = threadIdx.x;
  const BlockExt e = block_ext(g, i);
  const bool active = lane < e.len;
  const int tok = active ? block_token(g, e, lane) : 0;
  float qr[D], dor[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qr[d] = active ? to_f<T>(q[(bh * g.ct + tok) * D + d]) : 0.f;
    dor[d] = active ? to_f<T>(dout[(bh * g.ct + tok) * D + d]) : 0.f;
    acc[d] = 0.f;
  }
  const float L = active ? lse[bh * g.ct + tok] : 0.f;
  const float Dl = active ? delta[bh * g.ct + tok] : 0.f;
  for (int t = 0; t < g.S + g.K; ++t) {
    int n;
    const T *kb, *vb;
    BlockExt le;
    int loff = 0;
    const bool pers = t < g.S;
    if (pers) {
      n = min(plen[bh * g.S + t], g.C);
      kb = kp + (bh * g.S + t) * g.C * D;
      vb = vp + (bh * g.S + t) * g.C * D;
    } else {
      const int p = topk[(bh * g.nq + i) * g.K + (t - g.S)];
      if ((unsigned)p >= (unsigned)g.nl) continue;  // ids outside the cache are ignored
      le = block_ext(g, p % g.nq);
      loff = (p / g.nq) * g.ct;
      n = le.len;
      kb = kl + bh * (size_t)g.NL * D;
      vb = vl + bh * (size_t)g.NL * D;
    }
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
      for (int r = 0; r < nr; ++r) {
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(qr[d], ks[r][d], s);
          dp = fmaf(dor[d], vs[r][d], dp);
        }
        const float p = expf(s * g.scale - L);
        const float ds = p * (dp - Dl);
        for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, ks[r][d], acc[d]);
      }
    }
  }
  if (!active) return;
  for (int d = 0; d < D; ++d) dq[(bh * g.ct + tok) * D + d] = acc[d] * g.scale;
}

// dK, dV, key-outer.  grid (S + nl, H, B), 256 threads = 64 key rows x 4
// column quarters.  Persistent slots see every query token (ascending);
// local blocks see the tokens of the query blocks that selected them.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dkv_simple_kernel(Geo g, const T* __restrict__ q, const T* __restrict__ kp,
                                                             const T* __restrict__ vp, const int32_t* __restrict__ plen,
                                                             const T* __restrict__ kl, const T* __restrict__ vl,
                                                             const int32_t* __restrict__ tcount,
                                                             const int32_t* __restrict__ tlist,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ delta,
                                                             const T* __restrict__ dout, float* __restrict__ dkp,
                                                             float* __restrict__ dvp, float* __restrict__ dkl,
                                                             float* __restrict__ dvl) {
  constexpr int Q4 = D / 4;
  constexpr int kTq = 32;  // query tokens staged per tile
  __shared__ float qs[kTq][D];
  __shared__ float ds_[kTq][D];
  __shared__ float ls[kTq], dls[kTq];
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * g.H + h;
  const int r = threadIdx.x / 4, c = threadIdx.x & 3;
  const bool pers = (int)blockIdx.x < g.S;
  const int s_or_p = pers ? blockIdx.x : blockIdx.x - g.S;
  int n, loff = 0;
  BlockExt le;
  const T *kb, *vb;
  if (pers) {
    n = min(plen[bh * g.S + s_or_p], g.C);
    kb = kp + (bh * g.S + s_or_p) * g.C * D;
    vb = vp + (bh * g.S + s_or_p) * g.C * D;
  } else {
    le = block_ext(g, s_or_p % g.nq);
    loff = (s_or_p / g.nq) * g.ct;
    n = le.len;
    kb = kl + bh * (size_t)g.NL * D;
    vb = vl + bh * (size_t)g.NL * D;
  }
  const bool act = r < n;
  const size_t krow = act ? (pers ? (size_t)r : (size_t)(loff + block_token(g, le, r))) : 0;
  float kr[Q4], vr[Q4], dk[Q4], dv[Q4];
  for (int d = 0; d < Q4; ++d) {
    kr[d] = act ? to_f<T>(kb[krow * D + c * Q4 + d]) : 0.f;
    vr[d] = act ? to_f<T>(vb[krow * D + c * Q4 + d]) : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  // query token list: all tokens (persistent) or the selecting query blocks' tokens
  const int nsel = pers ? 1 : tcount[bh * g.nl + s_or_p];
  const int32_t* sel = pers ? nullptr : tlist + (bh * g.nl + s_or_p) * g.nq;
  for (int si = 0; si < nsel; ++si) {
    BlockExt qe;
    int ntok;
    if (pers) {
      ntok = g.ct;
    } else {
      qe = block_ext(g, sel[si]);
      ntok = qe.len;
    }
    for (int t0 = 0; t0 < ntok; t0 += kTq) {
      const int nt = min(kTq, ntok - t0);
      __syncthreads();
      for (int x = threadIdx.x; x < nt * D; x += 256) {
        const int tt = x / D, d = x - tt * D;
        const int tok = pers ? t0 + tt : block_token(g, qe, t0 + tt);
        qs[tt][d] = to_f<T>(q[(bh * g.ct + tok) * D + d]);
        ds_[tt][d] = to_f<T>(dout[(bh * g.ct + tok) * D + d]);
        if (d == 0) {
          ls[tt] = lse[bh * g.ct + tok];
          dls[tt] = delta[bh * g.ct + tok];
        }
      }
      __syncthreads();
      for (int tt = 0; tt < nt; ++tt) {
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < Q4; ++d) {
          s = fmaf(qs[tt][c * Q4 + d], kr[d], s);
          dp = fmaf(ds_[tt][c * Q4 + d], vr[d], dp);
        }
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        dp += __shfl_xor(dp, 1, 64);
        dp += __shfl_xor(dp, 2, 64);
        const float p = act ? expf(s * g.scale - ls[tt]) : 0.f;
        const float dsv = p * (dp - dls[tt]);
        for (int d = 0; d < Q4; ++d) {
          dv[d] = fmaf(p, ds_[tt][c * Q4 + d], dv[d]);
          dk[d] = fmaf(dsv, qs[tt][c * Q4 + d], dk[d]);
        }
      }
    }
  }
  if (pers) {
    if (r >= g.C) return;
    const size_t o = ((bh * g.S + s_or_p) * g.C + r) * D + c * Q4;
    for (int d = 0; d < Q4; ++d) {
      dkp[o + d] = act ? dk[d] * g.scale : 0.f;
      dvp[o + d] = act ? dv[d] : 0.f;
    }
  } else if (act) {
    const size_t o = (bh * g.NL + krow) * D + c * Q4;
    for (int d = 0; d < Q4; ++d) {
      dkl[o + d] = dk[d] * g.scale;
      dvl[o + d] = dv[d];
    }
  }
}

}  // namespace

hipError_t launch_bwd_delta(const Geo& g, const void* o, const void* dout, const float* lse, WsBwd ws,
                            hipStream_t s) {
#define PBSA_DELTA(T, DD)                                                                              \
  bwd_delta_kernel<T, DD><<<dim3((g.ct + 256 / (DD * sizeof(T) / 16) - 1) / (256 / (DD * sizeof(T) / 16)), g.H, g.B), \
                           256, 0, s>>>(g, (const T*)o, (const T*)dout, lse, ws.delta, ws.lse2, ws.zrow)
  if (g.dtype == PBSA_BF16) {
    if (g.D == 128) PBSA_DELTA(bf16_t, 128); else PBSA_DELTA(bf16_t, 64);
  } else {
    if (g.D == 128) PBSA_DELTA(float, 128); else PBSA_DELTA(float, 64);
  }
#undef PBSA_DELTA
  return hipGetLastError();
}

hipError_t launch_bwd_index(const Geo& g, const int32_t* topk, WsBwd ws, hipStream_t s) {
  const size_t shm = (size_t)g.nl * max(1, min(g.nq, kTindexLds / g.nl));
  bwd_tindex_kernel<<<dim3(g.H, g.B), 256, shm, s>>>(g, topk, ws.tcount, ws.tlist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_korder_kernel<<<8, 256, (size_t)(g.nq + 1 + 256) * 4, s>>>(g, ws.tcount, ws.korder);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const Geo& g, const void* o, const void* dout, const float* lse, const int32_t* topk,
                           WsBwd ws, hipStream_t s) {
  hipError_t e = launch_bwd_delta(g, o, dout, lse, ws, s);
  return e != hipSuccess ? e : launch_bwd_index(g, topk, ws, s);
}

hipError_t launch_bwd_simple(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                             const void* k_l, const void* v_l, const int32_t* topk, const float* lse,
                             const void* dout, float* dq, float* dk_p, float* dv_p, float* dk_l, float* dv_l,
                             WsBwd ws, hipStream_t s) {
#define PBSA_LAUNCH(T, D)                                                                                       \
  do {                                                                                                          \
    bwd_dq_simple_kernel<T, D><<<dim3(g.nq, g.H, g.B), 64, 0, s>>>(g, (const T*)q, (const T*)k_p, (const T*)v_p, \
                                                                  plen, (const T*)k_l, (const T*)v_l, topk, lse,  \
                                                                  ws.delta, (const T*)dout, dq);                  \
    bwd_dkv_simple_kernel<T, D><<<dim3(g.S + g.nl, g.H, g.B), 256, 0, s>>>(                                      \
        g, (const T*)q, (const T*)k_p, (const T*)v_p, plen, (const T*)k_l, (const T*)v_l, ws.tcount, ws.tlist,   \
        lse, ws.delta, (const T*)dout, dk_p, dv_p, dk_l, dv_l);                                                   \
  } while (0)
  if (g.dtype == PBSA_BF16) {
    if (g.D == 64) PBSA_LAUNCH(bf16_t, 64); else PBSA_LAUNCH(bf16_t, 128);
  } else {
    if (g.D == 64) PBSA_LAUNCH(float, 64); else PBSA_LAUNCH(float, 128);
  }
#undef PBSA_LAUNCH
  return hipGetLastError();
}

}  // namespace pbsa
