// Shared host/device definitions of the PBSA HIP library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pbsa.h"

namespace pbsa {

// Derived geometry, passed by value to every kernel.
struct Geo {
  int B, H, D;
  int fh, fw, bt, bh, bw, cf;
  int ft;      // tokens per frame
  int ct;      // tokens per chunk (= query tokens)
  int nbr;     // block rows per frame
  int nbc;     // block columns per frame
  int bpg;     // blocks per block_t-frame group
  int nq;      // blocks per chunk = query blocks
  int R;       // local ring chunk slots
  int nl;      // local blocks
  int NL;      // local tokens
  int S;       // persistent slots
  int C;       // rows per persistent slot
  int K;       // top-k
  float scale; // softmax scale
  int dtype;   // pbsa_dtype
  int Z;       // pinned sink slots (leading persistent slots)
  int ds;      // the MFMA backward stores the persistent dS tiles (else its dK pass recomputes dS)
};

// Extent of chunk block j: base token offset inside the chunk, frames, rows,
// columns and the total token count.  Block-row-major within a frame group.
struct BlockExt {
  int f0, r0, c0, nt, nh, nw, len;
};

__host__ __device__ inline BlockExt block_ext(const Geo& g, int j) {
  BlockExt e;
  int grp = j / g.bpg, rem = j - grp * g.bpg;
  int br = rem / g.nbc, bc = rem - br * g.nbc;
  e.f0 = grp * g.bt;
  e.r0 = br * g.bh;
  e.c0 = bc * g.bw;
  e.nt = g.bt;
  e.nh = min(g.bh, g.fh - e.r0);
  e.nw = min(g.bw, g.fw - e.c0);
  e.len = e.nt * e.nh * e.nw;
  return e;
}

// Token offset (inside the chunk) of the i-th token of a block, raster order.
__host__ __device__ inline int block_token(const Geo& g, const BlockExt& e, int i) {
  int hw = e.nh * e.nw;
  int f = i / hw, rem = i - f * hw;
  int r = rem / e.nw, c = rem - r * e.nw;
  return (e.f0 + f) * g.ft + (e.r0 + r) * g.fw + e.c0 + c;
}

// floor(n / d) for 0 <= n < 2^20 and 1 <= d < 2^20 by one multiply with the
// hardware reciprocal: (n + 1/2) / d lies at least 1 / (2d) from an integer,
// and the product's relative error (reciprocal 1 ulp, product 1/2 ulp) keeps
// it closer than that for n below 2^20.
__device__ __forceinline__ int small_div(int n, int d) {
  return (int)(((float)n + 0.5f) * __builtin_amdgcn_rcpf((float)d));
}

// Local block p of the ring (chunk slot p / nq, chunk block p mod nq): the
// ring token of its first row, its length, and the extents that place row r.
struct LocBlock {
  int base, len, nw, hw;
};

__device__ __forceinline__ LocBlock loc_block(const Geo& g, int p) {
  const int cp = p / g.nq, j = p - cp * g.nq;
  const BlockExt e = block_ext(g, j);
  return {cp * g.ct + e.f0 * g.ft + e.r0 * g.fw + e.c0, e.len, e.nw, e.nh * e.nw};
}

// Ring token of row r (0 <= r < b.len, r < 2^20) of a local block, raster order.
__device__ __forceinline__ int loc_row(const Geo& g, const LocBlock& b, int r) {
  const int f = small_div(r, b.hw), rem = r - f * b.hw;
  const int y = small_div(rem, b.nw);
  return b.base + f * g.ft + y * g.fw + (rem - y * b.nw);
}

// ---------------------------------------------------------------------------
// Device-resident ring state
// ---------------------------------------------------------------------------
// Sticky error bits of the library's device status word (pbsa_device_status).
constexpr uint32_t kStatusRingHead = 1u;     // a ring head outside [0, R) was read
constexpr uint32_t kStatusStepCounter = 2u;  // a step counter outside [0, 2^31 / blocks per chunk) was read

// A stored ring head reduced into [0, R): the non-negative remainder, so that
// every chunk slot derived from it is in bounds whatever the stored value.
__host__ __device__ inline int ring_wrap(int v, int R) {
  const int r = v % R;
  return r < 0 ? r + R : r;
}

// The ring head read on the device, reduced into [0, R); a stored value
// outside [0, R) raises kStatusRingHead in *status.
__device__ inline int read_ring_head(const int32_t* ring_head, int R, uint32_t* status) {
  const int v = *ring_head;
  if ((unsigned)v >= (unsigned)R) atomicOr(status, kStatusRingHead);
  return ring_wrap(v, R);
}

// The step counter read on the device; a value for which step*nq would leave
// the int32 source ids raises kStatusStepCounter (the ids it produces are
// then not unique, nothing is out of bounds).
__device__ inline int read_step(const int32_t* step_counter, int nq, uint32_t* status) {
  const int v = *step_counter;
  if (v < 0 || v > INT32_MAX / nq - 1) atomicOr(status, kStatusStepCounter);
  return v;
}

// Address of the device status word on the current device (looked up once
// per device).
hipError_t device_status_word(uint32_t** out);

// Wait until at most N of this wave's global loads are in flight and all of
// its LDS reads have returned, then the workgroup barrier.  Unlike
// __syncthreads this leaves the newest LDS-bound loads running.  The wait is
// the s_waitcnt builtin, which the compiler's own wait placement takes into
// account (it then knows every older load has landed); the empty asm
// statements keep memory accesses from moving across.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  asm volatile("" ::: "memory");
#if PBSA_LDS_RACE_CHECK
  __builtin_amdgcn_s_waitcnt(0);  // check build: every load and LDS access done first
#else
  __builtin_amdgcn_s_waitcnt(0x070 | N);  // vmcnt(N), lgkmcnt(0), expcnt not waited for
#endif
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One LDS-bound load (global_load_lds).  The LDS-race check build
// (PBSA_LDS_RACE_CHECK, a second library built beside the product one) waits
// for each at once, so its bytes land as early as its issue allows, and every
// step barrier drains all loads in flight: a kernel whose waves read a buffer
// before its rows land, or issue rows into a buffer that another wave still
// reads, then gives different results from the product build, which keeps
// the loads in flight across the barriers.  The two builds must agree bitwise.
#if PBSA_LDS_RACE_CHECK
#define PBSA_LDS_LOAD(src, dst, size, off, aux)                \
  do {                                                         \
    __builtin_amdgcn_global_load_lds(src, dst, size, off, aux); \
    __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */          \
  } while (0)
#else
#define PBSA_LDS_LOAD(src, dst, size, off, aux) __builtin_amdgcn_global_load_lds(src, dst, size, off, aux)
#endif

// The valid rows of a head's persistent slots numbered consecutively
// ("packed" rows, slot order): pre[s] = first packed row of slot s (prefix
// sums of the lengths clamped to [0, C]), pre[S] = the head's valid rows;
// with rowtab, rowtab[p] = s*C + r for packed row p (row r of slot s).  Every
// thread of the workgroup calls it (it has barriers); returns pre[S].
__device__ inline int packed_rows(const int32_t* plen, int S, int C, int* pre, int* rowtab, int nthreads) {
  const int lane = threadIdx.x & 63;
  for (int x = threadIdx.x; x < S; x += nthreads) pre[x] = min(max(plen[x], 0), C);
  __syncthreads();
  if (threadIdx.x < 64) {  // wave 0: exclusive scan, 64 slots per round
    int run = 0;
    for (int s0 = 0; s0 < S; s0 += 64) {
      const int sl = s0 + lane;
      const int n = sl < S ? pre[sl] : 0;
      int x = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      __builtin_amdgcn_wave_barrier();
      if (sl < S) pre[sl] = run + x - n;
      run += __shfl(x, 63, 64);
    }
    if (lane == 0) pre[S] = run;
  }
  __syncthreads();
  if (rowtab) {
    for (int x = threadIdx.x; x < S * C; x += nthreads) {
      const int sl = x / C, r = x - sl * C;
      const int b0 = pre[sl];
      if (r < pre[sl + 1] - b0) rowtab[b0 + r] = x;
    }
    __syncthreads();
  }
  return pre[S];
}

// Slot holding packed row p (0 <= p < pre[S]): the last s with pre[s] <= p
// (slots without rows share their start with the next slot).
__device__ inline int packed_slot(const int* pre, int S, int p) {
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= p) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Runs a set-up step (kernel attributes) once per device: run(f) calls f
// with the caller's device current the first time that device is seen and
// returns its status; later calls on that device return hipSuccess.  A failed
// f is tried again on the next call.  Thread-safe.
struct PerDeviceOnce {
  static constexpr int kMaxDevices = 64;
  std::mutex mu;
  bool done[kMaxDevices] = {};
  template <typename F>
  hipError_t run(F f) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (done[dev]) return hipSuccess;
    if ((e = f()) != hipSuccess) return e;
    done[dev] = true;
    return hipSuccess;
  }
};

// ---------------------------------------------------------------------------
// Element conversion
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// float -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t x) { return bf2f(x); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f2bf(x); }

constexpr int32_t kEmptySrc = INT32_MIN;

// ---------------------------------------------------------------------------
// Launchers implemented in the kernel translation units.  Each returns the
// hipError_t of its launches.
// ---------------------------------------------------------------------------
// Bytes of the persistent dS tiles that the MFMA backward passes from its dQ
// kernel to its dK kernel, whether or not g.ds selects that path.
size_t bwd_ds_tile_bytes(const Geo& g);
// The same where g.ds is set, else 0.
size_t bwd_ds_bytes(const Geo& g);
bool bwd_mfma_supported(const Geo& g);

// Query blocks per score workgroup at a geometry (4, 2 or 1: the largest whose LDS fits).
int score_qpw(const Geo& g);
struct WsScore {
  float* part;  // [B,H,groups,S+nl]  column sums of each score workgroup's softmax rows
};
size_t score_workspace(const Geo& g);
// Device address and size of the static scratch array of the allocation-free
// scoring entry point on the current device (looked up once per device).
hipError_t score_static_scratch(void** out, size_t* bytes);
hipError_t launch_pool_slots(const Geo& g, const void* k_p, const int32_t* plen, float* kbar, hipStream_t s);
// Pooled keys of every physical local block of the ring.
hipError_t launch_pool_local(const Geo& g, const void* k_l, float* kbar_l, hipStream_t s);
hipError_t launch_score_select(const Geo& g, const void* q, const float* kbar_l, const int32_t* ring_head,
                               const float* kbar_p, const int32_t* plen, int32_t* topk, float* mass, WsScore ws,
                               uint32_t* status, hipStream_t s);
// blse_p / blse_l: NULL, or [B,H,S,ct] / [B,H,K,ct] outputs of each query's
// log-sum-exp over each persistent slot / each of its selected local blocks,
// in base 2 (log2 of the sum of exp of the scaled scores; -inf where the slot
// or block holds no valid row).
hipError_t launch_fwd(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                      const void* k_l, const void* v_l, const int32_t* topk, void* o, float* lse, void* ws,
                      float* blse_p, float* blse_l, hipStream_t s);
size_t fwd_workspace(const Geo& g);
// Token-exact mass from the block log-sum-exps and the final LSE (natural
// log): mass[s] = sum_t 2^(blse_p[s][t] - lse[t]*log2e); mass[S+p] = sum over
// query blocks i and their selections k with topk[i][k] = p of
// sum_{t in i} 2^(blse_l[k][t] - lse[t]*log2e).  part: [B,H,nq,nl] scratch.
hipError_t launch_token_mass(const Geo& g, const int32_t* plen, const int32_t* topk, const float* lse,
                             const float* blse_p, const float* blse_l, float* part, float* mass, hipStream_t s);
struct WsBwd {
  float* delta;     // [B,H,Nq] + 1  rowsum(dO * O); the extra entry is 0
  float* zrow;      // 256 zero bytes after delta: a zero row (head_dim <= 128 bf16) for gathers
  float* lse2;      // [B,H,Nq] + 1  lse * log2(e); the extra entry is +inf (rows that do not exist)
  int32_t* tcount;  // [B,H,nl]      query blocks that selected each local block
  int32_t* tlist;   // [B,H,nl,nq]   their ids, ascending
  int32_t* korder;  // [B,H,nl]      local blocks in key-outer launch order (see bwd_korder_kernel)
  void* dsb;        // bwd_ds_bytes: dS of the persistent slots as bf16 32x32 tiles (MFMA path)
};
// Backward preparation: D = rowsum(dO * O) and lse * log2(e) (with the
// sentinel entries), and the key-block -> query-block index with its launch
// order.
hipError_t launch_bwd_delta(const Geo& g, const void* o, const void* dout, const float* lse, WsBwd ws,
                            hipStream_t s);
hipError_t launch_bwd_index(const Geo& g, const int32_t* topk, WsBwd ws, hipStream_t s);
hipError_t launch_bwd(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                      const void* k_l, const void* v_l, const int32_t* topk, const void* o,
                      const float* lse, const void* dout, float* dq, float* dk_p, float* dv_p,
                      float* dk_l, float* dv_l, WsBwd ws, hipStream_t s);
size_t update_workspace(const Geo& g);
hipError_t launch_persist_update(const Geo& g, const float* mass, const void* k_l, const void* v_l,
                                 const float* kbar_l, int32_t* ring_head, int32_t* step_counter, void* k_p,
                                 void* v_p, int32_t* plen, int32_t* psrc, float* pkbar, int32_t* n_rep,
                                 void* ws, uint32_t* status, hipStream_t s);
// Copy a new chunk into the newest ring slot and pool its keys into kbar_l.
hipError_t launch_ring_append(const Geo& g, const void* k_new, const void* v_new, const int32_t* ring_head,
                              void* k_l, void* v_l, float* kbar_l, uint32_t* status, hipStream_t s);

}  // namespace pbsa
