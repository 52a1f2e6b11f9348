// Sparse attention forward on the gfx950 matrix cores (bf16 inputs, head_dim
// 64 or 128).
//
// What is computed (abstract and project page of Sparse Forcing): every query
// token of query block i attends all valid rows of every persistent slot and
// every token of its K selected local blocks, with one softmax over that union.
//
// Mapping to CDNA4
// ----------------
//  * Two kernels.  The persistent slots are the same for every query of a
//    head, so the first kernel is a dense attention of all of a head's
//    queries (contiguous 256-row tiles, 8 waves x 32 rows, two waves per
//    SIMD so one wave's softmax overlaps the other's MFMAs) against the
//    compact persistent memory: the valid rows of all slots are numbered
//    through a row table in LDS and streamed as dense 64-key steps, each
//    staged once in LDS for the eight waves (fwd_pers2_kernel; the
//    token-mass variant, which needs per-slot sums, keeps one slot per step:
//    fwd_pers_kernel).  It writes a normalised fp32 partial output and its
//    log-sum-exp.
//    The second kernel handles the selected local blocks, which differ per
//    query block: one query block per workgroup (2 waves = 2 tiles of 32
//    queries, four workgroups per CU), so a step's barrier waits only for
//    the two waves of one block; it merges its result with the persistent
//    partial by log-sum-exp and writes O (bf16) and LSE.
//  * The products are computed transposed with v_mfma_f32_32x32x16_bf16:
//    S^T = K Q^T (keys x queries) and O^T += V^T P^T.  In the result layout a
//    lane holds one query and 16 of the tile's 32 keys, so the online softmax
//    is lane-local plus one exchange with lane^32 (v_permlane32_swap), the
//    P^T operand of the second product is already in the right registers
//    (keys reordered consistently on both operands), and the O rescale is a
//    per-lane scalar multiply.
//  * K is read from LDS as the A operand with 16-byte reads; V is read
//    transposed with ds_read_b64_tr_b16 (two per 8-key operand).  Both LDS
//    tiles are XOR-swizzled at 16-byte granularity to spread banks.
//  * Rows reach LDS by LDS-bound loads (global_load_lds_dwordx4), with no
//    staging registers.  The persistent kernels load two steps ahead into
//    three buffers and end each step with a barrier that waits for all but
//    the newest loads (the token-mass variant, which stores inside the loop,
//    prefetches the next slot into registers instead); the local kernel
//    gathers the next step's rows into two buffers.
//  * exp2 with softmax_scale*log2(e) folded into one FMA; the running max is
//    only raised when a tile's max exceeds it by more than 2^8 (P values stay
//    below 256, safe in bf16 and fp32), which makes O rescales rare.
//  * Workgroup ids are remapped so that each XCD (ids i, i+8, ...) works on a
//    contiguous range of (head, query tile): a head's persistent K/V is then
//    read by one or two XCDs instead of all eight.
//  * Optional (MASS): for the token-exact attention mass, each query also
//    writes the log-sum-exp of its scores over every persistent slot and
//    every selected local block (base 2, in the units of the running max).
//    The tile already forms the row sum of its probabilities (relative to the
//    running max) for the online softmax, so this costs one lane exchange and
//    one native log2 per (query, block).
#include "common.h"

namespace pbsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBufBytes = 64 * 1024;

template <int D> struct Shape {
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int KS = D / 16;    // k-steps of S^T = K Q^T
  static constexpr int DT = D / 32;    // 32-wide d tiles of O^T
  static constexpr int ROWB = D * 2;   // bytes per bf16 row
};

__device__ __forceinline__ int swz_k(int r, int c, int cpr) { return c ^ (r & (cpr - 1)); }
__device__ __forceinline__ int swz_v(int r, int c, int cpr) { return c ^ (((r & 3) << 2) & (cpr - 1)); }

__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(char* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

struct FwdArgs {
  Geo g;
  const bf16_t* q;
  const bf16_t* kp;
  const bf16_t* vp;
  const int32_t* plen;
  const bf16_t* kl;
  const bf16_t* vl;
  const int32_t* topk;
  bf16_t* o;
  float* lse;
  float* o_part;    // [B,H,ct,D] persistent-part output (normalised), fp32
  float* lse_part;  // [B,H,ct]   its log-sum-exp (-inf when no slot is valid)
  float* blse_p;    // MASS: [B,H,S,ct] log2-sum-exp2 of each query's scaled scores (log2 units) over each slot's rows
  float* blse_l;    // MASS: [B,H,K,ct] ... over each of its selected local blocks
  int ntiles;       // work items per (batch, head)
};

// Per-wave online-softmax state for NT tiles of 32 queries.
template <int D, int NT> struct WaveState {
  bf16x8_t qf[NT][Shape<D>::KS];
  f32x16_t o[NT][Shape<D>::DT];
  float m[NT];  // running max in log2 units (scores times scale*log2e)
  float l[NT];  // partial row sum over this lane's keys
};

constexpr float kLn2 = 0.6931471805599453f;

struct NoMid {
  __device__ void operator()() const {}
};

// V^T operands of O^T += V^T P^T for keys row0 .. row0+31, read transposed
// from LDS (two ds_read_b64_tr_b16 per 8-key operand).
template <int D>
__device__ __forceinline__ void read_vt(const char* vbase, int row0, bf16x8_t (&va)[Shape<D>::DT][2]) {
  using Sh = Shape<D>;
  const int lane = threadIdx.x & 63, G = lane >> 4, s16 = lane & 15;
#pragma unroll
  for (int dt = 0; dt < Sh::DT; ++dt) {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      s16x4_t part[2];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int r = row0 + 16 * ks2 + 8 * h8 + 4 * (G >> 1) + (s16 >> 2);
        const int col = 32 * dt + 16 * (G & 1) + 4 * (s16 & 3);
        const char* p = vbase + r * Sh::ROWB + swz_v(r, col >> 3, Sh::CPR) * 16 + (col & 7) * 2;
        part[h8] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
      }
      va[dt][ks2] = __builtin_bit_cast(bf16x8_t, (__attribute__((ext_vector_type(8))) short){
          part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]});
    }
  }
}

// The same operands read by one asm block that waits for its own reads: the
// compiler cannot tell a ds_read_tr builtin's LDS array and waits for every
// LDS-bound load in flight before one, which would drain the loads of the
// slots after this one.  The V swizzle depends on the row mod 4 only, so the
// four reads of column tile dt share one address, 8 and 16 rows apart.
#define PBSA_TRV(o, i, off) "ds_read_b64_tr_b16 %" #o ", %" #i " offset:" #off "\n\t"
template <int D>
__device__ __forceinline__ void read_vt_asm(const char* vbase, int row0, bf16x8_t (&va)[Shape<D>::DT][2]) {
  using Sh = Shape<D>;
  static_assert(D == 64 || D == 128, "head dimension");
  const int lane = threadIdx.x & 63, G = lane >> 4, s16 = lane & 15;
  const int r = row0 + 4 * (G >> 1) + (s16 >> 2);
  unsigned ad[Sh::DT];
#pragma unroll
  for (int dt = 0; dt < Sh::DT; ++dt) {
    const int col = 32 * dt + 16 * (G & 1) + 4 * (s16 & 3);
    const char* p = vbase + r * Sh::ROWB + swz_v(r, col >> 3, Sh::CPR) * 16 + (col & 7) * 2;
    ad[dt] = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
  }
  s16x4_t v[Sh::DT][2][2];  // [dt][ks2][h8]: rows +16*ks2 +8*h8
  if constexpr (D == 128) {
    asm volatile(PBSA_TRV(0, 16, 0) PBSA_TRV(1, 16, 2048) PBSA_TRV(2, 16, 4096) PBSA_TRV(3, 16, 6144)
                 PBSA_TRV(4, 17, 0) PBSA_TRV(5, 17, 2048) PBSA_TRV(6, 17, 4096) PBSA_TRV(7, 17, 6144)
                 PBSA_TRV(8, 18, 0) PBSA_TRV(9, 18, 2048) PBSA_TRV(10, 18, 4096) PBSA_TRV(11, 18, 6144)
                 PBSA_TRV(12, 19, 0) PBSA_TRV(13, 19, 2048) PBSA_TRV(14, 19, 4096) PBSA_TRV(15, 19, 6144)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]),
                   "=&v"(v[1][0][0]), "=&v"(v[1][0][1]), "=&v"(v[1][1][0]), "=&v"(v[1][1][1]),
                   "=&v"(v[2][0][0]), "=&v"(v[2][0][1]), "=&v"(v[2][1][0]), "=&v"(v[2][1][1]),
                   "=&v"(v[3][0][0]), "=&v"(v[3][0][1]), "=&v"(v[3][1][0]), "=&v"(v[3][1][1])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]));
  } else {
    asm volatile(PBSA_TRV(0, 8, 0) PBSA_TRV(1, 8, 1024) PBSA_TRV(2, 8, 2048) PBSA_TRV(3, 8, 3072)
                 PBSA_TRV(4, 9, 0) PBSA_TRV(5, 9, 1024) PBSA_TRV(6, 9, 2048) PBSA_TRV(7, 9, 3072)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]),
                   "=&v"(v[1][0][0]), "=&v"(v[1][0][1]), "=&v"(v[1][1][0]), "=&v"(v[1][1][1])
                 : "v"(ad[0]), "v"(ad[1]));
  }
#pragma unroll
  for (int dt = 0; dt < Sh::DT; ++dt)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const s16x4_t x = v[dt][k2][0], y = v[dt][k2][1];
      va[dt][k2] = __builtin_bit_cast(bf16x8_t, (__attribute__((ext_vector_type(8))) short){
                                                    x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]});
    }
}
#undef PBSA_TRV

// One 32-key tile in LDS: K rows kbase[row0 .. row0+31], V rows likewise,
// the first nvalid (1..32) keys valid.  ntq (<= NT) query tiles are active.
// Returns this lane's part of the tile's probability sum for query tile 0,
// relative to the running max after the tile.  EARLY: read the V^T operands
// first and then call mid() (the local kernel issues its next LDS-bound
// gather there: the compiler cannot tell transposed LDS reads from such a
// load in flight and would wait for it).
template <int D, int NT, bool EARLY = false, bool ASMV = false, typename Mid = NoMid>
__device__ __forceinline__ float tile(const char* kbase, const char* vbase, int row0, int nvalid, int ntq, float c2,
                                     WaveState<D, NT>& st, Mid mid = Mid{}) {
  using Sh = Shape<D>;
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  bf16x8_t va[Sh::DT][2];
  if (EARLY) {
    read_vt<D>(vbase, row0, va);
    __builtin_amdgcn_sched_barrier(0);  // keep mid() after the reads
  }
  mid();
  f32x16_t s[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) s[n] = f32x16_t{};
  {
    const int r = row0 + l32;
    const char* krow = kbase + r * Sh::ROWB;
    bf16x8_t ka[Sh::KS];  // all K operands issued before the first product
#pragma unroll
    for (int ks = 0; ks < Sh::KS; ++ks)
      ka[ks] = *reinterpret_cast<const bf16x8_t*>(krow + swz_k(r, 2 * ks + h, Sh::CPR) * 16);
#pragma unroll
    for (int ks = 0; ks < Sh::KS; ++ks) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
        if (n < ntq) s[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], st.qf[n][ks], s[n], 0, 0, 0);
    }
    if constexpr (EARLY) {
      // the local kernel: every K read issued before the first product, then
      // one partial wait per product (the scheduler would interleave them a
      // pair at a time with full waits; 68 -> 66 us).  The persistent kernels
      // measured slower with it: their eight waves read the same tile.
      __builtin_amdgcn_sched_group_barrier(0x100, Sh::KS, 0);    // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, Sh::KS * NT, 0);  // MFMAs
    }
  }
  // V^T operands read now if not yet: they do not depend on P, so their
  // latency is covered by the softmax below
  if (!EARLY) {
    if constexpr (ASMV)
      read_vt_asm<D>(vbase, row0, va);
    else
      read_vt<D>(vbase, row0, va);
  }
  if (nvalid < 32) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kk = 8 * (j >> 2) + 4 * h + (j & 3);
      if (kk >= nvalid) {
#pragma unroll
        for (int n = 0; n < NT; ++n) s[n][j] = -INFINITY;
      }
    }
  }
  bf16x8_t pk[NT][2];
  float ret = 0.f;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (n < ntq) {
      // tree reductions (max, then the row sum below): short dependency
      // chains; the max of this lane's 16 scores in eight 3-input maxes
      auto mx3 = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
      const float* sv = reinterpret_cast<const float*>(&s[n]);
      const float tl = fmaxf(mx3(mx3(sv[0], sv[1], sv[2]), mx3(sv[3], sv[4], sv[5]), mx3(sv[6], sv[7], sv[8])),
                             mx3(mx3(sv[9], sv[10], sv[11]), mx3(sv[12], sv[13], sv[14]), sv[15]));
      // raise the running max only when the tile exceeds it by more than 2^8:
      // a row does exactly when one of its two lanes does, so the lanes test
      // their own maxima and the row max is formed only then
      if (__builtin_amdgcn_ballot_w64(tl * c2 > st.m[n] + 8.0f)) {
        const float tm = half_max(tl) * c2;
        const float mn = fmaxf(st.m[n], tm);
        const float f = __builtin_amdgcn_exp2f(st.m[n] - mn);
        st.l[n] *= f;
#pragma unroll
        for (int dt = 0; dt < Sh::DT; ++dt) st.o[n][dt] *= f;
        st.m[n] = mn;
      }
      const float mneg = -st.m[n];
      float p16[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        p16[j] = __builtin_amdgcn_exp2f(fmaf(s[n][j], c2, mneg));
        pk[n][j >> 3][j & 7] = (__bf16)p16[j];
      }
#pragma unroll
      for (int w2 = 8; w2 >= 1; w2 >>= 1)
#pragma unroll
        for (int j = 0; j < w2; ++j) p16[j] += p16[j + w2];
      const float ls = p16[0];
      st.l[n] += ls;
      if (n == 0) ret = ls;
    }
  }
  // O^T += V^T P^T
#pragma unroll
  for (int dt = 0; dt < Sh::DT; ++dt) {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
        if (n < ntq) st.o[n][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][ks2], pk[n][ks2], st.o[n][dt], 0, 0, 0);
    }
  }
  return ret;
}

template <int D, int NT>
__device__ __forceinline__ void init_state(WaveState<D, NT>& st) {
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int dt = 0; dt < Shape<D>::DT; ++dt) st.o[n][dt] = f32x16_t{};
    st.m[n] = -INFINITY;
    st.l[n] = 0.f;
  }
}

template <int D, int NT>
__device__ __forceinline__ void load_q(const bf16_t* qrow, bool ok, int n, WaveState<D, NT>& st) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < Shape<D>::KS; ++ks) {
    const uint4 v = ok ? ld16(qrow + 16 * ks + 8 * h) : make_uint4(0, 0, 0, 0);
    st.qf[n][ks] = __builtin_bit_cast(bf16x8_t, v);
  }
}

// XCD-aware remap of a 1-D grid: hardware places workgroup i on XCD i % 8,
// so give each XCD a contiguous range of the linear work index.
__device__ __forceinline__ int xcd_remap(int total) {
  const int per_xcd = (total + 7) / 8;
  return (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
}

// ---------------------------------------------------------------------------
// Kernel 1: every query of a head against all persistent slots (dense over
// the compact memory).  8 waves x 32 contiguous query rows; slot K/V staged
// in LDS once per workgroup.  Writes the normalised partial output and its
// log-sum-exp.
// ---------------------------------------------------------------------------
constexpr int kPersWaves = 8;   // 2 waves per SIMD: one's softmax overlaps the other's MFMAs
constexpr int kPersNT = 1;      // 32-query tiles per wave
constexpr int kPersThreads = 64 * kPersWaves;
constexpr int kPersRows = 32 * kPersNT * kPersWaves;

template <int D> struct PersPrefetch {
  static constexpr int N = 64 * Shape<D>::CPR / kPersThreads;  // chunks per thread per tensor
  uint4 k[N], v[N];
};

template <int D>
__device__ __forceinline__ void pers_load(const FwdArgs& a, size_t bh, int s, PersPrefetch<D>& pf) {
  using Sh = Shape<D>;
  const Geo& g = a.g;
  const int n = min(a.plen[bh * g.S + s], g.C);
  const bf16_t* kb = a.kp + (bh * g.S + s) * (size_t)g.C * D;
  const bf16_t* vb = a.vp + (bh * g.S + s) * (size_t)g.C * D;
#pragma unroll
  for (int u = 0; u < PersPrefetch<D>::N; ++u) {
    const int id = threadIdx.x + kPersThreads * u, r = id / Sh::CPR, c = id % Sh::CPR;
    const bool ok = r < n;
    pf.k[u] = ok ? ld16(kb + (size_t)r * D + c * 8) : make_uint4(0, 0, 0, 0);
    pf.v[u] = ok ? ld16(vb + (size_t)r * D + c * 8) : make_uint4(0, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void pers_store(const PersPrefetch<D>& pf, char* buf) {
  using Sh = Shape<D>;
#pragma unroll
  for (int u = 0; u < PersPrefetch<D>::N; ++u) {
    const int id = threadIdx.x + kPersThreads * u, r = id / Sh::CPR, c = id % Sh::CPR;
    st16(buf + r * Sh::ROWB + swz_k(r, c, Sh::CPR) * 16, pf.k[u]);
    st16(buf + 64 * Sh::ROWB + r * Sh::ROWB + swz_v(r, c, Sh::CPR) * 16, pf.v[u]);
  }
}

// LDS-bound loads of one persistent slot: K rows 0-63 (swz_k) then V rows
// 0-63 (swz_v).  Every wave issues NU loads; rows past the slot's length take
// its last row (finite; the tile gives those keys no probability), so the
// count is the same on every path.
template <int D> struct PersSlotDma {
  using Sh = Shape<D>;
  static constexpr int RPK = 1024 / Sh::ROWB;    // rows per 1 KB unit
  static constexpr int UPT = 64 * Sh::ROWB / 1024;  // units per 64-row tensor
  static constexpr int NU = 2 * UPT / kPersWaves;   // units per wave
  static constexpr int BUF = 2 * 64 * Sh::ROWB;
  static_assert(NU * kPersWaves == 2 * UPT, "whole units per wave");
  static __device__ __forceinline__ void issue(const FwdArgs& a, size_t bh, int s, int n, char* buf) {
    const Geo& g = a.g;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rr = lane / Sh::CPR, pos = lane % Sh::CPR;
    const int nl = max(n, 1) - 1;
    const size_t sb = (bh * g.S + s) * (size_t)g.C * D;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave * NU + i, t = u / UPT, tu = u % UPT;  // t: 0 K, 1 V
      const int r = RPK * tu + rr;                             // slot row 0-63
      const int c = t ? swz_v(r, pos, Sh::CPR) : swz_k(r, pos, Sh::CPR);
      const bf16_t* src = (t ? a.vp : a.kp) + sb + (size_t)min(r, nl) * D + c * 8;
      PBSA_LDS_LOAD(src, (__attribute__((address_space(3))) void*)(buf + t * 64 * Sh::ROWB + tu * 1024), 16, 0, 0);
    }
  }
};

template <int D, bool MASS>
__global__ __launch_bounds__(kPersThreads, 1) void fwd_pers_kernel(FwdArgs a) {
  using Sh = Shape<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const Geo& g = a.g;
  const int total = g.B * g.H * a.ntiles;
  const int lin = xcd_remap(total);
  if (lin >= total) return;
  const int qt = lin % a.ntiles;
  const size_t bh = lin / a.ntiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int row_w = qt * kPersRows + 32 * kPersNT * wave;  // first query row of this wave
  const int ntq = max(0, min(kPersNT, (g.ct - row_w + 31) / 32));

  WaveState<D, kPersNT> st;
  init_state(st);
#pragma unroll
  for (int n = 0; n < kPersNT; ++n) {
    const int r = row_w + 32 * n + l32;
    load_q(a.q + (bh * g.ct + min(r, g.ct - 1)) * D, r < g.ct, n, st);
  }
  const float c2 = g.scale * 1.4426950408889634f;

  if (g.S > 0) {
    if constexpr (MASS) {
      // register prefetch (this variant stores per-slot values inside the
      // loop, which the counted waits of the other variant do not allow)
      PersPrefetch<D> pf;
      pers_load<D>(a, bh, 0, pf);
      pers_store<D>(pf, smem);
      __syncthreads();
      // unrolled by two so that each half's LDS buffer is a compile-time offset
      auto step = [&](int s, char* buf, char* nxt) {
        const int n = min(a.plen[bh * g.S + s], g.C);
        if (s + 1 < g.S) pers_load<D>(a, bh, s + 1, pf);
        float bl = 0.f;  // MASS: log2-sum-exp2 over the slot
        if (ntq > 0) {
          float bs = 0.f;  // this lane's probability sum over the slot
          if (n > 0) bs = tile<D, kPersNT>(buf, buf + 64 * Sh::ROWB, 0, min(n, 32), ntq, c2, st);
          if (n > 32) {
            const float m0 = st.m[0];
            const float t2 = tile<D, kPersNT>(buf, buf + 64 * Sh::ROWB, 32, n - 32, ntq, c2, st);
            bs = bs * __builtin_amdgcn_exp2f(m0 - st.m[0]) + t2;
          }
          if (MASS) {
            const float tot = half_sum(bs);
            bl = tot > 0.f ? st.m[0] + __builtin_amdgcn_logf(tot) : -INFINITY;
          }
        }
        if (s + 1 < g.S) pers_store<D>(pf, nxt);
        // stored after the LDS fill so that its wait for the prefetch does not also wait for this store
        if (MASS && ntq > 0 && h == 0 && row_w + l32 < g.ct) a.blse_p[(bh * g.S + s) * g.ct + row_w + l32] = bl;
        __syncthreads();
      };
      for (int s = 0; s < g.S; s += 2) {
        step(s, smem, smem + kBufBytes);
        if (s + 1 < g.S) step(s + 1, smem + kBufBytes, smem);
      }
    } else {
      // Every slot streams through LDS, loaded two steps ahead: step s
      // computes on buffer s%3 while slots s+1 and s+2 land.  The barrier
      // that ends a step waits for all but the loads it issued; V is read
      // transposed by asm that the compiler's own waits do not cover.  Every
      // step issues its loads (steps past the end repeat the last slot), so
      // the counts hold on every path.
      using Dm = PersSlotDma<D>;
      __shared__ __attribute__((aligned(1024))) char pb0[Dm::BUF];
      __shared__ __attribute__((aligned(1024))) char pb1[Dm::BUF];
      __shared__ __attribute__((aligned(1024))) char pb2[Dm::BUF];
      int* plen_s = reinterpret_cast<int*>(smem);  // [S] this head's slot lengths
      for (int x = threadIdx.x; x < g.S; x += kPersThreads) plen_s[x] = min(a.plen[bh * g.S + x], g.C);
      __syncthreads();
      const int last = g.S - 1;
      Dm::issue(a, bh, 0, plen_s[0], pb0);
      Dm::issue(a, bh, min(1, last), plen_s[min(1, last)], pb1);
      vm_barrier<Dm::NU>();
      auto step = [&](int s, char* cur, char* nx2) {
        const int s2 = min(s + 2, last);
        Dm::issue(a, bh, s2, plen_s[s2], nx2);
        if (ntq > 0 && s <= last) {
          const int n = plen_s[s];
          if (n > 0) tile<D, kPersNT, false, true>(cur, cur + 64 * Sh::ROWB, 0, min(n, 32), ntq, c2, st);
          if (n > 32) tile<D, kPersNT, false, true>(cur, cur + 64 * Sh::ROWB, 32, n - 32, ntq, c2, st);
        }
        vm_barrier<Dm::NU>();
      };
      for (int s = 0; s < g.S; s += 3) {
        step(s, pb0, pb2);
        step(s + 1, pb1, pb0);
        step(s + 2, pb2, pb1);
      }
      __builtin_amdgcn_s_waitcnt(0xF70);  // the last loads land before the workgroup can end
    }
  }

#pragma unroll
  for (int n = 0; n < kPersNT; ++n) {
    if (n < ntq) {
      const int r = row_w + 32 * n + l32;
      const float lt = half_sum(st.l[n]);
      if (r < g.ct) {
        float* orow = a.o_part + (bh * g.ct + r) * D;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
        for (int dt = 0; dt < Sh::DT; ++dt) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = 32 * dt + 8 * i4 + 4 * h;
            *reinterpret_cast<float4*>(orow + d0) =
                make_float4(st.o[n][dt][4 * i4] * inv, st.o[n][dt][4 * i4 + 1] * inv, st.o[n][dt][4 * i4 + 2] * inv,
                            st.o[n][dt][4 * i4 + 3] * inv);
          }
        }
        if (h == 0) a.lse_part[bh * g.ct + r] = lt > 0.f ? st.m[n] * kLn2 + logf(lt) : -INFINITY;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 1 for the plain forward: the persistent part with the slots' valid
// rows packed into dense 64-key steps.
//
// The valid rows of all slots are numbered consecutively through a row table
// built in LDS at the start (prefix sums of the slot lengths), so every step
// is 64 keys -- only the last is partial -- with no per-slot padding (slots of
// 24 or 48 rows no longer take a whole 32-key tile each) and one barrier per
// 64 keys instead of one per slot.  Same wave layout as fwd_pers_kernel (8
// waves x 32 queries, 2 waves per SIMD, 256 contiguous queries per
// workgroup), same per-tile product and softmax (tile()), rows reaching LDS by
// LDS-bound loads two steps ahead (three buffers).  (Two 32-query tiles per
// wave at one wave per SIMD halves the LDS operand reads per MFMA but measured
// slower: nothing hides a single wave's latencies, and its O-rescale path
// needs more than the 512 registers.)
// ---------------------------------------------------------------------------
constexpr int kP2Waves = 8;
constexpr int kP2Threads = 64 * kP2Waves;
constexpr int kP2Rows = 32 * kP2Waves;  // queries per workgroup

template <int D> struct P2 {
  using Sh = Shape<D>;
  static constexpr int KEYS = 64;                     // keys per step
  static constexpr int BUF = 2 * KEYS * Sh::ROWB;     // K rows, then V rows (swizzled)
  static constexpr int RPK = 1024 / Sh::ROWB;         // rows per 1 KB unit
  static constexpr int UPT = KEYS * Sh::ROWB / 1024;  // units per tensor per step
  static constexpr int NU = 2 * UPT / kP2Waves;       // units per wave per step
  static_assert(NU * kP2Waves == 2 * UPT, "whole units per wave");
};

// LDS the packed kernel needs besides its step buffers: the row table and
// the slot prefix sums.
size_t p2_table_bytes(const Geo& g) { return ((size_t)g.S * g.C + g.S + 1) * 4; }

// LDS-bound loads of packed step t (rows 64t .. 64t+63 of the head's valid
// rows) into buf; rows past the last valid one repeat it (finite; masked).
template <int D>
__device__ __forceinline__ void p2_issue(const FwdArgs& a, size_t bh, int t, int nvalid, const int* rowtab,
                                         char* buf) {
  using Sh = Shape<D>;
  using Q = P2<D>;
  const Geo& g = a.g;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rr = lane / Sh::CPR, pos = lane % Sh::CPR;
  const size_t base = bh * (size_t)g.S * g.C;
#pragma unroll
  for (int i = 0; i < Q::NU; ++i) {
    const int u = wave * Q::NU + i, tsel = u / Q::UPT, tu = u % Q::UPT;  // tsel: 0 K, 1 V
    const int r = Q::RPK * tu + rr;                                       // row of the step, 0-63
    const int grow = rowtab[min(Q::KEYS * t + r, nvalid - 1)];
    const int c = tsel ? swz_v(r, pos, Sh::CPR) : swz_k(r, pos, Sh::CPR);
    const bf16_t* src = (tsel ? a.vp : a.kp) + (base + grow) * D + c * 8;
    PBSA_LDS_LOAD(src, (__attribute__((address_space(3))) void*)(buf + tsel * Q::KEYS * Sh::ROWB + tu * 1024), 16, 0,
                  0);
  }
}

template <int D>
__global__ __launch_bounds__(kP2Threads, 1) void fwd_pers2_kernel(FwdArgs a) {
  constexpr int NT = 1;
  using Sh = Shape<D>;
  using Q = P2<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ __attribute__((aligned(1024))) char pb0[Q::BUF];
  __shared__ __attribute__((aligned(1024))) char pb1[Q::BUF];
  __shared__ __attribute__((aligned(1024))) char pb2[Q::BUF];
  const Geo& g = a.g;
  const int total = g.B * g.H * a.ntiles;
  const int lin = xcd_remap(total);
  if (lin >= total) return;
  const int qt = lin % a.ntiles;
  const size_t bh = lin / a.ntiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int row_w = qt * kP2Rows + 32 * NT * wave;  // first query row of this wave
  const int ntq = max(0, min(NT, (g.ct - row_w + 31) / 32));

  WaveState<D, NT> st;
  init_state(st);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int r = row_w + 32 * n + l32;
    load_q(a.q + (bh * g.ct + min(r, g.ct - 1)) * D, r < g.ct, n, st);
  }
  const float c2 = g.scale * 1.4426950408889634f;

  // row table: packed row -> slot * C + row, from prefix sums of the lengths
  int* rowtab = reinterpret_cast<int*>(smem);  // [S*C]
  int* pre = rowtab + g.S * g.C;               // [S+1]
  const int nvalid = packed_rows(a.plen + bh * g.S, g.S, g.C, pre, rowtab, kP2Threads);

  const int nsteps = (nvalid + Q::KEYS - 1) / Q::KEYS;
  if (nsteps > 0) {
    const int last = nsteps - 1;
    p2_issue<D>(a, bh, 0, nvalid, rowtab, pb0);
    p2_issue<D>(a, bh, min(1, last), nvalid, rowtab, pb1);
    vm_barrier<Q::NU>();
    auto step = [&](int t, char* cur, char* nx2) {
      p2_issue<D>(a, bh, min(t + 2, last), nvalid, rowtab, nx2);
      if (t <= last) {
        // two 32-key halves; each K / V^T operand read feeds both query tiles
        const int nk = min(Q::KEYS, nvalid - Q::KEYS * t);
        tile<D, NT, false, true>(cur, cur + Q::KEYS * Sh::ROWB, 0, min(nk, 32), NT, c2, st);
        if (nk > 32) tile<D, NT, false, true>(cur, cur + Q::KEYS * Sh::ROWB, 32, nk - 32, NT, c2, st);
      }
      vm_barrier<Q::NU>();
    };
    for (int t = 0; t < nsteps; t += 3) {
      step(t, pb0, pb2);
      step(t + 1, pb1, pb0);
      step(t + 2, pb2, pb1);
    }
    __builtin_amdgcn_s_waitcnt(0xF70);  // the last loads land before the workgroup can end
  }

#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (n < ntq) {
      const int r = row_w + 32 * n + l32;
      const float lt = half_sum(st.l[n]);
      if (r < g.ct) {
        float* orow = a.o_part + (bh * g.ct + r) * D;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
        for (int dt = 0; dt < Sh::DT; ++dt) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = 32 * dt + 8 * i4 + 4 * h;
            *reinterpret_cast<float4*>(orow + d0) =
                make_float4(st.o[n][dt][4 * i4] * inv, st.o[n][dt][4 * i4 + 1] * inv, st.o[n][dt][4 * i4 + 2] * inv,
                            st.o[n][dt][4 * i4 + 3] * inv);
          }
        }
        if (h == 0) a.lse_part[bh * g.ct + r] = lt > 0.f ? st.m[n] * kLn2 + logf(lt) : -INFINITY;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: each query block against its K selected local blocks, merged with
// the persistent partial by log-sum-exp.  A workgroup is kLocBlocks query
// blocks x 2 query tiles; per step it stages the next 32 rows of the query
// block's selected blocks, packed back to back (one LDS region per query
// block).  One block per workgroup
// measured 14% faster than four: the blocks' work differs (edge blocks of
// 24-48 tokens, short selected blocks) and a shared barrier per step made
// every block wait for the slowest.
// ---------------------------------------------------------------------------
constexpr int kLocBlocks = 1;
constexpr int kLocWaves = 2 * kLocBlocks;
constexpr int kLocThreads = 64 * kLocWaves;

// Rows of every step of this workgroup, built once in LDS: rowtab[32*j + r]
// = byte offset in the head's local K (or V) of row r of step j; binfo[t] =
// the t-th selected block's first ring token and its length and extents (8
// bits each), from which its rows follow by arithmetic.  Packed (the plain
// forward): the selected blocks' rows numbered consecutively, lentab[t] =
// block t's first packed row and lentab[K] the total, rows past the total up
// to the step boundary (and the whole first step when there is none) give 0.
// Otherwise (the token-mass forward, which sums per block): block t fills
// steps 2t and 2t+1, lentab[t] = its length (0 if absent), rows past its end
// repeat its first row (finite; the tile masks them), absent selections give
// 0 (no tile reads them).  Used when the tables fit in the LDS beside the two
// step buffers (four workgroups share a CU while they stay under about 8 KB,
// K <= 30); otherwise every gather places its rows itself, two steps per
// selected block.
template <int D>
constexpr size_t loc_tab_room() {
  return 160 * 1024 - 2 * (size_t)kLocBlocks * 64 * Shape<D>::ROWB;
}

constexpr size_t loc_tab_bytes(int K) { return (size_t)kLocBlocks * K * (64 * 4 + 8 + 4) + 4; }

template <int D, bool PACK>
__device__ __forceinline__ void build_rowtab(const FwdArgs& a, size_t bh, int qg, int nthreads, int* rowtab,
                                             int2* binfo, int* lentab) {
  const Geo& g = a.g;
  const int nb = kLocBlocks * g.K;
  // one thread per selected block: where it sits in the ring (all top-k
  // entries loaded at once, no table lookups behind them)
  for (int x = threadIdx.x; x < nb; x += nthreads) {
    const int w = x / g.K, qb = qg * kLocBlocks + w;
    int2 bi = make_int2(0, 0);
    if (qb < g.nq) {
      const int p = a.topk[(bh * g.nq + qb) * g.K + (x - w * g.K)];
      if ((unsigned)p < (unsigned)g.nl) {
        const LocBlock b = loc_block(g, p);  // len, nw, hw <= C <= 64
        bi = make_int2(b.base, b.len | b.nw << 8 | b.hw << 16);
      }
    }
    binfo[x] = bi;
    lentab[x] = bi.y & 255;
  }
  __syncthreads();
  if (PACK) {
    // packed: the selected blocks' rows numbered consecutively (lentab[t]
    // becomes block t's first packed row, lentab[nb] the total), so only
    // the last 32-row step is partial
    static_assert(kLocBlocks == 1, "one query block per workgroup");
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      int run = 0;
      for (int t0 = 0; t0 < nb; t0 += 64) {
        const int t = t0 + lane;
        const int n = t < nb ? lentab[t] : 0;
        int x = n;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(x, o, 64);
          if (lane >= o) x += y;
        }
        __builtin_amdgcn_wave_barrier();
        if (t < nb) lentab[t] = run + x - n;
        run += __shfl(x, 63, 64);
      }
      if (lane == 0) lentab[nb] = run;
    }
    __syncthreads();
    const int total = lentab[nb];
    for (int x = threadIdx.x; x < nb * 64; x += nthreads) {
      const int r = x & 63, t = x >> 6;
      const int2 bi = binfo[t];
      const LocBlock b{bi.x, bi.y & 255, (bi.y >> 8) & 255, bi.y >> 16};
      if (r < b.len) rowtab[lentab[t] + r] = loc_row(g, b, r) * D * 2;
    }
    // rows past the total up to the step boundary, and the whole first step
    // when no block is selected (the first gather is issued regardless): row
    // 0 of the head (finite; the tile masks them or no tile runs)
    for (int x = total + threadIdx.x; x < max(32, (total + 31) & ~31); x += nthreads) rowtab[x] = 0;
    return;
  }
  for (int x = threadIdx.x; x < nb * 64; x += nthreads) {
    const int r = x & 63;
    const int2 bi = binfo[x >> 6];
    const LocBlock b{bi.x, bi.y & 255, (bi.y >> 8) & 255, bi.y >> 16};
    const int tok = r < b.len ? loc_row(g, b, r) : b.base;
    rowtab[x] = tok * D * 2;
  }
}

// One local step gathered straight into LDS (global_load_lds_dwordx4): no
// staging registers and no LDS store instructions.  An instruction fills 1 KB
// of the buffer (lane l at byte 16*l); lane l fetches the global chunk whose
// swizzled position is l's, so K and V land in their swizzled layouts.  TAB:
// rows from the LDS row table as 32-bit byte offsets added to the head's base
// (one add per load; a compile-time choice: if the path that places rows per
// load shares the loop, the compiler joins the two with a full wait).  Without
// the table, rows past a selected block's end (and absent selections) load row 0
// of the head's queries: finite values whose keys the tile masks.
template <int D, bool TAB>
__device__ __forceinline__ void loc_gather(const FwdArgs& a, size_t bh, int qg, int j, char* buf,
                                           const int* rowtab) {
  using Sh = Shape<D>;
  constexpr int RPK = 1024 / Sh::ROWB;                 // rows per KB unit
  constexpr int UPT = 32 * Sh::ROWB / 1024;            // KB units per 32-row tile
  constexpr int PER_WAVE = kLocBlocks * 2 * UPT / kLocWaves;
  const Geo& g = a.g;
  const int t = j >> 1, half = j & 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rr = lane / Sh::CPR, pos = lane % Sh::CPR;
  const bf16_t* kb = a.kl + bh * (size_t)g.NL * D;
  const bf16_t* vb = a.vl + bh * (size_t)g.NL * D;
  const bf16_t* fill = a.q + bh * (size_t)g.ct * D;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int u = wave * PER_WAVE + i;
    const int w = u / (2 * UPT), tensor = (u / UPT) & 1;
    const int r = RPK * (u % UPT) + rr;  // row in the 32-row tile
    const int c = tensor ? swz_v(r, pos, Sh::CPR) : swz_k(r, pos, Sh::CPR);
    if (TAB) {
      const uint32_t off = (uint32_t)rowtab[(w * g.K + t) * 64 + 32 * half + r] + (uint32_t)(c * 16);
      const char* src = reinterpret_cast<const char*>(tensor ? vb : kb) + off;
      PBSA_LDS_LOAD(src, (__attribute__((address_space(3))) void*)(buf + u * 1024), 16, 0, 0);
      continue;
    }
    int tok = -1;
    {
      const int qb = qg * kLocBlocks + w;
      if (qb < g.nq) {
        const int p = a.topk[(bh * g.nq + qb) * g.K + t];
        if ((unsigned)p < (unsigned)g.nl) {
          const LocBlock b = loc_block(g, p);
          if (32 * half + r < b.len) tok = loc_row(g, b, 32 * half + r);
        }
      }
    }
    const bf16_t* src = (tok >= 0 ? (tensor ? vb : kb) + (size_t)tok * D : fill) + c * 8;
    PBSA_LDS_LOAD(src, (__attribute__((address_space(3))) void*)(buf + u * 1024), 16, 0, 0);
  }
}

template <int D, bool MASS, bool TAB>
// 2 waves per SIMD: the register budget of four such workgroups per CU
__global__ __launch_bounds__(kLocThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_local_kernel(FwdArgs a) {
  using Sh = Shape<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];  // row tables
  constexpr int BUF = kLocBlocks * 64 * Sh::ROWB;            // per block: 32 K rows, 32 V rows
  // the two step buffers are separate arrays so that the compiler can tell the
  // gather into one from the reads of the other
  __shared__ __attribute__((aligned(1024))) char kv0[BUF];
  __shared__ __attribute__((aligned(1024))) char kv1[BUF];
  const Geo& g = a.g;
  const int total = g.B * g.H * a.ntiles;
  const int lin = xcd_remap(total);
  if (lin >= total) return;
  const int qg = lin % a.ntiles;
  const size_t bh = lin / a.ntiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int qb = qg * kLocBlocks + (wave >> 1), nt = wave & 1;
  const bool has_q = qb < g.nq;
  const BlockExt qe = block_ext(g, has_q ? qb : 0);
  const int ntq = has_q && 32 * nt < qe.len ? 1 : 0;
  const int r = 32 * nt + l32;
  const bool row_ok = ntq && r < qe.len;
  const int tok = row_ok ? block_token(g, qe, r) : 0;

  WaveState<D, 1> st;
  init_state(st);
  load_q(a.q + (bh * g.ct + tok) * D, row_ok, 0, st);
  const float c2 = g.scale * 1.4426950408889634f;

  // PACK: the selected blocks' rows packed into consecutive 32-row steps
  // (the token-mass variant keeps one block per two steps: it sums per block)
  constexpr bool PACK = TAB && !MASS;
  int nsteps = 2 * g.K;
  int* rowtab = reinterpret_cast<int*>(smem);
  int2* binfo = reinterpret_cast<int2*>(rowtab + kLocBlocks * g.K * 64);
  int* lentab = reinterpret_cast<int*>(binfo + kLocBlocks * g.K);
  int nrows = 0;  // PACK: packed rows of all selected blocks
  if (TAB) {
    build_rowtab<D, PACK>(a, bh, qg, kLocThreads, rowtab, binfo, lentab);
    __syncthreads();
    if (PACK) {
      nrows = lentab[kLocBlocks * g.K];
      nsteps = (nrows + 31) / 32;
    }
  }
  loc_gather<D, TAB>(a, bh, qg, 0, kv0, rowtab);
  __syncthreads();  // its fence waits for the gather
  float bs = 0.f;   // this lane's probability sum over the current selected block (MASS)
  // unrolled by two so that each step's buffers are compile-time arrays
  auto step = [&](int j, char* cur, char* nxt) {
    int nv = 0;
    if (PACK) {
      nv = ntq ? min(nrows - 32 * j, 32) : 0;
    } else if (ntq) {
      int len = 0;
      if (TAB) {
        len = lentab[(wave >> 1) * g.K + (j >> 1)];
      } else {
        const int p = a.topk[(bh * g.nq + qb) * g.K + (j >> 1)];
        if ((unsigned)p < (unsigned)g.nl) len = block_ext(g, p % g.nq).len;
      }
      nv = min(len - 32 * (j & 1), 32);
    }
    nv = __builtin_amdgcn_readfirstlane(nv);  // uniform per wave: a scalar branch
    auto gather = [&]() {
      if (j + 1 < nsteps) loc_gather<D, TAB>(a, bh, qg, j + 1, nxt, rowtab);
    };
    if (nv > 0) {
      const char* region = cur + (wave >> 1) * (64 * Sh::ROWB);
      const float m0 = st.m[0];
      const float ts = tile<D, 1, true>(region, region + 32 * Sh::ROWB, 0, nv, 1, c2, st, gather);
      if (MASS) bs = (j & 1) ? bs * __builtin_amdgcn_exp2f(m0 - st.m[0]) + ts : ts;
    } else {
      gather();
      if (MASS && !(j & 1)) bs = 0.f;
    }
    if (MASS && (j & 1) && ntq) {
      const float tot = half_sum(bs);  // lane exchange: both halves of the wave take part
      if (h == 0 && row_ok)
        a.blse_l[(bh * g.K + (j >> 1)) * g.ct + tok] = tot > 0.f ? st.m[0] + __builtin_amdgcn_logf(tot) : -INFINITY;
    }
    __syncthreads();
  };
  for (int j = 0; j < nsteps; j += 2) {
    step(j, kv0, kv1);
    if (j + 1 < nsteps) step(j + 1, kv1, kv0);
  }

  // merge with the persistent partial and write O (bf16) and LSE
  const float lt = half_sum(st.l[0]);
  if (!row_ok) return;
  const size_t row = bh * g.ct + tok;
  const float lse_l = lt > 0.f ? st.m[0] * kLn2 + logf(lt) : -INFINITY;
  const float lse_p = a.lse_part[row];
  const float mx = fmaxf(lse_l, lse_p);
  const float wl = lse_l == -INFINITY ? 0.f : expf(lse_l - mx);
  const float wp = lse_p == -INFINITY ? 0.f : expf(lse_p - mx);
  const float den = wl + wp;
  const float fl = lt > 0.f ? wl / (den * lt) : 0.f;  // local accumulators are unnormalised
  const float fp = wp / den;
  const float* op = a.o_part + row * D;
  bf16_t* orow = a.o + row * D;
  float4 pvs[Sh::DT][4];  // all loads issued before the first use
#pragma unroll
  for (int dt = 0; dt < Sh::DT; ++dt) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) pvs[dt][i4] = *reinterpret_cast<const float4*>(op + 32 * dt + 8 * i4 + 4 * h);
  }
#pragma unroll
  for (int dt = 0; dt < Sh::DT; ++dt) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * dt + 8 * i4 + 4 * h;
      const float4 pv = pvs[dt][i4];
      uint2 w;
      w.x = (uint32_t)f2bf(fmaf(st.o[0][dt][4 * i4 + 0], fl, pv.x * fp)) |
            ((uint32_t)f2bf(fmaf(st.o[0][dt][4 * i4 + 1], fl, pv.y * fp)) << 16);
      w.y = (uint32_t)f2bf(fmaf(st.o[0][dt][4 * i4 + 2], fl, pv.z * fp)) |
            ((uint32_t)f2bf(fmaf(st.o[0][dt][4 * i4 + 3], fl, pv.w * fp)) << 16);
      *reinterpret_cast<uint2*>(orow + d0) = w;
    }
  }
  if (h == 0) a.lse[row] = mx + logf(den);
}

template <typename K>
hipError_t set_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Dynamic LDS of the packed persistent kernel (row table and prefix sums); its
// three 64-key step buffers are static (96 KB at head_dim 128).
constexpr int kP2TableMax = 60 * 1024;

template <int D, bool MASS>
hipError_t launch_d(const FwdArgs& base, hipStream_t s) {
  static PerDeviceOnce attr;
  // persistent kernel: the mass variant stages through dynamic LDS, the other
  // keeps only the slot lengths there (at most 2048 slots)
  const size_t shm = MASS ? 2 * kBufBytes : (size_t)base.g.S * 4;
  const Geo& g0 = base.g;
  const size_t tabb = loc_tab_bytes(g0.K);
  const bool tab = tabb <= loc_tab_room<D>() && (size_t)g0.NL * D * 2 < ((size_t)1 << 31);  // 32-bit row offsets
  const size_t shm_loc = tab ? tabb : 0;  // row tables (step buffers are static)
  {
    const hipError_t e = attr.run([] {
      hipError_t r = set_lds(fwd_pers_kernel<D, MASS>, MASS ? 2 * kBufBytes : 2048 * 4);
      if (r == hipSuccess) r = set_lds(fwd_local_kernel<D, MASS, true>, loc_tab_room<D>());
      return r;
    });
    if (e != hipSuccess) return e;
  }
  const Geo& g = base.g;
  FwdArgs a = base;
  hipError_t e = hipSuccess;
  int total = 0;
  const size_t tab2 = p2_table_bytes(g);
  if (!MASS && g.S > 0 && tab2 <= (size_t)kP2TableMax) {
    static PerDeviceOnce attr2;
    e = attr2.run([] { return set_lds(fwd_pers2_kernel<D>, kP2TableMax); });
    if (e != hipSuccess) return e;
    a.ntiles = (g.ct + kP2Rows - 1) / kP2Rows;
    total = g.B * g.H * a.ntiles;
    fwd_pers2_kernel<D><<<((total + 7) / 8) * 8, kP2Threads, tab2, s>>>(a);
  } else {
    a.ntiles = (g.ct + kPersRows - 1) / kPersRows;
    total = g.B * g.H * a.ntiles;
    fwd_pers_kernel<D, MASS><<<((total + 7) / 8) * 8, kPersThreads, shm, s>>>(a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  a.ntiles = (g.nq + kLocBlocks - 1) / kLocBlocks;
  total = g.B * g.H * a.ntiles;
  if (tab)
    fwd_local_kernel<D, MASS, true><<<((total + 7) / 8) * 8, kLocThreads, shm_loc, s>>>(a);
  else
    fwd_local_kernel<D, MASS, false><<<((total + 7) / 8) * 8, kLocThreads, shm_loc, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool fwd_mfma_supported(const Geo& g) {
  return g.dtype == PBSA_BF16 && (g.D == 64 || g.D == 128) && g.C <= 64;
}

size_t fwd_mfma_workspace(const Geo& g) {
  return ((size_t)g.B * g.H * g.ct * g.D * 4 + 255) / 256 * 256 +
         ((size_t)g.B * g.H * g.ct * 4 + 255) / 256 * 256;
}

hipError_t launch_fwd_mfma(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                           const void* k_l, const void* v_l, const int32_t* topk, void* o, float* lse, void* ws,
                           float* blse_p, float* blse_l, hipStream_t s) {
  float* o_part = (float*)ws;
  float* lse_part = (float*)((char*)o_part + ((size_t)g.B * g.H * g.ct * g.D * 4 + 255) / 256 * 256);
  FwdArgs a{g, (const bf16_t*)q, (const bf16_t*)k_p, (const bf16_t*)v_p, plen, (const bf16_t*)k_l,
            (const bf16_t*)v_l, topk, (bf16_t*)o, lse, o_part, lse_part, blse_p, blse_l, 0};
  if (blse_p) return g.D == 128 ? launch_d<128, true>(a, s) : launch_d<64, true>(a, s);
  return g.D == 128 ? launch_d<128, false>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace pbsa
