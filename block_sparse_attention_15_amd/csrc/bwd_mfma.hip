// Sparse attention backward on the gfx950 matrix cores (bf16 inputs, head_dim
// 64 or 128).
//
// For the fixed block mask of the forward (all persistent slots plus each
// query block's selected local blocks) the gradients are those of softmax
// attention ("full gradient support for training" on the Sparse Forcing
// project page):
//   P = exp(scale q.k - lse),  dP = dO.v,  dS = P (dP - D),  D = rowsum(dO*O)
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Five kernels, all deterministic (every output element is accumulated by one
// lane in a fixed order; no atomics):
//   dq_pers   query-outer over the persistent slots: 8 waves x 32 contiguous
//             query rows; S^T = K Q^T and dP^T = V dO^T put one query per
//             lane (lane-local P and dS), dQ^T += K^T dS^T reads K transposed
//             from LDS (ds_read_b64_tr_b16).  Writes dq, and every dS tile
//             (bf16) for dk_ds.
//   dq_local  the same over each query block's selected local blocks (one
//             query block x 2 query tiles = 2 waves per workgroup, four
//             workgroups per CU), rows gathered straight into LDS; adds into
//             dq.
//   dkv_pers  key-outer: 8 waves x 32 keys (four slots) stream every query of
//             the head through LDS in 32-row tiles; S = Q K^T (and dP =
//             dO V^T) put one key per lane, dV += P^T dO (or dK += dS^T Q)
//             reads dO (or Q) transposed from LDS.  The dV pass always; the
//             dK pass only where the dS tiles would not fit their cap.
//   dk_ds     key-outer like dkv_pers: dK += dS^T Q from the stored dS tiles,
//             one product where recomputing dS takes three.
//   dkv_local key-outer over a local block (4 waves: dV and dK for 2 x 32
//             keys; each dV wave passes P to its key tile's dK wave through
//             LDS), streaming only the query blocks that selected it (a
//             key-block -> query-block index built from the top-k lists),
//             rows gathered straight into LDS.
// LDS tiles hold 32 rows of 16-byte chunks XOR-swizzled so that both the
// natural 16-byte reads (rows of one chunk column) and the transposed
// ds_read_b64_tr_b16 reads (4 rows x 4 chunks per 16 lanes) avoid bank
// conflicts.
#include "common.h"

namespace pbsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

template <int D> struct Sh {
  static constexpr int CPR = D / 8;       // 16-byte chunks per row
  static constexpr int KS = D / 16;       // k-steps over the head dimension
  static constexpr int DT = D / 32;       // 32-wide tiles of the head dimension
  static constexpr int ROWB = D * 2;      // bytes per bf16 row
  static constexpr int TILEB = 32 * ROWB; // bytes per 32-row tile
};

__device__ __forceinline__ int swz(int r, int c, int cpr) {
  return c ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (cpr - 1));
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte chunk c of row r of a 32-row LDS tile.
template <int D>
__device__ __forceinline__ bf16x8_t rd_nat(const char* t, int r, int c) {
  return *reinterpret_cast<const bf16x8_t*>(t + r * Sh<D>::ROWB + swz(r, c, Sh<D>::CPR) * 16);
}

// Natural-layout operands by k-step, addressed from the LDS array `arr` that
// holds the tile (tile offset `rel` in it a multiple of 256 bytes): with the
// XOR swizzle the byte offset of chunk 2*ks+h of row r inside its row is
// (32*ks) ^ (16*h ^ 16*swizzle(r)), so one XOR with the lane's base offset
// per read stands in for a live offset register per k-step.  The empty asm
// keeps the base opaque so the per-k-step offsets are not hoisted out of the
// caller's loop.
template <int D>
__device__ __forceinline__ int nat_base(int rel, int r, int h) {
  int off = rel + r * Sh<D>::ROWB + ((16 * h) ^ (16 * swz(r, 0, Sh<D>::CPR)));
  asm volatile("" : "+v"(off));
  return off;
}
template <int D>
__device__ __forceinline__ bf16x8_t rd_nat_at(const char* arr, int base, int ks) {
  return *reinterpret_cast<const bf16x8_t*>(arr + (base ^ (32 * ks)));
}

// Transposed operand from a 32-row tile: lane l receives column 32*dt + l%32
// at rows 16*ks2 + 4*(l/32) + {0,1,2,3} and the same +8 (the row order that
// matches the packing of a 32x32 MFMA result into the next product).
template <int D>
__device__ __forceinline__ bf16x8_t rd_tr(const char* t, int ks2, int dt) {
  const int lane = threadIdx.x & 63, G = lane >> 4, s16 = lane & 15;
  s16x4_t part[2];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int r = 16 * ks2 + 8 * h8 + 4 * (G >> 1) + (s16 >> 2);
    const int col = 32 * dt + 16 * (G & 1) + 4 * (s16 & 3);
    const char* p = t + r * Sh<D>::ROWB + swz(r, col >> 3, Sh<D>::CPR) * 16 + (col & 7) * 2;
    part[h8] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  }
  return __builtin_bit_cast(bf16x8_t, s16x8_t{part[0][0], part[0][1], part[0][2], part[0][3], part[1][0],
                                              part[1][1], part[1][2], part[1][3]});
}

// All transposed operands of a 32-row tile, out[dt][ks2] = rd_tr(t, ks2, dt),
// read in one asm block that waits for its own reads.  The compiler cannot
// tell which LDS array a ds_read_tr builtin reads, so it waits for every
// LDS-bound global load in flight before one; reads it does not see let
// loads into the other step buffers stay in flight.  Rows 16*ks2 + r share
// the swizzle of row r, so ks2 = 1 is the offset 16 rows further.
#define PBSA_TR(o, i, off) "ds_read_b64_tr_b16 %" #o ", %" #i " offset:" #off "\n\t"
template <int D>
__device__ __forceinline__ void rd_tr_all(const char* t, bf16x8_t (&out)[Sh<D>::DT][2]) {
  static_assert(D == 64 || D == 128, "head dimension");
  const int lane = threadIdx.x & 63, G = lane >> 4, s16 = lane & 15;
  unsigned ad[Sh<D>::DT][2];
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      const int r = 8 * h8 + 4 * (G >> 1) + (s16 >> 2);
      const int col = 32 * dt + 16 * (G & 1) + 4 * (s16 & 3);
      const char* p = t + r * Sh<D>::ROWB + swz(r, col >> 3, Sh<D>::CPR) * 16 + (col & 7) * 2;
      ad[dt][h8] = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
    }
  s16x4_t v[Sh<D>::DT][2][2];  // [dt][ks2][h8]
  if constexpr (D == 128) {
    asm volatile(PBSA_TR(0, 16, 0) PBSA_TR(1, 17, 0) PBSA_TR(2, 16, 4096) PBSA_TR(3, 17, 4096)
                 PBSA_TR(4, 18, 0) PBSA_TR(5, 19, 0) PBSA_TR(6, 18, 4096) PBSA_TR(7, 19, 4096)
                 PBSA_TR(8, 20, 0) PBSA_TR(9, 21, 0) PBSA_TR(10, 20, 4096) PBSA_TR(11, 21, 4096)
                 PBSA_TR(12, 22, 0) PBSA_TR(13, 23, 0) PBSA_TR(14, 22, 4096) PBSA_TR(15, 23, 4096)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]),
                   "=&v"(v[1][0][0]), "=&v"(v[1][0][1]), "=&v"(v[1][1][0]), "=&v"(v[1][1][1]),
                   "=&v"(v[2][0][0]), "=&v"(v[2][0][1]), "=&v"(v[2][1][0]), "=&v"(v[2][1][1]),
                   "=&v"(v[3][0][0]), "=&v"(v[3][0][1]), "=&v"(v[3][1][0]), "=&v"(v[3][1][1])
                 : "v"(ad[0][0]), "v"(ad[0][1]), "v"(ad[1][0]), "v"(ad[1][1]), "v"(ad[2][0]), "v"(ad[2][1]),
                   "v"(ad[3][0]), "v"(ad[3][1]));
  } else {
    asm volatile(PBSA_TR(0, 8, 0) PBSA_TR(1, 9, 0) PBSA_TR(2, 8, 2048) PBSA_TR(3, 9, 2048)
                 PBSA_TR(4, 10, 0) PBSA_TR(5, 11, 0) PBSA_TR(6, 10, 2048) PBSA_TR(7, 11, 2048)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]),
                   "=&v"(v[1][0][0]), "=&v"(v[1][0][1]), "=&v"(v[1][1][0]), "=&v"(v[1][1][1])
                 : "v"(ad[0][0]), "v"(ad[0][1]), "v"(ad[1][0]), "v"(ad[1][1]));
  }
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const s16x4_t a = v[dt][k2][0], b = v[dt][k2][1];
      out[dt][k2] = __builtin_bit_cast(bf16x8_t, s16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
    }
}

// The two transposed operands of column tile dt, out[ks2] = rd_tr(t, ks2, dt),
// in one asm block that waits for its own reads (fewer live registers than
// rd_tr_all, one LDS round trip per column tile).
template <int D>
__device__ __forceinline__ void rd_tr_dt(const char* t, int dt, bf16x8_t (&out)[2]) {
  const int lane = threadIdx.x & 63, G = lane >> 4, s16 = lane & 15;
  unsigned ad[2];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int r = 8 * h8 + 4 * (G >> 1) + (s16 >> 2);
    const int col = 32 * dt + 16 * (G & 1) + 4 * (s16 & 3);
    const char* p = t + r * Sh<D>::ROWB + swz(r, col >> 3, Sh<D>::CPR) * 16 + (col & 7) * 2;
    ad[h8] = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
  }
  s16x4_t v[2][2];  // [ks2][h8]
  if constexpr (D == 128)
    asm volatile(PBSA_TR(0, 4, 0) PBSA_TR(1, 5, 0) PBSA_TR(2, 4, 4096) PBSA_TR(3, 5, 4096) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1])
                 : "v"(ad[0]), "v"(ad[1]));
  else
    asm volatile(PBSA_TR(0, 4, 0) PBSA_TR(1, 5, 0) PBSA_TR(2, 4, 2048) PBSA_TR(3, 5, 2048) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1])
                 : "v"(ad[0]), "v"(ad[1]));
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const s16x4_t x = v[k2][0], y = v[k2][1];
    out[k2] = __builtin_bit_cast(bf16x8_t, s16x8_t{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]});
  }
}
// A dS tile (32 queries x 32 keys, bf16) as the query-outer dQ kernel stores
// it: the 8-byte piece of query q holding keys 4m..4m+3 sits at byte
// 1024*(m/4) + 16*(2q + m%2) + 8*((m/2)%2), i.e. each lane's two packed
// 16-byte operands, lane-interleaved so that both the stores (1 KB per
// instruction) and the transposed reads below (4 queries x 32 contiguous
// bytes per 16 lanes) are dense.  out[ks2] as rd_tr(t, ks2, 0) would
// return them from a row-major tile.
__device__ __forceinline__ int ds_piece(int q, int m) {
  return 1024 * (m >> 2) + 16 * (2 * q + (m & 1)) + 8 * ((m >> 1) & 1);
}
__device__ __forceinline__ void rd_tr_ds(const char* t, bf16x8_t (&out)[2]) {
  const int lane = threadIdx.x & 63, G = lane >> 4, s16 = lane & 15;
  unsigned ad[2];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int q = 8 * h8 + 4 * (G >> 1) + (s16 >> 2);
    const int m = 4 * (G & 1) + (s16 & 3);
    ad[h8] = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)(t + ds_piece(q, m));
  }
  s16x4_t v[2][2];  // [ks2][h8]; queries 16..31 are 512 bytes further
  asm volatile(PBSA_TR(0, 4, 0) PBSA_TR(1, 5, 0) PBSA_TR(2, 4, 512) PBSA_TR(3, 5, 512) "s_waitcnt lgkmcnt(0)"
               : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1])
               : "v"(ad[0]), "v"(ad[1]));
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const s16x4_t x = v[k2][0], y = v[k2][1];
    out[k2] = __builtin_bit_cast(bf16x8_t, s16x8_t{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]});
  }
}
#undef PBSA_TR

__device__ __forceinline__ void st_chunk(char* tile, int rowb, int cpr, int r, int c, uint4 v) {
  *reinterpret_cast<uint4*>(tile + r * rowb + swz(r, c, cpr) * 16) = v;
}

__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& x, int ks2) {
  bf16x8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[8 * ks2 + i];
  return r;
}

__device__ __forceinline__ int xcd_remap(int total) {
  const int per_xcd = (total + 7) / 8;
  return (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
}

struct BwdArgs {
  Geo g;
  const bf16_t* q;
  const bf16_t* kp;
  const bf16_t* vp;
  const int32_t* plen;
  const bf16_t* kl;
  const bf16_t* vl;
  const int32_t* topk;
  const float* lse;
  const float* delta;
  const float* lse2;  // lse * log2(e)
  const bf16_t* dout;
  const int32_t* tcount;
  const int32_t* tlist;
  const int32_t* korder;
  const bf16_t* zrow;  // a zero row: the gathers' filler for key rows that do not exist
  bf16_t* dsb;         // persistent dS tiles [B,H][2S key tiles][query tiles][32 x 32], bf16
  float* dq;
  float* dkp;
  float* dvp;
  float* dkl;
  float* dvl;
  int ntiles;
  int pk;  // dq_pers / dk_ds run on packed persistent rows (dkv_pers then zeroes dK past the slot lengths)
};

// Which tiles read their transposed operands ahead of the VALU work (only
// where the registers allow it without spilling).
constexpr bool kHoistDqPers = true;

// ===========================================================================
// dQ, query-outer
// ===========================================================================
template <int D> struct QState {
  bf16x8_t qf[Sh<D>::KS];
  bf16x8_t df[Sh<D>::KS];
  f32x16_t acc[Sh<D>::DT];
  float lse2;   // lse * log2(e) of this lane's query
  float dl;     // rowsum(dO * O) of this lane's query
};

template <int D>
__device__ __forceinline__ void q_init(const BwdArgs& a, size_t bh, int tok, bool ok, QState<D>& st) {
  const int h = (threadIdx.x & 63) >> 5;
  const size_t row = bh * a.g.ct + tok;
#pragma unroll
  for (int ks = 0; ks < Sh<D>::KS; ++ks) {
    st.qf[ks] = __builtin_bit_cast(bf16x8_t, ok ? ld16(a.q + row * D + 16 * ks + 8 * h) : make_uint4(0, 0, 0, 0));
    st.df[ks] = __builtin_bit_cast(bf16x8_t, ok ? ld16(a.dout + row * D + 16 * ks + 8 * h) : make_uint4(0, 0, 0, 0));
  }
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt) st.acc[dt] = f32x16_t{};
  st.lse2 = ok ? a.lse[row] * kLog2e : INFINITY;
  st.dl = ok ? a.delta[row] : 0.f;
}

// One 32-key tile: K tile at arr + tk_rel, V tile at arr + tv_rel (32 rows
// each), nvalid leading keys.  HOIST: read the transposed K operands of dQ
// ahead of the VALU work (their LDS latency is then covered), at the cost of
// 2*DT more live registers; EARLY: read them first of all, then call mid()
// (the local kernel issues its next gather there: the compiler cannot tell
// transposed LDS reads from an LDS-bound load in flight and would wait for
// it).  XADDR: natural reads through per-read XOR offsets (nat_base) rather
// than one live offset register per k-step (fewer registers, more VALU).
// MASK: zero the probabilities of keys at or past nvalid.  Without it those
// keys must have zero K rows: their dS then meets a zero row in dQ += dS K,
// and the probability is clamped to [0, 1] (free, a modifier of the exp) so
// that it stays finite for any log-sum-exp; that saves a compare and a
// select per score.  STORE: also write the tile's dS (bf16, as rounded for
// the dQ product) to dso, a 2 KB tile in the layout rd_tr_ds reads.
struct NoMid {
  __device__ void operator()() const {}
};
template <int D, bool HOIST, bool EARLY = false, bool XADDR = false, bool MASK = true, bool STORE = false,
          typename Mid = NoMid>
__device__ __forceinline__ void q_tile(const char* arr, int tk_rel, int tv_rel, int nvalid, float c2,
                                       QState<D>& st, Mid mid = Mid{}, bf16_t* dso = nullptr) {
  static_assert(HOIST || !EARLY, "EARLY reads are hoisted reads");
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const char* tk = arr + tk_rel;
  bf16x8_t kt[HOIST ? Sh<D>::DT : 1][2];
  auto read_kt = [&]() {
#pragma unroll
    for (int dt = 0; dt < Sh<D>::DT; ++dt) {
      kt[HOIST ? dt : 0][0] = rd_tr<D>(tk, 0, dt);
      kt[HOIST ? dt : 0][1] = rd_tr<D>(tk, 1, dt);
    }
  };
  if (EARLY) {
    read_kt();
    __builtin_amdgcn_sched_barrier(0);  // keep mid() after the reads
  }
  mid();
  f32x16_t s = {}, dp = {};
  if (XADDR) {
    const int bk = nat_base<D>(tk_rel, l32, h), bv = nat_base<D>(tv_rel, l32, h);
#pragma unroll
    for (int ks = 0; ks < Sh<D>::KS; ++ks) {
      s = mfma(rd_nat_at<D>(arr, bk, ks), st.qf[ks], s);
      dp = mfma(rd_nat_at<D>(arr, bv, ks), st.df[ks], dp);
    }
  } else {
    const char* tv = arr + tv_rel;
#pragma unroll
    for (int ks = 0; ks < Sh<D>::KS; ++ks) {
      s = mfma(rd_nat<D>(tk, l32, 2 * ks + h), st.qf[ks], s);
      dp = mfma(rd_nat<D>(tv, l32, 2 * ks + h), st.df[ks], dp);
    }
  }
  if (HOIST && !EARLY) read_kt();
  f32x16_t ds;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int kk = 8 * (j >> 2) + 4 * h + (j & 3);
    const float e = __builtin_amdgcn_exp2f(fmaf(s[j], c2, -st.lse2));
    const float p = MASK ? (kk < nvalid ? e : 0.f) : __builtin_amdgcn_fmed3f(e, 0.f, 1.f);
    ds[j] = p * (dp[j] - st.dl);
  }
  const bf16x8_t d0 = pack8(ds, 0), d1 = pack8(ds, 1);
  if constexpr (STORE) {
    // d0 holds keys 4h..4h+3 and 8+4h..8+4h+3 of this lane's query (pieces
    // m = h and 2+h), d1 the same +16 (m = 4+h, 6+h); non-temporal: read
    // back only by the dK kernel, much later
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    u32x4_t* t = reinterpret_cast<u32x4_t*>(dso) + 2 * l32 + h;
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, d0), t);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, d1), t + 64);
  }
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt) {
    st.acc[dt] = mfma(HOIST ? kt[HOIST ? dt : 0][0] : rd_tr<D>(tk, 0, dt), d0, st.acc[dt]);
    st.acc[dt] = mfma(HOIST ? kt[HOIST ? dt : 0][1] : rd_tr<D>(tk, 1, dt), d1, st.acc[dt]);
  }
}

// Persistent part: 8 waves x 32 contiguous query rows; every slot staged once.
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRows = 32 * kDqWaves;

template <int D> struct SlotPf {
  static constexpr int N = 64 * Sh<D>::CPR / kDqThreads;  // chunks per thread per tensor
  uint4 k[N], v[N];
};

// Unconditional loads (rows clamped to the step's last): the rows at or
// past the step's row count are zeroed when staged, after the wait for the
// loads.  A step is one slot (its rows 0-63), or with a row table (PK) the
// packed rows 64s .. 64s+63 of the head (nvalid of them in all).
template <int D, bool PK>
__device__ __forceinline__ void slot_load(const BwdArgs& a, size_t bh, int s, SlotPf<D>& pf, const int* rowtab,
                                          int nvalid) {
  const Geo& g = a.g;
  const size_t hb = PK ? bh * g.S * (size_t)g.C * D : (bh * g.S + s) * (size_t)g.C * D;
#pragma unroll
  for (int u = 0; u < SlotPf<D>::N; ++u) {
    const int id = threadIdx.x + kDqThreads * u, c = id % Sh<D>::CPR;
    const int r = PK ? rowtab[min(64 * s + id / Sh<D>::CPR, nvalid - 1)] : min(id / Sh<D>::CPR, g.C - 1);
    pf.k[u] = ld16(a.kp + hb + (size_t)r * D + c * 8);
    pf.v[u] = ld16(a.vp + hb + (size_t)r * D + c * 8);
  }
}

// LDS: K rows 0-31, K rows 32-63, V rows 0-31, V rows 32-63 (four tiles)
template <int D>
__device__ __forceinline__ void slot_store(const SlotPf<D>& pf, char* buf, int n) {
#pragma unroll
  for (int u = 0; u < SlotPf<D>::N; ++u) {
    const int id = threadIdx.x + kDqThreads * u, r = id / Sh<D>::CPR, c = id % Sh<D>::CPR;
    const bool ok = r < n;
    st_chunk(buf + (r >> 5) * Sh<D>::TILEB, Sh<D>::ROWB, Sh<D>::CPR, r & 31, c, ok ? pf.k[u] : make_uint4(0, 0, 0, 0));
    st_chunk(buf + (2 + (r >> 5)) * Sh<D>::TILEB, Sh<D>::ROWB, Sh<D>::CPR, r & 31, c,
             ok ? pf.v[u] : make_uint4(0, 0, 0, 0));
  }
}

template <int D, bool DS, bool PK>
__global__ __launch_bounds__(kDqThreads, 1) void dq_pers_kernel(BwdArgs a) {
  // DS: also store every dS tile for dk_ds.  PK: the keys are the head's
  // valid slot rows packed (a row table in LDS), 64 per step, so only the
  // last step is partial; else one slot per step (its 64 rows, padded).
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int BUF = 4 * Sh<D>::TILEB;
  const Geo& g = a.g;
  const int total = g.B * g.H * a.ntiles;
  const int lin = xcd_remap(total);
  if (lin >= total) return;
  const int qt = lin % a.ntiles;
  const size_t bh = lin / a.ntiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int r = qt * kDqRows + 32 * wave + l32;
  const bool ok = r < g.ct;
  const bool active = qt * kDqRows + 32 * wave < g.ct;
  QState<D> st;
  q_init<D>(a, bh, ok ? r : 0, ok, st);
  const float c2 = g.scale * kLog2e;
  const int nqt = (g.ct + 31) / 32;  // query tiles of the head; this wave's is qt * kDqWaves + wave
  bf16_t* dsw = DS ? a.dsb + ((size_t)bh * 2 * g.S * nqt + qt * kDqWaves + wave) * 1024 : nullptr;
  // Slot lengths (or the packed row table) go to LDS before the first dS
  // store: a length read from global memory later would wait (vmcnt) for
  // every store in flight.
  int* plen_s = reinterpret_cast<int*>(smem + 2 * BUF);  // [S], or PK: prefix sums [S+1]
  int* rowtab = plen_s + g.S + 1;                        // PK: [S*C]
  int nsteps = g.S, nvalid = 0;
  if (PK) {
    nvalid = packed_rows(a.plen + bh * g.S, g.S, g.C, plen_s, rowtab, kDqThreads);
    nsteps = (nvalid + 63) / 64;
  } else {
    for (int i = threadIdx.x; i < g.S; i += kDqThreads) plen_s[i] = min(a.plen[bh * g.S + i], g.C);
    __syncthreads();
  }
  // rows of step s
  auto rows_of = [&](int s) { return PK ? min(nvalid - 64 * s, 64) : plen_s[s]; };
  if (nsteps > 0) {
    SlotPf<D> pf;
    slot_load<D, PK>(a, bh, 0, pf, rowtab, nvalid);
    slot_store<D>(pf, smem, rows_of(0));
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      if (s + 1 < nsteps) slot_load<D, PK>(a, bh, s + 1, pf, rowtab, nvalid);
      if (active) {
        // rows at or past n are staged as zeros: no key mask needed (see
        // q_tile); dS goes to the tiles of key tiles 2s and 2s+1
        const int n = rows_of(s), rb = (s & 1) * BUF;
        bf16_t* dso = DS ? dsw + (size_t)(2 * s) * nqt * 1024 : nullptr;
        if (n > 0)
          q_tile<D, kHoistDqPers, false, false, false, DS>(smem, rb, rb + 2 * Sh<D>::TILEB, 32, c2, st, NoMid{},
                                                           dso);
        if (n > 32)
          q_tile<D, kHoistDqPers, false, false, false, DS>(smem, rb + Sh<D>::TILEB, rb + 3 * Sh<D>::TILEB, 32,
                                                           c2, st, NoMid{}, DS ? dso + (size_t)nqt * 1024 : nullptr);
      }
      if (s + 1 < nsteps) slot_store<D>(pf, smem + ((s + 1) & 1) * BUF, rows_of(s + 1));
      __syncthreads();
    }
  }
  if (!ok) return;
  float* out = a.dq + (bh * g.ct + r) * D;
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      *reinterpret_cast<float4*>(out + 32 * dt + 8 * i4 + 4 * h) =
          make_float4(st.acc[dt][4 * i4] * g.scale, st.acc[dt][4 * i4 + 1] * g.scale,
                      st.acc[dt][4 * i4 + 2] * g.scale, st.acc[dt][4 * i4 + 3] * g.scale);
}

// Local part: kLocBlocks query blocks x 2 query tiles per workgroup; per step
// the 32-row half of each query block's current selected block (K and V) is
// staged.  One block per workgroup (four workgroups per CU) keeps a step's
// barrier to the two waves of one block, whose work differs from block to
// block (6% faster than four blocks sharing one barrier).
constexpr int kLocBlocks = 1;  // query blocks per workgroup (2 waves each)
constexpr int kDqlThreads = 64 * 2 * kLocBlocks;

// Row tokens of every step of this workgroup, built once in LDS (see the
// forward's local kernel): the selected blocks' rows packed into consecutive
// 32-row steps, rowtab[32*step + r] (-1 past the last row, up to the step
// boundary), binfo[t], and lentab[t] = block t's first packed row (lentab[K]
// = the total).  Used when they fit in the LDS beside the two step buffers;
// otherwise every gather places its rows, two steps per selected block.
template <int D>
constexpr size_t dql_tab_room() {
  return 160 * 1024 - 2 * (size_t)kLocBlocks * 2 * Sh<D>::TILEB;
}

__device__ __forceinline__ void build_rowtab(const BwdArgs& a, size_t bh, int qg, int nthreads, int* rowtab,
                                             int2* binfo, int* lentab) {
  static_assert(kLocBlocks == 1, "one query block per workgroup");
  const Geo& g = a.g;
  const int nb = kLocBlocks * g.K;
  // one thread per selected block: where it sits in the ring (binfo: first
  // ring token; length and extents, 8 bits each)
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
  if (threadIdx.x < 64) {  // wave 0: exclusive scan of the lengths, 64 blocks per round
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
  const int nrows = lentab[nb];
  for (int x = threadIdx.x; x < nb * 64; x += nthreads) {
    const int r = x & 63, t = x >> 6;
    const int2 bi = binfo[t];
    const LocBlock b{bi.x, bi.y & 255, (bi.y >> 8) & 255, bi.y >> 16};
    if (r < b.len) rowtab[lentab[t] + r] = loc_row(g, b, r);
  }
  // past the last row up to the step boundary, and the whole first step when
  // no block is selected (the first gather is issued regardless): the zero row
  for (int x = nrows + threadIdx.x; x < max(32, (nrows + 31) & ~31); x += nthreads) rowtab[x] = -1;
}

// One local step gathered straight into LDS (global_load_lds_dwordx4): no
// staging registers and no LDS store instructions.  An instruction fills 1 KB
// of the buffer (lane l at byte 16*l); lane l fetches the global chunk whose
// swizzled position is l's, so the tile lands in the swizzled layout.  Rows
// past a selected block's end (and absent selections) load the zero row
// instead, so the tile needs no key mask (see q_tile).  TAB:
// row tokens from the LDS table (compile-time, see the forward's local
// kernel).
template <int D, bool TAB>
__device__ __forceinline__ void loc_gather(const BwdArgs& a, size_t bh, int qg, int j, char* buf,
                                           const int* rowtab) {
  constexpr int RPK = 1024 / Sh<D>::ROWB;                // rows per KB unit
  constexpr int UPT = Sh<D>::TILEB / 1024;               // KB units per 32-row tile
  constexpr int PER_WAVE = kLocBlocks * 2 * UPT / (kDqlThreads / 64);
  const Geo& g = a.g;
  const int t = j >> 1, half = j & 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rr = lane / Sh<D>::CPR, pos = lane % Sh<D>::CPR;
  const bf16_t* kb = a.kl + bh * (size_t)g.NL * D;
  const bf16_t* vb = a.vl + bh * (size_t)g.NL * D;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int u = wave * PER_WAVE + i;
    const int w = u / (2 * UPT), tensor = (u / UPT) & 1;
    const int r = RPK * (u % UPT) + rr;  // row in the 32-row tile
    const int c = swz(r, pos, Sh<D>::CPR);
    int tok = -1;
    if (TAB) {
      tok = rowtab[32 * j + r];  // packed rows (one query block per workgroup)
    } else {
      const int qb = qg * kLocBlocks + w;
      if (qb < g.nq) {
        const int p = a.topk[(bh * g.nq + qb) * g.K + t];
        if ((unsigned)p < (unsigned)g.nl) {
          const LocBlock b = loc_block(g, p);
          if (32 * half + r < b.len) tok = loc_row(g, b, 32 * half + r);
        }
      }
    }
    const bf16_t* src = (tok >= 0 ? (tensor ? vb : kb) + (size_t)tok * D : a.zrow) + c * 8;
    PBSA_LDS_LOAD(src, (__attribute__((address_space(3))) void*)(buf + u * 1024), 16, 0, 0);
  }
}

template <int D, bool TAB>
// 2 waves per SIMD: the register budget of four such workgroups per CU
__global__ __launch_bounds__(kDqlThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_local_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];  // row tables
  constexpr int BUF = kLocBlocks * 2 * Sh<D>::TILEB;
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
  const bool active = has_q && 32 * nt < qe.len;
  const int r = 32 * nt + l32;
  const bool ok = active && r < qe.len;
  const int tok = ok ? block_token(g, qe, r) : 0;
  QState<D> st;
  q_init<D>(a, bh, tok, ok, st);
  const float c2 = g.scale * kLog2e;
  // TAB: the selected blocks' rows packed into consecutive 32-row steps
  // (only the last partial); otherwise two steps per selected block
  int nsteps = 2 * g.K;
  int* rowtab = reinterpret_cast<int*>(smem);
  int2* binfo = reinterpret_cast<int2*>(rowtab + kLocBlocks * g.K * 64);
  int* lentab = reinterpret_cast<int*>(binfo + kLocBlocks * g.K);
  int nrows = 0;
  if (TAB) {
    build_rowtab(a, bh, qg, kDqlThreads, rowtab, binfo, lentab);
    __syncthreads();
    nrows = lentab[kLocBlocks * g.K];
    nsteps = (nrows + 31) / 32;
  }
  loc_gather<D, TAB>(a, bh, qg, 0, kv0, rowtab);
  __syncthreads();  // its fence waits for the gather
  // unrolled by two so that each step's buffers are compile-time arrays
  auto step = [&](int j, char* cur, char* nxt) {
    int nv = 0;
    if (active) {
      if (TAB) {
        nv = min(nrows - 32 * j, 32);
      } else {
        const int p = a.topk[(bh * g.nq + qb) * g.K + (j >> 1)];
        const int len = (unsigned)p < (unsigned)g.nl ? block_ext(g, p % g.nq).len : 0;
        nv = min(len - 32 * (j & 1), 32);
      }
    }
    nv = __builtin_amdgcn_readfirstlane(nv);  // uniform per wave: a scalar branch
    auto gather = [&]() {
      if (j + 1 < nsteps) loc_gather<D, TAB>(a, bh, qg, j + 1, nxt, rowtab);
    };
    if (nv > 0) {
      const int rel = (wave >> 1) * 2 * Sh<D>::TILEB;
      q_tile<D, true, true, true, false>(cur, rel, rel + Sh<D>::TILEB, nv, c2, st, gather);
    } else {
      gather();
    }
    __syncthreads();
  };
  for (int j = 0; j < nsteps; j += 2) {
    step(j, kv0, kv1);
    if (j + 1 < nsteps) step(j + 1, kv1, kv0);
  }
  if (!ok) return;
  float* out = a.dq + (bh * g.ct + tok) * D;
  float4 prev[Sh<D>::DT][4];  // the persistent part, all loads issued before the first use
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) prev[dt][i4] = *reinterpret_cast<const float4*>(out + 32 * dt + 8 * i4 + 4 * h);
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4* o4 = reinterpret_cast<float4*>(out + 32 * dt + 8 * i4 + 4 * h);
      float4 v = prev[dt][i4];
      v.x += st.acc[dt][4 * i4] * g.scale;
      v.y += st.acc[dt][4 * i4 + 1] * g.scale;
      v.z += st.acc[dt][4 * i4 + 2] * g.scale;
      v.w += st.acc[dt][4 * i4 + 3] * g.scale;
      // gradients are written once and not read again here: non-temporal
      // stores keep them from evicting the gathered rows from L2
      typedef float nf4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(nf4{v.x, v.y, v.z, v.w}, reinterpret_cast<nf4*>(o4));
    }
}

// ===========================================================================
// dK, dV, key-outer
// ===========================================================================
// Key-outer state of one wave (32 keys).  A dV role needs K only
// (S = Q K^T, dV += P^T dO); a dK role needs K and V (dP = dO V^T,
// dK += dS^T Q).  Separate waves keep each under 256 registers so two
// waves share a SIMD.  The dK role holds -V: its dP product then starts from
// D (read from LDS straight into the accumulator) and ends at D - dP, so the
// tile forms -dS with one multiply per score, and the result is written
// negated.
template <int D, bool DV> struct KState {
  bf16x8_t kf[Sh<D>::KS];
  bf16x8_t vf[DV ? 1 : Sh<D>::KS];  // -V
  f32x16_t acc[Sh<D>::DT];
};

template <int D, bool DV>
__device__ __forceinline__ void k_init(const bf16_t* krow, const bf16_t* vrow, bool ok, KState<D, DV>& st) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < Sh<D>::KS; ++ks) {
    st.kf[ks] = __builtin_bit_cast(bf16x8_t, ok ? ld16(krow + 16 * ks + 8 * h) : make_uint4(0, 0, 0, 0));
    if (!DV) {
      const uint4 v = ok ? ld16(vrow + 16 * ks + 8 * h) : make_uint4(0, 0, 0, 0);
      const unsigned sg = 0x80008000u;  // bf16 sign bits
      st.vf[DV ? 0 : ks] = __builtin_bit_cast(bf16x8_t, make_uint4(v.x ^ sg, v.y ^ sg, v.z ^ sg, v.w ^ sg));
    }
  }
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt) st.acc[dt] = f32x16_t{};
}

// One 32-query tile in LDS: Q tile tq, dO tile td, per-row lse*log2e and D.
// Rows that do not exist carry lse*log2e = +inf (their probability is 0).
// The transposed B operands are read ahead of the VALU work (HOIST): after
// the first products, or with EARLY first of all, before mid().  XADDR:
// natural reads through per-read XOR offsets from the array arr holding the
// tiles (see q_tile).  ASMTR: transposed reads in asm blocks that wait for
// their own reads: all at once (rd_tr_all) in a dV role, per column tile
// after the softmax (rd_tr_dt, fewer live registers) in a dK role, which
// holds V as well.  PX (P exchange between the two waves of a key tile): 1,
// a dV role, stores its P tile (fp32, 4 float4 per lane) in pex and calls
// sync(); 2, a dK role, skips S = Q K^T and the exponentials, calls sync()
// after its dP product and reads P from pex: the same values, one product
// fewer per tile.
template <int D, bool DV, bool EARLY = false, bool XADDR = false, bool ASMTR = false, typename Mid = NoMid,
          int PX = 0, typename Sync = NoMid>
__device__ __forceinline__ void k_tile(const char* tq, const char* td, const float* lse2, const float* dl, float c2,
                                       KState<D, DV>& st, Mid mid = Mid{}, const char* arr = nullptr,
                                       float4* pex = nullptr, Sync sync = Sync{}) {
  constexpr bool HOIST = !ASMTR || DV;
  static_assert(HOIST || !EARLY, "EARLY reads are hoisted reads");
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const char* tb = DV ? td : tq;  // dV += P^T dO ; dK += dS^T Q
  bf16x8_t bt[HOIST ? Sh<D>::DT : 1][2];  // transposed B operands
  auto read_bt = [&]() {
    if constexpr (ASMTR && HOIST) {
      rd_tr_all<D>(tb, bt);
      return;
    }
#pragma unroll
    for (int dt = 0; dt < Sh<D>::DT; ++dt) {
      bt[HOIST ? dt : 0][0] = rd_tr<D>(tb, 0, dt);
      bt[HOIST ? dt : 0][1] = rd_tr<D>(tb, 1, dt);
    }
  };
  if (EARLY) {
    read_bt();
    __builtin_amdgcn_sched_barrier(0);  // keep mid() after the reads
  }
  mid();
  f32x16_t s = {}, dp = {};
  if (!DV) {  // dp starts at D (rows 8i + 4h + jj of element 4i + jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 Dv = *reinterpret_cast<const float4*>(dl + 8 * i + 4 * h);
      dp[4 * i] = Dv.x;
      dp[4 * i + 1] = Dv.y;
      dp[4 * i + 2] = Dv.z;
      dp[4 * i + 3] = Dv.w;
    }
  }
  if (XADDR) {
    const int bq = nat_base<D>((int)(tq - arr), l32, h);
    const int bd = DV ? 0 : nat_base<D>((int)(td - arr), l32, h);
#pragma unroll
    for (int ks = 0; ks < Sh<D>::KS; ++ks) {
      if (PX != 2) s = mfma(rd_nat_at<D>(arr, bq, ks), st.kf[ks], s);
      if (!DV) dp = mfma(rd_nat_at<D>(arr, bd, ks), st.vf[DV ? 0 : ks], dp);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < Sh<D>::KS; ++ks) {
      s = mfma(rd_nat<D>(tq, l32, 2 * ks + h), st.kf[ks], s);
      if (!DV) dp = mfma(rd_nat<D>(td, l32, 2 * ks + h), st.vf[DV ? 0 : ks], dp);
    }
  }
  if constexpr (HOIST && !EARLY) read_bt();
  f32x16_t x;
  if constexpr (PX == 2) {
    // P from the dV wave of this key tile
    sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 P = pex[i * 64 + lane];
      x[4 * i] = P.x * dp[4 * i];
      x[4 * i + 1] = P.y * dp[4 * i + 1];
      x[4 * i + 2] = P.z * dp[4 * i + 2];
      x[4 * i + 3] = P.w * dp[4 * i + 3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 L = *reinterpret_cast<const float4*>(lse2 + 8 * i + 4 * h);
      const float Ls[4] = {L.x, L.y, L.z, L.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * i + jj;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[j], c2, -Ls[jj]));
        x[j] = DV ? p : p * dp[j];  // P, or -dS = P (D - dP)
      }
    }
    if constexpr (PX == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pex[i * 64 + lane] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
      sync();
    }
  }
  const bf16x8_t x0 = pack8(x, 0), x1 = pack8(x, 1);
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt) {
    if constexpr (!HOIST) rd_tr_dt<D>(tb, dt, bt[0]);
    st.acc[dt] = mfma(x0, bt[HOIST ? dt : 0][0], st.acc[dt]);
    st.acc[dt] = mfma(x1, bt[HOIST ? dt : 0][1], st.acc[dt]);
  }
}

// Write this wave's 32 key rows: row kr of the tile goes to dst(kr) if kr < n, else zero.
// Non-temporal stores: the gradients are not read again by these kernels, and
// cached they would evict the query rows the other workgroups gather.
template <int D, bool DV, typename RowPtr>
__device__ __forceinline__ void k_write(const KState<D, DV>& st, int n, float scale, RowPtr rows) {
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int kr = 8 * (j >> 2) + 4 * h + (j & 3);
    float* dst;
    if (!rows(kr, dst)) continue;
    const bool ok = kr < n;
#pragma unroll
    for (int dt = 0; dt < Sh<D>::DT; ++dt)
      __builtin_nontemporal_store(ok ? st.acc[dt][j] * scale : 0.f, dst + 32 * dt + l32);
  }
}

constexpr int kKvWaves = 8;       // dkv_pers, dk_ds: 8 waves = 4 slots x 2 key tiles
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvSlots = kKvWaves / 2;

// LDS-bound loads of one contiguous 32-row query tile of a head (Q and dO
// rows XOR-swizzled as the tiles expect, then lse*log2(e) in lanes 0-31 and
// D in lanes 32-63).  Every wave issues the same NLD loads (the lse2 / D row
// by all waves, to the same place), so a wait for "all but the last NLD"
// means exactly "all but this tile".  Rows past the head's last query repeat
// its Q / dO (finite) and read the lse2 / D sentinel after the last head
// (lse2 = +inf: no probability, so they add nothing).
template <int D> struct PersDma {
  static constexpr int RPK = 1024 / Sh<D>::ROWB;   // rows per 1 KB unit
  static constexpr int UPT = Sh<D>::TILEB / 1024;  // units per tensor tile
  static constexpr int NU = 2 * UPT / kKvWaves;    // Q / dO units per wave
  static constexpr int NLD = NU + 1;
  static constexpr int BUF = 2 * Sh<D>::TILEB + 256;
  static_assert(NU * kKvWaves == 2 * UPT, "whole units per wave");
  static __device__ __forceinline__ void issue(const BwdArgs& a, size_t bh, int row0, char* buf) {
    const Geo& g = a.g;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rr = lane / Sh<D>::CPR, pos = lane % Sh<D>::CPR;
    const size_t hb = bh * g.ct;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave * NU + i, t = u / UPT, uu = u % UPT;  // t: 0 Q, 1 dO
      const int r = RPK * uu + rr;
      const bf16_t* src = (t ? a.dout : a.q) + (hb + min(row0 + r, g.ct - 1)) * D + swz(r, pos, Sh<D>::CPR) * 8;
      PBSA_LDS_LOAD(src, (__attribute__((address_space(3))) void*)(buf + t * Sh<D>::TILEB + uu * 1024), 16, 0, 0);
    }
    const int rl = row0 + (lane & 31);
    const size_t ro = rl < g.ct ? hb + rl : (size_t)g.B * g.H * g.ct;
    PBSA_LDS_LOAD(lane < 32 ? a.lse2 + ro : a.delta + ro,
                  (__attribute__((address_space(3))) void*)(buf + 2 * Sh<D>::TILEB), 4, 0, 0);
  }
};

// dV (DV) or dK of the persistent slots; dK comes from dk_ds where the dS
// tiles are stored.
// PK (the dV pass beside the packed dk_ds): every wave takes 32 consecutive
// valid rows of the head's slots (the rows numbered through the prefix sums
// of the slot lengths, as dq_pers and dk_ds number them), so slots shorter
// than 64 rows leave no half-empty key tiles and the head needs fewer
// workgroups; each workgroup also writes the zero dV and dK of the rows past
// the lengths of its share of the slots.
template <int D, bool DV, bool PK>
__global__ __launch_bounds__(kKvThreads, 1) void dkv_pers_kernel(BwdArgs a) {
  static_assert(!PK || DV, "packed rows: the dV pass");
  using Dm = PersDma<D>;
  // three step buffers, separate arrays so that the compiler can tell the
  // loads into one from the reads of another
  __shared__ __attribute__((aligned(1024))) char kb0[Dm::BUF];
  __shared__ __attribute__((aligned(1024))) char kb1[Dm::BUF];
  __shared__ __attribute__((aligned(1024))) char kb2[Dm::BUF];
  __shared__ int dst32[PK ? kKvWaves : 1][32];  // PK: slot*C + row of each key of each wave's tile
  extern __shared__ __attribute__((aligned(16))) int pre[];  // PK: [S+1] prefix sums of the slot lengths
  const Geo& g = a.g;
  const int total = g.B * g.H * a.ntiles;
  const int lin = xcd_remap(total);
  if (lin >= total) return;
  const int sp = lin % a.ntiles;  // slot group, or PK: group of packed key tiles
  const size_t bh = lin / a.ntiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31;
  const int slot = kKvSlots * sp + (wave >> 1), kh = wave & 1;
  const bool has_slot = slot < g.S;
  int nk;  // valid keys of this wave's tile
  size_t sbase = 0;
  bool busy = true;  // PK: the workgroup has a tile
  KState<D, DV> st;
  if constexpr (PK) {
    const int nvalid = packed_rows(a.plen + bh * g.S, g.S, g.C, pre, nullptr, kKvThreads);
    const int kt = kKvWaves * sp + wave;
    nk = __builtin_amdgcn_readfirstlane(min(max(nvalid - 32 * kt, 0), 32));
    busy = kKvWaves * sp * 32 < nvalid;
    int off = 0;
    const bool ok = l32 < nk;
    if (ok) {
      const int p = 32 * kt + l32, sl = packed_slot(pre, g.S, p);
      off = sl * g.C + (p - pre[sl]);
    }
    if (lane < 32) dst32[wave][lane] = off;
    const size_t hb = bh * (size_t)g.S * g.C * D;
    k_init<D, DV>(a.kp + hb + (size_t)off * D, a.vp + hb + (size_t)off * D, ok, st);
  } else {
    const int n = has_slot ? min(a.plen[bh * g.S + slot], g.C) : 0;
    nk = __builtin_amdgcn_readfirstlane(min(max(n - 32 * kh, 0), 32));
    sbase = (bh * g.S + (has_slot ? slot : 0)) * (size_t)g.C * D;
    const int kr = 32 * kh + l32;
    k_init<D, DV>(a.kp + sbase + (size_t)kr * D, a.vp + sbase + (size_t)kr * D, kr < n, st);
  }
  const float c2 = g.scale * kLog2e;

  // Every query tile of the head streams through LDS, loaded two steps
  // ahead: step i computes on buffer i%3 while the tiles of steps i+1 and
  // i+2 land.  The barrier that ends a step waits for all but the loads it
  // issued; the transposed operands are read by asm that the compiler's own
  // waits do not cover, so they do not drain the loads in flight either.
  // Every step issues its loads (steps past the end repeat the last tile),
  // so the counts hold on every path.  (PK: a workgroup without a tile, the
  // same for all its waves, skips the stream.)
  if (busy) {
    const int nsteps = (g.ct + 31) / 32, last = nsteps - 1;
    Dm::issue(a, bh, 0, kb0);
    Dm::issue(a, bh, 32 * min(1, last), kb1);
    vm_barrier<Dm::NLD>();
    auto step = [&](int i, char* cur, char* nx2) {
      Dm::issue(a, bh, 32 * min(i + 2, last), nx2);
      if (nk > 0 && i <= last) {
        const float* f = reinterpret_cast<const float*>(cur + 2 * Sh<D>::TILEB);
        k_tile<D, DV, false, false, true>(cur, cur + Sh<D>::TILEB, f, f + 32, c2, st);
      }
      vm_barrier<Dm::NLD>();
    };
    for (int i = 0; i < nsteps; i += 3) {
      step(i, kb0, kb2);
      step(i + 1, kb1, kb0);
      step(i + 2, kb2, kb1);
    }
    __builtin_amdgcn_s_waitcnt(0xF70);  // the last loads land before the workgroup can end
  }
  typedef float nf2 __attribute__((ext_vector_type(2)));
  if constexpr (PK) {
    const size_t hb = bh * (size_t)g.S * g.C * D;
    if (nk > 0)
      k_write<D, DV>(st, nk, 1.0f, [&](int r, float*& dst) {
        if (r >= nk) return false;
        dst = a.dvp + hb + (size_t)dst32[wave][r] * D;
        return true;
      });
    // the rows past the slot lengths of this workgroup's share of the slots:
    // zero dV here, zero dK for the packed dk_ds, which writes only the rows
    // that exist
    const int s0 = (int)((long long)sp * g.S / a.ntiles), s1 = (int)((long long)(sp + 1) * g.S / a.ntiles);
    for (int sl = s0; sl < s1; ++sl) {
      const int len = pre[sl + 1] - pre[sl];
      const int n2 = (g.C - len) * (D / 2);
      for (int x = threadIdx.x; x < n2; x += kKvThreads) {
        const size_t e = hb + ((size_t)sl * g.C + len + x / (D / 2)) * D + 2 * (x % (D / 2));
        __builtin_nontemporal_store(nf2{0.f, 0.f}, reinterpret_cast<nf2*>(a.dvp + e));
        __builtin_nontemporal_store(nf2{0.f, 0.f}, reinterpret_cast<nf2*>(a.dkp + e));
      }
    }
    return;
  }
  if (!has_slot || 32 * kh >= g.C) return;
  float* ob = (DV ? a.dvp : a.dkp) + sbase;
  k_write<D, DV>(st, nk, DV ? 1.0f : -g.scale, [&](int r, float*& dst) {
    const int row = 32 * kh + r;
    if (row >= g.C) return false;
    dst = ob + (size_t)row * D;
    return true;
  });
  if (DV && a.pk) {
    // the packed dk_ds writes only the rows that exist: the slot's rows past
    // its length get their zero dK here
    float* zk = a.dkp + sbase;
    for (int r = max(nk, 0); r < 32 && 32 * kh + r < g.C; ++r)
      __builtin_nontemporal_store(nf2{0.f, 0.f}, reinterpret_cast<nf2*>(zk + (size_t)(32 * kh + r) * D) + lane % (D / 2));
  }
}

// dK of the persistent slots from the dS tiles that dq_pers stored:
// dK = scale dS^T Q, one product instead of the three of a recomputing pass.
// Key-outer like dkv_pers (8 waves = 4 slots x 2 key tiles, 32 keys per
// wave): every query tile of the head streams through LDS with each wave's
// dS tile for it, loaded two steps ahead into three buffers; both operands
// are read transposed (dS^T with lane = key, Q with lane = column), so their
// query orders match.  Every wave issues the same loads in every step:
// waves past the last slot load key tile 0's dS tiles, and waves whose key
// tile holds no keys load tiles that nothing wrote; both skip the product.
// Where a Q tile has fewer 1 KB units than there are waves (head_dim 64),
// two waves load each unit, the same bytes to the same place.
template <int D> struct DsDma {
  static constexpr int RPK = 1024 / Sh<D>::ROWB;   // rows per 1 KB unit
  static constexpr int UPT = Sh<D>::TILEB / 1024;  // units per Q tile
  static constexpr int NQ = UPT >= kKvWaves ? UPT / kKvWaves : 1;
  static constexpr int NLD = NQ + 2;               // Q units, then the wave's 2 KB dS tile
  static constexpr int QB = Sh<D>::TILEB;          // the dS tiles follow the Q tile
  static constexpr int BUF = QB + kKvWaves * 2048;
  static_assert(UPT % kKvWaves == 0 || kKvWaves % UPT == 0, "whole Q units per wave");
  static __device__ __forceinline__ void issue(const BwdArgs& a, size_t bh, const bf16_t* dsw, int qtile,
                                               char* buf) {
    const Geo& g = a.g;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rr = lane / Sh<D>::CPR, pos = lane % Sh<D>::CPR;
    const int row0 = 32 * qtile;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int u = (wave * NQ + i) % UPT, r = RPK * u + rr;
      const bf16_t* src = a.q + (bh * g.ct + min(row0 + r, g.ct - 1)) * D + swz(r, pos, Sh<D>::CPR) * 8;
      PBSA_LDS_LOAD(src, (__attribute__((address_space(3))) void*)(buf + u * 1024), 16, 0, 0);
    }
    // the dS tile, read once: a streaming (nt) load, so that the 2 KB tiles
    // of the whole pass do not evict what the caches hold for later kernels
    const bf16_t* ds = dsw + (size_t)qtile * 1024 + lane * 8;
    constexpr int kNt = 2;  // cache-policy operand: nt
#pragma unroll
    for (int u = 0; u < 2; ++u)
      PBSA_LDS_LOAD(ds + u * 512, (__attribute__((address_space(3))) void*)(buf + QB + wave * 2048 + u * 1024), 16, 0,
                    kNt);
  }
};

// PK: the key tiles are the head's packed valid rows (as dq_pers<PK> stored
// their dS tiles).  The head's nkt tiles are split evenly over its
// workgroups (sp takes tiles [sp*nkt/G, (sp+1)*nkt/G), one per wave, G =
// ceil(S/4) workgroups per head), so that the compute units, two workgroups
// each, carry nearly equal numbers of busy waves: the kernel's time follows
// the most loaded unit.  Rows are written through the prefix sums of the
// slot lengths; the rows past the slots' lengths, which no tile covers, get
// their zeros from the dV pass of dkv_pers.
template <int D, bool PK>
__global__ __launch_bounds__(kKvThreads, 1) void dk_ds_kernel(BwdArgs a) {
  using Dm = DsDma<D>;
  __shared__ __attribute__((aligned(1024))) char db0[Dm::BUF];
  __shared__ __attribute__((aligned(1024))) char db1[Dm::BUF];
  __shared__ __attribute__((aligned(1024))) char db2[Dm::BUF];
  __shared__ int dst32[PK ? kKvWaves : 1][32];  // PK: slot*C + row of each key of each wave's tile
  extern __shared__ __attribute__((aligned(16))) int pre[];  // PK: [S+1] prefix sums of the slot lengths
  const Geo& g = a.g;
  const int total = g.B * g.H * a.ntiles;
  const int lin = xcd_remap(total);
  if (lin >= total) return;
  const int sp = lin % a.ntiles;  // slot group, or PK: group of packed key tiles
  const size_t bh = lin / a.ntiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = kKvSlots * sp + (wave >> 1), kh = wave & 1;
  const int nqt = (g.ct + 31) / 32, last = nqt - 1;
  int nk, kt;  // valid keys of this wave's tile, its key tile (dS tile row)
  if (PK) {
    const int nvalid = packed_rows(a.plen + bh * g.S, g.S, g.C, pre, nullptr, kKvThreads);
    const int nkt = (nvalid + 31) / 32;
    const int t0 = sp * nkt / a.ntiles, t1 = (sp + 1) * nkt / a.ntiles;  // at most kKvWaves tiles
    kt = t0 + wave;
    nk = kt < t1 ? __builtin_amdgcn_readfirstlane(min(nvalid - 32 * kt, 32)) : 0;
    if (nk > 0 && lane < 32) {
      const int p = 32 * kt + lane;
      if (p < nvalid) {
        const int sl = packed_slot(pre, g.S, p);
        dst32[PK ? wave : 0][lane] = sl * g.C + (p - pre[sl]);
      }
    }
    if (t0 >= t1) return;  // no tile for this workgroup (uniform)
    if (nk <= 0) kt = t0;  // loads of an existing tile, no product
  } else {
    const bool has_slot = slot < g.S;
    const int n = has_slot ? min(a.plen[bh * g.S + slot], g.C) : 0;
    nk = __builtin_amdgcn_readfirstlane(min(max(n - 32 * kh, 0), 32));
    kt = has_slot ? 2 * slot + kh : 0;
  }
  const bf16_t* dsw = a.dsb + ((size_t)bh * 2 * g.S + kt) * nqt * 1024;
  KState<D, true> st;
#pragma unroll
  for (int dt = 0; dt < Sh<D>::DT; ++dt) st.acc[dt] = f32x16_t{};
  Dm::issue(a, bh, dsw, 0, db0);
  Dm::issue(a, bh, dsw, min(1, last), db1);
  vm_barrier<Dm::NLD>();
  auto step = [&](int i, char* cur, char* nx2) {
    Dm::issue(a, bh, dsw, min(i + 2, last), nx2);
    if (nk > 0 && i <= last) {
      bf16x8_t as[2];
      rd_tr_ds(cur + Dm::QB + wave * 2048, as);
#pragma unroll
      for (int dt = 0; dt < Sh<D>::DT; ++dt) {
        bf16x8_t bt[2];
        rd_tr_dt<D>(cur, dt, bt);
        st.acc[dt] = mfma(as[0], bt[0], st.acc[dt]);
        st.acc[dt] = mfma(as[1], bt[1], st.acc[dt]);
      }
    }
    vm_barrier<Dm::NLD>();
  };
  for (int i = 0; i < nqt; i += 3) {
    step(i, db0, db2);
    step(i + 1, db1, db0);
    step(i + 2, db2, db1);
  }
  __builtin_amdgcn_s_waitcnt(0xF70);  // the last loads land before the workgroup can end
  if (PK) {
    if (nk <= 0) return;
    float* ob = a.dkp + bh * g.S * (size_t)g.C * D;
    k_write<D, true>(st, nk, g.scale, [&](int r, float*& dst) {
      if (r >= nk) return false;
      dst = ob + (size_t)dst32[PK ? wave : 0][r] * D;
      return true;
    });
    return;
  }
  if (slot >= g.S || 32 * kh >= g.C) return;
  float* ob = a.dkp + (bh * g.S + slot) * (size_t)g.C * D;
  k_write<D, true>(st, nk, g.scale, [&](int r, float*& dst) {
    const int row = 32 * kh + r;
    if (row >= g.C) return false;
    dst = ob + (size_t)row * D;
    return true;
  });
}

// dkv_local: one local block (64 keys = 2 key tiles) per workgroup, 4 waves:
// waves 0-1 accumulate dV and waves 2-3 dK of the two key tiles, over the
// same gathered query tiles, which are staged into LDS once for both passes.
// The dV wave of a key tile hands its probabilities to the dK wave through
// LDS (a barrier in mid-step), so the dK wave computes dP and dK^T only: 16
// products per wave and step in both roles instead of 16 and 24 (171 -> 157
// us at the decode shape).
// A step is one 32-row half of one query block that selected this local
// block (key-block -> query-block lists from bwd_tindex_kernel, copied to LDS
// with the step list).  Q and dO rows and their lse*log2(e) / D are
// gathered straight into LDS (global_load_lds_dwordx4 / _dword) into two
// static buffers; the row tokens of the next gather are loaded one step
// ahead.  Step counts per local block are heavy-tailed (a few blocks are
// selected by most query blocks), so workgroups take their blocks in the
// order of korder: within each XCD's range, most selecting query blocks
// first, which keeps the longest workgroups off the end of the launch.
constexpr int kKvlThreads = 256;
constexpr int kKvlWaves = kKvlThreads / 64;

template <int D, bool PACK> struct KvlGather {
  static constexpr int RPK = 1024 / Sh<D>::ROWB;   // rows per KB unit
  static constexpr int UPT = Sh<D>::TILEB / 1024;  // KB units per 32-row tile
  static constexpr int UPW = UPT / kKvlWaves;      // units of each tensor per wave
  static constexpr int BUF = 2 * Sh<D>::TILEB + 256;  // Q tile, dO tile, lse2[32], D[32]
  // The next step's rows, read from LDS by tokens() and put together by
  // gather() a step later (so nothing waits for the reads in between): the
  // block's first token and length, the step's half, and the in-block
  // offsets of this lane's rows (units, and row lane%32 for lse2 / D).
  int tbase, tlen, thalf;
  int toff[UPW];
  int toffl;

  // step = (selecting-list index << 3) | (shape class << 1) | half;
  // sbase[i], slen[i] = first token and length of selecting block i;
  // shape_off[c*64 + r] = offset of row r from the first token in class c.
  // (Plain int reads: reads of a vector type made the compiler wait for the
  // gather in flight.)
  __device__ __forceinline__ void tokens(const int* sbase, const int* slen, const int* shape_off, int step) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sidx = step >> 3, half = step & 1;
    const int* off = shape_off + ((step >> 1) & 3) * 64;
    tbase = sbase[sidx];
    tlen = slen[sidx];
    thalf = half;
#pragma unroll
    for (int i = 0; i < UPW; ++i) toff[i] = off[32 * half + RPK * (wave * UPW + i) + lane / Sh<D>::CPR];
    toffl = off[32 * half + (threadIdx.x & 31)];
  }
  // PACK: the selecting blocks' rows packed into consecutive 32-row steps,
  // rtab[32*step + r] = the chunk token of row r of the step (-1: none)
  __device__ __forceinline__ void tokens(const int* rtab, int step) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < UPW; ++i) toff[i] = rtab[32 * step + RPK * (wave * UPW + i) + lane / Sh<D>::CPR];
    toffl = rtab[32 * step + (threadIdx.x & 31)];
  }
  // Issue the gather of the step whose tokens are held into buf: Q and dO
  // rows, and (wave 0) the rows' lse2 and D, lanes 0-31 and 32-63.  Rows
  // without a token load Q / dO row 0 of the head (finite filler) and the
  // lse2 / D sentinel, which gives them no probability.
  __device__ __forceinline__ void gather(const BwdArgs& a, size_t bh, char* buf) {
    const Geo& g = a.g;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rr = lane / Sh<D>::CPR, pos = lane % Sh<D>::CPR;
    const bf16_t* qb = a.q + bh * g.ct * (size_t)D;
    const bf16_t* db = a.dout + bh * g.ct * (size_t)D;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int u = wave * UPW + i;
      const int r = RPK * u + rr;
      const int tok = PACK ? max(toff[i], 0) : 32 * thalf + r < tlen ? tbase + toff[i] : 0;
      const int off = tok * D + swz(r, pos, Sh<D>::CPR) * 8;
      PBSA_LDS_LOAD(qb + off, (__attribute__((address_space(3))) void*)(buf + u * 1024), 16, 0, 0);
      PBSA_LDS_LOAD(db + off, (__attribute__((address_space(3))) void*)(buf + Sh<D>::TILEB + u * 1024), 16, 0, 0);
    }
    if (wave == 0) {
      // rows without a token read the sentinel after the last head: lse2 = +inf
      // (probability 0, so their dV and dS terms vanish) and D = 0
      const bool has = PACK ? toffl >= 0 : 32 * thalf + (lane & 31) < tlen;
      const size_t ro = has ? bh * g.ct + (PACK ? toffl : tbase + toffl) : (size_t)g.B * g.H * g.ct;
      PBSA_LDS_LOAD(lane < 32 ? a.lse2 + ro : a.delta + ro,
                    (__attribute__((address_space(3))) void*)(buf + 2 * Sh<D>::TILEB), 4, 0, 0);
    }
  }
};

// LDS beyond the static arrays: the row offsets of the four block shapes,
// the selecting blocks' first tokens and their lengths and shape classes,
// and the steps (up to two per block).
constexpr size_t kvl_lds(int nq) { return 4 * 64 * 4 + (size_t)nq * (4 + 4 + 2 * 4); }
// PACK: the same lists plus the selecting blocks' first packed rows and the
// packed row table (up to 64 rows per selecting block, padded to a step)
constexpr size_t kvl_lds_pack(int nq) { return 4 * 64 * 4 + (size_t)nq * (4 + 4 + 4) + 4 + ((size_t)nq * 64 + 32) * 4; }
// dynamic LDS that keeps two workgroups per CU beside the static arrays (the
// two step buffers, each 1 KB aligned, and the probability hand-over)
template <int D>
constexpr size_t kvl_pack_room() {
  return 80 * 1024 - 2 * (((size_t)KvlGather<D, true>::BUF + 1023) & ~size_t(1023)) - 2 * 4 * 64 * 16;
}

// The key-outer pass of one role (dV or dK) over the workgroup's step list;
// every wave runs the same number of barriers and gathers whatever its role.
template <int D, bool DV, bool PACK>
__device__ __forceinline__ void kvl_pass(const BwdArgs& a, size_t bh, int p, int kt, const int* sbase,
                                         const int* slen, const int* shape_off, const int* steps, int nsteps,
                                         char* kv0, char* kv1, float4* pex) {
  const Geo& g = a.g;
  const int l32 = threadIdx.x & 31;
  const BlockExt ke = block_ext(g, p % g.nq);
  const int koff = (p / g.nq) * g.ct;
  const int nk = __builtin_amdgcn_readfirstlane(min(max(ke.len - 32 * kt, 0), 32));  // uniform per wave
  const int kr = 32 * kt + l32;
  const bool kok = kr < ke.len;
  const size_t krow = (bh * g.NL + koff + (kok ? block_token(g, ke, kr) : 0)) * (size_t)D;
  KState<D, DV> st;
  k_init<D, DV>(a.kl + krow, a.vl + krow, kok, st);
  const float c2 = g.scale * kLog2e;
  KvlGather<D, PACK> ga;
  // PACK: steps is the packed row table and the step index is the step
  auto toks = [&](int i) {
    if constexpr (PACK)
      ga.tokens(steps, i);
    else
      ga.tokens(sbase, slen, shape_off, steps[i]);
  };
  if (nsteps > 0) {
    toks(0);
    ga.gather(a, bh, kv0);
    if (nsteps > 1) toks(1);
  }
  __syncthreads();  // its fence waits for the gather
  // unrolled by two so that each step's buffers are compile-time arrays
  auto step = [&](int i, char* cur, char* nxt) {
    auto mid = [&]() {
      if (i + 1 < nsteps) {
        ga.gather(a, bh, nxt);
        if (i + 2 < nsteps) toks(i + 2);
      }
    };
    // mid-step barrier: the dV wave of each key tile has written its P
    auto sync = []() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); the LDS-bound loads stay in flight
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    if (nk > 0) {
      const float* f = reinterpret_cast<const float*>(cur + 2 * Sh<D>::TILEB);
      k_tile<D, DV, true, true, false, decltype(mid), DV ? 1 : 2, decltype(sync)>(cur, cur + Sh<D>::TILEB, f, f + 32,
                                                                                 c2, st, mid, cur, pex, sync);
    } else {
      mid();
      sync();
    }
    __syncthreads();
  };
  for (int i = 0; i < nsteps; i += 2) {
    step(i, kv0, kv1);
    if (i + 1 < nsteps) step(i + 1, kv1, kv0);
  }
  if (nk <= 0) return;
  float* ob = (DV ? a.dvl : a.dkl) + (bh * g.NL + koff) * (size_t)D;
  k_write<D, DV>(st, nk, DV ? 1.0f : -g.scale, [&](int r, float*& dst) {
    const int row = 32 * kt + r;
    if (row >= ke.len) return false;
    dst = ob + (size_t)block_token(g, ke, row) * D;
    return true;
  });
}

// PACK: the selecting blocks' rows packed into consecutive 32-row steps (only
// the last partial; used when the row table fits, see kvl_pack_room);
// otherwise one or two steps per selecting block from the step list.
template <int D, bool PACK>
__global__ __launch_bounds__(kKvlThreads, 2) void dkv_local_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];  // step lists
  // the two step buffers are separate arrays so that the compiler can tell the
  // gather into one from the reads of the other
  __shared__ __attribute__((aligned(1024))) char kv0[KvlGather<D, PACK>::BUF];
  __shared__ __attribute__((aligned(1024))) char kv1[KvlGather<D, PACK>::BUF];
  __shared__ float4 pex[2][4 * 64];  // P of each key tile's current step, from its dV wave
  const Geo& g = a.g;
  const int total = g.B * g.H * g.nl;
  const int slot = xcd_remap(total);
  if (slot >= total) return;
  const int lin = a.korder[slot];
  const int p = lin % g.nl;
  const size_t bh = lin / g.nl;
  const int wave = threadIdx.x >> 6;
  const int kt = wave & 1, role = wave >> 1;  // role 0: dV, role 1: dK

  // Row offsets inside a block by shape class (bit 1: a last block row of
  // fewer than block_h rows, bit 0: a last block column narrower than
  // block_w), one thread per (class, row).  Every block of a class places
  // its rows alike, so a row's token is one LDS read and an add.
  static_assert(kKvlThreads == 4 * 64, "one thread per shape class and row");
  int* shape_off = reinterpret_cast<int*>(smem);
  {
    const int c = threadIdx.x >> 6, r = threadIdx.x & 63;
    const int nh = (c & 2) ? g.fh - (g.nbr - 1) * g.bh : g.bh;
    const int nw = (c & 1) ? g.fw - (g.nbc - 1) * g.bw : g.bw;
    const int f = r / (nh * nw), rem = r - f * nh * nw, y = rem / nw;
    shape_off[threadIdx.x] = f * g.ft + y * g.fw + (rem - y * nw);
  }
  // selecting query blocks (ascending): each one's first token in the chunk
  // and its length and shape class, and the step list, in LDS
  const int ncount = a.tcount[bh * g.nl + p];
  const int32_t* lst = a.tlist + (bh * g.nl + p) * g.nq;
  int* sbase = shape_off + 4 * 64;
  int* slen = sbase + g.nq;
  int* steps = slen + g.nq;
  for (int x = threadIdx.x; x < ncount; x += kKvlThreads) {
    const BlockExt e = block_ext(g, lst[x]);
    const int cls = (e.nh != g.bh ? 2 : 0) | (e.nw != g.bw ? 1 : 0);
    sbase[x] = e.f0 * g.ft + e.r0 * g.fw + e.c0;
    slen[x] = e.len | cls << 8;  // the class moves into the steps below
  }
  __syncthreads();
  int nsteps = 0;
  if constexpr (PACK) {
    // first packed row of every selecting block (wave 0: exclusive scan, 64
    // blocks per round), then every row's chunk token, -1 past the last
    int* pre = steps;             // [ncount + 1]
    int* rtab = pre + g.nq + 1;   // [nq*64 + 32]
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      int run = 0;
      for (int x0 = 0; x0 < ncount; x0 += 64) {
        const int x = x0 + lane;
        const int n = x < ncount ? (slen[x] & 255) : 0;
        int v = n;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(v, o, 64);
          if (lane >= o) v += y;
        }
        __builtin_amdgcn_wave_barrier();
        if (x < ncount) pre[x] = run + v - n;
        run += __shfl(v, 63, 64);
      }
      if (lane == 0) pre[ncount] = run;
    }
    __syncthreads();
    const int nrows = pre[ncount];
    for (int x = threadIdx.x; x < ncount * 64; x += kKvlThreads) {
      const int r = x & 63, b = x >> 6, lc = slen[b];
      if (r < (lc & 255)) rtab[pre[b] + r] = sbase[b] + shape_off[(lc >> 8) * 64 + r];
    }
    for (int x = nrows + threadIdx.x; x < max(32, (nrows + 31) & ~31); x += kKvlThreads) rtab[x] = -1;
    __syncthreads();
    nsteps = (nrows + 31) / 32;
    if (role == 0)
      kvl_pass<D, true, true>(a, bh, p, kt, sbase, slen, shape_off, rtab, nsteps, kv0, kv1, pex[kt]);
    else
      kvl_pass<D, false, true>(a, bh, p, kt, sbase, slen, shape_off, rtab, nsteps, kv0, kv1, pex[kt]);
    return;
  }
  for (int x = 0; x < ncount; ++x) {
    const int lc = slen[x], nh = ((lc & 255) + 31) / 32;
    if ((int)threadIdx.x < nh) steps[nsteps + threadIdx.x] = (x << 3) | (lc >> 8) << 1 | threadIdx.x;
    nsteps += nh;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < ncount; x += kKvlThreads) slen[x] &= 255;
  __syncthreads();
  if (role == 0)
    kvl_pass<D, true, false>(a, bh, p, kt, sbase, slen, shape_off, steps, nsteps, kv0, kv1, pex[kt]);
  else
    kvl_pass<D, false, false>(a, bh, p, kt, sbase, slen, shape_off, steps, nsteps, kv0, kv1, pex[kt]);
}

template <typename K>
hipError_t set_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// The MFMA kernels, in order on the caller's stream: dK and dV of the local
// blocks, dV (and without stored dS tiles, dK) of the persistent slots, dQ
// of the persistent slots (with g.ds it also writes the dS tiles), dK of the
// slots from those tiles, then dQ of the local blocks.  (Running the dK/dV
// kernels on a second stream beside the dQ kernels measured within 1% of this
// order at the decode shape, so the library keeps to the caller's stream.)
// Most LDS for the packed row table of dq_pers (beside its 2 x 4 tiles).
constexpr size_t kDqTableMax = 60 * 1024;

template <int D>
hipError_t launch_d(const BwdArgs& base, hipStream_t s) {
  const Geo& g = base.g;
  // persistent keys packed (valid rows numbered consecutively) where the row table fits
  const size_t tab_dq = ((size_t)g.S * g.C + g.S + 1) * 4;
  const bool pk = g.S > 0 && tab_dq <= kDqTableMax;
  const size_t shm_dq = 2 * 4 * Sh<D>::TILEB + (pk ? tab_dq : g.S * 4);  // 2 x (K,K,V,V), row table or lengths
  const size_t tabb = (size_t)kLocBlocks * g.K * (64 * 4 + 8 + 4) + 4;
  const bool tab = tabb <= dql_tab_room<D>();
  const size_t shm_dql = tab ? tabb : 0;  // local: row tables (step buffers are static)
  const bool kvl_pack = kvl_lds_pack(g.nq) <= kvl_pack_room<D>();
  const size_t shm_kvl = kvl_pack ? kvl_lds_pack(g.nq) : kvl_lds(g.nq);
  static PerDeviceOnce attr;
  hipError_t e = attr.run([] {
    hipError_t r = set_lds(dq_pers_kernel<D, true, false>, 2 * 4 * Sh<D>::TILEB + 2048 * 4);
    if (r == hipSuccess) r = set_lds(dq_pers_kernel<D, false, false>, 2 * 4 * Sh<D>::TILEB + 2048 * 4);
    if (r == hipSuccess) r = set_lds(dq_pers_kernel<D, true, true>, 2 * 4 * Sh<D>::TILEB + kDqTableMax);
    if (r == hipSuccess) r = set_lds(dq_pers_kernel<D, false, true>, 2 * 4 * Sh<D>::TILEB + kDqTableMax);
    if (r == hipSuccess) r = set_lds(dq_local_kernel<D, true>, dql_tab_room<D>());
    if (r == hipSuccess) r = set_lds(dkv_local_kernel<D, false>, kvl_lds(2048));
    if (r == hipSuccess) r = set_lds(dkv_local_kernel<D, true>, kvl_pack_room<D>());
    return r;
  });
  if (e != hipSuccess) return e;
  BwdArgs a = base;
  const bool ds = g.ds && g.S > 0;
  a.pk = ds && pk;
  // dK, dV of the local blocks, then dV (and without dS tiles, dK) of the
  // persistent slots
  int total = g.B * g.H * g.nl;
  if (kvl_pack)
    dkv_local_kernel<D, true><<<((total + 7) / 8) * 8, kKvlThreads, shm_kvl, s>>>(a);
  else
    dkv_local_kernel<D, false><<<((total + 7) / 8) * 8, kKvlThreads, shm_kvl, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int kv_tiles = (g.S + kKvSlots - 1) / kKvSlots;
  // workgroups of eight packed key tiles: as many as the slots' rows could
  // fill (kv_tiles when the slots hold 64 rows)
  const int pk_tiles = (int)(((long long)g.S * g.C + 32 * kKvWaves - 1) / (32 * kKvWaves));
  if (g.S > 0) {
    // slots shorter than 64 rows: the dV pass on packed key tiles (eight per
    // workgroup), beside the packed dk_ds
    const size_t shm_pk = ((size_t)g.S + 1) * 4;
    const bool dv_pk = a.pk && g.C < 64 && 3 * PersDma<D>::BUF + 1024 + shm_pk <= 65536;
    a.ntiles = dv_pk ? pk_tiles : kv_tiles;
    total = g.B * g.H * a.ntiles;
    if (dv_pk)
      dkv_pers_kernel<D, true, true><<<((total + 7) / 8) * 8, kKvThreads, shm_pk, s>>>(a);
    else
      dkv_pers_kernel<D, true, false><<<((total + 7) / 8) * 8, kKvThreads, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    a.ntiles = kv_tiles;
    total = g.B * g.H * a.ntiles;
    if (!ds) {
      dkv_pers_kernel<D, false, false><<<((total + 7) / 8) * 8, kKvThreads, 0, s>>>(a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  // dq of the persistent slots (writes dq, and the dS tiles)
  a.ntiles = (g.ct + kDqRows - 1) / kDqRows;
  total = g.B * g.H * a.ntiles;
  const int grid_dq = ((total + 7) / 8) * 8;
  if (ds && pk)
    dq_pers_kernel<D, true, true><<<grid_dq, kDqThreads, shm_dq, s>>>(a);
  else if (ds)
    dq_pers_kernel<D, true, false><<<grid_dq, kDqThreads, shm_dq, s>>>(a);
  else if (pk)
    dq_pers_kernel<D, false, true><<<grid_dq, kDqThreads, shm_dq, s>>>(a);
  else
    dq_pers_kernel<D, false, false><<<grid_dq, kDqThreads, shm_dq, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ds) {
    // dK of the persistent slots from the dS tiles
    a.ntiles = pk ? pk_tiles : kv_tiles;
    total = g.B * g.H * a.ntiles;
    if (pk)  // the dS tiles are in packed key-tile order
      dk_ds_kernel<D, true><<<((total + 7) / 8) * 8, kKvThreads, ((size_t)g.S + 1) * 4, s>>>(a);
    else
      dk_ds_kernel<D, false><<<((total + 7) / 8) * 8, kKvThreads, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dq of the local blocks (adds)
  a.ntiles = (g.nq + kLocBlocks - 1) / kLocBlocks;
  total = g.B * g.H * a.ntiles;
  if (tab)
    dq_local_kernel<D, true><<<((total + 7) / 8) * 8, kDqlThreads, shm_dql, s>>>(a);
  else
    dq_local_kernel<D, false><<<((total + 7) / 8) * 8, kDqlThreads, shm_dql, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool bwd_mfma_supported(const Geo& g) { return g.dtype == PBSA_BF16 && (g.D == 64 || g.D == 128) && g.C <= 64; }

size_t bwd_ds_tile_bytes(const Geo& g) {
  if (!bwd_mfma_supported(g) || g.S <= 0) return 0;
  return (size_t)g.B * g.H * 2 * g.S * ((g.ct + 31) / 32) * 32 * 32 * 2;
}

size_t bwd_ds_bytes(const Geo& g) { return g.ds ? bwd_ds_tile_bytes(g) : 0; }

// Preparation (key-block index and its launch order, D and lse*log2(e)),
// then the MFMA kernels, all on the caller's stream.
hipError_t launch_bwd_mfma(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                           const void* k_l, const void* v_l, const int32_t* topk, const void* o, const float* lse,
                           const void* dout, float* dq, float* dk_p, float* dv_p, float* dk_l, float* dv_l,
                           WsBwd ws, hipStream_t s) {
  hipError_t e = hipSuccess;
  if ((e = launch_bwd_index(g, topk, ws, s)) != hipSuccess) return e;
  if ((e = launch_bwd_delta(g, o, dout, lse, ws, s)) != hipSuccess) return e;
  BwdArgs a{g, (const bf16_t*)q, (const bf16_t*)k_p, (const bf16_t*)v_p, plen, (const bf16_t*)k_l,
            (const bf16_t*)v_l, topk, lse, ws.delta, ws.lse2, (const bf16_t*)dout, ws.tcount, ws.tlist,
            ws.korder, (const bf16_t*)ws.zrow, (bf16_t*)ws.dsb, dq, dk_p, dv_p, dk_l, dv_l, 0};
  return g.D == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace pbsa
