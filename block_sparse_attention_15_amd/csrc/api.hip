// C ABI entry points: host-side validation, derived sizes, workspace
// carving and kernel launches.  No entry point allocates, frees or
// synchronizes; all work goes onto the caller's stream.
#include <math.h>
#include <stdlib.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "common.h"

namespace pbsa {

// Sticky error bits raised by the kernels of this device (one copy per
// device; pbsa_device_status reads and clears it).
__device__ uint32_t g_device_status;

hipError_t device_status_word(uint32_t** out) {
  static std::mutex mu;
  static uint32_t* addr[PerDeviceOnce::kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= PerDeviceOnce::kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_status))) != hipSuccess) return e;
    addr[dev] = (uint32_t*)p;
  }
  *out = addr[dev];
  return hipSuccess;
}

namespace {

__global__ void device_status_kernel(uint32_t* word, uint32_t* out, int clear) {
  *out = *word;
  if (clear) *word = 0u;
}

thread_local std::string g_err;

pbsa_status fail(pbsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pbsa_status fail(pbsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// float index of the zero row in the delta region: after the n entries and the
// sentinel, rounded up to 16 bytes
size_t zrow_offset(size_t n) { return (n + 1 + 3) & ~size_t(3); }

struct Plan {
  Geo g;
  pbsa_plan_info info;
};

// Derive the geometry of a configuration (block tiling of the project page's
// sparse_kv_block_size, cache sizes of its constructor) and check it.
pbsa_status make_plan(const pbsa_config* c, Plan* p) {
  if (!c) return fail(PBSA_ERR_INVALID_ARG, "config is NULL");
  if (c->batch <= 0 || c->heads <= 0 || c->head_dim <= 0)
    return fail(PBSA_ERR_INVALID_ARG, "batch, heads and head_dim must be positive");
  if (c->frame_h <= 0 || c->frame_w <= 0 || c->block_t <= 0 || c->block_h <= 0 || c->block_w <= 0 ||
      c->chunk_frames <= 0)
    return fail(PBSA_ERR_INVALID_ARG, "frame, block and chunk sizes must be positive");
  if (c->local_cache_size <= 0 || c->persistent_cache_size < 0)
    return fail(PBSA_ERR_INVALID_ARG, "cache sizes must be positive");
  if (c->total_cache_size != c->local_cache_size + c->persistent_cache_size)
    return fail(PBSA_ERR_INVALID_ARG, "total_cache_size (%lld) != local (%lld) + persistent (%lld)",
                (long long)c->total_cache_size, (long long)c->local_cache_size,
                (long long)c->persistent_cache_size);
  if (c->chunk_frames % c->block_t)
    return fail(PBSA_ERR_INVALID_ARG, "chunk_frames (%d) must be a multiple of block_t (%d)", c->chunk_frames,
                c->block_t);
  if (c->dtype != PBSA_BF16 && c->dtype != PBSA_FP32) return fail(PBSA_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
  if (c->use_local_block_sparse_attn && !(c->topk_ratio > 0.f && c->topk_ratio <= 1.f))
    return fail(PBSA_ERR_INVALID_ARG, "topk_ratio (%g) must be in (0, 1]", (double)c->topk_ratio);
  if (!(c->softmax_scale >= 0.f) || isinf(c->softmax_scale))
    return fail(PBSA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  const int64_t ft = (int64_t)c->frame_h * c->frame_w;
  const int64_t ct = ft * c->chunk_frames;
  if (c->local_cache_size % ct)
    return fail(PBSA_ERR_INVALID_ARG, "local_cache_size (%lld) is not a whole number of %lld-token chunks",
                (long long)c->local_cache_size, (long long)ct);
  if (c->persistent_cache_size % (ft * c->block_t))
    return fail(PBSA_ERR_INVALID_ARG, "persistent_cache_size (%lld) is not a whole number of %lld-token frame groups",
                (long long)c->persistent_cache_size, (long long)(ft * c->block_t));
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PBSA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", c->head_dim);
  const int C = c->block_t * c->block_h * c->block_w;
  if (C > 64) return fail(PBSA_ERR_UNSUPPORTED, "blocks of %d tokens unsupported (at most 64)", C);
  if (ct > (1 << 24) || c->local_cache_size > (1 << 26))
    return fail(PBSA_ERR_UNSUPPORTED, "chunk or cache too large");

  Geo& g = p->g;
  g.B = c->batch;
  g.H = c->heads;
  g.D = c->head_dim;
  g.fh = c->frame_h;
  g.fw = c->frame_w;
  g.bt = c->block_t;
  g.bh = c->block_h;
  g.bw = c->block_w;
  g.cf = c->chunk_frames;
  g.ft = (int)ft;
  g.ct = (int)ct;
  g.nbr = (g.fh + g.bh - 1) / g.bh;
  g.nbc = (g.fw + g.bw - 1) / g.bw;
  g.bpg = g.nbr * g.nbc;
  g.nq = g.bpg * (g.cf / g.bt);
  g.R = (int)(c->local_cache_size / ct);
  g.nl = g.R * g.nq;
  g.NL = (int)c->local_cache_size;
  g.S = (int)(c->persistent_cache_size / (ft * g.bt)) * g.bpg;
  g.C = C;
  if (c->use_local_block_sparse_attn) {
    // k = ceil(ratio * n) with a 1e-6 allowance so that products that are
    // integers in decimal (0.1 * 10) do not round up.
    double k = ceil((double)c->topk_ratio * g.nl - 1e-6);
    g.K = (int)fmin(fmax(k, 1.0), (double)g.nl);
  } else {
    g.K = g.nl;
  }
  g.scale = c->softmax_scale > 0.f ? c->softmax_scale : (float)(1.0 / sqrt((double)g.D));
  g.dtype = c->dtype;
  if (g.S > 2048 || g.nl > 2048 || g.nq > 2048)
    return fail(PBSA_ERR_UNSUPPORTED, "more than 2048 blocks per cache or chunk");
  if (c->sink_slots < 0 || c->sink_slots > g.S || c->sink_slots > g.nq)
    return fail(PBSA_ERR_INVALID_ARG, "sink_slots (%d) must be in [0, min(%d slots, %d blocks per chunk)]",
                c->sink_slots, g.S, g.nq);
  g.Z = c->sink_slots;
  // The backward stores dS of every (query, persistent key) pair in its
  // workspace when that takes at most bwd_ds_max_mb MiB (0: 8192; -1: never);
  // above it the dK pass recomputes dS instead (slower, no such workspace).
  if (c->bwd_ds_max_mb < -1)
    return fail(PBSA_ERR_INVALID_ARG, "bwd_ds_max_mb (%d) must be -1, 0 or positive", c->bwd_ds_max_mb);
  {
    const double cap_mb = c->bwd_ds_max_mb == 0 ? 8192.0 : (double)c->bwd_ds_max_mb;
    g.ds = 0;
    const size_t need = bwd_ds_tile_bytes(g);
    g.ds = need > 0 && c->bwd_ds_max_mb >= 0 && (double)need <= cap_mb * 1048576.0 ? 1 : 0;
  }

  pbsa_plan_info& in = p->info;
  memset(&in, 0, sizeof in);
  in.blocks_per_chunk = g.nq;
  in.local_blocks = g.nl;
  in.ring_chunks = g.R;
  in.persistent_slots = g.S;
  in.slot_rows = g.C;
  in.topk = g.K;
  in.chunk_tokens = g.ct;
  int mx = 0;
  for (int j = 0; j < g.nq; ++j) mx = mx > block_ext(g, j).len ? mx : block_ext(g, j).len;
  in.max_block_tokens = mx;
  const size_t BH = (size_t)g.B * g.H;
  in.ws_score_select = score_workspace(g);
  in.ws_fwd = fwd_workspace(g);
  in.ws_bwd = align256(zrow_offset(BH * g.ct) * 4 + 256) + align256(BH * g.ct * 4 + 4) + 2 * align256(BH * g.nl * 4) +
              align256(BH * g.nl * g.nq * 4) + align256(bwd_ds_bytes(g));
  in.ws_persist_update = update_workspace(g);
  in.ws_fwd_mass = align256(in.ws_fwd) + align256(BH * g.S * g.ct * 4) + align256(BH * g.K * g.ct * 4) +
                   align256(BH * g.nq * g.nl * 4);
  return PBSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

#define REQUIRE_PTR(p)                                                         \
  do {                                                                         \
    if (!(p)) return fail(PBSA_ERR_INVALID_ARG, "%s is NULL", #p);             \
  } while (0)
#define REQUIRE_ALIGNED(p)                                                                   \
  do {                                                                                       \
    REQUIRE_PTR(p);                                                                          \
    if (!aligned16(p)) return fail(PBSA_ERR_ALIGNMENT, "%s is not 16-byte aligned", #p);     \
  } while (0)

pbsa_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return PBSA_OK;
  if (!ws) return fail(PBSA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (!aligned16(ws)) return fail(PBSA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  if (have < need) return fail(PBSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return PBSA_OK;
}

pbsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err.clear();
    return PBSA_OK;
  }
  return fail(PBSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace
}  // namespace pbsa

using namespace pbsa;

extern "C" {

pbsa_status pbsa_plan(const pbsa_config* cfg, pbsa_plan_info* out) {
  if (!out) return fail(PBSA_ERR_INVALID_ARG, "out is NULL");
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  *out = p.info;
  g_err.clear();
  return PBSA_OK;
}

pbsa_status pbsa_pool_slots(const pbsa_config* cfg, const void* k_pers, const int32_t* persist_len,
                            float* persist_kbar, void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  if (p.g.S == 0) {  // no persistent memory: nothing to pool
    g_err.clear();
    return PBSA_OK;
  }
  REQUIRE_ALIGNED(k_pers);
  REQUIRE_PTR(persist_len);
  REQUIRE_ALIGNED(persist_kbar);
  return hip_status(launch_pool_slots(p.g, k_pers, persist_len, persist_kbar, (hipStream_t)stream),
                    "pbsa_pool_slots");
}

pbsa_status pbsa_pool_local(const pbsa_config* cfg, const void* k_local, float* kbar_local, void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  REQUIRE_ALIGNED(k_local);
  REQUIRE_ALIGNED(kbar_local);
  return hip_status(launch_pool_local(p.g, k_local, kbar_local, (hipStream_t)stream), "pbsa_pool_local");
}

pbsa_status pbsa_score_select(const pbsa_config* cfg, const void* q, const float* kbar_local,
                              const int32_t* ring_head, const float* persist_kbar, const int32_t* persist_len,
                              int32_t* topk_idx, float* mass, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  REQUIRE_ALIGNED(q);
  REQUIRE_ALIGNED(kbar_local);
  REQUIRE_PTR(ring_head);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(mass);
  if (p.g.S > 0) {
    REQUIRE_ALIGNED(persist_kbar);
    REQUIRE_PTR(persist_len);
  }
  if ((st = check_ws(ws, ws_bytes, p.info.ws_score_select)) != PBSA_OK) return st;
  WsScore w;
  w.part = (float*)ws;
  uint32_t* status = nullptr;
  hipError_t e = device_status_word(&status);
  if (e == hipSuccess)
    e = launch_score_select(p.g, q, kbar_local, ring_head, persist_kbar, persist_len, topk_idx, mass, w, status,
                            (hipStream_t)stream);
  return hip_status(e, "pbsa_score_select");
}

pbsa_status pbsa_score_select_noalloc(const pbsa_config* cfg, const void* q, const float* kbar_local,
                                      const int32_t* ring_head, const float* persist_kbar,
                                      const int32_t* persist_len, int32_t* topk_idx, float* mass, void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  void* ws = nullptr;
  size_t cap = 0;
  hipError_t e = score_static_scratch(&ws, &cap);
  if (e != hipSuccess) return hip_status(e, "pbsa_score_select_noalloc: static scratch");
  if (p.info.ws_score_select > cap)
    return fail(PBSA_ERR_WORKSPACE,
                "pbsa_score_select_noalloc: this configuration needs %zu bytes of scratch, the static array holds %zu "
                "(use pbsa_score_select with a workspace)",
                p.info.ws_score_select, cap);
  return pbsa_score_select(cfg, q, kbar_local, ring_head, persist_kbar, persist_len, topk_idx, mass, ws,
                           p.info.ws_score_select, stream);
}

pbsa_status pbsa_fwd(const pbsa_config* cfg, const void* q, const void* k_pers, const void* v_pers,
                     const int32_t* persist_len, const void* k_local, const void* v_local,
                     const int32_t* topk_idx, void* o, float* lse, void* ws, size_t ws_bytes,
                     void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  REQUIRE_ALIGNED(q);
  REQUIRE_ALIGNED(k_local);
  REQUIRE_ALIGNED(v_local);
  REQUIRE_PTR(topk_idx);
  REQUIRE_ALIGNED(o);
  REQUIRE_PTR(lse);
  if (p.g.S > 0) {
    REQUIRE_ALIGNED(k_pers);
    REQUIRE_ALIGNED(v_pers);
    REQUIRE_PTR(persist_len);
  }
  if ((st = check_ws(ws, ws_bytes, p.info.ws_fwd)) != PBSA_OK) return st;
  return hip_status(launch_fwd(p.g, q, k_pers, v_pers, persist_len, k_local, v_local, topk_idx, o, lse, ws,
                               nullptr, nullptr, (hipStream_t)stream),
                    "pbsa_fwd");
}

pbsa_status pbsa_fwd_mass(const pbsa_config* cfg, const void* q, const void* k_pers, const void* v_pers,
                          const int32_t* persist_len, const void* k_local, const void* v_local,
                          const int32_t* topk_idx, void* o, float* lse, float* mass, void* ws, size_t ws_bytes,
                          void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  REQUIRE_ALIGNED(q);
  REQUIRE_ALIGNED(k_local);
  REQUIRE_ALIGNED(v_local);
  REQUIRE_PTR(topk_idx);
  REQUIRE_ALIGNED(o);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(mass);
  if (p.g.S > 0) {
    REQUIRE_ALIGNED(k_pers);
    REQUIRE_ALIGNED(v_pers);
    REQUIRE_PTR(persist_len);
  }
  if ((st = check_ws(ws, ws_bytes, p.info.ws_fwd_mass)) != PBSA_OK) return st;
  const Geo& g = p.g;
  const size_t BH = (size_t)g.B * g.H;
  char* base = (char*)ws;
  void* ws_f = p.info.ws_fwd ? base : nullptr;
  base += align256(p.info.ws_fwd);
  float* blse_p = (float*)base;
  base += align256(BH * g.S * g.ct * 4);
  float* blse_l = (float*)base;
  base += align256(BH * g.K * g.ct * 4);
  float* part = (float*)base;
  hipError_t e = launch_fwd(g, q, k_pers, v_pers, persist_len, k_local, v_local, topk_idx, o, lse, ws_f, blse_p,
                            blse_l, (hipStream_t)stream);
  if (e == hipSuccess)
    e = launch_token_mass(g, persist_len, topk_idx, lse, blse_p, blse_l, part, mass, (hipStream_t)stream);
  return hip_status(e, "pbsa_fwd_mass");
}

pbsa_status pbsa_bwd(const pbsa_config* cfg, const void* q, const void* k_pers, const void* v_pers,
                     const int32_t* persist_len, const void* k_local, const void* v_local,
                     const int32_t* topk_idx, const void* o, const float* lse, const void* dout,
                     float* dq, float* dk_pers, float* dv_pers, float* dk_local, float* dv_local,
                     void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  REQUIRE_ALIGNED(q);
  REQUIRE_ALIGNED(k_local);
  REQUIRE_ALIGNED(v_local);
  REQUIRE_PTR(topk_idx);
  REQUIRE_ALIGNED(o);
  REQUIRE_PTR(lse);
  REQUIRE_ALIGNED(dout);
  REQUIRE_ALIGNED(dq);
  REQUIRE_ALIGNED(dk_local);
  REQUIRE_ALIGNED(dv_local);
  if (p.g.S > 0) {
    REQUIRE_ALIGNED(k_pers);
    REQUIRE_ALIGNED(v_pers);
    REQUIRE_PTR(persist_len);
    REQUIRE_ALIGNED(dk_pers);
    REQUIRE_ALIGNED(dv_pers);
  }
  if ((st = check_ws(ws, ws_bytes, p.info.ws_bwd)) != PBSA_OK) return st;
  const size_t BH = (size_t)p.g.B * p.g.H;
  WsBwd w;
  char* base = (char*)ws;
  w.delta = (float*)base;
  w.zrow = w.delta + zrow_offset(BH * p.g.ct);  // after the sentinel entry, 16-byte aligned
  base += align256(zrow_offset(BH * p.g.ct) * 4 + 256);
  w.lse2 = (float*)base;
  base += align256(BH * p.g.ct * 4 + 4);
  w.tcount = (int32_t*)base;
  base += align256(BH * p.g.nl * 4);
  w.tlist = (int32_t*)base;
  base += align256(BH * p.g.nl * p.g.nq * 4);
  w.korder = (int32_t*)base;
  base += align256(BH * p.g.nl * 4);
  w.dsb = base;
  return hip_status(launch_bwd(p.g, q, k_pers, v_pers, persist_len, k_local, v_local, topk_idx, o, lse, dout, dq,
                               dk_pers, dv_pers, dk_local, dv_local, w, (hipStream_t)stream),
                    "pbsa_bwd");
}

pbsa_status pbsa_persist_update(const pbsa_config* cfg, const float* mass, const void* k_local,
                                const void* v_local, const float* kbar_local, int32_t* ring_head,
                                int32_t* step_counter, void* k_pers, void* v_pers, int32_t* persist_len,
                                int32_t* persist_src, float* persist_kbar, int32_t* n_replaced,
                                void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  REQUIRE_PTR(mass);
  REQUIRE_ALIGNED(k_local);
  REQUIRE_ALIGNED(v_local);
  REQUIRE_ALIGNED(kbar_local);
  REQUIRE_PTR(ring_head);
  REQUIRE_PTR(n_replaced);
  REQUIRE_PTR(step_counter);
  if (p.g.S > 0) {
    REQUIRE_ALIGNED(k_pers);
    REQUIRE_ALIGNED(v_pers);
    REQUIRE_PTR(persist_len);
    REQUIRE_PTR(persist_src);
    REQUIRE_ALIGNED(persist_kbar);
  }
  if ((st = check_ws(ws, ws_bytes, p.info.ws_persist_update)) != PBSA_OK) return st;
  uint32_t* status = nullptr;
  hipError_t e = device_status_word(&status);
  if (e == hipSuccess)
    e = launch_persist_update(p.g, mass, k_local, v_local, kbar_local, ring_head, step_counter, k_pers, v_pers,
                              persist_len, persist_src, persist_kbar, n_replaced, ws, status, (hipStream_t)stream);
  return hip_status(e, "pbsa_persist_update");
}

pbsa_status pbsa_ring_append(const pbsa_config* cfg, const void* k_new, const void* v_new,
                             const int32_t* ring_head, void* k_local, void* v_local, float* kbar_local,
                             void* stream) {
  Plan p;
  pbsa_status st = make_plan(cfg, &p);
  if (st != PBSA_OK) return st;
  REQUIRE_ALIGNED(k_new);
  REQUIRE_ALIGNED(v_new);
  REQUIRE_PTR(ring_head);
  REQUIRE_ALIGNED(k_local);
  REQUIRE_ALIGNED(v_local);
  REQUIRE_ALIGNED(kbar_local);
  uint32_t* status = nullptr;
  hipError_t e = device_status_word(&status);
  if (e == hipSuccess)
    e = launch_ring_append(p.g, k_new, v_new, ring_head, k_local, v_local, kbar_local, status, (hipStream_t)stream);
  return hip_status(e, "pbsa_ring_append");
}

pbsa_status pbsa_device_status(uint32_t* out, int32_t clear, void* stream) {
  REQUIRE_PTR(out);
  uint32_t* word = nullptr;
  hipError_t e = device_status_word(&word);
  if (e == hipSuccess) {
    device_status_kernel<<<1, 1, 0, (hipStream_t)stream>>>(word, out, clear);
    e = hipGetLastError();
  }
  return hip_status(e, "pbsa_device_status");
}

const char* pbsa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
