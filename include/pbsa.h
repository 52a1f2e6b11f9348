/*
 * pbsa.h -- C ABI of the Persistent Block-Sparse Attention (PBSA) library for
 * AMD Instinct MI355X (gfx950).
 *
 * PBSA is the attention kernel of "Sparse Forcing: Native Trainable Sparse
 * Attention for Real-time Autoregressive Diffusion Video Generation".  The
 * abstract describes it as sparse attention of a query chunk over a persistent
 * set of salient blocks plus a dynamically selected neighbourhood of a sliding
 * local window, together with the update of that persistent memory.  The
 * project page ("Sparse Forcing") gives the module interface this ABI mirrors:
 * SparseForcingAttention(total_cache_size, local_cache_size,
 * persistent_cache_size, sparse_kv_block_size, local_block_sparse_topk_ratio,
 * use_local_block_sparse_attn, ...) called with (query, key_persistent,
 * value_persistent, key_local, value_local), and lists full gradient support.
 * The fragment of the paper's training algorithm on the review page fixes when
 * the update runs: the t=0 cache pass applies PBSA with top-K and updates the
 * persistent (P) and local (L) caches.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Ownership: the caller owns every buffer.  Device pointers point to device
 *    memory the caller allocated; the library never allocates, frees or
 *    synchronizes.  Host pointers (the config, the plan) are read during the
 *    call only.
 *  - Streams: every kernel is enqueued on `stream` (a hipStream_t; NULL means
 *    the default stream).  No entry point reads device data back to the host,
 *    so each call is asynchronous and may be captured into a hipGraph.
 *  - Errors: arguments are checked on the host before any launch.  On failure
 *    nothing is launched, a non-zero pbsa_status is returned and
 *    pbsa_last_error() describes the problem.  A failed kernel launch returns
 *    PBSA_ERR_HIP.
 *  - Layouts (all row-major, contiguous):
 *      q, o, dout, dq        [B, H, Nq, D]   Nq = chunk tokens, raster order
 *                                            (frame, row, column)
 *      k_local, v_local,     [B, H, NL, D]   NL = local_cache_size; physical
 *      dk_local, dv_local                    chunk slot c holds tokens
 *                                            [c*Nq, (c+1)*Nq), raster order
 *      k_pers, v_pers,       [B, H, S, C, D] S persistent slots of C rows
 *      dk_pers, dv_pers                      (C = block_t*block_h*block_w);
 *                                            rows >= persist_len are zero
 *      persist_len, persist_src  [B, H, S] int32
 *      persist_kbar          [B, H, S, D] float32 (mean of the slot's rows)
 *      kbar_local            [B, H, NL_blocks, D] float32, physical order
 *      topk_idx              [B, H, NQ_blocks, K] int32 physical local block
 *                                            ids, ascending
 *      mass                  [B, H, S + NL_blocks] float32 (slot s at s,
 *                                            physical local block p at S+p)
 *      lse                   [B, H, Nq] float32 (natural log)
 *      ring_head             one int32 on the device: physical chunk slot of
 *                                            the oldest local chunk
 *    Element type of q/k/v/o/dout is bf16 (PBSA_BF16) or fp32 (PBSA_FP32);
 *    gradients are always fp32.
 *  - Blocks: a frame of frame_h x frame_w tokens is tiled into
 *    ceil(h/block_h) x ceil(w/block_w) blocks in block-row-major order (edge
 *    blocks are smaller); with block_t > 1 a block spans block_t frames.  The
 *    chunk's blocks are the query blocks; local physical block p is block
 *    (p mod NQ_blocks) of chunk slot (p div NQ_blocks).
 */
#ifndef PBSA_H
#define PBSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PBSA_OK = 0,
  PBSA_ERR_INVALID_ARG = -1,  /* inconsistent sizes, null pointer, bad value */
  PBSA_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim 96) */
  PBSA_ERR_ALIGNMENT = -3,    /* a tensor pointer is not 16-byte aligned */
  PBSA_ERR_WORKSPACE = -4,    /* workspace missing or smaller than planned */
  PBSA_ERR_HIP = -5           /* the HIP runtime reported an error */
} pbsa_status;

typedef enum { PBSA_BF16 = 0, PBSA_FP32 = 1 } pbsa_dtype;

/* Mirrors the SparseForcingAttention constructor of the project page's usage
 * example, plus the latent frame grid and batch geometry it leaves implicit. */
typedef struct {
  int32_t batch, heads, head_dim;      /* head_dim in {64, 128} */
  int32_t frame_h, frame_w;            /* latent tokens per frame (e.g. 30 x 52) */
  int32_t block_t, block_h, block_w;   /* sparse_kv_block_size, e.g. [1, 8, 8] */
  int32_t chunk_frames;                /* frames per generated chunk (multiple of block_t) */
  int64_t total_cache_size;            /* tokens; must equal local + persistent */
  int64_t local_cache_size;            /* tokens; a whole number of chunks (the ring) */
  int64_t persistent_cache_size;       /* tokens; a whole number of block_t-frame groups */
  int32_t use_local_block_sparse_attn; /* 0: attend every local block (k = all) */
  float topk_ratio;                    /* local_block_sparse_topk_ratio, in (0, 1] */
  float softmax_scale;                 /* 0 means 1/sqrt(head_dim) */
  int32_t dtype;                       /* pbsa_dtype of q/k/v/o/dout */
  int32_t sink_slots;                  /* "sink" pattern: the first sink_slots persistent slots
                                          are pinned (see pbsa_persist_update); 0 = none;
                                          at most min(S, NQ_blocks) */
  int32_t bwd_ds_max_mb;               /* pbsa_bwd stores dS of the persistent keys in its
                                          workspace while that takes at most this many MiB
                                          (0 = 8192; -1 = never, the dK pass recomputes dS) */
} pbsa_config;

/* Derived sizes and workspace requirements (bytes). */
typedef struct {
  int32_t blocks_per_chunk;   /* NQ_blocks: query blocks = blocks per chunk */
  int32_t local_blocks;       /* NL_blocks */
  int32_t ring_chunks;        /* R = local_cache_size / chunk tokens */
  int32_t persistent_slots;   /* S */
  int32_t slot_rows;          /* C = block_t*block_h*block_w */
  int32_t topk;               /* K = clamp(ceil(ratio*NL_blocks - 1e-6), 1, NL_blocks) */
  int32_t chunk_tokens;       /* Nq */
  int32_t max_block_tokens;   /* largest block */
  size_t ws_score_select;
  size_t ws_fwd;
  size_t ws_bwd;
  size_t ws_persist_update;  /* new slot lengths and source ids, committed at the end */
  size_t ws_fwd_mass;
} pbsa_plan_info;

/* Validate a configuration and derive its sizes.  Host only; touches no GPU.
 * Returns PBSA_ERR_INVALID_ARG for inconsistent sizes (total != local +
 * persistent, a local cache that is not whole chunks, a persistent cache that
 * is not whole frame groups, ratio outside (0,1]) and PBSA_ERR_UNSUPPORTED for
 * head_dim outside {64,128} or blocks of more than 64 tokens. */
pbsa_status pbsa_plan(const pbsa_config* cfg, pbsa_plan_info* out);

/* Mean of each persistent slot's first persist_len rows -> persist_kbar (zero
 * for empty slots).  Used to initialise the pooled-key metadata of a
 * persistent cache that was filled from outside the library (reading: block
 * scores use mean-pooled keys). */
pbsa_status pbsa_pool_slots(const pbsa_config* cfg, const void* k_pers, const int32_t* persist_len,
                            float* persist_kbar, void* stream);

/* Pooled keys of every physical local block of the ring: kbar_local[b,h,p]
 * = mean of the keys of local block p (its valid tokens), float32.  The
 * pooled local keys are ring metadata, like persist_kbar for the slots:
 * pbsa_ring_append keeps them for the chunk it writes, so this call is needed
 * only for a ring whose keys were written from outside the library (or to
 * rebuild them).  Reading: block scores use mean-pooled keys. */
pbsa_status pbsa_pool_local(const pbsa_config* cfg, const void* k_local, float* kbar_local, void* stream);

/* Block scoring and top-k selection ("learned top-k selection" on the project
 * page; "dynamically selected local neighborhood" in the abstract), plus the
 * pooled attention masses that drive the persistent update.
 *   q               input (dtype)
 *   kbar_local      pooled keys of the local blocks (kept by pbsa_ring_append,
 *                   or pbsa_pool_local); they must describe the ring's
 *                   current keys
 *   ring_head       device int32, oldest chunk slot; ties in the top-k go to
 *                   the lower logical index (oldest chunk first)
 *   persist_kbar, persist_len   persistent slot metadata
 *   topk_idx        out [B,H,NQ_blocks,K] physical ids, ascending
 *   mass            out [B,H,S+NL_blocks]: for every query block a softmax of
 *                   scale*qbar.kbar over valid slots and all local blocks,
 *                   summed over query blocks in ascending order (empty slots
 *                   get 0); deterministic
 *   ws, ws_bytes    workspace of at least plan.ws_score_select bytes (the
 *                   column sums of the softmax rows of each group of query
 *                   blocks, written before they are read; no initial contents
 *                   needed) */
pbsa_status pbsa_score_select(const pbsa_config* cfg, const void* q, const float* kbar_local,
                              const int32_t* ring_head, const float* persist_kbar, const int32_t* persist_len,
                              int32_t* topk_idx, float* mass, void* ws, size_t ws_bytes, void* stream);

/* pbsa_score_select without a workspace, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as pbsa_score_select
 * minus ws / ws_bytes.  Its scratch is a static array of the library, 8 MiB
 * per device, held until the process ends; a configuration whose
 * plan.ws_score_select exceeds it is rejected with PBSA_ERR_WORKSPACE and
 * nothing is launched.  The call allocates nothing.  Every call on a device
 * shares that device's array, so calls that overlap on one device (on
 * different streams, or concurrent graphs) race; calls on one stream are
 * ordered and safe.  The scratch is fully written before it is read, so no
 * call depends on what an earlier call left in it. */
pbsa_status pbsa_score_select_noalloc(const pbsa_config* cfg, const void* q, const float* kbar_local,
                                      const int32_t* ring_head, const float* persist_kbar,
                                      const int32_t* persist_len, int32_t* topk_idx, float* mass, void* stream);

/* Sparse attention forward.  Every query token of query block i attends all
 * valid rows of all persistent slots and every token of the K local blocks
 * topk_idx[b,h,i,:], with one softmax over that union.  Writes o (dtype) and
 * lse (float32, natural log).  ws: at least plan.ws_fwd bytes (it holds the
 * persistent-part partial output of the bf16 path; 0 bytes and NULL allowed for
 * fp32). */
pbsa_status pbsa_fwd(const pbsa_config* cfg, const void* q, const void* k_pers, const void* v_pers,
                     const int32_t* persist_len, const void* k_local, const void* v_local,
                     const int32_t* topk_idx, void* o, float* lse, void* ws, size_t ws_bytes,
                     void* stream);

/* pbsa_fwd plus the token-exact attention mass of every candidate block: the
 * alternative to the pooled mass of pbsa_score_select as input of
 * pbsa_persist_update (the abstract only says the persistent memory keeps the
 * blocks most relevant to the queries; this reading takes relevance from the
 * attention itself).  mass[b,h,j] = sum over the chunk's query tokens t of the
 * softmax probability that t's attention puts on the rows of block j (slot s
 * at index s, physical local block p at S+p).  Every entry is written: empty
 * slots and local blocks that no query block selected get 0, and the entries
 * of a head sum to Nq.  o and lse are those of pbsa_fwd up to rounding (this
 * call adds the persistent keys slot by slot, pbsa_fwd in packed 64-key
 * steps).  Deterministic (fixed
 * summation order, no atomics).  ws: at least plan.ws_fwd_mass bytes
 * (per-query log-sum-exps over every slot and selected block, about
 * 4*B*H*(S+K)*Nq bytes, plus 4*B*H*NQ_blocks*NL_blocks). */
pbsa_status pbsa_fwd_mass(const pbsa_config* cfg, const void* q, const void* k_pers, const void* v_pers,
                          const int32_t* persist_len, const void* k_local, const void* v_local,
                          const int32_t* topk_idx, void* o, float* lse, float* mass, void* ws, size_t ws_bytes,
                          void* stream);

/* Backward of pbsa_fwd for a fixed block mask ("full gradient support for
 * training" on the project page).  Inputs as in pbsa_fwd plus o, lse (from
 * pbsa_fwd) and dout.  Writes float32 dq, dk_pers, dv_pers, dk_local,
 * dv_local, overwriting them entirely (rows that receive no gradient are set
 * to zero).  Deterministic: no floating-point atomics.  ws of at least
 * plan.ws_bwd bytes: for bf16 inputs it holds dS of every (query, persistent
 * key) pair as bf16 (about 2*B*H*2S*ceil(Nq/32)*1024 bytes: 1.2 GB at the
 * 30x52 decode shape), which the dq kernel writes and the dk kernel reads
 * instead of recomputing it, when that size is at most cfg->bwd_ds_max_mb
 * MiB (0: 8192; -1: never); otherwise the dk kernel recomputes dS and the
 * workspace is smaller.  The setting is part of the configuration, so the
 * plan that sizes the workspace and the call agree. */
pbsa_status pbsa_bwd(const pbsa_config* cfg, const void* q, const void* k_pers, const void* v_pers,
                     const int32_t* persist_len, const void* k_local, const void* v_local,
                     const int32_t* topk_idx, const void* o, const float* lse, const void* dout,
                     float* dq, float* dk_pers, float* dv_pers, float* dk_local, float* dv_local,
                     void* ws, size_t ws_bytes, void* stream);

/* Persistent-cache update of the cache pass ("update P and L" in the paper's
 * algorithm; "compress, preserve, and update these persistent blocks" in the
 * abstract).  Candidates are the valid slots and the NQ_blocks blocks of the
 * oldest local chunk (physical slot *ring_head).  The S candidates of largest
 * mass are kept (ties: incumbents first, then lower slot / block index).
 * Vacated slots, ascending, receive the admitted blocks, ascending: their rows
 * are copied (zero padding), len = block size, src = step*NQ_blocks + e where
 * step = *step_counter, kbar = kbar_local of the block.  Vacated slots left
 * over are emptied (len 0, rows 0, src INT32_MIN, kbar 0).  n_replaced[b,h]
 * receives the admitted count.  Finally *ring_head advances to
 * (ring_head+1) mod R, so the evicted chunk slot becomes the newest and is
 * free for the next chunk, and *step_counter advances by one.  Both are
 * device int32 values, so one captured graph serves every step of a rollout
 * (src ids are int32: step*NQ_blocks must stay below 2^31).  ws of at least
 * plan.ws_persist_update bytes.
 *
 * Sink slots (cfg.sink_slots = Z > 0; the project page lists "sink" among the
 * sparsity patterns): slots s < Z are not candidates.  A valid sink slot is
 * always kept; an empty one receives block s of the evicted chunk (so a
 * rollout that starts from an empty persistent cache pins the blocks of the
 * first frame to leave the local window).  The other candidates compete for
 * the remaining S - Z slots as above. */
pbsa_status pbsa_persist_update(const pbsa_config* cfg, const float* mass, const void* k_local,
                                const void* v_local, const float* kbar_local, int32_t* ring_head,
                                int32_t* step_counter, void* k_pers, void* v_pers, int32_t* persist_len,
                                int32_t* persist_src, float* persist_kbar, int32_t* n_replaced,
                                void* ws, size_t ws_bytes, void* stream);

/* Write a new chunk's keys and values ([B,H,Nq,D] each) into the newest local
 * ring slot, physical slot (ring_head + R - 1) mod R, reading ring_head on the
 * device (so one captured graph serves every step of a rollout), and pool the
 * chunk's keys into kbar_local (the rows of that slot's NQ_blocks blocks).
 * The per-chunk schedule of the paper's algorithm calls it once per pass:
 * every denoising pass and the cache pass write their own keys and values
 * into this slot before scoring, so the local window holds the current
 * chunk. */
pbsa_status pbsa_ring_append(const pbsa_config* cfg, const void* k_new, const void* v_new,
                             const int32_t* ring_head, void* k_local, void* v_local, float* kbar_local,
                             void* stream);

/* Device status word: sticky error bits that kernels raise when they find
 * device-resident state out of range, without faulting.  The project page
 * lists "flexible KV-cache management"; the ring head and step counter of that
 * cache live on the device, so a corrupt value can only be seen there.  Bits:
 *   PBSA_DEVICE_BAD_RING_HEAD     a ring head outside [0, R) was read by
 *                                 pbsa_score_select, pbsa_persist_update or
 *                                 pbsa_ring_append; the call used it reduced
 *                                 into [0, R) (non-negative remainder), so every
 *                                 access stayed in bounds, but it is not the
 *                                 caller's ring phase
 *   PBSA_DEVICE_BAD_STEP_COUNTER  pbsa_persist_update read a step counter
 *                                 outside [0, 2^31 / NQ_blocks): source ids
 *                                 are then not unique
 * The word is per device and shared by every call on it.  pbsa_device_status
 * enqueues on `stream` a copy of the word into `out` (one device uint32) and,
 * when `clear` is non-zero, resets it; asynchronous like every entry point. */
#define PBSA_DEVICE_BAD_RING_HEAD 1u
#define PBSA_DEVICE_BAD_STEP_COUNTER 2u
pbsa_status pbsa_device_status(uint32_t* out, int32_t clear, void* stream);

/* Text of the last error on the calling thread ("" if none). */
const char* pbsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PBSA_H */
