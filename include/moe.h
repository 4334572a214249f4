/*
 * moe.h — C ABI of the MI355X (gfx950) routed-MoE-layer library with a shared
 * expert-slot cache.
 *
 * Sources (cited by page title and section):
 *   [FT]   "FreeToken 完全拆解" (pinghaoyang.com.cn/aigc/posts/freetoken/)
 *   [FTK]  "개인 장치에서 MoE 모델을 서빙하는 FreeToken" (aitrends.kr/articles/99620)
 *   [OSDI] "OSDI'26 | 双路 CPU + 两张 5090 ..." (marsggbo.github.io, 2026-07-23)
 *
 * Conventions for every call:
 *   - Returns moe_status: MOE_OK (0) or a negative error.  Arguments are
 *     validated on the host before anything is enqueued; on an error nothing
 *     is enqueued.  moe_last_error() returns a message for the calling thread.
 *   - Pointers named d_* / "device" are device memory (hipMalloc or torch
 *     CUDA tensors) owned by the caller.  "host" pointers are ordinary host
 *     memory.  "pinned" pointers are page-locked host memory from hipHostMalloc
 *     (torch pin_memory); the library reads them from kernels and DMA.
 *   - The caller owns every buffer, the pinned host pool and the streams.  The
 *     library owns only its opaque handles (small host structs), and the
 *     events of a prefill pool.  Device state of a cache lives in a caller
 *     workspace whose size moe_cache_workspace_bytes() reports.
 *   - Work is enqueued on the given stream, in stream order, and the calls
 *     marked "capturable" neither allocate, synchronise the host nor copy
 *     device data to the host, so they may be recorded into a hipGraph.
 *   - BF16 values are passed as uint16_t bit patterns; FP8 values as uint8_t
 *     OCP E4M3FN codes.
 *   - A handle is used by one host thread and one stream at a time.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,        /* null pointer, bad enum, misaligned pointer        */
  MOE_ERR_SHAPE = -2,      /* a size outside the supported range                */
  MOE_ERR_NO_SPACE = -3,   /* not enough slots / workspace                      */
  MOE_ERR_NOT_PINNED = -4, /* a host-pool pointer is not device-accessible      */
  MOE_ERR_HIP = -5,        /* a HIP runtime call failed (see moe_last_error)    */
  MOE_ERR_STATE = -6,      /* call out of order (e.g. acquire before prefetch)  */
  MOE_ERR_DEVICE = -7      /* a kernel flagged bad data (see moe_cache_error)   */
} moe_status;

/* Stored weight formats of one expert. */
typedef enum {
  MOE_W_BF16 = 0,          /* BF16 weights                                        */
  MOE_W_FP8_B128 = 1       /* E4M3FN codes + one float32 scale per 128x128 tile   */
} moe_wtype;

/*
 * Slot pool: every tensor of one (layer, expert) in one slot ([FT] section
 * "全层双缓冲"; [FTK] paragraph on the elastic expert cache).  One bank per
 * tensor kind, slot-major, 16-byte aligned:
 *   w_gate_up : [n_slots][2*I*H] elements, gate and up weights in the packed
 *               brick format below (BF16 bits or E4M3 codes)
 *   w_down    : [n_slots][H*I] elements, down weights in the brick format
 *   s_gate, s_up : [n_slots][I/128][H/128] float32  (FP8 only, else NULL)
 *   s_down       : [n_slots][H/128][I/128] float32  (FP8 only, else NULL)
 * Brick format of a matrix W [N][K] (stored [out, in]): 1 KB bricks, one per
 * 16 rows x KB columns (KB = 32 for BF16, 64 for FP8), brick (t, kt) at
 * element offset (t * (K/KB) + kt) * 16*KB; inside a brick the 64 lanes of an
 * MFMA operand follow each other, lane l = 16*j + r holding W[16t + r][KB*kt
 * + (KB/4)*j + e] for e < KB/4.  The gate/up bank is the brick format of the
 * 2I-row matrix whose row 16t + r is W_gate row 8t + r (r < 8) or W_up row
 * 8t + r - 8 (r >= 8).  moe_pack_weights produces both banks from row-major
 * matrices.  Scales stay row-major per 128 x 128 tile of the original
 * matrices.  A view of slots [a, a+n) is the same struct with every base
 * advanced by a slots and n_slots = n.
 */
typedef struct moe_slots {
  int32_t wtype;           /* moe_wtype */
  int32_t H, I;            /* hidden and SwiGLU intermediate sizes */
  int32_t n_slots;
  void* w_gate_up;
  void* w_down;
  float* s_gate;
  float* s_up;
  float* s_down;
} moe_slots;

/*
 * Host expert pool: the ground truth of every routed expert, addressed by
 * logical id l*E + e ([FT] section "FTW 权重格式与平台适配": banks keyed by
 * lE+e, the rows of one id across banks form one expert).  Each field is a
 * HOST array of L*E pointers into PINNED host memory, one per logical id
 * (aliasing allowed: several ids may point at the same bytes).  Scale tables
 * are NULL for BF16.  The arrays are copied at moe_cache_create; the pinned
 * memory they point to must outlive the cache.
 */
typedef struct moe_host_pool {
  const void* const* w_gate_up;   /* packed gate/up bank rows, per logical id */
  const void* const* w_down;      /* packed down bank rows                    */
  const float* const* s_gate;
  const float* const* s_up;
  const float* const* s_down;
} moe_host_pool;

typedef struct moe_cache_cfg {
  int32_t L;               /* MoE layers sharing the cache                       */
  int32_t E;               /* routed experts per layer (<= 4096)                 */
  int32_t k;               /* picks per token                                    */
  int32_t T_max;           /* max tokens per moe_cache_step call (T_max*k<=1024) */
  int32_t C;               /* cache slots (<= 16384, == slots->n_slots)          */
  uint32_t bp, bh;         /* B_P and B_H in one unit (e.g. 0.1 GB/s); bh > 0    */
} moe_cache_cfg;

typedef struct moe_cache* moe_cache_t;
typedef struct moe_prefill* moe_prefill_t;

/* Indices into moe_step_out.counts. */
enum {
  MOE_CNT_UNIQ = 0,        /* u: distinct logical ids routed this call            */
  MOE_CNT_HIT = 1,         /* h                                                   */
  MOE_CNT_MISS = 2,        /* m                                                   */
  MOE_CNT_QSTAR = 3,       /* q*: the split's fill count before the victim clamp  */
  MOE_CNT_FILL = 4,        /* q = min(q*, free victims): valid entries of fill_*  */
  MOE_CNT_HOST = 5,        /* m - q: valid entries of host_id                     */
  MOE_CNT_N = 8
};

/*
 * Fixed-shape outputs of one cache step, all DEVICE arrays owned by the
 * caller ([FT] section "Device-side 缓存控制": fixed-shape work buffers plus a
 * device-resident valid count).  U_max = min(T_max*k, E).  Entries past the
 * valid count are written -1.
 */
typedef struct moe_step_out {
  int32_t* pick_slot;      /* [T_max*k] slot of each pick, or -1 = host set       */
  int32_t* uniq;           /* [U_max] distinct logical ids, ascending             */
  int32_t* is_hit;         /* [U_max] 1 if uniq[i] was resident                   */
  int32_t* fill_id;        /* [U_max] logical ids filled, ascending               */
  int32_t* fill_slot;      /* [U_max] their victim slots                          */
  int32_t* fill_evicted;   /* [U_max] id evicted from that slot, -1 if empty      */
  int32_t* host_id;        /* [U_max] logical ids left to the host, ascending     */
  int32_t* counts;         /* [MOE_CNT_N]                                         */
} moe_step_out;

#define MOE_STEP_NO_COPY 1u   /* decisions and tables only; skip the fill copy  */
#define MOE_STEP_FILL_ALL 2u  /* q* = m: fill every miss that finds a non-hit
                                 slot (on-demand loading, see
                                 moe_cache_prefill_load)                        */

#define MOE_FWD_DECODE 0u     /* grouped GEMV, T <= 16                           */
#define MOE_FWD_PREFILL 1u    /* sorted grouped GEMM on MFMA                     */
#define MOE_FWD_DECODE_SPLIT 2u /* MOE_FWD_DECODE in two launches (see below)    */

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/*
 * Top-k router ([FTK] paragraphs on MoE routing and the GPU router).
 * logits: device float32 [T, E]; ids: device int32 [T, k]; w: device float32
 * [T, k].  Per token, experts are ranked by logit descending, ties to the
 * lower index; ids are written in rank order and w = softmax over the k kept
 * logits.  1 <= k <= min(E, 32), 1 <= E <= 1024, T >= 0.  Capturable.
 */
moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                          int32_t* ids, float* w, hipStream_t stream);

/* Bytes of device workspace a cache with this configuration needs. */
moe_status moe_cache_workspace_bytes(const moe_cache_cfg* cfg, size_t* bytes);

/*
 * Create a cache over `slots` (which must have n_slots == cfg->C) and the host
 * pool `host` (L*E ids).  dev_ws: device workspace of at least
 * moe_cache_workspace_bytes, 256-byte aligned, owned by the caller and kept
 * alive until moe_cache_destroy.  Every host-pool pointer is checked to be
 * pinned and device-accessible (else MOE_ERR_NOT_PINNED).  Initialises the
 * tables to empty on `stream` (not capturable).
 */
moe_status moe_cache_create(const moe_cache_cfg* cfg, const moe_slots* slots,
                            const moe_host_pool* host, void* dev_ws, size_t ws_bytes,
                            hipStream_t stream, moe_cache_t* out);

/*
 * Reset the cache to empty, then place logical id host_ids[i] in slot i with
 * recency older than any step (stamp 1 + i), copying its bytes from the host
 * pool unless flags has MOE_STEP_NO_COPY.  host_ids: host array of n distinct
 * ids, n <= C.  Not capturable.
 */
moe_status moe_cache_seed(moe_cache_t c, const int32_t* host_ids, int32_t n,
                          uint32_t flags, hipStream_t stream);

/*
 * One layer call of the cache ([FT] sections "Device-side 缓存控制", "q* 策略",
 * "语义感知专家缓存"; [FTK] decode and dynamic-LRU paragraphs).  One kernel:
 * dedup of the routed experts -> hit/miss against the residency table ->
 * q* = clamp(round(m*bp/bh), 1, m) -> one scan selecting the least recently
 * used non-hit slots -> table update and recency stamps -> rewrite of every
 * pick to its slot or -1 (host set).  Then, unless MOE_STEP_NO_COPY, one
 * fixed-grid copy kernel moves every bank of each filled expert from the
 * pinned host pool into its slot, masked by the device fill count ([FT]
 * section "Device-side 缓存控制": one fused transfer over all banks).
 * d_layer: DEVICE int32 scalar holding the layer (0 <= layer < L), read by
 * the kernel when it runs, so one captured graph of a layer call serves
 * every layer ([FT] section "执行顺序与工程细节": the per-layer control flow is
 * captured once and replayed; [FT] section "Device-side 缓存控制": no host
 * decision per layer).  A layer outside [0, L) sets the device error word
 * (moe_cache_error) and the call decides nothing: tables unchanged, every
 * pick -1, lists -1, counts 0 (counts[6] = the bad layer), no fill.
 * ids: device int32 [T, k] expert indices of that layer.  1 <= T <= T_max.
 * An id outside [0, E) sets the device error word and is treated as routed
 * to the host.  Capturable.
 */
moe_status moe_cache_step(moe_cache_t c, const int32_t* d_layer, const int32_t* ids, int32_t T,
                          uint32_t flags, const moe_step_out* out, hipStream_t stream);

/*
 * Router and cache step in one launch: the same results as
 * moe_route_topk(logits, T, E, k, ids, w) followed by
 * moe_cache_step(c, d_layer, ids, T, flags, out) (bit for bit: the same
 * selection and softmax code), with one kernel instead of two on the decode
 * path ([FT] section "Device-side 缓存控制": routing feeds the one control
 * kernel; [FTK] GPU-router paragraph).  d_layer: device int32 scalar, as
 * for moe_cache_step (a bad layer also leaves ids and w unwritten).
 * logits: device float32 [T, E]; ids: device int32 [T, k] and w: device
 * float32 [T, k], both written.  Needs E <= 1024 and k <= 32.  Capturable.
 */
moe_status moe_cache_route_step(moe_cache_t c, const int32_t* d_layer, const float* logits, int32_t T,
                                int32_t* ids, float* w, uint32_t flags, const moe_step_out* out,
                                hipStream_t stream);

/*
 * The fused fill copy alone: copy every bank of the out->counts[MOE_CNT_FILL]
 * experts listed in out->fill_id / out->fill_slot from the pinned host pool
 * into their slots, with one fixed-grid launch masked by the device count
 * ([FT] section "Device-side 缓存控制").  moe_cache_step with
 * MOE_STEP_NO_COPY followed by this call equals moe_cache_step without the
 * flag.  Capturable.
 */
moe_status moe_cache_fill(moe_cache_t c, const moe_step_out* out, hipStream_t stream);

/*
 * On-demand loading of one layer for a prefill batch, the fallback when the
 * pool has no room for the full-layer buffers ([FT] section "全层双缓冲";
 * [FTK] prefill paragraph: without two whole-layer buffers prefill loads
 * what the layer needs instead of oversubscribing memory).  One layer call
 * of the cache over the batch's routed experts with MOE_STEP_FILL_ALL: the
 * dedup, hit/miss, victim scan, table update and stamps of moe_cache_step
 * with q* = m (every miss is filled while non-hit slots remain; the rest
 * stay on the host), then pick_slot[p] = slot of the expert of pick p, or -1
 * for a pick left to the host, then (unless MOE_STEP_NO_COPY) the fused fill
 * copy.  Decisions, tables and counts equal moe_cache_step(c, layer, ids, T,
 * flags | MOE_STEP_FILL_ALL, out) would give for a T within T_max.
 * ids: device int32 [T, k], any T >= 1; pick_slot: device int32 [T, k],
 * written (out->pick_slot is not used).  Needs ceil(E/k) <= T_max (the
 * layer's expert set goes to the decision kernel as rows of k).  Ids outside
 * [0, E) set the device error word and go to the host.  Capturable.
 */
moe_status moe_cache_prefill_load(moe_cache_t c, int32_t layer, const int32_t* ids, int32_t T,
                                  uint32_t flags, const moe_step_out* out, int32_t* pick_slot,
                                  hipStream_t stream);

/*
 * Copy the residency tables to HOST arrays (any pointer may be NULL):
 * slot_id [C] (-1 empty, -2 reserved by a prefill pool), stamp [C] (0 empty,
 * (tick << 16) | (1 + rank) otherwise), id_slot [L*E], tick, and counters[6] =
 * calls, uniq, hits, misses, fills, host summed over all steps.  Synchronises
 * `stream`; not capturable.
 */
moe_status moe_cache_read_state(moe_cache_t c, int32_t* slot_id, uint64_t* stamp,
                                int32_t* id_slot, uint64_t* tick, uint64_t* counters,
                                hipStream_t stream);

/* Read and clear the device error word (0 = none).  Synchronises; not capturable. */
moe_status moe_cache_error(moe_cache_t c, int32_t* code, hipStream_t stream);

moe_status moe_cache_destroy(moe_cache_t c);

/*
 * Change the cache's slot count at a safe point (between layer calls, no
 * prefill pool alive) ([FTK] safe-point paragraph: the memory budget between
 * KV cache and expert cache is re-split at run time, and since the host pool
 * is the ground truth a smaller GPU cache changes no output; [FT] section
 * "挑战三": the budget shrinks or grows without a restart).  The new
 * capacity is slots->n_slots (same weight type, H and I).  The cache keeps
 * its min(residents, new C) most recent residents with their stamps: one in
 * a slot below the new C stays there, the others move, in ascending order of
 * their old slots, to the free slots below the new C in ascending order
 * (evicting the least recently used); slots added by growth are empty; tick
 * and counters carry over.  slots: either every bank at the same address as
 * now (in place: shrink, or grow into banks allocated that large) or every
 * bank in new memory that does not overlap the old (kept experts are copied
 * there).  dev_ws: a new workspace of moe_cache_workspace_bytes for the new
 * configuration, not overlapping the current one; afterwards the cache uses
 * it and the old workspace (and old banks, if moved) may be freed.
 * Synchronises `stream`; not capturable.  On MOE_ERR_HIP the cache must be
 * destroyed.
 */
moe_status moe_cache_resize(moe_cache_t c, const moe_slots* slots, void* dev_ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * Pack n experts from row-major device matrices into the brick format of the
 * slot pool (see moe_slots): w_gate, w_up [n][I][H] and w_down [n][H][I]
 * (BF16 bits or E4M3 codes) -> w_gate_up [n][2*I*H], w_down_packed [n][H*I].
 * Requires I % 8 == 0 and H, I multiples of 32 (BF16) or 128 (FP8).  The
 * outputs must not overlap the inputs.  Device pointers; enqueued on stream.
 */
moe_status moe_pack_weights(int32_t wtype, int32_t H, int32_t I, int32_t n, const void* w_gate, const void* w_up,
                            const void* w_down, void* w_gate_up, void* w_down_packed, hipStream_t stream);

/* Bytes of device workspace moe_expert_forward needs for these sizes. */
moe_status moe_forward_workspace_bytes(int32_t T_max, int32_t k, int32_t H, int32_t I,
                                       int32_t n_slots, uint32_t mode, size_t* bytes);

/*
 * Grouped SwiGLU expert evaluation of G = H u F ([FT] section "执行顺序与工程细节":
 * grouped evaluation of the hits and fills; [OSDI] section 4.3 expert
 * structure; [OSDI] section 4.2 FP8 expansion and post-scaling).
 *   y[t] = sum over picks j with pick_slot[t,j] >= 0 of
 *          w[t,j] * W_down (silu(W_gate x_t) * (W_up x_t))   (slot's weights)
 * x: device BF16 [T, H]; pick_slot: device int32 [T, k] (slot index in
 * `slots`, -1 = skip); w: device float32 [T, k]; y: device float32 [T, H],
 * fully overwritten.  FP8 weights are expanded exactly to BF16 in registers
 * (the gfx950 two-codes-per-instruction E4M3 -> BF16 conversion with unit
 * scale) and each 128x128 tile's scale is applied once to its block partial
 * sum.  Accumulation is FP32; the
 * SwiGLU activations h are rounded to BF16 before the down projection, and
 * in prefill mode each pick's gate-weighted row is rounded to BF16 before a
 * token's k rows are summed (in FP32, pick order).
 *   mode MOE_FWD_DECODE: T <= 16 and T*k <= 256 (grouped GEMV streaming each
 *     slot once; y is the same bits on every run).
 *   mode MOE_FWD_DECODE_SPLIT: the decode evaluation in two launches of the
 *     same kernel (gate/up + SwiGLU, then down + gate weight), the same
 *     bits.  MOE_FWD_DECODE hands h from the gate/up to the down work inside
 *     one launch, so its down workgroups wait for gate/up work of the same
 *     grid: it needs the whole grid resident at once (the grid is sized to
 *     the compute units' capacity; a GPU whose units are shared with other
 *     work can break that, and the bounded wait then reports it, below).
 *     The split form waits for nothing and completes on any share of the
 *     GPU, at the cost of a second launch.
 *   mode MOE_FWD_PREFILL: any T (tokens sorted by slot, grouped GEMM).
 * ws: device workspace of moe_forward_workspace_bytes(T_max >= T, ...),
 * owned by the caller, 256-byte aligned and ZERO-FILLED before its first
 * use: decode mode keeps its hand-over counters there and leaves them at
 * zero on exit, so the same workspace serves any later call on the same
 * stream without clearing; calls that overlap on one workspace race.  A
 * MOE_FWD_DECODE call whose internal wait timed out (only possible when its
 * workgroups cannot all be resident, e.g. a shared GPU) sets the first
 * 32-bit word of ws to a non-zero value; y is then not valid, and ws must be
 * zero-filled again before its next use (a late hand-over store may leave a
 * control word set).
 * Requires H, I multiples of 128 (FP8) or of 32 (BF16).  Capturable.
 */
moe_status moe_expert_forward(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot,
                              const float* w, int32_t T, int32_t k, float* y,
                              void* ws, size_t ws_bytes, uint32_t mode, hipStream_t stream);

/*
 * moe_expert_forward followed by moe_merge_partial in one call, with the
 * same bits: y_out = y_gpu + y_host and, if y_out_bf16 != NULL, its BF16
 * ([FT] section "q* 策略": the GPU and host partial sums are added).  The
 * sum is formed where the GPU partial sum leaves the expert kernels, so the
 * merge needs no launch of its own.  y_gpu: device float32 [T, H], written
 * if not NULL; y_host: device or pinned host float32 [T, H]; y_out: device
 * float32 [T, H] (may not alias y_host).  Same modes, sizes and workspace as
 * moe_expert_forward.  Capturable.
 */
moe_status moe_expert_forward_merge(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot,
                                    const float* w, int32_t T, int32_t k, float* y_gpu, const float* y_host,
                                    float* y_out, uint16_t* y_out_bf16, void* ws, size_t ws_bytes, uint32_t mode,
                                    hipStream_t stream);

/*
 * Launch shape of the decode forward (MOE_FWD_DECODE and _SPLIT in
 * moe_expert_forward and _merge): n_workgroups > 0 fixes the grid of every
 * later decode launch in this process, 0 restores the automatic grid (as
 * many workgroups as the compute units hold at once).  For tests and
 * tuning: in MOE_FWD_DECODE_SPLIT mode every grid completes, with the bits
 * of MOE_FWD_DECODE on the same grid (the grid decides which workgroup sums
 * which terms, so other grids may round differently, within the layer
 * tolerance); MOE_FWD_DECODE with more workgroups than the GPU holds at once
 * times out (see moe_expert_forward).  Host only, takes effect at the next launch;
 * MOE_ERR_ARG outside [0, 4096].
 */
moe_status moe_decode_grid_override(int32_t n_workgroups);

/*
 * Exercises the bounded wait of MOE_FWD_DECODE (for tests of its error path,
 * which otherwise needs a GPU shared with other work).  Same arguments as
 * moe_expert_forward in MOE_FWD_DECODE mode (T <= 16, the same workspace),
 * except that it launches only the down phase, with the waits of the
 * one-launch form for the start signal that the gate/up phase would raise;
 * nothing in this launch raises it, so each waiting workgroup gives up after
 * `polls` polls (in [1, 4194304]; the one-launch form allows 4194304, about
 * 1-2 s), sets the first 32-bit word of ws non-zero and finishes its work on
 * whatever h the workspace holds.  Every workgroup exits; y is written but
 * not valid, and ws must be zero-filled again before its next use, as after a
 * time-out of moe_expert_forward.  MOE_ERR_ARG for polls outside the range,
 * otherwise the errors of moe_expert_forward.  Capturable.
 */
moe_status moe_decode_wait_test(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot,
                                const float* w, int32_t T, int32_t k, float* y, void* ws, size_t ws_bytes,
                                uint32_t polls, hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under hipGraph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * as moe_expert_forward_merge in MOE_FWD_DECODE mode (the same kernels, the
 * same bits), with the workspace taken from a static device array of the
 * library (8.5 MiB per GPU, held until the process ends) instead of a
 * caller buffer.  The library allocates nothing in this call (no hipMalloc,
 * hipFree or allocating library routine).  Limit: the call needs
 * min(T*k, n_slots) * 16 * I * 2 bytes of h within 8 MiB (for example T*k
 * <= 128 at I = 2048, or <= 256 at I = 1024), else MOE_ERR_NO_SPACE with
 * nothing enqueued; T <= 16 and T*k <= 256 as in decode mode.  Every call
 * clears the array's hand-over words with a small kernel before the
 * forward, so a call that timed out leaves nothing behind.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  The
 * first call on a device looks up the array's address (hipGetSymbolAddress):
 * make it outside graph capture.  Capturable after that.
 */
moe_status moe_expert_forward_merge_static(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot,
                                           const float* w, int32_t T, int32_t k, float* y_gpu,
                                           const float* y_host, float* y_out, uint16_t* y_out_bf16,
                                           hipStream_t stream);

/*
 * Merge of the GPU and host partial sums ([FT] section "q* 策略": the two
 * partial sums are combined exactly; [FT] "Graph 内的 CPU 执行分支").
 * y_out[i] = y_gpu[i] + y_host[i] over T*H floats; if y_out_bf16 != NULL it
 * also receives the BF16 (round-to-nearest-even) of y_out.  y_host may be
 * device memory or pinned host memory.  y_out may alias y_gpu.  Capturable.
 */
moe_status moe_merge_partial(const float* y_gpu, const float* y_host, int32_t T, int32_t H,
                             float* y_out, uint16_t* y_out_bf16, hipStream_t stream);

/*
 * Full-layer double buffer for prefill ([FT] section "全层双缓冲"; [FTK]
 * prefill paragraph).  Reserves the last 2E slots of the cache's pool as two
 * full-layer buffers (evicting what they held; they leave the LRU), else
 * MOE_ERR_NO_SPACE (then prefill falls back to moe_cache_prefill_load).
 * Layer l uses buffer l % 2.  Synchronises the device.
 */
moe_status moe_prefill_create(moe_cache_t c, moe_prefill_t* out);

/*
 * The same with `depth` full-layer buffers (2 <= depth <= 64) in a ring:
 * reserves the last depth*E slots, layer l uses buffer l % depth, so up to
 * depth - 1 layers load ahead of the one computing ([OSDI] section 3.2,
 * the expert ring of stream-loading prefill: deep while transfer is the
 * bottleneck, two buffers once compute is).  MOE_ERR_NO_SPACE if depth*E > C.
 */
moe_status moe_prefill_create_ring(moe_cache_t c, int32_t depth, moe_prefill_t* out);

/*
 * Enqueue on copy_stream: wait until buffer (layer % depth) is released, copy ALL
 * E experts of `layer` (every bank) from the pinned host pool into it
 * (without waiting for routing), then mark it ready.  MOE_ERR_STATE (nothing
 * enqueued) if the layer the buffer holds has not been released by
 * moe_prefill_release since its own prefetch: the copy would overwrite
 * weights that compute may still be reading.
 */
moe_status moe_prefill_prefetch(moe_prefill_t p, int32_t layer, hipStream_t copy_stream);

/*
 * Make `compute` wait until layer's buffer is ready and return its view: a
 * moe_slots of E slots whose slot e holds expert e of `layer` (pick_slot in
 * prefill mode is then the expert index).  MOE_ERR_STATE if `layer` was not
 * prefetched into that buffer.
 */
moe_status moe_prefill_acquire(moe_prefill_t p, int32_t layer, hipStream_t compute,
                               moe_slots* view);

/* Record on `compute` that layer's buffer may be overwritten by a later prefetch. */
moe_status moe_prefill_release(moe_prefill_t p, int32_t layer, hipStream_t compute);

/*
 * End prefill and seed decode with what the buffers hold ([FT] section
 * "全层双缓冲" and [FTK] prefill paragraph: the buffers are slots of the
 * shared pool, so the experts that survive prefill are decode's first
 * residents, with no copy).  Waits for the device, then every expert of a
 * layer a buffer holds becomes resident in its buffer slot, more recent than
 * every earlier entry: buffers in load order (least recent first), experts
 * ascending, stamps (tick << 16) | (1 + rank); an expert already resident in
 * a decode slot keeps that slot and takes the new stamp, its buffer slot and
 * every buffer that holds nothing return empty; the tick advances by one.
 * Frees the pool.  Not capturable.
 */
moe_status moe_prefill_finish(moe_prefill_t p, hipStream_t stream);

/* End prefill discarding the buffers: their slots return to the LRU empty. */
moe_status moe_prefill_destroy(moe_prefill_t p, hipStream_t stream);


/*
 * Expand n E4M3FN codes to BF16 bit patterns with the conversion the decode
 * kernels run in registers ([OSDI] section 4.2: every E4M3 value is exactly a
 * BF16 value; here gfx950's E4M3 -> BF16 pack conversion with unit scale,
 * NaN codes give a BF16 NaN).  codes: device uint8 [n]; out: device uint16
 * [n].  Capturable.
 */
moe_status moe_e4m3_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, hipStream_t stream);

/*
 * Measurement reference, not a step of the method: one launch that reads
 * `bytes` from `src` with the decode kernels' wide non-temporal loads and
 * does nothing else (each workgroup folds what it read into sink[0..255]
 * with atomic XORs, so the loads stay).  Its duration bounds what any single
 * launch streaming the same bytes can reach on this GPU, start-up and tail
 * included.  src: device, 16-byte aligned; bytes a multiple of 16; sink:
 * device uint32 [256].  Capturable.
 */
moe_status moe_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * moe_stream_read with its launch shape chosen: n_wg workgroups of 256
 * threads (1 <= n_wg <= 65536), each thread keeping `unroll` 16-byte loads
 * in flight (1, 2, 4, 8 or 16); moe_stream_read is n_wg 512, unroll 4.  A
 * sweep of the two gives the fastest single launch that only reads a given
 * byte count.  Capturable.
 */
moe_status moe_stream_read_cfg(const void* src, size_t bytes, uint32_t* sink, int32_t n_wg, int32_t unroll,
                               hipStream_t stream);

/*
 * Host executor for the host set C ([FT] section "q* 策略": the misses a step
 * does not fill are computed by the CPU while the GPU evaluates G, and the two
 * partial sums are added; [OSDI] section 4.2: FP8 codes expanded on the CPU,
 * each 128-wide block dotted first and multiplied by its scale once;
 * [OSDI] section 4.3: gate, up, SiLU(gate) * up, down).  This is the CPU side
 * of the method, never a substitute for the GPU evaluation of G.
 *
 * moe_host_exec_create starts n_threads - 1 worker threads (the calling
 * thread is the n-th); after a call they spin for a quarter of a
 * millisecond, so calls one layer apart find them awake, then sleep.  The executor uses AVX-512
 * where the CPU has it (AVX512F, BW and VL), else portable C++; flags
 * MOE_HOST_PORTABLE selects the portable path everywhere.  Both sum in the
 * same order within a 16-row brick row but group the additions differently,
 * so their results agree to FP32 rounding, not bitwise.
 * moe_host_exec_destroy joins the threads; no call may be running.
 * moe_host_exec_simd returns 512 for an executor on the AVX-512 path, else 0.
 */
#define MOE_HOST_PORTABLE 1u
#define MOE_HOST_PIN 2u
typedef struct moe_host_exec* moe_host_exec_t;
moe_status moe_host_exec_create(int32_t n_threads, uint32_t flags, moe_host_exec_t* out);
moe_status moe_host_exec_destroy(moe_host_exec_t h);
int32_t moe_host_exec_simd(moe_host_exec_t h);

/*
 * Core placement ([FT] section "Graph 内的 CPU 执行分支": a resident pool of
 * worker threads pinned to physical cores).  With MOE_HOST_PIN in the flags
 * of moe_host_exec_create, the pool is n_threads worker threads, worker i
 * pinned to entry i (modulo its length) of this list: the CPUs of the
 * process's affinity set, one per physical core first (the lowest allowed
 * SMT sibling of each core), the cores of the NUMA node the current HIP
 * device is attached to before the others, then the remaining siblings in
 * the same order; the calling thread (or the signalled form's dispatcher)
 * then only waits for them.  Without the flag the pool is n_threads - 1
 * unpinned workers plus the calling thread.  moe_host_exec_cpus writes the
 * CPU of workers 0 .. n-1 (-1: not pinned, or beyond the pool) and the
 * device's NUMA node (-1 if unknown).
 */
moe_status moe_host_exec_cpus(moe_host_exec_t h, int32_t* cpus, int32_t n, int32_t* numa_node);

/*
 * y_host[t] = sum over picks j with pick_slot[t,j] < 0 of
 *             w[t,j] * W_down (silu(W_gate x_t) * (W_up x_t))   (expert ids[t,j])
 * computed on the executor's threads from the packed rows of `pool` (the
 * rows fills copy: the brick format, gate/up interleaved; FP8 with its
 * 128x128 scales).  All pointers are host memory: x BF16 [T, H]; ids int32
 * [T, k] logical ids (indices into the pool's tables; must be >= 0 where
 * pick_slot < 0); pick_slot int32 [T, k] as written by moe_cache_step (only
 * its sign is read); w float32 [T, k]; y_host float32 [T, H], fully
 * overwritten (0 for tokens with no host pick).  Accumulation is FP32 and h
 * stays FP32; each output element is summed by one thread in a fixed order,
 * so the result has the same bits on every call and for any thread count.
 * Calls on one executor are serialised.  Requires H, I multiples of 32 (BF16)
 * or 128 (FP8) and I % 8 == 0.  Returns MOE_ERR_ARG on a NULL pointer or a
 * negative host id, MOE_ERR_SHAPE on bad sizes.  Synchronous; not a HIP call.
 */
moe_status moe_host_forward(moe_host_exec_t h, const moe_host_pool* pool, int32_t wtype, int32_t H, int32_t I,
                            const uint16_t* x, const int32_t* ids, const int32_t* pick_slot, const float* w,
                            int32_t T, int32_t k, float* y_host);

/*
 * moe_host_forward in stream order: records the arguments in the executor
 * (one descriptor per executor, replaced by the next enqueue) and enqueues on
 * `stream` a host function that runs the call when the stream reaches it;
 * later work on `stream` waits for it.  The host arrays (x, ids, pick_slot,
 * w: written by earlier copies on the stream; y_host: read by later work)
 * must stay valid until then, pinned if the GPU reads or writes them.
 * Capturable: the host function becomes a graph node, and replays run the
 * recorded descriptor again, so capture one enqueue per executor per graph.
 * The host function makes no HIP call.  A failure inside it is kept until
 * moe_host_exec_status reads it (returns and clears the first failure).
 */
moe_status moe_host_forward_enqueue(moe_host_exec_t h, const moe_host_pool* pool, int32_t wtype, int32_t H,
                                    int32_t I, const uint16_t* x, const int32_t* ids, const int32_t* pick_slot,
                                    const float* w, int32_t T, int32_t k, float* y_host, hipStream_t stream);
moe_status moe_host_exec_status(moe_host_exec_t h);

/*
 * The host branch of a decode step without host callbacks: pinned words hand
 * the step over between a GPU stream and the executor's dispatcher thread.
 *   moe_host_signal: in stream order, store seq into *word (pinned host
 *     memory) at system scope: put after the copies of the step's inputs.
 *   moe_host_forward_signal: queue moe_host_forward on the executor's
 *     dispatcher thread (started by the first call; calls run in order):
 *     it waits until *ready - seq >= 0 (serial numbers modulo 2^32; at most
 *     2 s, then the call is skipped and its failure kept for
 *     moe_host_exec_status), runs the call, and stores seq into *done after
 *     y_host.  Returns at once; the host arrays must stay valid until *done
 *     reaches seq.  ready, done: pinned host words, zero before the first
 *     seq (seq = 1, 2, ...).
 *   moe_merge_partial_after: moe_merge_partial whose workgroups first wait
 *     until *done - seq >= 0 (a bounded poll, seconds; on time-out
 *     *err |= 1 and the merge goes on with whatever y_host holds).  y_host
 *     is pinned host memory read after the wait; err: device or pinned word,
 *     or NULL.
 * Not capturable (the dispatcher is fed per call); moe_host_forward_enqueue
 * is the capturable form.
 */
moe_status moe_host_signal(uint32_t* word, uint32_t seq, hipStream_t stream);
moe_status moe_host_forward_signal(moe_host_exec_t h, const moe_host_pool* pool, int32_t wtype, int32_t H,
                                   int32_t I, const uint16_t* x, const int32_t* ids, const int32_t* pick_slot,
                                   const float* w, int32_t T, int32_t k, float* y_host, const uint32_t* ready,
                                   uint32_t* done, uint32_t seq);
moe_status moe_merge_partial_after(const float* y_gpu, const float* y_host, const uint32_t* done, uint32_t seq,
                                   int32_t T, int32_t H, float* y_out, uint16_t* y_out_bf16, uint32_t* err,
                                   hipStream_t stream);

/*
 * Bandwidth calibration for the q* split ([FT] section "q* 策略": B_P and B_H
 * are measured on the deployed machine at the deployed tensor shapes before
 * serving; [FT] section "挑战二": the right split is machine-specific).
 * Copies the n experts `ids` (host array of logical ids of the cache's host
 * pool) into scratch slots 0 .. n-1, once untimed and then `reps` times
 * timed with HIP events on `stream`, through
 *   - the fused fill kernel (mapped pinned host memory; the decode fill path):
 *     fill_GBps, and bp = round(10 * fill_GBps), the cache's B_P unit;
 *   - hipMemcpyAsync per bank (the DMA engines; the prefill buffers' path):
 *     dma_GBps;
 * and, if hx is not NULL, evaluates them on the host executor as the host
 * set of decode-shaped calls (one token, min(8, n) host picks per call,
 * cycling through the ids), once untimed and then `reps` times:
 * host_GBps and bh = round(10 * host_GBps) (else 0).  Rates count every
 * bank's bytes (expert_bytes per expert).  The cache's tables and slots are
 * not touched; the fill list uses the cache's seed scratch.  scratch:
 * device slots of the cache's weight type, H and I with n_slots >= n
 * (caller-owned; overwritten).  1 <= n <= C, 1 <= reps <= 1000.
 * Synchronises `stream`; not capturable.
 */
typedef struct moe_bandwidth {
  uint32_t bp, bh;         /* B_P (fill kernel) and B_H (host executor) in 0.1 GB/s */
  double fill_GBps;        /* fused fill kernel, pinned host -> device       */
  double dma_GBps;         /* hipMemcpyAsync, pinned host -> device           */
  double host_GBps;        /* host executor, expert bytes evaluated per second */
  double expert_bytes;     /* bytes of one expert over every bank            */
} moe_bandwidth;
moe_status moe_calibrate_bandwidth(moe_cache_t c, moe_host_exec_t hx, const int32_t* ids, int32_t n,
                                   const moe_slots* scratch, int32_t reps, hipStream_t stream, moe_bandwidth* out);

/*
 * Measurement: the calls of moe_host_forward (direct or enqueued) that had
 * host picks, and the wall time spent in them (ns), since the executor was
 * created.
 */
moe_status moe_host_exec_stats(moe_host_exec_t h, uint64_t* calls, uint64_t* ns);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
