/*
 * moe.h - C ABI of libmoe: the routed MoE expert-layer forward for one
 * AMD Instinct MI355X (gfx950), with an HBM expert cache over a pinned host
 * expert pool.
 *
 * What it computes comes from the FreeToken pages:
 *  - experts live in host memory and are brought to the GPU on demand, only
 *    a few of many experts being active per token (aiforradalom.hu article
 *    "Egyetlen munkaállomás-GPU-n futtatja a 753 milliárdos GLM-5.2 modellt
 *    a FreeToken", section "A Mixture-of-Experts (MoE) kihívásai és a
 *    FreeToken megoldásai");
 *  - offloading is exact: no simplified expert, no modified router, partial
 *    results summed at the end (jansverre.net FreeToken article, section
 *    "Hva er FreeToken?");
 *  - decode uses one global LRU expert cache across the MoE layers, prefill
 *    streams the next layer's experts in while the current layer computes
 *    (jansverre.net article, section "Hvorfor er båndbredden viktigere enn
 *    antall kjerner?"; aipolix.com article "FreeToken مدلهای عظیم MoE را روی
 *    GPUهای مصرفی اجرا میکند", fourth and fifth paragraphs);
 *  - the GPU expert cache can be resized without restarting or reloading
 *    the host-resident pool (aipolix.com article, sixth paragraph).
 * The pages give no formulas; the readings used (softmax router, top-k by
 * logit then lower id, renormalised gates, SwiGLU experts, MXFP4 weights
 * with E2M1 elements and one E8M0 scale per 32 along K, or bf16 weights) are
 * stated at each call.  Two other cache placements (per-layer shares, a
 * static set) exist for comparing the global LRU with them.
 *
 * Conventions
 *  - Every call returns a moe_status (int32_t); MOE_OK is 0, errors are
 *    negative.  moe_last_error() returns a thread-local message describing
 *    the last failure on the calling thread.  No C++ exception crosses the
 *    ABI; invalid arguments are reported before any GPU work is enqueued.
 *  - "d_" pointers are device pointers owned by the caller; they must be
 *    16-byte aligned and stay valid until the enqueued work completes.
 *    "h_" pointers are host pointers read (or written) before the call
 *    returns.
 *  - GPU work is enqueued on the caller's stream (a hipStream_t passed as
 *    void*; NULL means the default stream) and, for prefill, on an internal
 *    copy stream joined by events.  Calls marked (sync) wait for completion.
 *  - A context is not thread-safe; use it from one thread and one stream at
 *    a time.  Calls that overlap on one context race.
 *  - bf16 tensors are IEEE bfloat16 bit patterns (uint16).  Row-major.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad pointer, size, index or config field   */
  MOE_ERR_OOM = -2,         /* device or pinned host allocation failed     */
  MOE_ERR_HIP = -3,         /* a HIP runtime call failed                   */
  MOE_ERR_CAPACITY = -4,    /* request exceeds a configured capacity       */
  MOE_ERR_STATE = -5,       /* call not valid in the current state         */
  MOE_ERR_UNSUPPORTED = -6  /* valid request this build does not handle    */
};

typedef struct moe_ctx moe_ctx;

/*
 * Placement policy of the decode expert cache (moe_config.cache_policy).
 * The pages use one global LRU across the MoE layers instead of locking
 * chosen experts into GPU memory at start-up, and compare its miss rate with
 * other placements at equal capacity (jansverre.net FreeToken article,
 * section "Hvorfor er båndbredden viktigere enn antall kjerner?").  The two
 * alternatives exist for that comparison; every policy uses the lookup rule
 * of moe_layer_forward:
 *  - GLOBAL: all C slots are one LRU over (layer, expert) keys;
 *  - PER_LAYER: layer l owns slots floor(l*C/L) .. floor((l+1)*C/L) - 1, and
 *    a lookup of layer l takes victims only from them;
 *  - STATIC: lookups never insert (every miss bypasses through staging);
 *    only expert_cache_fill places experts, with the GLOBAL rule.
 * expert_cache_resize is supported under GLOBAL only.
 */
enum {
  MOE_CACHE_GLOBAL = 0,
  MOE_CACHE_PER_LAYER = 1,
  MOE_CACHE_STATIC = 2
};

/*
 * Expert weight format (moe_config.weight_format).  MXFP4: E2M1 codes with
 * one E8M0 scale per 32 along K, DeepSeek-V4-Flash's format on the pages.
 * BF16: plain bf16 matrices, the format the pages run their 35B-A3B model
 * in (jansverre.net FreeToken article, section "Hvor raskt kjører
 * modellene?").  BF16 experts run the decode path for up to 16 tokens per
 * call: moe_create requires max_tokens <= 16 and max_prefill_tokens = 0
 * with them (else UNSUPPORTED).
 */
enum {
  MOE_WEIGHTS_MXFP4 = 0,
  MOE_WEIGHTS_BF16 = 1
};

/* Layer-stack shape and capacities, fixed at moe_create. */
typedef struct moe_config {
  int32_t hidden;          /* H: multiple of 128, 128..6144                  */
  int32_t inter;           /* I: expert intermediate size, multiple of 128,
                              128..6144                                      */
  int32_t n_experts;       /* E: routed experts, top_k <= E <= 1024          */
  int32_t top_k;           /* k: 1..16                                       */
  int32_t n_layers;        /* L >= 1                                         */
  int32_t has_shared;      /* 1: each layer has one always-on shared expert  */
  int32_t renormalize;     /* 1: top-k gates renormalised to sum to 1        */
  int32_t max_tokens;      /* T_max of moe_layer_forward, 1..64              */
  int32_t cache_slots;     /* C: HBM LRU slots, 0..min(n_layers*n_experts,
                              4096)                                          */
  int32_t staging_slots;   /* S: HBM slots for misses that bypass the cache  */
  int32_t max_prefill_tokens; /* 0 disables moe_prefill_forward; at most
                              what keeps T*H*2 and T*(k+1)*I*2 bytes (and
                              the prefill h records) below 2 GiB (else
                              UNSUPPORTED)                                  */
  int32_t cache_policy;    /* MOE_CACHE_GLOBAL (0), _PER_LAYER or _STATIC  */
  int32_t weight_format;   /* MOE_WEIGHTS_MXFP4 (0) or MOE_WEIGHTS_BF16     */
} moe_config;

/* Counters since creation or the last moe_reset_stats. */
typedef struct moe_stats {
  uint64_t forward_calls;   /* moe_layer_forward calls with T > 0           */
  uint64_t lookups;         /* unique (layer, expert) keys looked up         */
  uint64_t hits;            /* keys found resident                           */
  uint64_t fills;           /* keys inserted (host-to-device copies)         */
  uint64_t bypasses;        /* keys served from staging, state unchanged     */
  uint64_t evictions;       /* resident keys displaced by fills or resizes   */
  uint64_t bytes_h2d;       /* expert bytes copied from the host pool        */
  uint64_t bytes_d2d;       /* expert bytes moved by resizes                 */
  uint64_t resizes;         /* expert_cache_resize calls                     */
  uint64_t prefill_layers;  /* layers run by moe_prefill_forward             */
} moe_stats;

/* Message for the last error on this thread ("" if none).  Never NULL. */
const char* moe_last_error(void);

/* Number of bytes of one expert in the MXFP4 layout: 3*H*I*17/32. */
size_t moe_expert_bytes(int32_t hidden, int32_t inter);

/*
 * Create a context on the current HIP device: allocates the pinned host
 * expert pool (n_layers * n_experts expert records), the HBM router
 * matrices, shared experts, cache slots, staging slots and scratch, and
 * the device-resident cache state (all slots empty, clock 0).
 * Errors: INVALID_ARG (NULL or field out of range), UNSUPPORTED (H or I not
 * a multiple of 128 or above 6144, cache_slots above 4096), OOM, HIP.  *out
 * is set only on success.
 */
moe_status moe_create(const moe_config* cfg, moe_ctx** out);

/* (sync) Wait for the context's work, free everything.  NULL is a no-op. */
moe_status moe_destroy(moe_ctx* ctx);

/*
 * (sync) Set one layer's router matrix W_r, fp32 [H][E] row-major (E
 * contiguous).  Copied to HBM.  Errors: INVALID_ARG, HIP.
 */
moe_status moe_set_router(moe_ctx* ctx, int32_t layer, const float* h_router);

/*
 * (sync) Set one expert's MXFP4 weights from the canonical layout:
 *   h_qg [I][H/2], h_qu [I][H/2], h_qd [H][I/2]: E2M1 codes, rows are output
 *     features, K contiguous, element 2i in the low nibble of byte i;
 *   h_sg [I][H/32], h_su [I][H/32], h_sd [H][I/32]: E8M0 scale bytes, one per
 *     32 consecutive K elements of a row (value 2^(s-127)).
 * The FFN is W_d (silu(W_g x) * (W_u x)).  expert in [0, E) writes the
 * record into the pinned host pool (an existing cached copy is NOT
 * refreshed: set weights before the first forward); expert = -1 sets the
 * layer's shared expert, held in HBM.  The library repacks into its own
 * MFMA-tiled layout.  With weight_format = MOE_WEIGHTS_BF16 the three
 * matrices are bf16 instead: h_qg and h_qu [I][H], h_qd [H][I] (2 bytes per
 * element, same row order), and h_sg, h_su, h_sd must be NULL.  Errors:
 * INVALID_ARG (NULL, bad index, scale byte 255 which is NaN, scale pointers
 * given with bf16 weights), STATE (expert = -1 without has_shared), HIP.
 */
moe_status moe_set_expert(moe_ctx* ctx, int32_t layer, int32_t expert,
                          const uint8_t* h_qg, const uint8_t* h_qu,
                          const uint8_t* h_qd, const uint8_t* h_sg,
                          const uint8_t* h_su, const uint8_t* h_sd);

/*
 * (sync) Set a whole layer: router plus all E routed experts plus the shared
 * expert.  h_q holds E consecutive records of [qg | qu | qd] (3*H*I/2
 * bytes each) and h_s E consecutive records of [sg | su | sd] (3*H*I/32
 * bytes each), each part laid out as in moe_set_expert; h_shared_q /
 * h_shared_s hold one such record, or are NULL when has_shared is 0.  With
 * bf16 weights a record of h_q is [wg | wu | wd] (3*H*I*2 bytes) and h_s
 * and h_shared_s are NULL.
 */
moe_status moe_set_layer(moe_ctx* ctx, int32_t layer, const float* h_router,
                         const uint8_t* h_q, const uint8_t* h_s,
                         const uint8_t* h_shared_q, const uint8_t* h_shared_s);

/*
 * Decode forward of one layer for T tokens (0 <= T <= max_tokens):
 *   logits l = fp32(x W_r + bias) accumulated in fp64; top-k ids ordered by
 *   (logit descending, expert ascending); gates = softmax over the chosen
 *   logits (renormalize = 1) or the full-softmax probabilities of the chosen
 *   experts (renormalize = 0); pairs (t, j) permuted stably by expert;
 *   the unique experts looked up in the LRU cache (hits stamped in
 *   ascending expert order, then misses take the empty slots in ascending
 *   index and then the least recently used slots not hit in this call, among
 *   the slots the cache policy lets this layer fill; misses beyond those
 *   bypass through staging slots without changing the state),
 *   misses copied from the pinned pool by a device kernel; the SwiGLU FFN of
 *   every (token, expert) pair on MXFP4 weights dequantised to bf16 inside
 *   the MFMA loads, fp32 accumulation, h carried between the two matrices as
 *   bf16 plus a second bf16 plane of its remainder (about 16 significant
 *   bits), expert outputs in fp32;
 *   y[t] = sum_j g[t,j] o[t,j] (+ shared expert output), fp32, rounded to
 *   bf16 (nearest, ties to even).  Nothing is synchronised with the host.
 * d_x: bf16 [T][H].  d_bias: fp32 [T][E] or NULL.  d_y: bf16 [T][H].
 * d_y32: fp32 [T][H] or NULL; when given it also receives y before the bf16
 * rounding.  d_ids (int32 [T][k]) and d_gates (fp32 [T][k]) receive the
 * routing when not NULL.  Errors: INVALID_ARG (T out of range, NULL x/y, bad layer), STATE
 * (router not set), CAPACITY (staging_slots cannot cover the worst-case
 * bypass count max(0, min(T*k, E) - C'), C' the slots this layer may fill:
 * C, its share under PER_LAYER, 0 under STATIC), HIP.
 */
moe_status moe_layer_forward(moe_ctx* ctx, int32_t layer, const void* d_x,
                             int32_t T, const float* d_bias, void* d_y,
                             float* d_y32, int32_t* d_ids, float* d_gates,
                             void* stream);

/*
 * Prefill forward of layers 0..n_layers-1 for T tokens each
 * (0 < T <= max_prefill_tokens).  Layer l's experts are uploaded whole from
 * the pinned pool into one of two HBM layer buffers on an internal copy
 * stream; the upload of layer l+1 overlaps the compute of layer l and waits
 * for layer l-1 (the previous reader of that buffer).  Expert FFNs run as
 * grouped MFMA GEMMs.  The cache state is not used or changed.  Math as in
 * moe_layer_forward, except that h's remainder travels as fp6 (E2M3) with one
 * power-of-two scale per 32 values, which keeps h to about 2^-14 of each
 * block's largest value.  h_x, h_bias, h_y are host arrays of n_layers device
 * pointers (bf16 [T][H] in, fp32 [T][E] bias or NULL entries / NULL array,
 * bf16 [T][H] out, and optionally fp32 [T][H] pre-rounding outputs in h_y32,
 * a NULL array or NULL entries when not wanted).  Errors: INVALID_ARG, STATE
 * (prefill disabled or router not set), HIP.
 */
moe_status moe_prefill_forward(moe_ctx* ctx, int32_t n_layers,
                               const void* const* h_x, int32_t T,
                               const float* const* h_bias, void* const* h_y,
                               float* const* h_y32, void* stream);

/*
 * Look up n unique experts (ascending, in [0, E)) of one layer in the cache
 * with the moe_layer_forward rule and fill the misses.  d_experts: int32
 * [>= *d_n]; d_n: int32 on the device, 0 <= *d_n <= min(E, max_tokens*k)
 * (larger values are clamped); d_slot: int32 [*d_n] receives the slot
 * (>= 0) or -1-b for staging slot b.  Errors: INVALID_ARG, CAPACITY
 * (staging_slots below the worst-case bypass count, as for
 * moe_layer_forward), HIP.
 */
moe_status expert_cache_lookup(moe_ctx* ctx, int32_t layer,
                               const int32_t* d_experts, const int32_t* d_n,
                               int32_t* d_slot, void* stream);

/*
 * Preload experts of one layer: the same rule as a lookup of h_experts
 * (ascending unique, 0 <= n <= min(E, max_tokens*k)), without compute.  It
 * inserts under every policy (it is how the STATIC set is placed).
 * Errors: INVALID_ARG (unsorted, duplicate or out-of-range ids), CAPACITY
 * (bypass would exceed staging_slots), HIP.
 */
moe_status expert_cache_fill(moe_ctx* ctx, int32_t layer,
                             const int32_t* h_experts, int32_t n,
                             void* stream);

/*
 * (sync) Resize the cache to new_slots (0 <= new_slots <= L*E) without
 * touching the host pool.  Growing appends empty slots.  Shrinking evicts
 * occupied slots in ascending recency while more than new_slots are
 * occupied, moves the survivors held in slots >= new_slots (ascending) into
 * the lowest empty slots < new_slots (ascending) keeping their recency,
 * then releases the tail of the slot memory.  Errors: INVALID_ARG,
 * UNSUPPORTED (above 4096 slots, or a policy other than GLOBAL), OOM, HIP.
 */
moe_status expert_cache_resize(moe_ctx* ctx, int32_t new_slots, void* stream);

/*
 * (sync) Copy the cache state to the host: *h_slots = C always; when
 * capacity >= C also h_key[C] (layer*E + expert, -1 empty), h_stamp[C]
 * (recency number, 0 empty) and *h_clock.  Errors: INVALID_ARG, CAPACITY
 * (capacity < C; *h_slots still written), HIP.
 */
moe_status expert_cache_snapshot(moe_ctx* ctx, int32_t capacity,
                                 int32_t* h_key, uint64_t* h_stamp,
                                 uint64_t* h_clock, int32_t* h_slots);

/*
 * (sync) Copy the dispatch of the last moe_layer_forward to the host, for
 * inspection: h_counts [E], h_offsets [E+1], h_sorted [T*k] (pair f = t*k+j
 * at each permuted position), h_inv [T*k], h_unique [E] (ascending experts
 * used; *h_n_unique of them), h_slot [E] (slot code per unique expert, as in
 * expert_cache_lookup).  Any pointer may be NULL.  *h_T receives T.
 */
moe_status moe_inspect_dispatch(moe_ctx* ctx, int32_t* h_T, int32_t* h_counts,
                                int32_t* h_offsets, int32_t* h_sorted,
                                int32_t* h_inv, int32_t* h_unique,
                                int32_t* h_n_unique, int32_t* h_slot);

/*
 * (sync) Copy the routing of the last layer run by moe_prefill_forward:
 * h_ids int32 [T][k], h_gates fp32 [T][k] (either may be NULL); *h_T
 * receives that call's T (0 if none ran).
 */
moe_status moe_inspect_prefill(moe_ctx* ctx, int32_t* h_T, int32_t* h_ids, float* h_gates);

/* (sync) Read / clear the counters. */
moe_status moe_get_stats(moe_ctx* ctx, moe_stats* out);
moe_status moe_reset_stats(moe_ctx* ctx);

/*
 * Kernel timing for measurement: when enabled, moe_layer_forward records HIP
 * events on the caller's stream around its expert FFN kernels and
 * moe_prefill_forward around each layer's grouped GEMMs (up to 65536
 * records, then recording stops).  moe_get_timing (sync) returns the number
 * of records and the summed milliseconds for each of the two paths, and
 * clears them.
 */
moe_status moe_set_timing(moe_ctx* ctx, int32_t enable);
moe_status moe_get_timing(moe_ctx* ctx, int32_t* h_n_decode, double* h_ms_decode,
                          int32_t* h_n_prefill, double* h_ms_prefill);

/*
 * (sync) As moe_get_timing, split per kernel: each record holds an event
 * before the gate/up kernel, one between it and the down kernel and one
 * after the down kernel.  h_n[2] = {decode records, prefill layer records};
 * h_ms[6] = {decode total, decode gate/up, decode down, prefill total,
 * prefill gate/up, prefill down}, summed milliseconds.  Clears the records.
 * Errors: INVALID_ARG (NULL context or arrays), HIP.
 */
moe_status moe_get_timing_split(moe_ctx* ctx, int32_t* h_n, double* h_ms);

/*
 * Bandwidth probe: copy n_bytes (multiple of 16) from d_src to d_dst with a
 * plain streaming copy kernel on the stream.  d_src may be device memory or
 * pinned host memory mapped for the device.  Used to calibrate traffic
 * counters and to measure HBM and PCIe rates.  Errors: INVALID_ARG, HIP.
 */
moe_status moe_probe_copy(const void* d_src, void* d_dst, size_t n_bytes,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
