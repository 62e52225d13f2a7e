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
 * modellene?").  NVFP4: E2M1 codes with one E4M3 scale per 16 along K and
 * one fp32 scale per matrix, the format the pages run the 35B-A3B model in
 * on a laptop GPU (same section); NVIDIA's definition, which the pages do
 * not spell out.  Decode runs every format through the expert-streaming
 * kernels; prefill runs grouped GEMMs in every format, carrying h between
 * them as two bf16 planes for BF16 and NVFP4 experts (the MXFP8 prefill
 * mode is MXFP4 only).  BF16 experts above 16 tokens per decode call need
 * H and I <= 4096 (else UNSUPPORTED).
 */
enum {
  MOE_WEIGHTS_MXFP4 = 0,
  MOE_WEIGHTS_BF16 = 1,
  MOE_WEIGHTS_NVFP4 = 2
};

/*
 * Arithmetic of the prefill expert GEMMs (moe_config.prefill_format).
 * BF16 (default): bf16 activations, weights dequantised exactly to bf16,
 * fp32 accumulation, h carried as bf16 plus an fp6 remainder (about 2^-14 of
 * each 32-block's largest value): the plain layer to within 4e-3 x rms.
 * MXFP8 (opt-in, this build's native-MX mode): the activations of both
 * products (x for gate/up, h for down) are block-quantised to MXFP8 (E4M3
 * elements, one E8M0 scale 2^e per 32 along K with e = floor(log2 amax) - 8,
 * elements rounded to nearest even and clamped to +-448: the OCP MX v1.0
 * rule) and multiplied with the MXFP4 weights as stored on the scaled
 * FP8 x FP4 matrix instructions.  It computes the layer on those quantised
 * activations (the router still sees the bf16 x): about 5.5% relative rms
 * and up to about 0.55 x rms max-abs from the plain layer on N(0,1)
 * activations (two E4M3 roundings), at half the matrix-instruction cost and
 * half the activation bytes of the bf16 mode.  h is quantised from the
 * kernel's fp32 values, so an element within rounding error of an E4M3
 * midpoint (or a block whose amax is within rounding error of a power of
 * two) may round either way; moe_inspect_prefill_mx exposes the decisions
 * taken.  The pages run
 * MXFP4 experts (jansverre.net FreeToken article, section "Hvor raskt
 * kjører modellene?"); quantised activations are this build's reading.
 */
enum {
  MOE_PREFILL_BF16 = 0,
  MOE_PREFILL_MXFP8 = 1
};

/*
 * Layer-stack shape and capacities, fixed at moe_create.  The shapes the
 * pages name: many experts with few active per token (DeepSeek-V4-Flash: 6
 * of 256) and an optional always-on shared expert (aiforradalom.hu article,
 * section "A Mixture-of-Experts (MoE) kihívásai és a FreeToken
 * megoldásai").  H and I must be multiples of 128: the weights are tiled in
 * 16-row x 128-K atoms (four MX blocks of 32 per lane of a wave, the operand
 * the MFMA and the one-load-per-lane streaming are built around); every
 * shape the pages name has such sizes.
 */
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
  int32_t weight_format;   /* MOE_WEIGHTS_MXFP4 (0), _BF16 or _NVFP4       */
  int32_t prefill_format;  /* MOE_PREFILL_BF16 (0) or MOE_PREFILL_MXFP8 (MXFP4
                              weights only); moe_set_prefill_format changes it */
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
  uint64_t bytes_d2d;       /* expert bytes copied by resizes (moved records) */
  uint64_t resizes;         /* expert_cache_resize calls                     */
  uint64_t prefill_layers;  /* layers run by moe_prefill_forward             */
  uint64_t prefetch_lookups; /* keys named by prefetches (moe_set_prefetch)  */
  uint64_t prefetch_hits;   /* of those, keys already resident               */
  uint64_t prefetch_fills;  /* keys a prefetch inserted (copies; also in
                               bytes_h2d)                                    */
} moe_stats;

/* Message for the last error on this thread ("" if none).  Never NULL. */
const char* moe_last_error(void);

/* Number of bytes of one expert in the MXFP4 layout: 3*H*I*17/32. */
size_t moe_expert_bytes(int32_t hidden, int32_t inter);

/*
 * Create a context on the current HIP device: allocates the pinned host
 * expert pool (n_layers * n_experts expert records; the experts live in host
 * memory and come to the GPU on demand: aiforradalom.hu article, section "A
 * Mixture-of-Experts (MoE) kihívásai és a FreeToken megoldásai"), the HBM
 * router matrices, shared experts, cache slots, staging slots and scratch,
 * and the device-resident cache state (all slots empty, clock 0).
 * Errors: INVALID_ARG (NULL or field out of range), UNSUPPORTED (H or I not
 * a multiple of 128 or above 6144, cache_slots above 4096), OOM, HIP.  *out
 * is set only on success.
 */
moe_status moe_create(const moe_config* cfg, moe_ctx** out);

/* (sync) Wait for the context's work, free everything.  NULL is a no-op. */
moe_status moe_destroy(moe_ctx* ctx);

/*
 * (sync) Set one layer's router matrix W_r, fp32 [H][E] row-major (E
 * contiguous).  Copied to HBM.  Offloading leaves the router unchanged
 * (jansverre.net FreeToken article, section "Hva er FreeToken?"), so it is
 * always resident.  Errors: INVALID_ARG, HIP.
 */
moe_status moe_set_router(moe_ctx* ctx, int32_t layer, const float* h_router);

/*
 * (sync) Set one expert's weights (MXFP4 for DeepSeek-V4-Flash on the pages:
 * jansverre.net FreeToken article, section "Hvor raskt kjører modellene?";
 * the element and scale encodings are OCP MX v1.0's) from the canonical
 * layout:
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
 * element, same row order), and h_sg, h_su, h_sd must be NULL.  With
 * MOE_WEIGHTS_NVFP4 the codes are as for MXFP4 and each scale array holds
 * its matrix's E4M3 block scales, one byte per 16 consecutive K elements of
 * a row ([I][H/16] or [H][I/16]), followed by the matrix's fp32 scale (4
 * bytes, little-endian): an element's value is e2m1 x e4m3 x that scale.
 * Errors: INVALID_ARG (NULL, bad index, E8M0 scale byte 255 which is NaN;
 * E4M3 block scale negative or NaN, or a matrix scale not finite; scale
 * pointers given with bf16 weights), STATE (expert = -1 without
 * has_shared), HIP.
 */
moe_status moe_set_expert(moe_ctx* ctx, int32_t layer, int32_t expert,
                          const uint8_t* h_qg, const uint8_t* h_qu,
                          const uint8_t* h_qd, const uint8_t* h_sg,
                          const uint8_t* h_su, const uint8_t* h_sd);

/*
 * (sync) Set a whole layer, loaded once into the host pool (the pages load
 * the model into host memory and stream experts from there: aiforradalom.hu
 * article, section "A Mixture-of-Experts (MoE) kihívásai és a FreeToken
 * megoldásai"): router plus all E routed experts plus the shared expert.  h_q holds E consecutive records of [qg | qu | qd] (3*H*I/2
 * bytes each) and h_s E consecutive records of [sg | su | sd] (3*H*I/32
 * bytes each), each part laid out as in moe_set_expert; h_shared_q /
 * h_shared_s hold one such record, or are NULL when has_shared is 0.  With
 * bf16 weights a record of h_q is [wg | wu | wd] (3*H*I*2 bytes) and h_s
 * and h_shared_s are NULL.  With NVFP4 weights a record of h_s is the three
 * scale arrays of moe_set_expert back to back (3*(H*I/16 + 4) bytes).
 */
moe_status moe_set_layer(moe_ctx* ctx, int32_t layer, const float* h_router,
                         const uint8_t* h_q, const uint8_t* h_s,
                         const uint8_t* h_shared_q, const uint8_t* h_shared_s);

/*
 * Decode forward of one layer for T tokens (0 <= T <= max_tokens).  The
 * pages' decode path: only the experts a token activates are needed, they
 * are served from one global LRU cache across the MoE layers and fetched
 * from host memory on a miss (jansverre.net FreeToken article, section
 * "Hvorfor er båndbredden viktigere enn antall kjerner?"), with no
 * approximation: the router is unchanged and the experts' partial results
 * are summed at the end (same article, section "Hva er FreeToken?").
 * Computed:
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
 * When one expert record is at least 4 MiB (its copy takes hundreds of
 * microseconds), the resident experts and the shared expert are computed on
 * the context's internal stream while the copies run on `stream`, and the
 * copied experts are computed on `stream` once their copies have landed;
 * the internal stream is joined back into `stream` before them, so work
 * queued on `stream` afterwards sees the call complete.  Outputs and cache state are
 * the same either way (not under stream capture, where the call stays on
 * `stream`).
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
 * Execution order of moe_layer_forward's copies (an execution knob: outputs
 * and cache state do not depend on it).  mode -1 (the default): copies run
 * beside the resident experts' kernels when one expert record is at least
 * 4 MiB; 0: never (fills, then every expert, all on the caller's stream);
 * 1: always.  The pages stream experts in while the GPU computes (aipolix.com
 * FreeToken article, fourth paragraph); this applies it within a decode
 * layer.  Errors: INVALID_ARG (mode outside -1..1).
 */
moe_status moe_set_copy_overlap(moe_ctx* ctx, int32_t mode);

/*
 * Cross-layer miss prefetch: arm a request that the next decode call
 * (moe_layer_forward or moe_layer_forward_noalloc with T >= 1, of any layer)
 * carries out, typically for the layer after that call's.  The pages carry
 * the next layer's upload under the current layer's compute in prefill
 * (aipolix.com FreeToken article, fourth paragraph) and name preloading of
 * experts that activation patterns make likely as one of the engine's
 * techniques, without a rule or a predictor (world.tibi.club FreeToken
 * article, section "Cum reușește FreeToken să ruleze 753B pe un singur
 * GPU?", third item).  The predictor is the caller's: the request names n
 * experts of `layer`, d_experts[0..n) (device int32, ascending and unique;
 * read when the call runs, so a kernel queued before the call may write it;
 * from the first entry that is not above its predecessor, or out of range,
 * on, entries are ignored).  Once the call's own copies are done it looks
 * them up with the lookup rule except that a miss may take only an empty
 * slot (ascending) or a slot whose stamp is at most the clock before the
 * call's own lookup (ascending stamp) -- never one the call uses -- and a
 * miss with no such slot is skipped (no staging copy); hits are stamped and
 * the clock advances as in a lookup.  The misses it inserts are copied from
 * the pool on an internal stream, beside the call's expert kernels and on
 * into the next call, and are hits for later lookups: the next decode call
 * (its routing runs meanwhile), expert_cache_lookup and expert_cache_fill
 * wait for those copies on their stream, the calls that synchronize the
 * device do, and a call under stream capture fails with STATE while they
 * run (synchronize before capturing).  Under capture a request is carried
 * out in order on the capturing stream.  Outputs never depend on it.  Counted in moe_stats' prefetch_* fields (its evictions in
 * evictions).  n = 0 disarms.  A request not yet carried out is replaced by
 * the next moe_set_prefetch.  Errors: INVALID_ARG (layer out of range, n
 * outside [0, n_experts], NULL list with n > 0), UNSUPPORTED (cache policy
 * other than GLOBAL), STATE (after a failed copy).
 */
moe_status moe_set_prefetch(moe_ctx* ctx, int32_t layer, const int32_t* d_experts, int32_t n);

/*
 * moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, arithmetic and cache behaviour; the
 * per-call device scratch (logits, routing, dispatch, work and fill lists,
 * h, fp32 expert outputs) lives in a fixed 16 MiB device array of the
 * library instead of the context's own buffer, and the call allocates
 * nothing (no hipMalloc, no event creation; kernel timing is not
 * recorded).  Each
 * GPU holds one such array for the life of the process, resolved at
 * moe_create, and every call on that GPU shares it, so calls that overlap
 * on one GPU (from any context or stream) race; nothing in it needs to
 * start at zero.  Errors: as moe_layer_forward, and CAPACITY when the call
 * needs more scratch than the array holds (about 2*T*(k+1)*(H+I) bytes plus
 * T*E*4; T=32 tokens at H=4096, I=2048, top-6 with a shared expert need
 * 5.5 MiB).
 */
moe_status moe_layer_forward_noalloc(moe_ctx* ctx, int32_t layer, const void* d_x,
                                     int32_t T, const float* d_bias, void* d_y,
                                     float* d_y32, int32_t* d_ids, float* d_gates,
                                     void* stream);

/*
 * Prefill forward of layers 0..n_layers-1 for T tokens each
 * (0 < T <= max_prefill_tokens): the pages stream the next layer's experts
 * over PCIe while the GPU computes the current layer (aipolix.com FreeToken
 * article, fourth paragraph; jansverre.net article, section "Hvorfor er
 * båndbredden viktigere enn antall kjerner?").  Layer l's experts are uploaded whole from
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
 * (sync) Switch the arithmetic of later moe_prefill_forward calls
 * (MOE_PREFILL_BF16 or MOE_PREFILL_MXFP8).  Errors: INVALID_ARG (unknown
 * format), UNSUPPORTED (MXFP8 with bf16 experts).
 */
moe_status moe_set_prefill_format(moe_ctx* ctx, int32_t format);

/*
 * Look up n unique experts (ascending, in [0, E)) of one layer in the cache
 * with the moe_layer_forward rule and fill the misses: the cache step of the
 * decode path on its own, for custom pipelines (one global LRU across
 * layers, misses fetched from the host pool on demand: jansverre.net
 * FreeToken article, section "Hvorfor er båndbredden viktigere enn antall
 * kjerner?").  d_experts: int32 [>= *d_n]; d_n: int32 on the device,
 * 0 <= *d_n <= min(E, max_tokens*k) (larger values are clamped); d_slot:
 * int32 [*d_n] receives the slot (>= 0) or -1-b for staging slot b.  The
 * list is read on the device, so it is checked there: an entry outside
 * [0, E), and every entry from the first one that is not above its
 * predecessor on, receives INT_MIN and changes no state.  Errors:
 * INVALID_ARG, CAPACITY (staging_slots below the worst-case bypass count,
 * as for moe_layer_forward), HIP.
 */
moe_status expert_cache_lookup(moe_ctx* ctx, int32_t layer,
                               const int32_t* d_experts, const int32_t* d_n,
                               int32_t* d_slot, void* stream);

/*
 * Preload experts of one layer (placing a set beforehand, the placement the
 * pages compare their LRU against: jansverre.net FreeToken article, section
 * "Hvorfor er båndbredden viktigere enn antall kjerner?"): the same rule as
 * a lookup of h_experts
 * (ascending unique, 0 <= n <= min(E, max_tokens*k)), without compute.  It
 * inserts under every policy (it is how the STATIC set is placed).
 * Errors: INVALID_ARG (unsorted, duplicate or out-of-range ids), CAPACITY
 * (bypass would exceed staging_slots), HIP.
 */
moe_status expert_cache_fill(moe_ctx* ctx, int32_t layer,
                             const int32_t* h_experts, int32_t n,
                             void* stream);

/*
 * (sync) Resize the cache to new_slots (0 <= new_slots <= min(L*E, 4096))
 * without touching the host pool or restarting: the GPU expert-cache budget
 * changes at run time (aipolix.com FreeToken article, sixth paragraph).
 * Growing maps memory for the new, empty slots.  Shrinking evicts occupied
 * slots in ascending recency while more than new_slots are occupied, moves
 * the survivors held in slots >= new_slots (ascending) into the lowest empty
 * slots < new_slots (ascending) keeping their recency, and releases the slot
 * memory past the new capacity.  Only the moved records are copied (at most
 * new_slots of them; moe_stats.bytes_d2d counts their bytes).  The slots live
 * in one reserved device address range backed by chunks of 64 MiB to 1 GiB,
 * so up to one chunk past the last slot stays mapped.  Errors: INVALID_ARG,
 * UNSUPPORTED (a policy other than GLOBAL), OOM (growing: the state is
 * unchanged), HIP (when a copy or upload fails after records were moved the
 * cache is left empty, which is consistent because outputs never depend on
 * the cache).
 */
moe_status expert_cache_resize(moe_ctx* ctx, int32_t new_slots, void* stream);

/*
 * (sync) Empty the expert cache: every slot empty, every (layer, expert)
 * absent (map, keys, stamps and recency order); the clock and the counters
 * are kept, the host pool and the slot memory are untouched.  A cold
 * restart of the cache without recreating the context or reloading the
 * pool: the way back after a failed copy (see moe_set_debug), and usable at
 * any time.  The pages list early failure reports of the engine, a prefill
 * that hung on a cold server's first request and a request left queued
 * without an error (jansverre.net FreeToken article, section "Hva betyr
 * dette for en vanlig RTX 4090?"); failing loudly and recovering the cache
 * in place is this build's answer.  Errors: HIP.
 */
moe_status expert_cache_reset(moe_ctx* ctx);

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
 * (sync) Copy the routing and dispatch of one layer of the last
 * moe_prefill_forward call: h_ids int32 [T][k], h_gates fp32 [T][k],
 * h_counts [E], h_offsets [E+1] (h_offsets[E] = T*k), h_sorted [T*k] (pair
 * f = t*k+j at each permuted position, stable by f within an expert), h_inv
 * [T*k].  Any of them may be NULL.  *h_T receives that call's T (0 if none
 * ran; nothing else is written then).  Errors: INVALID_ARG (NULL h_T, layer
 * outside [0, n_layers of that call)), HIP.
 */
moe_status moe_inspect_prefill(moe_ctx* ctx, int32_t layer, int32_t* h_T, int32_t* h_ids,
                               float* h_gates, int32_t* h_counts, int32_t* h_offsets,
                               int32_t* h_sorted, int32_t* h_inv);

/*
 * (sync) Copy the block-quantised operands of the LAST layer of the last
 * moe_prefill_forward call, when that call ran in the MXFP8 mode: h_xq
 * uint8 [T][H] (E4M3 codes of x), h_xs uint8 [T][H/32] (their E8M0 scale
 * bytes, exponent + 127), h_hq uint8 [R][I] (E4M3 codes of h = silu(gate) *
 * up) and h_hs uint8 [R][I/32] (their scale bytes), R = T*k, plus T with a
 * shared expert.  Row r < T*k of h belongs to pair sorted[r] of that layer
 * (moe_inspect_prefill); row T*k + t is token t's shared-expert row.  These
 * are the quantisation decisions the mode takes (OCP MX rule: the block
 * exponent floor(log2 amax) - 8, elements rounded to nearest even and
 * clamped to +-448), exposed so that a caller can check them.  Any array
 * may be NULL.  *h_T receives T (0 if no prefill ran; nothing else is
 * written then).  Errors: INVALID_ARG (NULL h_T), UNSUPPORTED (the last
 * call ran in the bf16 mode), HIP.
 */
moe_status moe_inspect_prefill_mx(moe_ctx* ctx, int32_t* h_T, uint8_t* h_xq, uint8_t* h_xs,
                                  uint8_t* h_hq, uint8_t* h_hs);

/* (sync) Read / clear the counters. */
moe_status moe_get_stats(moe_ctx* ctx, moe_stats* out);
moe_status moe_reset_stats(moe_ctx* ctx);

/*
 * Debug switches (host-initiated; no GPU fault is involved), so that a
 * failing step is reported rather than left silent (the failure reports
 * cited at expert_cache_reset).
 * MOE_DEBUG_SYNC: every stage of moe_layer_forward (router, finalize, fill,
 *   gate/up, down, combine; both parts of a split call) and every layer of
 *   moe_prefill_forward is followed by a synchronisation of the streams it
 *   used and an error check, so that a failing stage is named in the error
 *   message; results and cache state are bit-identical to an unsynchronised
 *   run (not under stream capture, where nothing is synchronised).
 * MOE_DEBUG_FAIL_NEXT_FILL: the next copy step (of moe_layer_forward,
 *   expert_cache_lookup or expert_cache_fill) issues no copies and fails
 *   with MOE_ERR_HIP, as a failed copy would, after the lookup has stamped
 *   and inserted this call's misses.  The flag clears itself.
 * After any failed copy, injected or real, slots may name experts whose
 * bytes did not land: moe_layer_forward, moe_layer_forward_noalloc and the
 * expert_cache_lookup / fill / resize calls return MOE_ERR_STATE until
 * expert_cache_reset.  expert_cache_snapshot still reads the state.
 * Errors: INVALID_ARG (unknown flag).
 */
enum {
  MOE_DEBUG_SYNC = 1,
  MOE_DEBUG_FAIL_NEXT_FILL = 2
};
moe_status moe_set_debug(moe_ctx* ctx, int32_t flags);

/*
 * Kernel timing for measurement.  When enabled, every kernel of
 * moe_layer_forward and every stage of moe_prefill_forward is launched with
 * a start and a stop event recorded by its own dispatch, so that an
 * interval is the kernel's duration (up to 65536 calls or layers are
 * recorded, then recording stops).  moe_get_timing (sync) returns the
 * number of records and the summed milliseconds per kernel, and clears
 * them.  Decode kernels: router, finalize (top-k, dispatch, cache lookup,
 * work list), fill (copies from the pinned pool), gate/up + SwiGLU, down,
 * combine.  A call that ran its copies beside the resident experts' kernels
 * (see moe_layer_forward) launches gate/up and down twice; both launches
 * count to gate/up and down, and n_decode_split counts such calls.  A
 * kernel's time is its stop minus the later of its start and the stops of
 * the kernels it waits for.  Prefill stages, per layer: routing (router
 * start to dispatch end), gate/up GEMM, down GEMM, combine.
 */
typedef struct moe_timing {
  int32_t n_decode;        /* moe_layer_forward calls recorded              */
  int32_t n_prefill;       /* prefill layers recorded                        */
  int32_t n_decode_split;  /* of n_decode, calls with two gate/up and down
                              launches                                       */
  int32_t reserved;
  double decode_ms[6];     /* router, finalize, fill, gate/up, down, combine */
  double prefill_ms[4];    /* routing, gate/up GEMM, down GEMM, combine      */
} moe_timing;

moe_status moe_set_timing(moe_ctx* ctx, int32_t enable);
moe_status moe_get_timing(moe_ctx* ctx, moe_timing* out);

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
