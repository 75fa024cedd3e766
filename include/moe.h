/*
 * moe.h — C ABI of the MI355X (gfx950) MoE decode library (libmoe.so).
 *
 * The method: the DeepSeek-V4.1-Flash MoE layer at decode as described on
 * the spark_model documentation pages [moe_v41.rs, module doc]:
 *   router   logits = bf16 x . bf16 gate weight, f32 accumulation;
 *            score = sqrt(softplus(logit / temp)); the top-k by
 *            score + correction bias; weights = the unbiased scores of the
 *            picks, renormalised and scaled by route_scale
 *            [moe_v41.rs, fn softplus, fn route_from_logits];
 *   experts  each pick: gate/up GEMVs on raw Q2_K blocks against the q8_1
 *            input, a clamped SwiGLU, q8_1 again, a down GEMV on raw Q3_K
 *            blocks [moe_v41.rs, module doc; Kernels];
 *   combine  a weighted sum of the expert outputs plus the resident bf16
 *            shared expert [moe_v41.rs, module doc; fn shared_side].
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The
 *     library allocates no memory on these paths and keeps no state between
 *     calls beyond what the caller's workspace holds, with two exceptions:
 *     the glibc score mode's registered table (moe_set_score_table), and
 *     the prefill of a layer with a bf16 shared expert (moe_layer_forward
 *     and moe_stack_forward at m > 8), which creates, on its first use on a
 *     device, one non-blocking stream and two events of the library's own,
 *     kept until the process ends: the shared expert's GEMMs run there,
 *     forked from and joined back into `stream` by event record/wait pairs
 *     before the call's last launch, so to the caller all of it is ordered
 *     on `stream` (a graph capture of `stream` takes it in). That enqueue
 *     holds a per-device lock. Every other call runs on `stream` alone.
 *   - bf16 and fp16 values are passed as their uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work and returns; nothing synchronises. Errors found on
 *     the device (non-finite ranking keys, invalid picks) are reported in the
 *     header's status word and in the workspace status word, visible once
 *     the caller synchronises.
 *   - Return value: MOE_OK (0) or a negative MOE_E* code; moe_last_error()
 *     gives a thread-local message for the last failing call.
 *   - Supported shapes: n_routed <= 1024, 1 <= topk <= 8, dim and inter
 *     multiples of 256 with dim/256 and inter/256 powers of two <= 16 (the
 *     K-quant kernels give each 256-weight super-block of a row to one lane
 *     and stage whole row tiles in LDS). Anything else: MOE_EUNSUPPORTED.
 *   - Tokens per call: 1 <= m <= 65535 with m * (topk + 1) * max(dim, inter) < 2^31
 *     (the kernels index the per-pair activations with 32-bit offsets); m < 1
 *     is MOE_EINVAL, more is MOE_EUNSUPPORTED (also for the workspace calls,
 *     where moe_workspace_bytes then returns 0).
 *   - Calls that share one workspace on one stream run in order; calls that
 *     overlap on different streams must use different workspaces.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)        /* null pointer, m out of range, bad cfg value */
#define MOE_EUNSUPPORTED (-2)  /* shape outside the supported set above        */
#define MOE_EWORKSPACE (-3)    /* workspace smaller than moe_workspace_bytes   */
#define MOE_EHIP (-4)          /* a HIP launch or attribute call failed        */

/* Header status bits (word 0 of a token's header). */
#define MOE_STATUS_MISS 1        /* a pick was not resident in an expert cache (moe_cache_forward) */
#define MOE_STATUS_NAN_KEY 2     /* a ranking key score+bias was NaN (the pages' "finite scores") */
#define MOE_STATUS_BAD_PICK 4    /* moe_experts_decode: a pick outside [0,n_routed) or repeated    */

/* Layer configuration [moe_v41.rs, struct MoeV41Cfg]. max_tokens is not a
 * field: the workspace is sized per call through moe_workspace_bytes. */
typedef struct moe_cfg {
  int32_t dim;            /* model width                                   */
  int32_t inter;          /* expert hidden width                           */
  int32_t n_routed;       /* routed experts (384)                          */
  int32_t topk;           /* experts per token (6)                         */
  int32_t norm_topk_prob; /* 1: renormalise the picked scores              */
  float gate_temp;        /* logits are divided by this before softplus    */
  float route_scale;      /* weights are multiplied by this                */
  float swiglu_limit;     /* SwiGLU clamp L                                */
  int32_t score_mode;     /* MOE_SCORE_CR (0) or MOE_SCORE_GLIBC (1)       */
} moe_cfg;

/* Score modes. MOE_SCORE_CR: every step of sqrt(softplus(logit / temp)) is
 * correctly rounded to f32 (any libm that rounds correctly gives these bits).
 * MOE_SCORE_GLIBC: the scores of the host's glibc, bit for bit, as the pages'
 * host reference computes them with f32 expf / log1pf / sqrtf [device_route.rs,
 * module doc: glibc-exact softplus; moe_v41.rs, fn softplus]: the device
 * computes the correctly rounded chain and replaces it, for the inputs where
 * glibc's differs, by glibc's value from a table the host builds from its own
 * libm (moe_glibc_score_table) and registers for the device
 * (moe_set_score_table). A call with MOE_SCORE_GLIBC and no table registered
 * for the current device fails with MOE_EINVAL. */
#define MOE_SCORE_CR 0
#define MOE_SCORE_GLIBC 1

/* The resident routed experts: expert e's blocks start at base + e*stride.
 * Inside: gate (w1) and up (w3) at gate_off / up_off, Q2_K [inter rows]
 * [dim/256 super-blocks of 84 B], row-major; down (w2) at down_off, Q3_K
 * [dim rows][inter/256 super-blocks of 110 B]. The raw GGUF blocks are read
 * as they are (no repacking). base, stride and the offsets must be multiples
 * of 16 bytes [moe_v41.rs, module doc; device_route.rs, fn arena_of]. */
typedef struct moe_experts {
  const void* base;
  uint64_t stride;
  uint64_t gate_off;
  uint64_t up_off;
  uint64_t down_off;
} moe_experts;

/* One layer's resident weights [moe_v41.rs, struct MoeV41LayerWeights]:
 * gate_w bf16 [n_routed][dim]; bias f32 [n_routed] (correction bias); the
 * shared expert either as bf16 matrices (shared_kind MOE_SHARED_BF16) sh_w1
 * [inter][dim], sh_w3 [inter][dim], sh_w2 [dim][inter], or as K-quant blocks
 * (MOE_SHARED_KQUANT) in shared_q laid out like one routed expert: Q2_K gate
 * (w1) and up (w3) [inter][dim/256] at base + gate_off / up_off, Q3_K down
 * (w2) [dim][inter/256] at base + down_off (stride unused), 16-byte aligned
 * [moe_v41.rs, struct MoeV41LayerWeights: the shared matrices resident as
 * bf16 or as the GGUF's Q2_K (w1, w3) / Q3_K (w2) blocks on the routed
 * experts' kernels]. The K-quant shared expert runs exactly as one more
 * routed expert of every token with weight 1 (q8_1 of x, gate/up GEMVs,
 * clamped SwiGLU, q8_1 of h, down GEMV), and is added after the routed sum
 * like the bf16 one [moe_v41.rs, fn shared_side]. A struct whose trailing
 * fields are zero is a bf16-shared layer. */
#define MOE_SHARED_BF16 0
#define MOE_SHARED_KQUANT 1
typedef struct moe_layer {
  const uint16_t* gate_w;
  const float* bias;
  moe_experts experts;
  const uint16_t* sh_w1;     /* bf16 shared expert (MOE_SHARED_BF16); may be NULL otherwise */
  const uint16_t* sh_w3;
  const uint16_t* sh_w2;
  int32_t shared_kind;       /* MOE_SHARED_BF16 or MOE_SHARED_KQUANT */
  moe_experts shared_q;      /* the K-quant shared expert's blocks (MOE_SHARED_KQUANT) */
} moe_layer;

/* Words of one token's routing header: 1 + 3*topk int32
 * [device_route.rs, module doc; fn header_words; fn parse_header]:
 *   [0]                  status bits (MOE_STATUS_*)
 *   [1 .. topk]          the picks, in pick (rank) order
 *   [1+topk .. 2*topk]   the f32 bits of the pick-order weights
 *   [1+2topk .. 3*topk]  the plan: the picks in ascending expert id
 *                        (the pages' plan slots; all experts are resident, so
 *                        an expert's slot is its id) */
int32_t moe_header_words(const moe_cfg* cfg);

/* Bytes of workspace the calls below need for up to max_m tokens (>= 1):
 * the caller-owned counterpart of the pages' per-layer device buffers
 * (logits, the group's q8_1 rows, gate/up/h/down outputs, the shared
 * expert's sg/su/sh/sd, the routing header and plan tables) [moe_v41.rs,
 * struct MoeV41]. Returns 0 for an invalid or unsupported cfg. The workspace must be
 * 256-byte aligned device memory. Its control region (the first 256 bytes,
 * for every m: the counter through which the last router workgroup of
 * moe_layer_forward learns that it is last) must be zero before the first
 * call: moe_workspace_init does that, and every call leaves it zero again.
 * The rest needs no initialisation. A workspace sized for max_m serves every
 * call with m <= max_m. */
size_t moe_workspace_bytes(const moe_cfg* cfg, int32_t max_m);

/* Zero the workspace's control region (asynchronous, on `stream`, with a
 * kernel: safe inside a captured graph). Call once after allocating a
 * workspace, before its first use. */
int moe_workspace_init(const moe_cfg* cfg, int32_t max_m, void* ws, size_t ws_bytes, void* stream);

/* Offsets (bytes from the workspace start) of the intermediate results, for
 * inspection after a call has completed [the pages' workspace buffers,
 * moe_v41.rs, struct MoeV41]. Pair p = one (expert, token) of the plan, in
 * ascending expert id, then ascending token; a K-quant shared expert is the
 * plan's expert id n_routed (weight 1), so its pairs come last. The plan
 * words hold n_u, n_pairs, then max_pairs entries each of u_expert, u_first,
 * u_npairs, pair_tok, pair_expert, pair_w (f32 bits), then tok_pairs
 * [max_m][topk + 1]: each token's pairs in plan order, the last entry its
 * K-quant shared expert's pair (-1 = none). */
typedef struct moe_ws_layout {
  uint64_t total;
  uint64_t xq;       /* int8  [max_m][dim]        q8_1 codes of x                  */
  uint64_t xd;       /* fp16  [max_m][dim/32]     q8_1 scales of x                 */
  uint64_t xs;       /* int32 [max_m][dim/16]     sums of 16 consecutive codes     */
  uint64_t logits;   /* f32   [max_m][n_routed]                                    */
  uint64_t scores;   /* f32   [max_m][n_routed]   sqrt(softplus(logit/temp))       */
  uint64_t plan;     /* int32 plan words (n_u, per-expert and per-pair tables)     */
  uint64_t g;        /* f32   [pairs][inter]      gate GEMV                        */
  uint64_t u;        /* f32   [pairs][inter]      up GEMV                          */
  uint64_t h;        /* f32   [pairs][inter]      clamped SwiGLU                   */
  uint64_t hq;       /* int8  [pairs][inter]      q8_1 codes of h                  */
  uint64_t hd;       /* fp16  [pairs][inter/32]   q8_1 scales of h                 */
  uint64_t hs;       /* int32 [pairs][inter/16]   sums of 16 consecutive codes     */
  uint64_t y;        /* f32   [pairs][dim]        down GEMV                        */
  uint64_t sg;       /* f32   [max_m][inter]      shared gate                      */
  uint64_t su;       /* f32   [max_m][inter]      shared up                        */
  uint64_t sh;       /* bf16  [max_m][inter]      shared SwiGLU, rounded to bf16   */
  uint64_t sd;       /* f32   [max_m][dim]        shared down                      */
  uint64_t yr;       /* f32   [max_m][dim]        routed sum (layer forward)       */
  uint64_t status;   /* int32 [4] device status words (word 0: OR of MOE_STATUS_*) */
  uint64_t ctl;      /* 256 B control words (zero between calls); always offset 0  */
  uint64_t grp;      /* int32 [max_m + 2*(n_routed+1)] grouping scratch (prefill)   */
  uint64_t xd64;     /* f64   [max_m][dim/32]     q8_1 scales of x (prefill)       */
  uint64_t hd64;     /* f64   [pairs][inter/32]   q8_1 scales of h (prefill)       */
  int32_t max_pairs; /* max_m * (topk + 1)                                        */
  int32_t plan_words;
} moe_ws_layout;

int moe_workspace_layout(const moe_cfg* cfg, int32_t max_m, moe_ws_layout* out);

/* Route m tokens (A1-A3): router logits, scores, the top-k selection and
 * the header [moe_v41.rs, fn route_from_logits; device_route.rs, module doc].
 *   x       bf16 [m][dim]
 *   gate_w  bf16 [n_routed][dim]
 *   bias    f32  [n_routed]
 *   logits  f32  [m][n_routed] output, may be NULL (always also in the workspace)
 *   header  int32 [m][moe_header_words] output
 * The logits of a token depend only on that token's row: they are identical
 * for any m. Also writes the q8_1 of x into the workspace. */
int moe_route_select(const moe_cfg* cfg, const uint16_t* x, int32_t m, const uint16_t* gate_w, const float* bias,
                     float* logits, int32_t* header, void* ws, size_t ws_bytes, void* stream);

/* The routed experts of m <= 8 tokens (A4-A6 and the routed half of A7):
 * for every pick in the headers, gate/up on Q2_K, clamped SwiGLU, q8_1,
 * down on Q3_K; then per token y_routed = the sum over its picks in plan
 * order (ascending id) of weight * y, in f32 starting from +0. Experts
 * picked by several tokens are read once for all of them.
 *   x        bf16 [m][dim]  (quantised to q8_1 again here)
 *   header   int32 [m][moe_header_words] (as written by moe_route_select)
 *   y_routed f32  [m][dim] output
 * A pick outside [0, n_routed) or repeated within a token zeroes that
 * token's output and sets MOE_STATUS_BAD_PICK in the workspace status. */
int moe_experts_decode(const moe_cfg* cfg, const uint16_t* x, int32_t m, const int32_t* header,
                       const moe_experts* experts, float* y_routed, void* ws, size_t ws_bytes, void* stream);

/* The routed experts of any number m >= 1 of tokens (prefill, A9): the
 * same values as moe_experts_decode (each token's output is defined exactly
 * as at m = 1), computed with the (token, expert) pairs grouped by expert
 * and each expert's blocks read once per 16 of its tokens: gate/up on Q2_K
 * and down on Q3_K as int8 MFMA tiles with exact integer block sums and a
 * float64 epilogue [moe_v41.rs, module doc; struct Kernels: gather,
 * scatter_add, mmq_q2k_* / mmq_q3k_*; struct MoeV41: one expert group's
 * gathered rows and q8_1 activations, group-major token rows and weights];
 * the int8 MFMA tiling is this library's own. Arguments and error behaviour as
 * moe_experts_decode (x bf16 [m][dim], header int32 [m][moe_header_words],
 * y_routed f32 [m][dim]); the workspace is sized for m. */
int moe_experts_prefill(const moe_cfg* cfg, const uint16_t* x, int32_t m, const int32_t* header,
                        const moe_experts* experts, float* y_routed, void* ws, size_t ws_bytes, void* stream);

/* The whole layer for m >= 1 tokens (A1-A7): route, routed experts, shared
 * expert (bf16 SwiGLU MLP, its SwiGLU output rounded to bf16), and
 * out = acc + shared where acc is the routed sum; the shared output is added
 * after the routed experts [moe_v41.rs, fn shared_side]. m <= 8 runs the
 * decode kernels (GEMVs over the union of the picked experts); m > 8 runs
 * the prefill kernels (router waves per 8 tokens, grouping by expert, int8
 * MFMA expert GEMMs, bf16 MFMA shared expert, A9). Every token's logits,
 * header, q8_1 codes and GEMV values are the same bits either way.
 *   x        bf16 [m][dim]
 *   out_bf16 bf16 [m][dim] output (round to nearest even of out_f32)
 *   out_f32  f32  [m][dim] output, may be NULL
 *   header   int32 [m][moe_header_words] output, may be NULL */
int moe_layer_forward(const moe_cfg* cfg, const moe_layer* layer, const uint16_t* x, int32_t m, uint16_t* out_bf16,
                      float* out_f32, int32_t* header, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): moe_layer_forward
 * for 1 <= m <= 8 tokens with no workspace argument. Its workspace is a
 * fixed 6 MiB array of the library's own on each GPU, held from the
 * library's load until the process ends; a shape whose workspace would not
 * fit returns MOE_EWORKSPACE, m outside 1..8 MOE_EINVAL. The first call on a
 * device looks the array's device address up and zeroes its control words
 * with a kernel on `stream`; no call allocates or frees anything. Every call
 * on one GPU shares the array: calls that overlap on one GPU (different
 * streams, or host threads) race and must not be issued. The intermediate
 * results stay in that array and are not exposed. Arguments, outputs and
 * the other errors as moe_layer_forward. */
int moe_layer_forward_noalloc(const moe_cfg* cfg, const moe_layer* layer, const uint16_t* x, int32_t m,
                              uint16_t* out_bf16, float* out_f32, int32_t* header, void* stream);

/* One step through a stack of n_layers MoE layers for m >= 1 tokens:
 * for l = 0 .. n_layers-1, out_l = layer l applied to x_l exactly as
 * moe_layer_forward computes it, and x_{l+1} = bf16(f32(x_l) + out_l), the
 * residual stream between layers (the pages' step runs the layers back to
 * back [step_seg.rs, module doc]; they name no norm between MoE layers and
 * none is applied here). All launches are enqueued on `stream` in order,
 * with no host synchronisation; the workspace is reused by every layer.
 *   layers   HOST array of n_layers moe_layer (device pointers inside)
 *   xs       bf16 [n_layers+1][m][dim]: xs[0] is the input, xs[l+1] is written
 *   out_f32  f32  [n_layers][m][dim] per-layer output before the residual add, may be NULL
 *   headers  int32 [n_layers][m][moe_header_words] per-layer headers, may be NULL */
int moe_stack_forward(const moe_cfg* cfg, const moe_layer* layers, int32_t n_layers, uint16_t* xs, int32_t m,
                      float* out_f32, int32_t* headers, void* ws, size_t ws_bytes, void* stream);

/* ---- Expert streaming beyond HBM ----------------------------------------
 * An expert cache holds the routed experts of n_layers layers in host memory
 * and keeps n_slots of them in a device slot pool, with a device slot table
 * [n_layers][n_routed] (the slot of each expert, -1 = not resident)
 * [device_route.rs, module doc, fn route_device_m1, fn slot_table_update;
 * moe_v41.rs, module doc: the LRU gathers the picked experts' raw blocks into
 * device slots, misses read from storage]. For each layer the routing runs
 * against the slot table, its header is read back once, the least recently
 * used slots take the missing picks (copied from host memory), the changed
 * table rows are uploaded, and the experts run from the slots; every value
 * is the same as with the experts resident. The cache owns device memory
 * (the pool, the table, a predicted-header buffer), pinned host buffers and a
 * copy stream, from moe_cache_create to moe_cache_destroy; its calls are not
 * thread-safe and must use the device that was current at its creation. */
typedef struct moe_cache moe_cache;

typedef struct moe_cache_stats {
  int64_t hits;           /* picks found resident                                     */
  int64_t misses;         /* picks copied in on demand                                */
  int64_t prefetched;     /* experts copied in ahead of need                          */
  int64_t prefetch_used;  /* picks found resident because a prefetch brought them in   */
  int64_t bytes_copied;   /* host-to-device expert bytes                              */
  int64_t reads_back;     /* header read-backs (one per layer call)                   */
} moe_cache_stats;

/* host_experts: n_layers host pointers, layer l's expert e at
 * host_experts[l] + e * stride with the moe_experts offsets (pinned memory
 * makes the copies asynchronous); n_slots device slots of stride bytes;
 * max_m: the largest m of a later moe_cache_forward. */
int moe_cache_create(const moe_cfg* cfg, int32_t n_layers, const void* const* host_experts, uint64_t stride,
                     uint64_t gate_off, uint64_t up_off, uint64_t down_off, int32_t n_slots, int32_t max_m,
                     moe_cache** out);
int moe_cache_destroy(moe_cache* cache);

/* Layers first_layer .. first_layer + n_layers - 1 of the cache, one step for
 * m tokens, as moe_stack_forward (xs [n_layers+1][m][dim], out_f32 and
 * headers per layer, may be NULL; layers[i] gives layer first_layer+i's
 * router, bias and shared expert; its `experts` field is not used). Each
 * layer's header has MOE_STATUS_MISS set when a pick was not resident at
 * routing time, and its plan words hold the picks' slots then (-1 = absent).
 * prefetch_k in 0..topk: also run the next layer's router on this layer's
 * input and copy the first prefetch_k predicted picks of each token into
 * slots while this layer computes [moe_v41.rs, fn prefetch_k; struct MoeV41:
 * pred_logits]. Blocks the calling thread once per layer (the header's
 * read-back). MOE_EUNSUPPORTED when a layer's distinct picks need more slots
 * than the cache has. */
int moe_cache_forward(moe_cache* cache, const moe_cfg* cfg, const moe_layer* layers, int32_t first_layer,
                      int32_t n_layers, uint16_t* xs, int32_t m, float* out_f32, int32_t* headers, int32_t prefetch_k,
                      void* ws, size_t ws_bytes, void* stream);

/* Copies the listed experts of a layer into slots ahead of need (on `stream`,
 * after the work enqueued there), evicting least recently used slots. */
int moe_cache_prefetch(moe_cache* cache, int32_t layer, const int32_t* experts, int32_t n, void* stream);
int moe_cache_get_stats(const moe_cache* cache, moe_cache_stats* out);
/* The cache's slot of each expert of a layer (host int32 [n_routed], -1 = not resident). */
int moe_cache_resident(const moe_cache* cache, int32_t layer, int32_t* slots);

/* The cache's slot assignment alone, on the host (checking only): keys in
 * 0..n_keys-1 requested in n_batches batches of batch_len keys; each
 * request's slot (-1: no slot free of the batch) and whether it missed. */
int moe_lru_simulate(int32_t n_slots, int64_t n_keys, const int64_t* keys, const int32_t* batch_len,
                     int32_t n_batches, int32_t* slots_out, int32_t* miss_out);

/* The glibc score table, computed on the host from its libm: every f32 input
 * z <= 20 (z = logit / temp) where sqrtf(log1pf(expf(z))) differs from the
 * correctly rounded chain, ascending in its bit pattern: keys[i] = the bits of
 * z, vals[i] = the bits of glibc's score; index[p] (p < 2^24, plus one end
 * entry, MOE_SCORE_INDEX_LEN words) = the first i with keys[i] >> 8 >= p.
 * Pass keys = NULL to get the count in *n (vals and index are then ignored);
 * otherwise keys and vals hold cap >= *n entries and index
 * MOE_SCORE_INDEX_LEN, else MOE_EINVAL. The first call sweeps all 2^32 inputs
 * on the host's cores (seconds); later calls copy its result. Host memory. */
#define MOE_SCORE_INDEX_LEN ((1 << 24) + 1)
int moe_glibc_score_table(uint32_t* keys, uint32_t* vals, uint32_t* index, int64_t cap, int64_t* n);

/* Registers the device copies of the glibc score table (keys, vals [n],
 * index [MOE_SCORE_INDEX_LEN]: the arrays moe_glibc_score_table returned,
 * copied unchanged; device pointers owned by the caller and kept alive while
 * the mode is used) for the current device; NULL keys unregisters. Calls that
 * route with MOE_SCORE_GLIBC read the registration of the device current when
 * they are made; the kernels index the table as given, without checks. */
int moe_set_score_table(const uint32_t* keys, const uint32_t* vals, const uint32_t* index, int64_t n);

/* The score chain of A3 alone on device data: out[i] = sqrt(softplus(
 * logits[i] / temp)) with correctly rounded exp, log1p, division and sqrt
 * [moe_v41.rs, fn softplus, fn route_from_logits]. flags bit 0 forces the
 * extended-precision path of exp/log1p for every element (checking only);
 * flags bit 1 gives the glibc mode's scores (the table registered for the
 * current device; MOE_EINVAL when there is none); flags bit 2 returns the
 * chain's exp step alone, out[i] = RN32(exp(logits[i] / temp)), the function
 * the SwiGLU also uses (checking only; not with bit 1). Other bits:
 * MOE_EINVAL. */
int moe_scores(const float* logits, int64_t n, float temp, float* out, int32_t flags, void* stream);

/* The same score chain computed on the host CPU by the library's own code
 * (the device functions compiled for the host); for checking the library's
 * arithmetic where no GPU is present. flags as moe_scores (bit 1: the glibc
 * mode through the host's copy of the table, built on first use; bit 2: the
 * exp step alone). All pointers are host pointers. */
int moe_scores_host(const float* logits, int64_t n, float temp, float* out, int32_t flags);

/* The clamped SwiGLU of the library on the host: out[i] = silu(min(g,L)) *
 * clamp(u,-L,L) (checking only, host pointers). */
int moe_swiglu_host(const float* g, const float* u, int64_t n, float limit, float* out);

/* Kernel timing hook: the next launch of kernel `which` (MOE_K_*) on the
 * calling thread records the two events (hipEvent_t, created by the caller)
 * at its dispatch's start and end (hipExtLaunchKernelGGL), on the stream it
 * is launched on. One-shot; pass NULL events to clear. For measurement only.
 *   MOE_K_GATEUP  the routed gate/up (Q2_K) kernel (at m = 1 with the
 *                 selection and the shared expert's gate/up rows)
 *   MOE_K_DOWN    the routed down (Q3_K) kernel (with the shared down rows
 *                 and the combine at m = 1)
 *   MOE_K_ROUTER  the front kernel (q8_1 of x and the router; for m > 1 also
 *                 the selection, the plan and the shared gate/up) */
#define MOE_K_GATEUP 1
#define MOE_K_DOWN 2
#define MOE_K_ROUTER 3
#define MOE_K_SHARED_GU 4    /* prefill: the shared expert's gate/up GEMM with its SwiGLU */
#define MOE_K_SHARED_DOWN 5  /* prefill: the shared expert's down GEMM                    */
#define MOE_K_GATEUP2 6      /* prefill: the gate/up kernel of the experts with more than 8 pairs
                                (MOE_K_GATEUP is then the one of the experts with at most 8) */
#define MOE_K_DOWN2 7        /* prefill: the down kernel of the experts with more than 8 pairs
                                (MOE_K_DOWN is then the one of the experts with at most 8)   */
#define MOE_K_READ_PROBE 8   /* moe_read_probe's streaming kernel                         */
int moe_time_next_launch(int32_t which, void* ev_begin, void* ev_end);

/* Measurement only: a plain read-only stream over `bytes` bytes of device
 * memory at `buf` (16-byte aligned, bytes a multiple of 16) with `blocks`
 * workgroups of 256 threads (each a contiguous share), 16-byte loads, nothing written
 * (sink: one device word, written only if the data XOR to a fixed value).
 * Timed through moe_time_next_launch(MOE_K_READ_PROBE, ...), it gives the
 * achievable HBM read rate that the kernels' rates are set beside. */
int moe_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, int32_t blocks, void* stream);


const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
