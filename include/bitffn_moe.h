/*
 * bitffn_moe.h -- C ABI of the routed-expert MoE layer library (gfx950).
 *
 * One MoE layer of a 2-3-bit block-quantized mixture-of-experts model: the
 * router's top-k choice, the split of the chosen experts into those resident
 * in the GPU expert cache and those that are not, the fused
 * dequantize + gate/up + SiLU-gating + down expert FFN, and the
 * routing-weighted sum into the residual.
 *
 * Sources: the pages on the "Strata" engine.
 *   - "Strata" (news.blueqat.app post 3262), section "Strataとは": 48 layers,
 *     512 experts per layer, 10 chosen per token plus one shared expert.
 *   - same page, section "GPU・CPU・RAM・SSDの分担": router, shared expert and a
 *     cache of the most used experts live on the GPU; long inputs are taken
 *     8,192 tokens at a time.
 *   - same page, section "投機的デコード" and "Strataとは？VRAM 12GBのGPUで
 *     Qwen3.8-Flash-Nextを動かす方法" (vramglass.com), section "その3": up to
 *     3 drafted tokens are verified in one pass over the layers; the weights
 *     are read once however many tokens are verified.
 *   - vramglass.com page, sections "その1" and "その2": about 72% of a
 *     token's experts are found in the GPU cache; the others are computed
 *     from host memory at the same time instead of being copied over.
 *   - "FreeToken vs Strata" (geekoyaji.com), section "共通の仕組み": the GPU
 *     part and the host part of a layer are joined before the next layer.
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless marked (host).  The caller owns
 *     every buffer; the library allocates nothing and keeps no state between
 *     calls except what a caller-provided workspace holds.
 *   - Work is enqueued asynchronously on `stream`; results are ready when
 *     the stream reaches that point.  Calls on one stream are ordered.
 *   - Arguments are checked on the host before any HIP call; a check that
 *     fails returns a negative status and enqueues nothing.  MOE_EHIP means
 *     a HIP launch failed; moe_last_hip_error() gives the HIP code (kept per
 *     calling thread).
 *   - Device pointers must be 16-byte aligned (MOE_EALIGN otherwise).
 *   - Results never depend on timing: every reduction has a fixed order, so
 *     two runs on the same inputs are bitwise equal.
 */
#ifndef BITFFN_MOE_H
#define BITFFN_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* status codes */
#define MOE_OK 0
#define MOE_EINVAL (-1)   /* null pointer, size or count out of range     */
#define MOE_EALIGN (-2)   /* device pointer not 16-byte aligned           */
#define MOE_EFORMAT (-3)  /* unknown block format or slot size mismatch  */
#define MOE_ENOSPC (-4)   /* workspace smaller than the query returned   */
#define MOE_EHIP (-5)     /* a HIP call failed                           */

/* Block formats: 32 consecutive weights of a row share one block.
 *   MOE_FMT_Q2S : 2-bit code q, fp16 scale s:          w = s * (q - 1.5)
 *   MOE_FMT_Q2SM: 2-bit code q, fp16 scale s, min m:   w = m + s * q
 *   MOE_FMT_Q3G : 3-bit code q, fp16 scale s:          w = s * (2q - 7) / 7
 *                 (the grid -3.5..3.5 in steps of 1, times s / 3.5)
 * Slot layout (bytes of one expert): matrix G = 2*d_ff rows x d_model
 * columns (row 2j = gate row j, row 2j+1 = up row j), then matrix
 * D = d_model rows x d_ff columns (down projection).  Rows are cut into
 * 32-weight blocks.  A matrix is stored in units of U consecutive blocks of
 * one row (U = 2 for G, U = 1 for D); with R rows, unit c of row r has index
 * c*R + r, so one unit of consecutive rows is contiguous.  Each matrix is a
 * sequence of planes, each starting 256-byte aligned from the slot start and
 * holding its units in index order (inside a unit the U blocks follow each
 * other):
 *   codes (8 B/block: code i at bits [2i,2i+2) of the little-endian 64-bit
 *          word; for Q3G the low two bits),
 *   hi    (Q3G only, 4 B/block: bit 2i+1 holds bit 2 of code i for i < 16,
 *          bit 2(i-16) holds it for i >= 16),
 *   scale (fp16, 2 B/block),
 *   min   (Q2SM only, fp16, 2 B/block).
 * The slot size is rounded up to 256 bytes; moe_slot_bytes() returns it. */
#define MOE_FMT_Q2S 1
#define MOE_FMT_Q2SM 2
#define MOE_FMT_Q3G 3

#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

/* Limits checked on the host. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 64
#define MOE_MAX_DECODE_T 4
#define MOE_MAX_DECODE_PAIRS 64
#define MOE_MAX_CACHE_SLOTS 4096

/* One MoE layer as it sits in device memory (host struct, read during the
 * call only). */
typedef struct moe_layer {
  int32_t d_model;     /* multiple of 64 in 64..2048                        */
  int32_t d_ff;        /* multiple of 32 in 32..4096                        */
  int32_t n_experts;   /* 1..MOE_MAX_EXPERTS routed experts                  */
  int32_t top_k;       /* 1..min(n_experts, MOE_MAX_TOPK)                    */
  int32_t fmt;         /* MOE_FMT_*                                          */
  int32_t n_slots;     /* slots in the pool                                  */
  int32_t shared_slot; /* slot of the always-used shared expert, -1 = none   */
  int32_t reserved;    /* must be 0                                          */
  int64_t slot_bytes;  /* must equal moe_slot_bytes(fmt, d_model, d_ff)      */
  const void* pool;    /* device: n_slots * slot_bytes packed experts, 256-B
                          aligned                                            */
} moe_layer;

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* (host) Static text for a status code. */
const char* moe_status_str(int status);

/* (host) HIP error code of this thread's last MOE_EHIP. */
int moe_last_hip_error(void);

/* (host) Bytes of one packed expert slot; MOE_EFORMAT / MOE_EINVAL (as a
 * negative value) for an unknown format or unsupported sizes. */
int64_t moe_slot_bytes(int fmt, int d_model, int d_ff);

/* Router projection (vramglass.com page, "なぜVRAM 12GBで足りるのか", and
 * "Strata" page, "GPU・CPU・RAM・SSDの分担": the router belongs to the
 * common part that stays on the GPU; it gives each routed expert a logit
 * from the token's hidden state).  For a decode or verify step of
 * 1 <= T <= MOE_MAX_DECODE_T tokens:
 *   logits[t][e] = sum_j x[t][j] * w[e][j]
 * x fp32 [T][d_model], w bfloat16 bits [n_experts][d_model] row-major (the
 * pages give no precision; bf16 router weights are this library's reading),
 * logits fp32 [T][n_experts] (may not alias x or w); all device memory,
 * 16-byte aligned.  Products and sums in fp32 in a fixed order (bitwise
 * reproducible).  Limits: d_model a multiple of 64 in 64..2048,
 * 1 <= n_experts <= MOE_MAX_EXPERTS.  The logits then feed moe_route_topk,
 * moe_decode_layer or moe_decode_stack. */
int moe_router_logits(const float* x, int T, int d_model, const uint16_t* w,
                      int n_experts, float* logits, hipStream_t stream);

/* Router top-k ("Strata" page, "Strataとは": 10 of 512 per token).
 * logits fp32 [T][E] row-major.  Per token the experts are ranked by
 * (logit descending, expert id ascending); NaN ranks as -inf and -0.0 as
 * +0.0.  idx int32 [T][k] receives the first k ids in rank order, w fp32
 * [T][k] the softmax over those k logits, exp(l_i - l_0) / sum_j
 * exp(l_j - l_0) with l_0 the largest (the difference of two equal values,
 * infinities included, is taken as 0).
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 64), 0 <= T < 2^24 (T = 0 is a
 * no-op). */
int moe_route_topk(const float* logits, int T, int E, int k,
                   int32_t* idx, float* w, hipStream_t stream);

/* Expert-cache lookup (vramglass.com page, "その1"/"その2": the GPU caches
 * the most used experts; the others are computed elsewhere).
 * slot_of_expert int32 [E]: slot holding expert e, or -1.
 * slot int32 [T*k] = slot_of_expert[idx]; miss_expert int32 [T*k] receives
 * the distinct missed expert ids in ascending order; miss_pair int32 [T*k]
 * (may be NULL) receives t*k+i of every missed pair, ordered by
 * (expert, t, i); n_miss int32 [2] = {distinct missed experts, missed
 * pairs}.  Entries past the counts are left as they were.
 * Expert ids in idx must be in [0, E) and distinct within a token (as
 * moe_route_topk returns them); neither is checked.
 * ws: device workspace of moe_lookup_workspace_bytes(T, k, E) bytes (0 for
 * T*k <= 1024, then ws may be NULL), 256-byte aligned. */
size_t moe_lookup_workspace_bytes(int T, int k, int E);
int moe_cache_lookup(const int32_t* idx, int T, int k,
                     const int32_t* slot_of_expert, int E,
                     int32_t* slot, int32_t* miss_expert, int32_t* miss_pair,
                     int32_t* n_miss, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* (host) Workspace bytes that moe_expert_ffn_decode needs for T tokens. */
size_t moe_decode_workspace_bytes(const moe_layer* L, int T);

/* Decode / verify layer for T = 1..4 tokens routed independently
 * ("Strata" page "投機的デコード": one real and up to 3 drafted tokens).
 *   y[t] = x[t] + sum_{i: slot[t*k+i] >= 0} w[t*k+i] * FFN_{slot}(x[t])
 *               + FFN_{shared_slot}(x[t])          (if shared_slot >= 0)
 * with FFN(x) = D (silu(G_gate x) * (G_up x)), silu(z) = z / (1 + e^-z),
 * summed for each token in k-slot order, shared expert last.  Misses
 * (slot < 0) are skipped: the caller adds them (moe_combine can).  A slot
 * at or past L->n_slots is a miss as well: no byte outside the pool is read.
 * Each distinct resident expert chosen by any of the T tokens is streamed
 * from memory once for all tokens that chose it.  x, y fp32 [T][d_model]
 * (y may not alias x); idx, slot int32 [T][k]; w fp32 [T][k].
 * Requires T * top_k <= 64.  ws: device workspace of at least
 * moe_decode_workspace_bytes(L, T) bytes, 256-byte aligned; its contents on
 * entry do not matter. */
int moe_expert_ffn_decode(const moe_layer* L, const float* x, int T,
                          const int32_t* idx, const int32_t* slot,
                          const float* w, float* y, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* One whole decode / verify layer step: moe_route_topk, moe_cache_lookup
 * and moe_expert_ffn_decode in one call, with identical results in every
 * output ("Strata" page, "Strataとは" and "投機的デコード": the router picks
 * 10 of 512 experts plus the shared one, the cached ones run on the GPU,
 * the misses are handed on).  logits fp32 [T][n_experts]; slot_of_expert
 * int32 [n_experts], an entry outside [0, L->n_slots) meaning not resident
 * (such an expert's slot output is -1 and it is in the miss list); outputs
 * as those three calls define them: idx, slot
 * int32 [T][k], w fp32 [T][k], miss_expert int32 [T*k], miss_pair int32
 * [T*k] (may be NULL), n_miss int32 [2], y fp32 [T][d_model] (may not alias
 * x).  Limits: as moe_expert_ffn_decode (T * top_k <= 64); n_experts <= 1024.
 * ws: at least moe_decode_workspace_bytes(L, T) bytes, 256-byte aligned.
 * Runs as two kernels; routing is repeated in every workgroup of the first,
 * so no routing result makes a round trip through memory before the expert
 * weights are requested. */
int moe_decode_layer(const moe_layer* L, const float* x, int T,
                     const float* logits, const int32_t* slot_of_expert,
                     int32_t* idx, float* w, int32_t* slot,
                     int32_t* miss_expert, int32_t* miss_pair, int32_t* n_miss,
                     float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_decode_layer with no workspace argument and no allocation, for
 * callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a 16 MiB array
 * in device memory that the library holds on every GPU it runs on until the
 * process ends; its address is looked up once per device.  Sizes whose
 * moe_decode_workspace_bytes(L, T) exceeds 16 MiB give MOE_ENOSPC (the
 * model's layer, d_model 2048, d_ff 768, top-10, needs 8.7 MB at T = 4).
 * Every call on one GPU uses the same array: calls that overlap on a GPU
 * (on different streams, without ordering between them) race and give
 * undefined results.  Arguments, outputs and limits as moe_decode_layer. */
int moe_decode_layer_noalloc(const moe_layer* L, const float* x, int T,
                             const float* logits, const int32_t* slot_of_expert,
                             int32_t* idx, float* w, int32_t* slot,
                             int32_t* miss_expert, int32_t* miss_pair,
                             int32_t* n_miss, float* y, hipStream_t stream);

/* Decode / verify through a stack of layers ("Strata" page, "Strataとは":
 * 48 MoE layers, each choosing 10 of 512 experts plus a shared one per
 * token; "FreeToken vs Strata", "共通の仕組み": a layer's output is complete
 * before the next layer starts; "投機的デコード": up to 3 drafted tokens are
 * checked in the same pass, the weights read once for all of them).
 * For l = 0 .. n_layers-1, with T = 1..4 tokens routed independently:
 *   x_0 = x,   x_l = y_{l-1} + layers[l].addend   (addend NULL: + 0)
 *   y_l = moe_decode_layer's y for layer l from x_l, its logits and its slot
 *         table (resident chosen experts in k-slot order, the shared expert
 *         last; misses left out and listed), bit for bit.
 * The addend stands for whatever the caller's model adds to the residual
 * between two MoE layers; the call itself only chains y into the next x.
 * Per layer the call runs moe_decode_layer's two kernels; the second also
 * forms x_{l+1}, and layer l+1's kernels start once it is complete.  Every
 * sum has a fixed order that does not depend on the other tokens of the
 * step: a token's y_l has the same bits at T = 1 and as one of T = 4 tokens,
 * and two calls on the same inputs give the same bits.
 *   layers    (host) array of n_layers descriptors, read during the call:
 *             pool, slot_bytes, n_slots, fmt (may differ between layers),
 *             shared_slot as in moe_layer; slot_of_expert int32 [n_experts];
 *             logits fp32 [T][n_experts]; addend fp32 [T][d_model] or NULL
 *             (ignored for layer 0); y fp32 [T][d_model] output or NULL (the
 *             last layer's y is required); idx, w, slot [T][k] routing
 *             outputs (all three or none), miss_expert, miss_pair, n_miss as
 *             moe_cache_lookup (miss_expert and n_miss together or neither;
 *             miss_pair may be NULL).
 *   x         fp32 [T][d_model], the first layer's input.
 * Limits: as moe_decode_layer (T * top_k <= 64, n_experts <= 1024, d_model a
 * multiple of 64 up to 2048, d_ff a multiple of 32 up to 4096),
 * 1 <= n_layers.  Outputs may not overlap x or any input.
 * ws: at least moe_decode_stack_workspace_bytes() bytes, 256-byte aligned;
 * its contents on entry do not matter. */
typedef struct moe_stack_layer {
  const void* pool;
  int64_t slot_bytes;
  int32_t n_slots;
  int32_t fmt;
  int32_t shared_slot;
  int32_t reserved;                 /* must be 0 */
  const int32_t* slot_of_expert;
  const float* logits;
  const float* addend;
  float* y;
  int32_t* idx;
  float* w;
  int32_t* slot;
  int32_t* miss_expert;
  int32_t* miss_pair;
  int32_t* n_miss;
} moe_stack_layer;

/* (host) Workspace bytes of moe_decode_stack (0 for sizes it does not take). */
size_t moe_decode_stack_workspace_bytes(int d_model, int d_ff, int n_experts, int top_k, int T);

int moe_decode_stack(int d_model, int d_ff, int n_experts, int top_k, int T, int n_layers,
                     const moe_stack_layer* layers, const float* x, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Miss execution and the per-layer join of a decode / verify step.  The
 * chosen experts not resident in the GPU cache are computed from the host
 * tier, a copy of the layer's experts in host memory, and added to the GPU
 * part ("Strataとは？VRAM 12GBのGPUで…" (vramglass.com), section "その2":
 * the misses run at the same time as the resident experts, from host memory,
 * instead of being copied to the GPU; "FreeToken vs Strata", "共通の仕組み":
 * both parts meet before the next layer).  Optionally misses of low rank are
 * left out ("Strata" page, section "どう見るか": a setting that drops missed
 * experts of low rank, which changes the output slightly).
 *   H          host tier: same d_model, d_ff, n_experts, top_k and fmt as
 *              the GPU layer; H->pool points to H->n_slots packed slots in
 *              pinned host memory that this device can address (hipHostMalloc)
 *              or in device memory; pageable memory gives MOE_EINVAL.
 *              H->shared_slot must be -1 (the shared expert is resident).
 *   x          fp32 [T][d_model], the layer input.
 *   idx, w     int32 / fp32 [T][k], the routing of this step (rank order;
 *              ids distinct within a token, as moe_route_topk gives them).
 *   slot       int32 [T][k], the GPU slots of this step as the GPU part
 *              wrote them (-1 = miss; any value >= 0 counts as computed
 *              there).
 *   host_slot_of_expert  int32 [n_experts], slot of each expert in H; a
 *              value outside [0, H->n_slots) means not there, and such a
 *              miss adds nothing.
 *   max_rank   0..top_k: a miss in k-slot i runs only if i < max_rank
 *              (top_k: every miss; 0: nothing is enqueued).  The weights
 *              of the terms kept are not rescaled.
 *   y          fp32 [T][d_model], in and out: on entry the GPU part (the y
 *              of moe_expert_ffn_decode / moe_decode_layer for the same
 *              step); on return
 *   y[t] += sum_{i < max_rank: slot[t*k+i] < 0, h >= 0} w[t*k+i] * FFN_h(x[t]),
 *              h = host_slot_of_expert[idx[t*k+i]], terms in k-slot order.
 * Each distinct missed expert is read from the host tier once for all
 * tokens that chose it, by the GPU's own loads (no copy engine, no host
 * wait), so the call can sit in a captured graph after the GPU part.
 * Limits as moe_expert_ffn_decode (T * top_k <= 64).  ws: at least
 * moe_decode_workspace_bytes(H, T) bytes, 256-byte aligned (the GPU part's
 * workspace may be reused once that part is done). */
int moe_decode_misses(const moe_layer* H, const float* x, int T,
                      const int32_t* idx, const int32_t* slot, const float* w,
                      const int32_t* host_slot_of_expert, int max_rank,
                      float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_decode_misses in two phases that the caller may put on different
 * streams, so that the host-tier reads overlap the GPU part ("Strataとは？
 * VRAM 12GBのGPUで…" (vramglass.com), section "その2": the missed experts
 * are computed at the same time as the resident ones; "FreeToken vs
 * Strata", "共通の仕組み": the parts meet before the next layer).
 *   MOE_MISSES_READ  the missed experts' products into ws (reads x, idx,
 *                    slot, host_slot_of_expert and the host tier; w and y
 *                    are not used and may be NULL);
 *   MOE_MISSES_JOIN  y += those products, as moe_decode_misses adds them
 *                    (reads ws, idx, slot, w, host_slot_of_expert; x may be
 *                    NULL).
 * phases = READ | JOIN is moe_decode_misses.  The JOIN of a step must run
 * after its READ has completed and after y holds the GPU part (the caller
 * orders the streams, e.g. with events); between the two, ws belongs to the
 * call.  The result is the same, bit for bit, as moe_decode_misses.  Other
 * arguments and limits as moe_decode_misses. */
#define MOE_MISSES_READ 1
#define MOE_MISSES_JOIN 2
int moe_decode_misses_phases(const moe_layer* H, const float* x, int T,
                             const int32_t* idx, const int32_t* slot, const float* w,
                             const int32_t* host_slot_of_expert, int max_rank,
                             float* y, void* ws, size_t ws_bytes, int phases,
                             hipStream_t stream);

/* One decode / verify layer with both tiers in the same two kernels: the
 * routing and lookup of moe_decode_layer, then the chosen experts resident in
 * L's pool read from there and the missed ones read from the host tier H in
 * the same launch, all terms joined in one sum ("Strataとは？VRAM 12GBのGPUで
 * …" (vramglass.com), section "その2": the missed experts are computed from
 * host memory at the same time as the resident ones; "FreeToken vs Strata",
 * "共通の仕組み": both parts meet before the next layer; "Strata" page,
 * section "どう見るか": missed experts of low rank may be left out).  The
 * layer time is that of the larger part, not of the two parts in turn.
 *   L, x, T, logits, slot_of_expert, idx, w, slot, miss_expert, miss_pair,
 *   n_miss   as moe_decode_layer; slot (and the miss lists) describe the GPU
 *            cache only: -1 for a pair not resident there, whether or not
 *            the host tier computed it.
 *   H, host_slot_of_expert, max_rank   as moe_decode_misses (same fmt,
 *            d_model, d_ff, n_experts and top_k as L; H->shared_slot = -1;
 *            H->pool pinned host or device memory).
 *   y        fp32 [T][d_model] output:
 *   y[t] = x[t] + sum_i term(t,i) + FFN_shared(x[t]), term(t,i) =
 *            w * FFN of GPU slot slot[t*k+i]                if that slot >= 0,
 *            w * FFN of host slot h = host_slot_of_expert[idx[t*k+i]]
 *                                       if the pair missed, i < max_rank and
 *                                       0 <= h < H->n_slots,
 *            0 otherwise;
 *            terms in k-slot order, then the shared expert (the same sum as
 *            moe_decode_layer's when nothing misses, so then the same bits).
 * Limits as moe_decode_layer.  ws: at least moe_decode_workspace_bytes(L, T)
 * bytes, 256-byte aligned. */
int moe_decode_layer_tiers(const moe_layer* L, const moe_layer* H,
                           const int32_t* host_slot_of_expert, int max_rank, const float* x,
                           int T, const float* logits, const int32_t* slot_of_expert,
                           int32_t* idx, float* w, int32_t* slot, int32_t* miss_expert,
                           int32_t* miss_pair, int32_t* n_miss, float* y, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Expert-cache admission and eviction.  The cache starts from a table of
 * usage frequencies and is updated as the conversation moves on ("FreeToken
 * vs Strata", comparison table, row "VRAMのエキスパートの入れ替え";
 * vramglass.com page, "その1"; "Strata" page, "GPU・CPU・RAM・SSDの分担").
 * The pages give no rule; these four calls implement one:
 *   moe_cache_count   after each routing, count the uses of every expert;
 *   moe_cache_plan    pick the swaps (best missing experts for the worst
 *                     slots), evict at once, decay the counts;
 *   moe_cache_fill    copy the admitted experts' bytes from the host tier
 *                     into their slots (may run on another stream);
 *   moe_cache_commit  make the admitted experts visible in the slot table.
 * Between plan and commit an admitted expert is still a miss, so decode
 * calls on the compute stream stay correct while the fill runs elsewhere;
 * the fill must not start before the work that read the evicted slots is
 * done, and the commit must follow the fill (events or one stream).
 * All four are kernels: nothing waits on the host, so they can be captured
 * in a graph. */

/* counts uint32 [E] += the number of times each expert appears in idx int32
 * [n_pairs] (ids outside [0, E) are ignored).  Counts wrap at 2^32.
 * Limits: 0 <= n_pairs < 2^24, 1 <= E <= MOE_MAX_EXPERTS. */
int moe_cache_count(const int32_t* idx, int n_pairs, int E, uint32_t* counts,
                    hipStream_t stream);

/* Plan up to max_swaps swaps.  slot_of_expert int32 [E] (slot or -1) and
 * expert_of_slot int32 [n_slots] (expert id, -1 = empty, the shared slot
 * holding anything) describe the cache and are updated in place; slot
 * shared_slot (-1 = none) is never touched.  host_slot_of_expert int32 [E]:
 * slot of each expert in the host tier (outside [0, host_n_slots) = none).
 *   candidates: experts with slot_of_expert < 0, a host slot and a count
 *     above 0, ranked by (count descending, id ascending);
 *   victims: slots other than shared_slot, ranked by (count of the expert
 *     held ascending, an empty slot or an id outside [0, E) counting as -1;
 *     then slot ascending);
 *   swap i (i = 0, 1, ...) puts candidate i into victim slot i while
 *     i < max_swaps and the candidate's count is strictly larger.
 * For each swap: slot_of_expert[old] = -1, expert_of_slot[slot] = new;
 * swaps int32 [max_swaps][4] receives (slot, old expert or -1, new expert,
 * its host slot) and n_swaps int32 [1] the number of swaps.  Then every
 * count becomes count >> decay_shift.  The newcomers stay out of
 * slot_of_expert until moe_cache_commit.
 * Limits: 1 <= E <= MOE_MAX_EXPERTS, 1 <= n_slots <= MOE_MAX_CACHE_SLOTS,
 * 1 <= max_swaps <= MOE_MAX_EXPERTS, 0 <= decay_shift <= 31.  One
 * workgroup; the result is unique (every ranking is total). */
int moe_cache_plan(uint32_t* counts, int E, int32_t* slot_of_expert,
                   int32_t* expert_of_slot, int n_slots, int shared_slot,
                   const int32_t* host_slot_of_expert, int host_n_slots,
                   int max_swaps, int decay_shift, int32_t* swaps,
                   int32_t* n_swaps, hipStream_t stream);

/* Copy the planned experts: for i < n_swaps, slot swaps[4i] of L's pool
 * receives the slot_bytes of slot swaps[4i+3] of H's pool.  L is the GPU
 * cache (its pool is written); H the host tier (pinned host memory this
 * device can address, or device memory; pageable memory gives MOE_EINVAL).
 * Both must have the same fmt, d_model and d_ff.  Entries whose slots lie
 * outside either pool are skipped.  max_swaps: as given to the plan. */
int moe_cache_fill(const moe_layer* L, const moe_layer* H, const int32_t* swaps,
                   const int32_t* n_swaps, int max_swaps, hipStream_t stream);

/* slot_of_expert[swaps[4i+2]] = swaps[4i] for i < min(n_swaps, max_swaps). */
int moe_cache_commit(int32_t* slot_of_expert, int E, const int32_t* swaps,
                     const int32_t* n_swaps, int max_swaps, hipStream_t stream);

/* Stage a whole layer for a prefill chunk ("Strata" page,
 * "GPU・CPU・RAM・SSDの分担": long inputs are processed 8,192 tokens at a
 * time while the next layer's experts travel to the GPU over PCIe).
 * Copies every expert's packed slot into `staging` in expert order: slot e
 * holds expert e (e < n_experts), slot n_experts the shared expert of C (if
 * C->shared_slot >= 0).  Resident experts (slot_of_expert[e] in C's pool)
 * are copied device to device, the others from H's pool at
 * host_slot_of_expert[e].  Copies go through the DMA engines
 * (hipMemcpyAsync on `stream`), consecutive source slots merged, so on a
 * stream of their own they overlap the compute kernels of the previous
 * layer.  Then moe_expert_ffn_prefill runs on a layer whose pool is
 * `staging` (n_slots = n_experts + 1, shared_slot = n_experts) with the
 * identity slot table, and gives the same bits as with the experts in any
 * other slots.
 *   C: the GPU cache of the layer; H: its host tier (pinned host memory or
 *   device memory; same fmt, d_model, d_ff, n_experts).
 *   slot_of_expert, host_slot_of_expert: (host) int32 [n_experts]; every
 *   expert must be resident in C (not in the shared slot) or have a host
 *   slot in H, else MOE_EINVAL and nothing is copied.
 *   staging: device memory of at least (n_experts + 1) * slot_bytes bytes,
 *   256-byte aligned.  The caller orders the copies after the last kernel
 *   that read `staging` and before the prefill that reads it. */
int moe_stage_layer(const moe_layer* C, const int32_t* slot_of_expert,
                    const moe_layer* H, const int32_t* host_slot_of_expert,
                    void* staging, size_t staging_bytes, hipStream_t stream);

/* (host) Workspace bytes that moe_expert_ffn_prefill needs for T tokens. */
size_t moe_prefill_workspace_bytes(const moe_layer* L, int T);

/* Prefill chunk ("Strata" page, "GPU・CPU・RAM・SSDの分担": up to 8,192
 * tokens at a time).  x_bf16 [T][d_model] bfloat16 bits.  Pairs (t,i) with
 * 0 <= slot[t*k+i] < L->n_slots are grouped by expert id (groups ascending,
 * inside a group by t then i); expert_offsets int32 [E+1] receives the group
 * bounds, pair_pos int32 [T*k] each pair's row in out_pairs (-1 for a miss,
 * which is any other slot value).  For
 * every pair the expert FFN runs with bf16 inputs and weights (weights
 * dequantized to bf16 round-to-nearest-even), fp32 accumulation, and
 * h = silu(g) * u rounded to bf16 before the down product:
 *   out_pairs fp32 [T*k][d_model] (rows past the pair count untouched),
 *   out_shared fp32 [T][d_model] = FFN_shared(x[t]) (NULL if no shared
 *   expert is wanted; must be NULL when shared_slot < 0).
 * moe_combine then forms y.  Limits: 1 <= T <= 65536, d_model a multiple
 * of 128, d_ff a multiple of 64, T * (top_k + 1) * d_ff * 2 < 2^32 (the bf16
 * h rows the GEMMs address with 32-bit offsets).
 * ws: at least moe_prefill_workspace_bytes(L, T) bytes, 256-byte aligned. */
int moe_expert_ffn_prefill(const moe_layer* L, const uint16_t* x_bf16, int T,
                           const int32_t* idx, const int32_t* slot,
                           float* out_pairs, int32_t* pair_pos,
                           int32_t* expert_offsets, float* out_shared,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Routing-weighted combine into the residual ("FreeToken vs Strata",
 * "共通の仕組み": a layer's parts are joined before the next layer).
 *   y[t] = x[t] + sum_{i: pair_pos[t*k+i] >= 0} w[t*k+i] * rows[pair_pos[t*k+i]]
 *               + shared[t]                       (if shared != NULL)
 * summed in i order, shared last, in fp32.  x is fp32 or bf16 bits
 * (x_dtype), [T][d]; rows fp32 [*][d]; y fp32 [T][d] and may alias x only
 * when x is fp32.  d must be a multiple of 4. */
int moe_combine(const void* x, int x_dtype, int T, int d, int k,
                const float* rows, const int32_t* pair_pos, const float* w,
                const float* shared, float* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BITFFN_MOE_H */
