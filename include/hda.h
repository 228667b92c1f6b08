/*
 * hda.h -- dynamic split-KV paged decode attention on MI355X (gfx950).
 *
 * C ABI of libhda.so.  Plain C types and pointers only; no HIP or torch
 * types appear here (a HIP stream is passed as an opaque void*).
 *
 * What the library computes (the method the pages describe as "Dynamic
 * Attention"): one decode step of grouped-query attention for a batch of
 * requests whose cached context lengths differ widely.  A host planner cuts
 * every request's KV range into uniform tiles and spreads the tiles over a
 * fixed set of persistent workgroups, rebuilt each step from the current
 * lengths; the kernel computes per-item partial softmax results and merges
 * partials of one request by log-sum-exp.  Sources: page "Tencent HPC llega
 * a SGLang y desafía a los kernels de inferencia predeterminados"
 * (remio.ai), section "Por qué Tencent HPC importa para el serving de
 * modelos en línea" (uniform tiles assigned to thread blocks by the current
 * workload, rebuilt as lengths change; a static split leaves units idle or
 * launches empty chunks); page "腾讯混元三算子杀入 SGLang…" (arex-research.com),
 * the Dynamic Attention paragraphs (a persistent kernel allocating tiles at
 * every decode step by the actual KV length); page "vLLM × HPC-Ops:
 * High-Performance Attention and MoE Backends from Tencent Hunyuan" (8sync
 * summary): a per-step load-balanced scheduler replacing fixed split-KV,
 * with a fused RoPE + QK-Norm + KV-write prologue.
 *
 * Conventions
 *   - Every function that can fail returns an int status (HDA_OK = 0, errors
 *     negative).  No C++ exception crosses this boundary.
 *   - All memory is owned by the caller, except hda_decode_noalloc's
 *     workspace (a fixed array in the library's device code).  The library
 *     allocates no device memory and never synchronises the stream
 *     (hda_decode_check, a debug aid, does).
 *   - Host pointers are marked [host], device pointers [device].  Device
 *     pointers must stay valid until the work enqueued on the stream ends.
 *   - Functions are reentrant; the only global state is the per-device
 *     address of hda_decode_noalloc's workspace array, set once per device
 *     under a lock.
 */
#ifndef HDA_H
#define HDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HDA_VERSION 1
#define HDA_PLAN_VERSION 1
#define HDA_PLAN_HEADER_INTS 8

/* status codes */
#define HDA_OK 0
#define HDA_ERR_INVALID_ARG (-1)   /* null pointer, non-positive size, bad length */
#define HDA_ERR_CAPACITY (-2)      /* plan buffer too small; *plan_len = ints needed */
#define HDA_ERR_UNSUPPORTED (-3)   /* shape or dtype the library has no kernel for */
#define HDA_ERR_PLAN_MISMATCH (-4) /* plan built for another batch / other lengths */
#define HDA_ERR_HIP (-5)           /* a HIP launch or runtime call failed */
#define HDA_ERR_WORKSPACE (-6)     /* workspace missing or smaller than required */
#define HDA_ERR_BAD_PLAN (-7)      /* plan array malformed (format, coverage, slots) */

/* KV cache element types */
#define HDA_KV_BF16 0      /* bfloat16 */
#define HDA_KV_FP8_E4M3 1  /* OCP FP8 E4M3FN code, value = decode(code) * scale */

/* Scale granularity (hda_params.scale_mode).  The value of a stored K
 * element is decode(element) * k_scale * f, where f is
 *   HDA_SCALE_TENSOR  1
 *   HDA_SCALE_HEAD    k_scales[h]                    (float [Hkv])
 *   HDA_SCALE_PAGE    k_scales[page * Hkv + h]       (float [num_pages][Hkv]),
 *                     page = the physical page holding the row
 * for kv head h; V likewise with v_scale and v_scales.  The pages name
 * quantisation scales as a per-model integration parameter without fixing a
 * granularity (remio.ai page, section "Lo que la afirmación de un 48,8 % de
 * TPOT no demuestra"); these three cover the usual cache quantisers. */
#define HDA_SCALE_TENSOR 0
#define HDA_SCALE_HEAD 1
#define HDA_SCALE_PAGE 2   /* fp8 cache only */

/* Product arithmetic (hda_params.math).
 *   HDA_MATH_BF16  cache elements widened exactly to bf16, q in bf16,
 *                  softmax weights rounded to bf16; fp32 accumulation
 *   HDA_MATH_FP8   fp8 cache only: QK^T and PV on fp8 matrix-core operands.
 *                  q is quantised per (request, q head) with scale
 *                  s = amax/448 as x = q/s (float32) = hi + lo/16, hi =
 *                  E4M3(x), lo = E4M3(16 (x - hi)), both round-to-nearest-
 *                  even (two QK products: the high part and the residual
 *                  kept at 16x scale, as the pages' Router GEMM keeps its
 *                  weights: remio.ai page, Router GEMM section); the
 *                  softmax weights z = p 2^8 enter PV as E4M3(z) plus
 *                  the E4M3 of its residual (two products into one
 *                  accumulator), the normaliser summing the same weights.
 *                  Needs v_layout HDA_V_DIM_MAJOR, D 128,
 *                  page_size >= 64 and tensor or head scales.
 * The pages report FP8 execution and name cache precision as a setting the
 * results depend on (remio.ai page, section "Lo que la afirmación de un
 * 48,8 % de TPOT no demuestra"); fp8 attention arithmetic is this library's
 * own option. */
#define HDA_MATH_BF16 0
#define HDA_MATH_FP8 1

/* V page layout (hda_params.v_layout); K pages are always token-major.
 *   HDA_V_TOKEN_MAJOR  [num_pages][Hkv][page_size][D]
 *   HDA_V_DIM_MAJOR    [num_pages][Hkv][D][page_size]: the tokens of one
 *                      head dim are contiguous (the V layout of the original
 *                      vLLM paged-attention cache); HDA_MATH_FP8 only */
#define HDA_V_TOKEN_MAJOR 0
#define HDA_V_DIM_MAJOR 1

/*
 * Plan format (int32 array), produced by hda_plan / hda_plan_static:
 *   [0..7]   header: VERSION, B, tile_len (0 for a static plan), W, T, N, P, 0
 *            W workgroups, T tiles (chunks for a static plan), N items,
 *            P partial slots
 *   [8 ..]   wg_ptr[W+1]: items of workgroup w are wg_ptr[w] .. wg_ptr[w+1]-1
 *   then     items[N][4] = (b, kv_begin, kv_end, slot); slot -1 means the item
 *            covers its whole request and writes the output directly
 *   then     req_part_ptr[B+1]: partial slots of request b are
 *            req_part_ptr[b] .. req_part_ptr[b+1]-1
 * Items of one request appear in token order and tile [0, len_b) exactly once.
 * Total length: 8 + (W+1) + 4N + (B+1) ints.
 */

/*
 * Upper bound on the plan length for `batch` requests over `n_workgroups`
 * workgroups: 8 + (W+1) + 4(W+B-1) + (B+1).  Also bounds a static plan with
 * n_workgroups = batch * n_splits.  Returns -1 for non-positive arguments.
 * (The plan is the per-step tile assignment of the remio.ai page, section
 * "Por qué Tencent HPC importa para el serving de modelos en línea".)
 */
int64_t hda_plan_capacity(int32_t batch, int32_t n_workgroups);

/*
 * Per-step tile plan: the planner the remio.ai page describes (section "Por
 * qué Tencent HPC importa para el serving de modelos en línea": each
 * request's KV work cut into uniform tiles and assigned to thread blocks by
 * the current workload, rebuilt as lengths change; arex-research page,
 * Dynamic Attention paragraphs: tiles allocated every decode step by the
 * actual KV length).  Tiles of `tile_len` tokens are taken request-major
 * (tile j of request b covers [j*tile_len, min((j+1)*tile_len, len_b)));
 * the T tiles are split contiguously over the W workgroups, the first
 * (T mod W) taking one extra; consecutive tiles of one request within a
 * workgroup form one item; requests with more than one item get partial
 * slots numbered in item order.  Cost O(B + W + N), no allocation.
 *
 *   seq_lens   [host] int32[batch], every length >= 1 (the current KV length,
 *              including a new token the prologue will write)
 *   plan       [host] output array of `capacity` ints (may be NULL when
 *              capacity is 0, to query the size)
 *   plan_len   [host] receives the number of ints used (or needed)
 * Errors: HDA_ERR_INVALID_ARG (null pointers, batch/tile_len/W < 1, a length
 * < 1, T or W+B beyond int32), HDA_ERR_CAPACITY (buffer too small).
 */
int hda_plan(const int32_t* seq_lens, int32_t batch, int32_t tile_len,
             int32_t n_workgroups, int32_t* plan, int64_t capacity,
             int64_t* plan_len);

/*
 * A launch width for hda_plan: *n_workgroups = W for tiles of tile_len over
 * seq_lens [host] int32[batch] (each >= 1), at most W_max = the width that
 * puts wg_per_cu workgroups on each of n_cu compute units over all
 * n_kv_heads (and at most the tile count).  The step lasts about as long as
 * its busiest unit, which holds ceil(W Hkv / n_cu) workgroups of
 * ceil(T / W) tiles; among the widths whose busiest unit holds at most 1/32
 * more tiles than the least possible, the one with the fewest partial
 * slots, then the widest.  (The pages size the tiles and their assignment
 * to the current workload: remio.ai page, section "Por qué Tencent HPC
 * importa para el serving de modelos en línea"; the width rule is this
 * library's.)  Cost O(batch x W_max).  Errors: HDA_ERR_INVALID_ARG.
 */
int hda_launch_config(const int32_t* seq_lens, int32_t batch, int32_t n_kv_heads, int32_t n_cu,
                      int32_t wg_per_cu, int32_t tile_len, int32_t* n_workgroups);

/*
 * Static split baseline -- the fixed split-KV schedule the pages compare
 * against (remio.ai page, same section: a static split leaves units idle or
 * launches empty chunks; "vLLM × HPC-Ops" summary: fixed split-KV
 * scheduling) -- in the same format: request b is cut into n_splits
 * chunks [floor(c*len_b/S), floor((c+1)*len_b/S)), chunk c handled by
 * workgroup b*S + c (W = B*S); empty chunks leave their workgroup without an
 * item.  This is the fixed split-KV schedule the dynamic plan is compared to.
 * Errors as hda_plan.
 */
int hda_plan_static(const int32_t* seq_lens, int32_t batch, int32_t n_splits,
                    int32_t* plan, int64_t capacity, int64_t* plan_len);

/*
 * Checks a plan (the tile assignment of the remio.ai page's planner, section
 * "Por qué Tencent HPC importa para el serving de modelos en línea")
 * against the lengths it will be used with: format and total
 * length, wg_ptr monotone, items in range and covering each [0, len_b)
 * exactly once in token order, slot numbering, and (for a dynamic plan) the
 * tile count.  [host] pointers.  Returns HDA_OK, HDA_ERR_INVALID_ARG,
 * HDA_ERR_PLAN_MISMATCH (batch or lengths differ) or HDA_ERR_BAD_PLAN.
 */
int hda_plan_validate(const int32_t* plan, int64_t plan_len,
                      const int32_t* seq_lens, int32_t batch);

/*
 * Bytes of workspace hda_decode needs for this plan, in this order, each
 * region starting on a 256-byte boundary: the device check words int32
 * [W][Hkv] (one per tile workgroup, rewritten by every call; read by
 * hda_decode_check), partial outputs float32 [P][Hq][D], partial
 * log-sum-exp float32 [P][Hq], the prologue's normalised, rotated q as bf16
 * [B][Hq][D] (used only when the prologue is on), and per-request slot
 * ranges int32 [B][2] (written by the tile kernel when the plan is built on
 * the device or travels in the launch arguments, and read by the merge).
 * Its contents need no initialisation.  Returns -1 for a malformed plan
 * header or non-positive sizes.  The plan is the one described above
 * (remio.ai page, section "Por qué Tencent HPC importa para el serving de
 * modelos en línea": the split requests' partial results are what the
 * workspace holds).
 */
int64_t hda_workspace_bytes(const int32_t* plan, int64_t plan_len,
                            int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim);

/* Shapes, dtypes, scales, prologue inputs and workspace of a step: the
 * inputs the pages' attention backend takes from the serving framework's KV
 * cache (remio.ai page, section "Lo que la afirmación de un 48,8 % de TPOT
 * no demuestra": head dims, cache layout, quantisation scales, RoPE and
 * normalisation are per-model parameters). */
typedef struct hda_params {
  int32_t batch;              /* B, must equal the plan's batch */
  int32_t n_q_heads;          /* Hq; Hq / Hkv (the group) in 1..16 */
  int32_t n_kv_heads;         /* Hkv */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t page_size;          /* tokens per page: power of two, 16..1024 */
  int32_t max_pages_per_req;  /* row length of block_table */
  int64_t num_pages;          /* pages in each pool; ids outside are never read */
  int32_t kv_dtype;           /* HDA_KV_BF16 or HDA_KV_FP8_E4M3 */
  float sm_scale;             /* softmax scale, e.g. 1/sqrt(D) */
  float k_scale;              /* per-tensor scale of K: value = stored * k_scale
                                 (either dtype; 1 for a plain bf16 cache) */
  float v_scale;              /* per-tensor scale of V, likewise */
  /* fused new-token prologue (RMSNorm then rotate-half RoPE on q and k, then
   * k and v stored into slot len_b - 1 of the cache, then attention) */
  int32_t prologue;           /* 0 off, 1 on */
  float rms_eps;
  float rope_theta;
  const void* q_norm_w;       /* [device] bf16 [D] */
  const void* k_norm_w;       /* [device] bf16 [D] */
  const void* k_new;          /* [device] bf16 [B][Hkv][D], pre-norm k of the new token */
  const void* v_new;          /* [device] bf16 [B][Hkv][D] */
  /* scratch for split requests' partial results, hda_workspace_bytes()
   * bytes, any contents; calls sharing a workspace must be ordered on one
   * stream */
  void* workspace;            /* [device] */
  int64_t workspace_bytes;
  /* optional profiling hook: a hipEvent_t recorded on the stream between the
   * tile kernel and the merge kernel; NULL for none */
  void* split_event;
  /* scale granularity (HDA_SCALE_*) and, for HEAD and PAGE, the factor
   * arrays: positive finite floats, read on the device, never written.  The
   * prologue stores the new token with the scale of its slot (it never
   * changes a scale: a caller that rescales a page does so itself). */
  int32_t scale_mode;
  int32_t math;               /* HDA_MATH_BF16 or HDA_MATH_FP8 */
  const float* k_scales;      /* [device] [Hkv] or [num_pages][Hkv]; NULL for TENSOR */
  const float* v_scales;      /* [device] likewise */
  int32_t v_layout;           /* HDA_V_TOKEN_MAJOR or HDA_V_DIM_MAJOR */
  int32_t reserved0;          /* must be 0 */
} hda_params;

/* Longest plan hda_decode accepts in its launch arguments (plan_dev NULL). */
#define HDA_PLAN_ARG_INTS 896

/*
 * One decode step -- the pages' "Dynamic Attention": single-token decode
 * attention over the paged KV cache by the per-step tile plan, per-item
 * partial softmax results merged by log-sum-exp (remio.ai page, section "Por
 * qué Tencent HPC importa para el serving de modelos en línea";
 * arex-research page, Dynamic Attention paragraphs; the fused RoPE +
 * QK-Norm + KV-write prologue of the "vLLM × HPC-Ops" summary) -- enqueued
 * on `stream`: the optional new-token prologue
 * kernel (RMSNorm + RoPE of q and k, k/v stored to slot len-1, all fused in
 * one kernel), the tile attention kernel, then the log-sum-exp merge of
 * split requests (only when the plan has partial slots).  Asynchronous; no
 * host synchronisation, no allocation.
 *
 *   q            [device] bf16 [B][Hq][D] (pre-norm when the prologue is on)
 *   k_pages,
 *   v_pages      [device] page pools [num_pages][Hkv][page_size][D] of bf16
 *                or fp8 codes; written only by the prologue (slot len_b-1)
 *   block_table  [device] int32 [B][max_pages_per_req]; token t of request b
 *                is row t % page_size of page block_table[b][t / page_size]
 *   seq_lens     [device] int32 [B], the lengths the plan was built for (see
 *                the device check below when they may differ)
 *   plan_host    [host] the plan (header read for the launch shape)
 *   plan_dev     [device] an identical copy of the plan, plan_len ints; or
 *                NULL when plan_len <= HDA_PLAN_ARG_INTS: the plan then
 *                travels in the tile kernel's launch arguments (no upload
 *                on the stream; plan_host is free once the call returns),
 *                and the tile kernel records each request's slot range in
 *                the workspace for the merge
 *   out          [device] float32 [B][Hq][D]
 *   stream       hipStream_t, or NULL for the default stream
 * q head h reads kv head floor(h * Hkv / Hq).  Rows past len_b are never
 * used, whatever they hold: every item's range is cut at the device length
 * seq_lens[b] before its tokens are read or scored.
 * Device check: the plan and the device lengths can disagree (a plan kept
 * from an earlier step while lengths changed -- the pages require the tiles
 * to be rebuilt as lengths change: remio.ai page, section "Por qué Tencent
 * HPC importa para el serving de modelos en línea").  Each tile workgroup
 * records in its check word whether one of its items ended past its
 * request's device length (HDA_CHECK_PAST_LEN: those tokens were masked, so
 * the output is still exact attention over seq_lens[b] as long as every
 * token below it is covered) or whether a request's last item ended before
 * it (HDA_CHECK_SHORT: the tokens after the plan's end were not attended).
 * hda_decode_check reads the words back.  The words live in the workspace;
 * without a workspace (P = 0, no prologue) nothing is recorded.
 * Errors (all detected on the host before any launch): HDA_ERR_INVALID_ARG,
 * HDA_ERR_UNSUPPORTED (also: plan_dev NULL with a longer plan),
 * HDA_ERR_PLAN_MISMATCH, HDA_ERR_BAD_PLAN (header, length or workgroup item
 * ranges), HDA_ERR_WORKSPACE (workspace missing or too small); HDA_ERR_HIP if
 * a launch fails.  Device faults
 * surface at the caller's next synchronisation.
 */
int hda_decode(const hda_params* p, const void* q, void* k_pages,
               void* v_pages, const int32_t* block_table,
               const int32_t* seq_lens, const int32_t* plan_host,
               const int32_t* plan_dev, int64_t plan_len, float* out,
               void* stream);

/* Workspace bytes available to hda_decode_noalloc (16 MiB). */
#define HDA_NOALLOC_WORKSPACE_BYTES 16777216

/*
 * hda_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and results, with the workspace taken from an array the
 * library keeps in device memory -- HDA_NOALLOC_WORKSPACE_BYTES on every GPU
 * it runs on, held until the process ends -- instead of p->workspace and
 * p->workspace_bytes, which are ignored.  The caller still passes every
 * input and output.  A plan whose hda_workspace_bytes exceeds that size
 * returns HDA_ERR_WORKSPACE before any launch.  Every call on one GPU shares
 * its array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that overlap on one GPU -- on different streams, or
 * from threads without ordering -- race; order them on one stream.  The
 * device check words go to that array and hda_decode_check cannot read
 * them.  `stream` must belong to the current device (else
 * HDA_ERR_INVALID_ARG); the first call on each device looks up the array's
 * address (HDA_ERR_HIP if that fails).  Allocates nothing, on the device or
 * in any library it calls.  Other arguments and errors as hda_decode.
 */
int hda_decode_noalloc(const hda_params* p, const void* q, void* k_pages, void* v_pages,
                       const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* plan_host, const int32_t* plan_dev, int64_t plan_len,
                       float* out, void* stream);

/*
 * Debug form of hda_decode (plan in device memory, plan_dev not NULL) that
 * also counts coverage: every token a tile wave scores adds one visit to
 * its cache row for its kv head, in visits [device] int32
 * [num_pages][page_size][Hkv] (index (page * page_size + row) * Hkv + h),
 * which the caller zeroes first.  A plan that tiles each [0, len_b) exactly
 * once leaves 1 on every row below len_b of every request -- a row shared
 * by several requests' block tables, once per request -- and 0 elsewhere.
 * The pages' planner hands every tile of every request to exactly one
 * thread block (remio.ai page, section "Por qué Tencent HPC importa para el
 * serving de modelos en línea"); this checks the kernels' loops keep that.
 * Outputs as hda_decode (slower: one atomic add per token and kv head).
 * Errors as hda_decode; HDA_ERR_INVALID_ARG also for visits or plan_dev NULL.
 */
int hda_decode_coverage(const hda_params* p, const void* q, void* k_pages, void* v_pages,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* plan_host, const int32_t* plan_dev, int64_t plan_len,
                        float* out, int32_t* visits, void* stream);

/* Device check bits (hda_decode_check). */
#define HDA_CHECK_PAST_LEN 1  /* an item reached past its request's device length (masked) */
#define HDA_CHECK_SHORT 2     /* a request's last item ended before its device length */

/*
 * Reads the device check words the last hda_decode, hda_decode_auto or
 * hda_prefill call with this workspace wrote: n_workgroups (the plan's W)
 * times p->n_kv_heads int32 words at the start of p->workspace.  Waits for
 * `stream` (the stream of that call) to finish, then copies the words to the
 * host; *flags receives their bitwise OR (HDA_CHECK_* bits).  Returns HDA_OK
 * when no bit is set, HDA_ERR_PLAN_MISMATCH when one is, HDA_ERR_INVALID_ARG
 * (null pointers, n_workgroups < 1, a workspace too small for the words) or
 * HDA_ERR_HIP.  A device-planned call always records 0 (its plan is built
 * from the device lengths).  This is a synchronising debug aid, not part of
 * the per-step path.
 */
int hda_decode_check(const hda_params* p, int32_t n_workgroups, int32_t* flags, void* stream);

/*
 * The same decode step with the plan built on the device: each workgroup
 * derives its own items from the device lengths with exactly the hda_plan
 * rule (request-major tiles of tile_len, contiguous balanced split over
 * n_workgroups), so no host planning or plan upload is needed per step and
 * the step has fixed arguments (it can be captured in a HIP graph while the
 * lengths change in device memory).  This follows the persistent kernel of
 * the arex-research page that allocates tiles every decode step by the
 * actual KV length.
 *
 *   seq_lens    [device] int32 [B], every length >= 1 (a request with a
 *               length < 1 gets no item and its output rows are not written)
 *   workspace   at least hda_workspace_bytes_bound(B, n_workgroups, Hq, D)
 * Other arguments and errors as hda_decode.  Outputs are bitwise identical
 * to hda_decode with hda_plan(seq_lens, B, tile_len, n_workgroups).
 */
int hda_decode_auto(const hda_params* p, const void* q, void* k_pages, void* v_pages,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int32_t tile_len, int32_t n_workgroups, float* out, void* stream);

/*
 * Workspace bytes that suffice for any plan over `batch` requests and
 * `n_workgroups` workgroups (partial slots <= W + B - 1), in the layout of
 * hda_workspace_bytes (the check words counted as W x Hq, a bound on
 * W x Hkv).  -1 for non-positive arguments.
 */
int64_t hda_workspace_bytes_bound(int32_t batch, int32_t n_workgroups,
                                  int32_t n_q_heads, int32_t head_dim);

/*
 * Writes, on `stream`, the hda_plan-format plan for the device lengths
 * `seq_lens` [device] into `plan` [device] (capacity ints, at least
 * hda_plan_capacity(batch, n_workgroups)), computed on the GPU with the
 * device-side planning of hda_decode_auto.  Asynchronous.  Errors:
 * HDA_ERR_INVALID_ARG, HDA_ERR_CAPACITY, HDA_ERR_HIP.
 */
int hda_plan_device(const int32_t* seq_lens, int32_t batch, int32_t tile_len,
                    int32_t n_workgroups, int32_t* plan, int64_t capacity, void* stream);

/* Plan ints carried by one launch of hda_plan_upload. */
#define HDA_PLAN_UPLOAD_CHUNK 1000

/*
 * Copies a host plan (plan_len ints, any size) to plan_dev [device, 4-byte
 * aligned] on `stream` inside the kernel arguments of a small store kernel,
 * one launch per HDA_PLAN_UPLOAD_CHUNK ints: the per-step upload of the plan
 * (the arex-research page has the tile allocation redone every decode step)
 * without a separate copy on the stream.  Launch arguments are copied when
 * the launch is enqueued, so plan_host may be pageable memory and may be
 * reused as soon as the call returns.  Asynchronous on the device.  Any
 * int32 array travels the same way (hda_prefill's row blocks and plan side
 * by side in one buffer, for one launch).  Errors: HDA_ERR_INVALID_ARG (null
 * pointer, plan_len < 1, misaligned plan_dev), HDA_ERR_HIP (a launch failed).
 */
int hda_plan_upload(const int32_t* plan_host, int64_t plan_len, int32_t* plan_dev,
                    void* stream);

/* Largest row block of hda_prefill, in units of hda_prefill_rows_per_block(). */
#define HDA_PREFILL_MAX_TILES 16

/*
 * ---- Multi-token queries (prefill, chunked prefill, speculative checks) ----
 *
 * The backend's attention also serves the prefill phase (the pages report
 * lower time to first token: remio.ai page, section "Por qué Tencent HPC
 * importa para el serving de modelos en línea") but describe no prefill
 * algorithm.  Here: request b brings q_len_b new query rows whose K and V are
 * already in the cache, which holds kv_len_b >= q_len_b tokens; row r sits at
 * position kv_len_b - q_len_b + r and attends causally to tokens 0..pos.
 * q and out are packed request after request: [sum q_len][Hq][D].
 *
 * The rows of each request are grouped into blocks; the (row, q head) pairs
 * of hda_prefill_rows_per_block() rows -- a tile -- fill the 16 matrix-core
 * columns the decode kernel gives one kv head's q heads.  Each block enters
 * the decode tile planner as one "request" whose length is its causal
 * extent, so hda_plan is used unchanged (its batch = the number of blocks)
 * and a block's partial results are merged as a request's are.  The largest
 * block picks the kernel shape:
 *   1 tile        the decode kernel's column shape, an item's chunks split
 *                 over the 4 waves;
 *   2 to 4 tiles  each K/V chunk loaded once into LDS and shared by 4 waves,
 *                 wave w taking tile w;
 *   5 to 8 tiles  the same with 8 waves;
 *   9 to 16       8 waves, wave w taking tiles w and w + 8.
 * K/V bytes requested per query row fall with the block size; a block longer
 * than a request's run leaves tiles idle (hda_prefill_block_rows picks one).
 */

/* Rows per block that fill the 16 columns (one tile): 16 / (Hq / Hkv), or
 * -1 for a group above 16.  hda_prefill accepts blocks of up to
 * HDA_PREFILL_MAX_TILES times this many rows. */
int32_t hda_prefill_rows_per_block(int32_t n_q_heads, int32_t n_kv_heads);

/* A block size for a batch: 1, 2, 4, 8 or 16 tiles of hda_prefill_rows_per_block
 * rows, the smallest power of two at least the mean query run
 * (q_lens [host] int32[batch], each >= 1) in tiles, at most
 * HDA_PREFILL_MAX_TILES.  -1 on a bad argument or group. */
int32_t hda_prefill_block_rows(const int32_t* q_lens, int32_t batch, int32_t n_q_heads,
                               int32_t n_kv_heads);

/*
 * The row blocks of a batch.  q_lens, kv_lens [host] int32[batch] with
 * 1 <= q_len <= kv_len.  Writes rows [host] int32[n][4] = (request, packed
 * index of the first row, rows in the block, position of the first row) and
 * row_lens [host] int32[n] (position of the last row + 1: the lengths to give
 * hda_plan), blocks in request order.  *n_rows receives n (also when the
 * buffers are NULL or smaller than capacity, which returns HDA_ERR_CAPACITY).
 * Errors: HDA_ERR_INVALID_ARG, HDA_ERR_CAPACITY.
 */
int hda_prefill_rows(const int32_t* q_lens, const int32_t* kv_lens, int32_t batch,
                     int32_t rows_per_block, int32_t* rows, int32_t* row_lens,
                     int64_t capacity, int64_t* n_rows);

/* Workspace bytes for hda_prefill with this plan and blocks of at most
 * rows_per_block rows (1 .. HDA_PREFILL_MAX_TILES x
 * hda_prefill_rows_per_block): the device check words int32 [W][Hkv] (as
 * for hda_decode), partial outputs float32 [P][rows_per_block][Hq][D], then
 * partial log-sum-exps float32 [P][rows_per_block][Hq], each region aligned
 * to 256 bytes (hda_prefill lays them out with the largest block's row
 * count).  -1 on a malformed header or sizes. */
int64_t hda_prefill_workspace_bytes(const int32_t* plan, int64_t plan_len, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim,
                                    int32_t rows_per_block);

/*
 * One multi-token attention step enqueued on `stream`: the tile kernel over
 * the plan's items (each covering a row block's KV range), then the
 * log-sum-exp merge of split blocks.  Asynchronous; allocates nothing.
 *
 *   p            as for hda_decode, with batch = B requests; prologue 0,
 *                math HDA_MATH_BF16, v_layout HDA_V_TOKEN_MAJOR (other
 *                settings: HDA_ERR_UNSUPPORTED); all scale modes
 *   q            [device] bf16 [n_q][Hq][D], packed
 *   block_table  [device] int32 [B][max_pages_per_req]
 *   kv_lens      [device] int32 [B], cache lengths (new rows included)
 *   n_q          total query rows (sum of q_len)
 *   rows_host,
 *   rows_dev     [host] and [device] copies of hda_prefill_rows' blocks,
 *                n_rows = the plan's batch
 *   plan_host,
 *   plan_dev     hda_plan(row_lens, n_rows, tile_len, W), as for hda_decode
 *   out          [device] float32 [n_q][Hq][D]
 * Tokens at or past kv_lens[b] are never scored (an item's range is cut at
 * the device length); an item that reached past it sets HDA_CHECK_PAST_LEN
 * in its workgroup's check word (hda_decode_check with the plan's W).
 * Errors (host, before any launch): HDA_ERR_INVALID_ARG (incl. a block out
 * of range or with more than HDA_PREFILL_MAX_TILES x
 * hda_prefill_rows_per_block rows),
 * HDA_ERR_UNSUPPORTED, HDA_ERR_BAD_PLAN (header, length or workgroup item
 * ranges), HDA_ERR_WORKSPACE; HDA_ERR_HIP if a launch fails.
 */
int hda_prefill(const hda_params* p, const void* q, const void* k_pages, const void* v_pages,
                const int32_t* block_table, const int32_t* kv_lens, int32_t n_q,
                const int32_t* rows_host, const int32_t* rows_dev, const int32_t* plan_host,
                const int32_t* plan_dev, int64_t plan_len, float* out, void* stream);

/*
 * ---- Router GEMM (MoE expert-selection logits) ----
 *
 * The router multiplies bf16 activations by fp32 weights whose small
 * differences can change the selected experts.  The pages describe keeping
 * each fp32 weight as two bf16 parts -- the high part and a residual stored
 * with a scale of 1/256 -- and running the two bf16 products in one kernel
 * that shares the input loads, keeps both accumulators in registers and
 * writes the combined result once (remio.ai page, Router GEMM section;
 * arex-research page, Router GEMM paragraph).  Here hi = bf16(w),
 * lo = bf16(256 (w - hi)), both round-to-nearest-even, and
 *   out[t][e] = sum_h x[t][h] hi[e][h] + (sum_h x[t][h] lo[e][h]) / 256
 * with fp32 accumulation.
 */

/* Splits fp32 weights [device] w[n] into hi and lo [device] bf16[n] on
 * `stream` (a one-time weight preparation).  Errors: HDA_ERR_INVALID_ARG,
 * HDA_ERR_UNSUPPORTED, HDA_ERR_HIP. */
int hda_router_split_weights(const float* w, int64_t n, void* w_hi, void* w_lo, void* stream);

/* Workspace bytes hda_router_gemm needs for this shape (0 when none), or -1
 * for a shape it does not take (hidden not a positive multiple of 32). */
int64_t hda_router_workspace_bytes(int32_t tokens, int32_t experts, int32_t hidden);

/*
 * Logits out[tokens][experts] (fp32, [device]) = x w^T from
 *   x      [device] bf16 [tokens][hidden], 16-byte aligned
 *   w_hi,
 *   w_lo   [device] bf16 [experts][hidden] from hda_router_split_weights
 * hidden must be a multiple of 32; tokens x hidden and experts x hidden
 * below 2^30.  The workspace (hda_router_workspace_bytes; [device],
 * 16-byte aligned, any content -- nothing needs clearing) holds partial
 * tiles when the hidden dimension is split across workgroups, and for 9 to
 * 64 tokens one arrival counter per output tile as well: the last
 * workgroup of a tile to finish adds its partials, so the call is one
 * launch.  Partials are added in a fixed (slot) order, so results do not
 * vary between runs.  Calls that overlap in time on one workspace race.
 * Asynchronous on `stream`.  Errors: HDA_ERR_INVALID_ARG (also a workspace
 * not 16-byte aligned), HDA_ERR_UNSUPPORTED, HDA_ERR_WORKSPACE, HDA_ERR_HIP.
 */
int hda_router_gemm(const void* x, const void* w_hi, const void* w_lo, int32_t tokens,
                    int32_t experts, int32_t hidden, float* out, void* workspace,
                    int64_t workspace_bytes, void* stream);

/*
 * ---- Measurement ----
 *
 * Not part of the attention method: a streaming-read probe that gives the
 * attention roofline a measured ceiling next to the published 8 TB/s.  One
 * kernel on `stream` reads buf [device] (16-byte aligned; bytes a multiple
 * of 16) once with the attention kernels' access pattern -- each wave a
 * contiguous region, 16-byte non-temporal loads, sixteen in flight per lane --
 * over n_workgroups workgroups of 256 threads, and writes to sink [device]
 * uint32[n_workgroups * 256] the XOR of the words each thread read (their
 * XOR is the XOR of the whole buffer).  The caller times it.  Asynchronous.
 * Errors: HDA_ERR_INVALID_ARG, HDA_ERR_HIP.
 */
int hda_read_probe(const void* buf, int64_t bytes, int32_t n_workgroups, uint32_t* sink,
                   void* stream);

/* Static description of a status code (this library's error convention;
 * the pages define none). */
const char* hda_status_string(int status);

/* HDA_VERSION of the built library. */
int hda_version(void);

/* sizeof(hda_params) as the library was compiled, for bindings that lay the struct out
 * themselves. */
int64_t hda_params_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* HDA_H */
