/*
 * pkvmla.h -- batched paged-KV Multi-head Latent Attention decode, absorbed
 * form, for AMD Instinct MI355X (gfx950).  Plain C ABI: no HIP, no torch types.
 *
 * What is computed.  Every request b has one query token with H heads.  All
 * heads share one compressed KV "head" per token: a ckv row of
 * head_dim_ckv = kv_lora_rank (512) values and a kpe row of
 * head_dim_kpe = qk_rope_head_dim (64) values (vLLM-metax pull request
 * "[WIP] support flashinfer_mla", review of the decode_wrapper.plan call).
 * For each head h and each of the kv_len[b] tokens t of request b:
 *     s_t    = sm_scale * (q_nope[b,h] . ckv_t + q_pe[b,h] . kpe_t)
 *     out    = sum_t softmax(s)_t * ckv_t                 (bf16, fp32 accumulation)
 *     lse    = ln sum_t exp(s_t)                          (fp32, natural log)
 * Attention is not causal (the same review sets causal=False) and the default
 * scale is 1/sqrt(ckv_dim + kpe_dim).
 *
 * Paged cache.  Token t of request b is stored in page
 * kv_indices[kv_indptr[b] + t / page_size] at slot t % page_size.  The
 * descriptors follow the same pull request's metadata review: an indptr of
 * batch+1 entries and a per-request length array of batch entries, both host
 * arrays; there is no last_page_len for MLA.  Slots past kv_len and pages no
 * request lists are never read.
 *
 * Cascade.  A two-level plan attends each request to a prefix page list shared
 * by its group, then to its own suffix pages, and merges the two states by
 * log-sum-exp; the result equals flat attention over prefix-then-suffix tokens
 * (vLLM pull request "[V1][Core] FlashInfer attention backend for V1", which
 * requires cascade and normal attention to agree, with KV dtype = query dtype).
 *
 * Device tensor layouts (all contiguous, row-major, bf16 unless noted):
 *     q_nope    [batch, num_heads, 512]
 *     q_pe      [batch, num_heads, 64]
 *     ckv_cache [num_pages, page_size, 512]
 *     kpe_cache [num_pages, page_size, 64]
 *     out       [batch, num_heads, 512]
 *     lse       [batch, num_heads]            float32
 * Device pointers must be 16-byte aligned.
 *
 * Errors.  Every call returns a pkvmla_status; on failure
 * pkvmla_last_error() returns a message for the calling thread.  An
 * unsupported request is a hard error, never a silent fallback.
 */
#ifndef PKVMLA_H_
#define PKVMLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKVMLA_OK = 0,
  PKVMLA_EINVAL = 1,       /* malformed argument (null pointer, bad indptr, ...) */
  PKVMLA_EUNSUPPORTED = 2, /* well-formed but not supported (dims, heads, page size) */
  PKVMLA_EHIP = 3,         /* HIP runtime or launch failure */
  PKVMLA_ENOMEM = 4        /* device allocation failed */
} pkvmla_status;

typedef struct pkvmla_plan_s* pkvmla_plan;

/* Build a flat decode plan.
 *   batch >= 1 (an empty batch is PKVMLA_EINVAL: a caller skips the run).
 *   kv_indptr  host int32[batch+1]: kv_indptr[0] == 0, non-decreasing.
 *   kv_indices host int32[kv_indptr[batch]]: page ids in [0, num_pages).
 *   kv_lens    host int32[batch]: 1 <= kv_lens[b] <= pages(b) * page_size.
 *   num_heads in {16, 32, 64, 128}; ckv_dim must be 512 and kpe_dim 64 (a
 *   ckv_dim equal to the KV head count, 1, is the mistake the plan review
 *   flags, and is rejected); page_size a power of two in [1, 256].
 *   sm_scale: 0 selects 1/sqrt(ckv_dim + kpe_dim); otherwise finite and > 0.
 *   stream: hipStream_t (as void*) used for the table upload; 0 = null stream.
 * The host arrays are read during the call only.  The plan owns device copies
 * of the page table and of the work schedule, and its split workspace; it is
 * bound to the device that was current at creation.  Output: *out. */
int pkvmla_plan_create(const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* kv_lens, int32_t batch, int32_t num_pages,
                       int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim,
                       int32_t page_size, float sm_scale, void* stream,
                       pkvmla_plan* out);

/* Build a flat decode plan whose device tables, split workspace and launch
 * shapes are sized once for later page-table updates (pkvmla_plan_update),
 * so that a HIP graph captured around pkvmla_run stays valid while the
 * batch's pages and lengths change between replays.  The vLLM pull-request
 * page "[WIP][Kernel] Flashinfer MLA support" reports graph capture of the
 * MLA decode path as the recurring failure; this is the capture-safe form.
 *   Arguments as pkvmla_plan_create, plus
 *   index_capacity: the most page ids (kv_indptr[batch]) any later update may
 *   bring, >= the first table's count; 0 builds an ordinary plan (exact launch
 *   shapes, as pkvmla_plan_create).
 * With index_capacity > 0 every pkvmla_run launches the decode kernel over
 * all schedule lanes (lanes without work return at once) and the merge
 * kernel over one record slot per request (unused slots are skipped), so the
 * sequence of kernels and their arguments never changes.  Units, partial
 * slots and lanes need no capacity: a lane boundary splits at most one
 * request, so units <= batch + lanes always.  Output: *out. */
int pkvmla_plan_create_with_capacity(const int32_t* kv_indptr, const int32_t* kv_indices,
                                     const int32_t* kv_lens, int32_t batch, int32_t num_pages,
                                     int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim,
                                     int32_t page_size, float sm_scale, int64_t index_capacity,
                                     void* stream, pkvmla_plan* out);

/* Replace a flat plan's page table and lengths (same batch; host arrays as in
 * pkvmla_plan_create, read during the call only) and recompute its schedule,
 * in place, without allocation.  A plan built with an index_capacity keeps
 * every pointer and launch shape, so a graph captured around pkvmla_run stays
 * valid.  An ordinary plan (index_capacity 0) accepts updates up to its first
 * table's page count, but its launch shapes follow the new schedule: eager
 * runs after the update are correct, a graph captured before it is not.  The new tables
 * are copied on `stream` and the call waits for that copy, so every run queued
 * earlier on `stream` has finished with the old tables and every later run
 * (eager, or a graph replayed on `stream`) sees the new ones; work on other
 * streams must be ordered by the caller.  PKVMLA_EINVAL when the arrays are
 * malformed or kv_indptr[batch] exceeds the plan's page-id capacity (the
 * plan is then unchanged, as it is for a cascade plan, which takes
 * pkvmla_plan_update_cascade). */
int pkvmla_plan_update(pkvmla_plan plan, const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* kv_lens, void* stream);

/* Build a plan in which request b brings qo_len(b) = qo_indptr[b+1] - qo_indptr[b]
 * new query tokens instead of one (speculative or multi-token decode, and the
 * prefill/decode mixes of the "[V1][Core] FlashInfer attention backend for V1"
 * page, where one batched wrapper serves requests with one and with several
 * query tokens).  Attention is causal among a request's new tokens: the new
 * tokens are the last qo_len(b) of its kv_lens[b] tokens, and query token j
 * (0-based) sits at position kv_lens[b] - qo_len(b) + j and attends the tokens
 * 0 .. that position.  With qo_len = 1 everywhere this is pkvmla_plan_create.
 *   qo_indptr host int32[batch+1]: qo_indptr[0] == 0, qo_len(b) >= 1 and
 *   qo_len(b) <= kv_lens[b].  Other arguments as pkvmla_plan_create.
 * The run's query, output and lse tensors have one row per query token:
 * q_nope [qo_indptr[batch], num_heads, 512], q_pe [.., 64], out [.., 512],
 * lse [qo_indptr[batch], num_heads], row qo_indptr[b] + j for token j of b.
 * The layout is chosen as pkvmla_plan_create_qo_layout does with
 * PKVMLA_QO_AUTO.  Plans of this kind are updated in place with
 * pkvmla_plan_update_qo (pkvmla_plan_update refuses them). */
int pkvmla_plan_create_qo(const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_lens, int32_t batch,
                          int32_t num_pages, int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim,
                          int32_t page_size, float sm_scale, void* stream, pkvmla_plan* out);

/* Work layouts of a plan with several query tokens per request. */
enum {
  PKVMLA_QO_AUTO = 0,        /* row blocks when the rule below picks them, else tokens */
  PKVMLA_QO_TOKENS = 1,      /* one work item per query token (any head count) */
  PKVMLA_QO_ROW_BLOCKS = 2   /* 16 or 32 heads: blocks of 64 query rows */
};

/* pkvmla_plan_create_qo with an explicit layout (same semantics and results,
 * up to rounding).
 *   PKVMLA_QO_TOKENS: each query token is its own work item over request b's
 *   pages, of its causal length; the tokens of a request read its KV tiles
 *   once each.
 *   PKVMLA_QO_ROW_BLOCKS (num_heads 16 or 32, else PKVMLA_EUNSUPPORTED): the
 *   query rows t * H + h of request b's tokens are cut into blocks of 64 rows
 *   (64 / H tokens each, the last block possibly short); a block is one work
 *   item over the positions its last token sees, split over lanes like a flat
 *   request, and every 64-row workgroup scores each KV tile once for all of
 *   its tokens, each row masked at its own causal bound.  A block left whole
 *   writes out and lse itself; a split one writes a partial state per token
 *   and piece, merged per token (see pkvmla_schedule_qo_rows_host).
 *   PKVMLA_QO_AUTO: row blocks when num_heads is 16 or 32 and some request
 *   brings more than one query token (qo_indptr[batch] > batch), else tokens
 *   (a 64-row workgroup costs about what a 16- or 32-head one does per KV
 *   tile, so blocks gain as soon as one tile serves two tokens).
 * pkvmla_plan_export reports the layout in header word 26 (1: tokens, 2: row
 * blocks; the blocks' units, slot list and merges are in the level-0 fields).
 * PKVMLA_EINVAL for an unknown layout. */
int pkvmla_plan_create_qo_layout(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                 const int32_t* kv_indices, const int32_t* kv_lens, int32_t batch,
                                 int32_t num_pages, int32_t num_heads, int32_t ckv_dim,
                                 int32_t kpe_dim, int32_t page_size, float sm_scale,
                                 int32_t layout, void* stream, pkvmla_plan* out);

/* pkvmla_plan_create_qo_layout sized for later pkvmla_plan_update_qo calls
 * (index_capacity > 0: page ids the device table holds, at least the first
 * table's; 0 is pkvmla_plan_create_qo_layout).  The "[WIP][Kernel] Flashinfer
 * MLA support" page reports graph capture of the MLA decode path as broken;
 * a plan with a capacity keeps its device tables, split workspace and
 * launch shapes, sized for any split of the same qo_indptr[batch] query
 * tokens over the same batch, so a HIP graph captured around its run stays
 * valid across updates (as for pkvmla_plan_create_with_capacity). */
int pkvmla_plan_create_qo_with_capacity(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                        const int32_t* kv_indices, const int32_t* kv_lens,
                                        int32_t batch, int32_t num_pages, int32_t num_heads,
                                        int32_t ckv_dim, int32_t kpe_dim, int32_t page_size,
                                        float sm_scale, int32_t layout, int64_t index_capacity,
                                        void* stream, pkvmla_plan* out);

/* Rewrite a plan of several query tokens per request in place for new page
 * tables and a new split of its query tokens: the same batch, the same total
 * qo_indptr[batch] (the run's tensors keep their shapes), each request 1 ..
 * kv_lens[b] tokens.  The plan keeps its layout (as pkvmla_plan_export header
 * word 26 reports it).  Ordering and capacity rules as pkvmla_plan_update;
 * PKVMLA_EINVAL for a different token count, malformed arrays or a table
 * beyond the plan's capacities (the plan is then unchanged). */
int pkvmla_plan_update_qo(pkvmla_plan plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_lens, void* stream);

/* Build a two-level (cascade) plan.  Requests are partitioned into
 * num_groups contiguous groups by group_req_indptr (host int32[G+1], from 0
 * to batch).  Group g's shared prefix is prefix_lens[g] tokens in pages
 * prefix_indices[prefix_indptr[g] ...] (host arrays).  kv_indptr, kv_indices
 * and kv_lens describe each request's own suffix as in a flat plan, except
 * that kv_lens[b] may be 0.  prefix_lens[g] + kv_lens[b] >= 1 for every b.
 * The two levels follow the cascade attention of the vLLM page "[V1][Core]
 * FlashInfer attention backend for V1" (shared-prefix level, per-request
 * level, merged; it must equal normal attention).  A run launches level 0
 * (each group's query rows b * H + head, 64 to a workgroup, several requests
 * per workgroup below 64 heads, scoring the group's prefix tiles: see
 * pkvmla_schedule_rows_host), then level 1 (each suffix, split like a flat
 * plan), then the log-sum-exp merge of every request's states. */
int pkvmla_plan_create_cascade(const int32_t* group_req_indptr, int32_t num_groups,
                               const int32_t* prefix_indptr, const int32_t* prefix_indices,
                               const int32_t* prefix_lens,
                               const int32_t* kv_indptr, const int32_t* kv_indices,
                               const int32_t* kv_lens, int32_t batch, int32_t num_pages,
                               int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim,
                               int32_t page_size, float sm_scale, void* stream,
                               pkvmla_plan* out);

/* pkvmla_run_strided for fp8 KV caches: ckv_cache and kpe_cache hold OCP
 * E4M3 codes (one byte per element, the format of the OCP 8-bit floating
 * point specification: bias 7, no infinity, S.1111.111 NaN), a token's ckv
 * value being ckv_scale times its code's value and its kpe value kpe_scale
 * times its code's (per-tensor scales, finite and > 0).  Queries, out and lse
 * are as in pkvmla_run.  The vLLM page "[V1][Core] FlashInfer attention
 * backend for V1" lists a KV-cache dtype other than the query dtype as the
 * limitation of its cascade path; here both flat and cascade plans take fp8
 * caches with bf16 queries.  The codes are widened exactly to bf16 and the
 * scales applied in fp32 (scores: ckv part + kpe_scale / ckv_scale times the
 * kpe part, times sm_scale * ckv_scale; outputs times ckv_scale).  Row
 * strides are in BYTES: ckv >= 512 and a multiple of 16, kpe >= 64 and a
 * multiple of 8 (packed caches: 512 and 64; the two views of one
 * [pages, page_size, 576] fp8 cache: 576 and 576).  ckv_cache 16-byte, kpe_cache
 * 8-byte aligned.  Errors as pkvmla_run, PKVMLA_EINVAL for bad scales. */
int pkvmla_run_fp8(pkvmla_plan plan, const void* q_nope, const void* q_pe,
                   const void* ckv_cache, const void* kpe_cache, int64_t ckv_row_stride,
                   int64_t kpe_row_stride, float ckv_scale, float kpe_scale, void* out,
                   float* lse, void* stream);

/* pkvmla_plan_create_cascade with device tables, split workspace and launch
 * shapes sized once (index_capacity > 0: page ids of prefixes and suffixes
 * together) for later pkvmla_plan_update_cascade calls, so that a HIP graph
 * captured around pkvmla_run stays valid across them.  The vLLM page "[WIP]
 * [Kernel] Flashinfer MLA support" names graph capture of the decode path as
 * the part that did not yet work there.  Every level-0 and level-1 lane and
 * every merge record is launched on each run (empty ones return at once).
 * index_capacity 0 is pkvmla_plan_create_cascade. */
int pkvmla_plan_create_cascade_with_capacity(
    const int32_t* group_req_indptr, int32_t num_groups, const int32_t* prefix_indptr,
    const int32_t* prefix_indices, const int32_t* prefix_lens, const int32_t* kv_indptr,
    const int32_t* kv_indices, const int32_t* kv_lens, int32_t batch, int32_t num_pages,
    int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim, int32_t page_size, float sm_scale,
    int64_t index_capacity, void* stream, pkvmla_plan* out);

/* Replace a cascade plan's groups (same num_groups and batch), prefixes and
 * suffixes (arrays as in pkvmla_plan_create_cascade, read during the call
 * only) and recompute both levels' schedules and the merge lists, in place,
 * without allocation.  Ordering and graph validity as for
 * pkvmla_plan_update.  PKVMLA_EINVAL when the arrays are malformed, a flat
 * plan is given, or the page ids exceed the plan's capacity (the plan is then
 * unchanged). */
int pkvmla_plan_update_cascade(pkvmla_plan plan, const int32_t* group_req_indptr,
                               const int32_t* prefix_indptr, const int32_t* prefix_indices,
                               const int32_t* prefix_lens, const int32_t* kv_indptr,
                               const int32_t* kv_indices, const int32_t* kv_lens, void* stream);

/* Run the decode for one set of tensors (e.g. one layer) on `stream`.  The
 * plan-then-run split and the run's operands (q_nope, q_pe, the ckv and kpe
 * caches in, output and log-sum-exp out) follow the decode-wrapper calls in
 * the vLLM-metax page "[WIP] support flashinfer_mla" (the plan-argument and
 * metadata reviews).
 * Asynchronous: only kernel launches on `stream`; no allocation, no host
 * synchronisation, no host<->device copies.  Device pointers are owned by the
 * caller and must stay valid until the stream reaches the end of the call;
 * out/lse must not alias the inputs.  One plan must not run on two streams at
 * once (the split workspace is shared).  Results are bitwise reproducible for
 * a fixed plan and inputs. */
int pkvmla_run(pkvmla_plan plan, const void* q_nope, const void* q_pe,
               const void* ckv_cache, const void* kpe_cache, void* out, float* lse,
               void* stream);

/* pkvmla_run for caches whose rows are not packed: ckv row r starts at
 * ckv_cache + r * ckv_row_stride elements and kpe row r at kpe_cache + r *
 * kpe_row_stride (r = page * page_size + slot).  A cache kept as one
 * [pages, page_size, 576] tensor (each row the 512 compressed-KV values, then
 * the 64 rope values; dims as in the plan-argument review of the vLLM-metax
 * page "[WIP] support flashinfer_mla") is passed as its two views:
 * ckv_cache = base, kpe_cache = base + 512, both strides 576.
 * Strides are in bf16 elements, multiples of 8 (whole 16-byte chunks), at
 * least 512 (ckv) and 64 (kpe), at most 2^20; both base pointers 16-byte
 * aligned; every row of the pool must lie inside the caller's allocation.
 * pkvmla_run is this call with strides 512 and 64.  Same semantics and
 * errors as pkvmla_run, plus PKVMLA_EINVAL for a stride out of range. */
int pkvmla_run_strided(pkvmla_plan plan, const void* q_nope, const void* q_pe,
                       const void* ckv_cache, const void* kpe_cache, int64_t ckv_row_stride,
                       int64_t kpe_row_stride, void* out, float* lse, void* stream);

/* pkvmla_run for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * split workspace the decode and merge kernels use for partial outputs is a
 * static device array of the library (64 MiB per device, held from the
 * library's first use on a device until the process ends) instead of the
 * plan's own buffer.  The call itself allocates nothing; its address lookup on
 * a device happens once, at the first call on that device.  Arguments,
 * layouts and results as pkvmla_run (packed caches), bitwise equal to
 * pkvmla_run of the same plan and inputs.  Every call on one device shares
 * that device's array: calls that overlap on one device (two streams, or two
 * threads) race and must be ordered by the caller.  PKVMLA_EUNSUPPORTED when
 * the plan's partial states (slots x num_heads x 1028 bytes) exceed 64 MiB. */
int pkvmla_run_noalloc(pkvmla_plan plan, const void* q_nope, const void* q_pe,
                       const void* ckv_cache, const void* kpe_cache, void* out, float* lse,
                       void* stream);

/* Bounded waits of the 16- and 32-head decode kernels (bf16 caches), whose
 * roles synchronise through progress counters in LDS instead of a per-tile
 * barrier: a wave polls a counter at most `polls` times (default 2^20, about
 * 0.1 s) and then gives up; a wave that gave up writes NaN to out and lse for
 * every unit it finishes afterwards (a stall anywhere in a workgroup reaches
 * the waits of the waves that write), so a broken protocol shows as
 * non-finite results and never as a launch that does not end.  0 makes every
 * such wait give up at once (the failure path, for tests); other kernels are
 * unaffected.  PKVMLA_EINVAL for polls < 0.  Applies to later runs of the
 * plan; not for use while a run is being captured. */
int pkvmla_plan_set_wait_limit(pkvmla_plan plan, int32_t polls);

/* Kernel timing for benchmarks.  enable 1: in every later pkvmla_run each
 * workgroup of the decode launch(es) stores its start and its end (wave 0
 * after the workgroup's final barrier; at 16 and 32 heads, where no barrier
 * ends the workgroup, the first PV wave after its last tile) on the GPU's
 * 100 MHz real-time counter into its own words of a per-run record (plain
 * stores, no atomics and no stream events, so the timed launches run as they
 * do untimed); a run's span is its earliest workgroup start to its latest
 * workgroup end.  enable 2: the same plus a HIP event pair on the stream
 * around the decode launch(es) (events between kernels change how the
 * launches that follow run).  0: off.
 * The record and event buffers are created here, so run still allocates
 * nothing; the run counter is reset.  pkvmla_plan_timing synchronises the
 * device and returns, over the last min(n, 256) timed runs, the summed event
 * intervals (ms; 0 without events), the summed spans (ms) and that count.
 * Timing must be off while a run is being captured into a HIP graph. */
int pkvmla_plan_set_timing(pkvmla_plan plan, int32_t enable);
int pkvmla_plan_timing(pkvmla_plan plan, double* event_ms, double* span_ms, int64_t* n_runs);

/* Per timed run (the last min(n, 256), oldest first): span_us[i] the run's
 * decode span, start_us[i] its earliest decode workgroup start and
 * merge_start_us[i] its earliest merge block start (-1: no merge launch), the
 * last two relative to the first returned run's start (microseconds).  With
 * back-to-back runs, consecutive starts give each step's period and
 * merge_start_us[i] - start_us[i] the decode launches' duration as a trace
 * counts it (dispatch to the next kernel's start), without events between
 * them.  *n_runs = the count; PKVMLA_EINVAL when it exceeds cap. */
int pkvmla_plan_timing_runs(pkvmla_plan plan, double* span_us, double* start_us,
                            double* merge_start_us, int64_t cap, int64_t* n_runs);

/* Free the plan's device buffers (synchronises the device first).  NULL is a
 * no-op.  The plan is built once per batch of page tables and reused across
 * runs (e.g. layers), as the metadata builder reviewed on the vLLM-metax page
 * "[WIP] support flashinfer_mla" does; this ends that lifetime. */
void pkvmla_plan_destroy(pkvmla_plan plan);

/* Message of the calling thread's last failed call ("" if none).  Every
 * unsupported request fails with a status and this message instead of falling
 * back to another path: the backend-selection reviews on the vLLM-metax page
 * "[WIP] support flashinfer_mla" ask for a hard error when the MLA backend
 * cannot serve a configuration. */
const char* pkvmla_last_error(void);

/* Kernel configuration used for num_heads (values the schedule depends on):
 * cfg[0] = KV tile tokens, cfg[1] = compute waves per workgroup (the QK
 * waves, one per 16 heads, and four PV waves; two copy waves come on top),
 * cfg[2] = heads per QK wave, cfg[3] = LDS stages, cfg[4] = workgroups per CU, cfg[5] = fixed cost
 * per segment in tiles, cfg[6] = head groups (workgroups that share one
 * token range, each holding num_heads / head_groups heads; the schedule has
 * num_cu * workgroups_per_cu / head_groups lanes).  Host only; needs no GPU. */
int pkvmla_kernel_config(int32_t num_heads, int32_t* cfg7);

/* The split-KV work schedule, computed on the host exactly as plan_create
 * does (no GPU needed).  items: host int32[n_items*3] of (request, sequence,
 * length).  num_wg: workgroup budget.  Outputs (capacities in elements):
 * wg_indptr int32[grid+1], units int32[n_units*8] records
 * (request, sequence, kv_begin, kv_end, slot, row, 0, 0) where row is the
 * number of tokens in all earlier units, merges int32[n*4]
 * records (request, first_slot, count, 0).  counts[0..2] = grid, n_units,
 * n_merges.  PKVMLA_EINVAL if a capacity is too small. */
int pkvmla_schedule_host(const int32_t* items, int32_t n_items, int32_t batch,
                         int32_t num_wg, int32_t tile, int32_t fixed_cost,
                         int32_t* wg_indptr, int64_t cap_wg,
                         int32_t* units, int64_t cap_units,
                         int32_t* merges, int64_t cap_merges, int32_t* counts);

/* The level-0 schedule of a cascade plan, computed on the host exactly as
 * pkvmla_plan_create_cascade does (no GPU needed).  Query rows rho = b * H +
 * head; group g owns rows [group_req_indptr[g] * H, group_req_indptr[g+1] * H),
 * cut into blocks of max(64, H) rows (groups with an empty prefix have none).
 * With nb blocks on num_wg lanes: nb <= num_wg cuts every block's prefix into
 * S = num_wg / nb token pieces (at most its tile count; piece p of T tiles
 * covers tiles [p*T/P, (p+1)*T/P) of P pieces) with piece p of block k on
 * lane k*S + p; nb > num_wg puts block k whole on lane k mod num_wg.  Unit
 * records (row0, group, kv_begin, kv_end, slot offset, row_end, 0, 0): slots
 * are numbered from 0 in lane order, one per request of a unit's rows, and
 * the offset is (first slot) * H - row0, so row rho's partial state is row
 * rho + offset of the partial-state rows.  counts[0..2] = grid, n_units,
 * n_slots.  A plan uses num_wg = CUs / max(1, H / 64). */
int pkvmla_schedule_rows_host(const int32_t* group_req_indptr, int32_t num_groups,
                              const int32_t* prefix_lens, int32_t num_heads, int32_t num_wg,
                              int32_t tile, int32_t* wg_indptr, int64_t cap_wg,
                              int32_t* units, int64_t cap_units, int32_t* counts);

/* The one-launch cascade schedule, computed on the host exactly as
 * pkvmla_plan_create_cascade does for an ordinary plan with num_heads >= 64
 * and every prefix non-empty (no GPU needed).  Request b of group g is one
 * block over g's prefix, cut over num_wg lanes as in
 * pkvmla_schedule_rows_host (batch <= num_wg: S = num_wg / batch pieces,
 * piece p on lane b*S + p; else request b whole on lane b mod num_wg).  Its
 * non-empty suffix (sequence num_groups + b, tokens 0 .. kv_lens[b]) follows
 * its last piece on that lane, and that piece's slot field is INT32_MIN: the
 * softmax state carries into the suffix unit.  A request with one piece
 * writes out directly (slot -1); otherwise each of its states takes the next
 * slot (emission order) and it gets a merge record (b, first list entry,
 * count, 1).  Unit records: (b, sequence, kv_begin, kv_end, slot, 0, 0, 0).
 * counts[0..3] = grid, n_units, n_merges, slot-list length. */
int pkvmla_schedule_chain_host(const int32_t* group_req_indptr, int32_t num_groups,
                               const int32_t* prefix_lens, const int32_t* kv_lens,
                               int32_t batch, int32_t num_wg, int32_t tile, int32_t* wg_indptr,
                               int64_t cap_wg, int32_t* units, int64_t cap_units,
                               int32_t* merges, int64_t cap_merges, int32_t* slot_list,
                               int64_t cap_list, int32_t* counts);

/* The row-block schedule of a plan with several query tokens per request
 * (PKVMLA_QO_ROW_BLOCKS), computed on the host exactly as the plan does (no
 * GPU needed; a plan uses num_wg = CUs, fixed_cost = 4, tile = 32).  Request
 * b's rows [qo_indptr[b] * H, qo_indptr[b+1] * H) are cut into blocks of 64
 * rows in request order; block k is the work item (k, b, t_last + c_b) of
 * pkvmla_schedule_host's walk, t_last being the block's last token (the
 * positions it sees; no row of the block sees more).  Each walk unit becomes the record
 * (row0, c_b, kv_begin, kv_end, slot field, row_end, 0, 0) with
 * c_b = kv_lens[b] - qo_len(b) + 1 - qo_indptr[b] (query token t, rows
 * t * H .. t * H + H - 1, attends the positions below t + c_b) and slot field
 * INT32_MIN + 1 for a block the walk left whole (it writes out and lse), else
 * walk slot * 64 - row0 (row rho's partial state is partial row
 * field + rho; partial slots hold H rows).  A split block's walk merge
 * (k, first, count) becomes, for each of its tokens t in order, the merge
 * record (t, first slot-list entry, count, 1) whose list holds the token's
 * slot (first + i) * 64 / H + (t - row0 / H) of every piece i.
 * counts[0..5] = grid, n_units, n_merges, slot-list length, partial slots
 * (of H rows), and 1 when PKVMLA_QO_AUTO would pick row blocks, else 0. */
int pkvmla_schedule_qo_rows_host(const int32_t* qo_indptr, const int32_t* kv_lens,
                                 int32_t batch, int32_t num_heads, int32_t num_wg, int32_t tile,
                                 int32_t fixed_cost, int32_t* wg_indptr, int64_t cap_wg,
                                 int32_t* units, int64_t cap_units, int32_t* merges,
                                 int64_t cap_merges, int32_t* slot_list, int64_t cap_list,
                                 int32_t* counts);

/* Copy the plan's uploaded device tables back to the host, for bit-exact
 * checking.  Layout of host int32 buf (cap elements):
 *   [0..15]  header: version(1), batch, num_heads, page_size, ckv_dim,
 *            kpe_dim, tile, waves, heads_per_wave, stages, wg_per_cu,
 *            fixed_cost, grid, n_units, n_merges, n_slots
 *   [16..31] header 2: num_seqs, n_indices, num_cu, sm_scale (float bits),
 *            is_cascade, num_groups, head_groups, launched workgroups,
 *            fixed launch shapes (0/1), page-id capacity, several query tokens
 *            per request (0: no, 1: one item per token, 2: row blocks),
 *            number of requests of such a plan,
 *            cascade level 0: grid0, n_units0, slot-list length, and 1 when the
 *            cascade runs in one launch (level-0 table: requests' prefix
 *            pieces with their suffixes chained; no level-1 units), else 0
 *   then wg_indptr[grid+1], units[n_units*8], merges[n_merges*4],
 *   seq_indptr[num_seqs+1], seq_lens[num_seqs], seq_indices[n_indices],
 *   and for a cascade plan wg_indptr0[grid0+1], units0[n_units0*8] (the
 *   records of pkvmla_schedule_rows_host with the page fields filled), the
 *   slot list; a row-block plan of several query tokens has the same three
 *   (records of pkvmla_schedule_qo_rows_host with the page fields of request
 *   b's pages) and its merges in the merge field, with no level-1 units.  A cascade plan's units are its suffixes', every one with a
 *   partial slot numbered after level 0's (in emission order), and its merge
 *   records are (request, first slot-list entry, count, 1): the request's
 *   level-0 slots in level-0 emission order, then its suffix slots.
 *   The unit records are those of pkvmla_schedule_host with their last two
 *   fields filled: page_base = seq_indptr[sequence] and first_page =
 *   seq_indices[page_base + kv_begin / page_size].
 * *used = number of int32 written (or needed, when cap is too small:
 * PKVMLA_EINVAL).  Synchronises the device. */
int pkvmla_plan_export(pkvmla_plan plan, int32_t* buf, int64_t cap, int64_t* used);

/* Page-table gather through the same device address path as the decode
 * kernel: rows (device bf16 [sum of attended tokens, 576]) receives, for every
 * work unit of the plan in request order and then token order, the ckv row
 * followed by the kpe row of each token.  For a flat plan this is
 * [sum(kv_lens), 576] in (request, token) order.  For a cascade plan: the
 * level-0 units (prefix token ranges, in level-0 emission order), then the
 * suffix units.  Bit-exact copy. */
int pkvmla_gather(pkvmla_plan plan, const void* ckv_cache, const void* kpe_cache,
                  void* rows, void* stream);

/* Number of rows pkvmla_gather writes for this plan. */
int pkvmla_gather_rows(pkvmla_plan plan, int64_t* n_rows);

#ifdef __cplusplus
}
#endif

#endif /* PKVMLA_H_ */
