/*
 * pa_verify.h -- C ABI of the paged verify-attention library (MI355X, gfx950).
 *
 * The operation (one speculative-decoding verify step of attention):
 * every sequence b brings q_b query tokens (q_b = k + 1 for k draft tokens,
 * 6 at MTP-5, up to 8) that attend, causally among themselves, to the
 * sequence's own KV context. The context lives in a paged pool of 16-token
 * blocks reached through a per-sequence block table; KV is bf16, or FP8 e4m3
 * with one fp32 scale per token and KV head. The query heads that share a KV
 * head are packed together (rows = q_b x G, G = Hq / Hkv).
 *
 * Sources:
 *  - ATOM #2843, "keep MTP-5 decode on FlyDSL pa_decode past the gluon
 *    query-length limit": Motivation (query length 6 at MTP-5; rows = query
 *    length x GQA group = 48; per-token FP8 KV scales), Change (the decode
 *    call receives the lengths, the block table, the query length, the K/V
 *    scales, the sliding window and the context bound; sinks and windows are
 *    layer properties), and the review thread on run_pa_decode (feasibility
 *    is checked before any plan or scratch exists; a plan's cached scratch
 *    means the call itself allocates nothing; a refused call fails loudly).
 *  - ATOM #3091, "High-interactivity monokernel decode for
 *    DeepSeek-V4.1-Flash on MI355X": Summary (contexts up to 1 Mi tokens;
 *    paged-pool stores masked by row liveness, so padded requests write
 *    nothing) and "How to reproduce" (16-token blocks, full graph capture).
 *  - ATOM #3038, "[MiniMax-M3.1] P/D from a PP4 prefill into a TP4 decode
 *    (2/2: DSpark)": Results (verify of 7 drafts + 1 = 8 tokens) and the KV
 *    export commit message (pages are head-major per page); its review on
 *    page geometry (no defaulted page size: the block size is an explicit,
 *    checked argument).
 *
 * Meaning of a call (the plain definition the library computes, up to fp32
 * rounding): for sequence b with context length L (the cache holds L tokens,
 * the q new ones included), query row i in [0, q) sits at position
 * p = L - q + i and sees the keys j with lo <= j <= p, where
 * lo = max(0, p - W + 1) for a window of W keys (W = 0: lo = 0). With scores
 * s_j = sigma * <Q[row], dequant(K_j)>, an optional sink logit z of the row's
 * head, M = max(max_j s_j, z) and Z = sum_j e^(s_j - M) + e^(z - M):
 *     out[row] = sum_j e^(s_j - M) dequant(V_j) / Z.
 * dequant is the identity for bf16 and code x scale[token][kv head] for FP8.
 *
 * Layouts (all row-major, no padding between rows):
 *  q            [T][Hq][D] bf16, T = sum_b q_b, sequence-major: sequence b's
 *               rows start at t_b = q_0 + ... + q_(b-1)
 *  k_pool/v_pool [num_blocks][Hkv][16][D] bf16, or uint8 e4m3 codes (OCP
 *               e4m3fn: bias 7, max 448, NaN = 0x7F/0xFF)
 *  k_scales/v_scales [num_blocks][Hkv][16] fp32 (a trailing [1] is the same
 *               memory)
 *  block_table  [B][max_blocks_per_seq] int32; entry n of row b is the pool
 *               block holding tokens 16n..16n+15 of sequence b
 *  sinks        mode 1: [Hq] fp32, one logit per head for every sequence;
 *               mode 2: [B][Hq] fp32, -inf meaning "no sink"
 *  out          [T][Hq][D], bf16 (round to nearest even) or fp32
 *
 * Ownership: every tensor belongs to the caller, who keeps it alive and
 * unmodified until the stream work of the call has finished. A plan owns its
 * work list, its copy of the lengths and windows, and its scratch; one plan
 * serves one stream at a time (the scratch is not shared between calls in
 * flight). Block-table contents (ids < num_blocks for every entry a sequence
 * uses) and pointer validity are the caller's contract and are not checked.
 */
#ifndef PA_VERIFY_H
#define PA_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_plan_s pa_plan_t; /* opaque plan */

typedef enum {
  PA_OK = 0,
  PA_E_INVALID = 1,     /* a null pointer, a negative size, q_b > L_b, ... */
  PA_E_UNSUPPORTED = 2, /* a meaningful shape this library does not serve */
  PA_E_HIP = 3,         /* a HIP runtime call or a kernel launch failed */
  PA_E_NOMEM = 4        /* device or host memory could not be allocated */
} pa_status;

typedef enum { PA_BF16 = 0, PA_FP8_E4M3 = 1, PA_FP32 = 2 } pa_dtype;

/* Limits (a shape beyond them is refused with PA_E_UNSUPPORTED). */
#define PA_BLOCK_TOKENS 16      /* tokens per KV block */
#define PA_MAX_QUERY_LEN 8      /* q_b <= 8: verify of 7 drafts + 1 */
#define PA_MAX_ROWS 128         /* q_b x G <= 128 packed rows per KV head */
#define PA_MAX_CONTEXT 1048576  /* L_b <= 1 Mi tokens */
#define PA_MAX_ITEM_KEYS 8192   /* partition_tokens <= 8192 */

typedef struct {
  int32_t num_seqs;           /* B >= 1 */
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;           /* D: 64 or 128 (bf16 or FP8 KV), or 256
                                 (FP8 KV only) */
  int32_t block_size;         /* must be 16 (explicit: never defaulted) */
  int32_t num_blocks;         /* pool capacity, >= 1 */
  int32_t max_blocks_per_seq; /* block-table row stride in entries, >= 1 */
  pa_dtype q_dtype;           /* PA_BF16 */
  pa_dtype kv_dtype;          /* PA_BF16 or PA_FP8_E4M3 */
  pa_dtype out_dtype;         /* PA_BF16 or PA_FP32 */
  float softmax_scale;        /* sigma, finite and > 0 (e.g. 1/sqrt(D)) */
  int32_t partition_tokens;   /* keys per work item (split-K unit): a
                                 multiple of 16 up to PA_MAX_ITEM_KEYS, or 0
                                 to let the plan choose */
  int32_t sinks_mode;         /* 0 none, 1 sinks[Hq], 2 sinks[B][Hq] */
  int32_t lengths_are_bounds; /* 0: context_lens are the lengths; 1: they
                                 are per-sequence upper bounds for calls
                                 that read the lengths from device memory
                                 (pa_decode_verify_dev); the work items
                                 then cover every key a length up to the
                                 bound can make visible (a windowed
                                 sequence from key 0) */
} pa_shape;

/*
 * Validate a shape and the per-sequence lengths, cut every sequence's
 * visible keys into work items, and allocate the plan's device work list and
 * scratch on `device`.
 *   context_lens  host [B]: L_b, KV tokens in the cache including the q_b new
 *                 ones; q_b <= L_b <= PA_MAX_CONTEXT
 *   query_lens    host [B]: q_b in 0..PA_MAX_QUERY_LEN; 0 marks a padded slot
 *                 that reads nothing and writes nothing
 *   window        host [B] or NULL: W_b >= 0 keys per row including its own;
 *                 0 = no window
 *   device        HIP device ordinal, or -1 for a host-only plan (validation
 *                 and work list, no HIP call and no device memory; useful for
 *                 inspection; pa_decode_verify refuses it)
 *   out           receives the plan; on any error *out = NULL and nothing
 *                 stays allocated
 * Every check runs before the first HIP call or allocation, so a refused
 * shape costs nothing and leaks nothing. The host arrays are copied; the
 * caller may free them on return. Thread-safe (no shared state).
 */
pa_status pa_plan(const pa_shape* shape, const int32_t* context_lens,
                  const int32_t* query_lens, const int32_t* window, int device,
                  pa_plan_t** out);

/*
 * Run one verify-attention call with a plan: the partition kernel, then (if
 * any sequence was split) the log-sum-exp reduce kernel (two launches when
 * some (sequence, KV head) has more than 512 partials), all enqueued on
 * `stream` (a hipStream_t; NULL = the null stream) of the plan's device,
 * which must be the current device. Asynchronous: it allocates nothing,
 * never synchronises, and may be captured in a HIP graph. Pointers are device
 * pointers in the layouts above; k_scales/v_scales must be non-NULL exactly
 * for FP8 KV, sinks non-NULL exactly for sinks_mode != 0. Rows of sequences
 * with q_b = 0 are not written. Returns PA_E_INVALID for a missing pointer or
 * a host-only plan (nothing is launched then) and PA_E_HIP if a launch fails.
 */
pa_status pa_decode_verify(const pa_plan_t* plan, const void* q,
                           const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const float* k_scales,
                           const float* v_scales, const float* sinks, void* out,
                           void* stream);

/*
 * pa_decode_verify with the context lengths read from device memory at run
 * time, so that one captured graph serves every step of a decode loop while
 * the lengths advance on the device. Source: ATOM #3091 ("High-interactivity
 * monokernel decode for DeepSeek-V4.1-Flash on MI355X", Summary: the next
 * step is laid out from the device-resident verdict; How to reproduce: full
 * graph capture); ATOM #2843 (Motivation: plans built on upper bounds,
 * scratch sized by the largest query).
 *   context_lens_dev  device [B] int32: L_b for this call. The plan's
 *                     context_lens are upper bounds; the kernels clamp L_b
 *                     to [q_b, bound_b]. Query lengths, windows and sinks
 *                     are the plan's.
 * The block table must hold valid page ids for the first ceil(L_b / 16)
 * entries of each row (entries past the length are not read). A plan with
 * windows must have been built with lengths_are_bounds = 1 (PA_E_INVALID
 * otherwise). Everything else as pa_decode_verify.
 */
pa_status pa_decode_verify_dev(const pa_plan_t* plan, const int32_t* context_lens_dev,
                               const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const float* k_scales,
                               const float* v_scales, const float* sinks, void* out,
                               void* stream);

/*
 * The verify-attention call as a single persistent launch: a grid of at most
 * the device's resident workgroups takes the plan's work items in turn (each
 * workgroup starts with its own and fetches the next from a device counter),
 * and the partition kernel merges the partial results of every split
 * (sequence, KV head) itself, so no reduce kernel follows. Source: ATOM
 * #3091 ("High-interactivity monokernel decode for DeepSeek-V4.1-Flash on
 * MI355X", Summary: a decode layer runs as one persistent kernel; How to
 * reproduce: full graph capture); ATOM #2843
 * ("keep MTP-5 decode on FlyDSL pa_decode past the gluon query-length
 * limit", Change: persistent and non-persistent decode calls are routed
 * apart).
 *   context_lens_dev  device [B] int32 lengths read at run time, with the
 *                     plan's lengths as upper bounds (as pa_decode_verify_dev),
 *                     or NULL for the plan's own lengths
 * The work items of a split pair write their partials and then count their
 * arrival on a device counter of the pair's merge node (a node merges at
 * most 16 partials; pairs with more go through a tree of nodes, one level
 * per factor of 16). The workgroup whose arrival completes a node's count
 * merges that node's partials: into the output at the root, else into an
 * input of the parent node, where it arrives in turn. The counters are
 * part of the plan's device memory, zero when pa_plan returns and reset by
 * each node's last arriver (the work-list counters by the last workgroup to
 * finish), so every call leaves them at zero (graph replays included). No
 * workgroup ever waits for another. Calls with one plan that overlap on the
 * device (different streams or threads) race on the counters and partials
 * and must be serialised by the caller. Results are pa_decode_verify's up to the order
 * of the log-sum-exp merge (float rounding). Otherwise as pa_decode_verify:
 * asynchronous, allocation-free, graph-capturable, the same errors (and
 * PA_E_INVALID for a windowed plan read with device lengths unless it was
 * built with lengths_are_bounds = 1).
 */
pa_status pa_decode_verify_fused(const pa_plan_t* plan, const int32_t* context_lens_dev,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const float* k_scales,
                                 const float* v_scales, const float* sinks, void* out,
                                 void* stream);

/*
 * pa_decode_verify for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the call allocates nothing, and the plan may be a host-only
 * one (pa_plan with device = -1, which owns no device memory either).
 * The work list, the reduce lists and the partial results go into the
 * library's static scratch, a device array of 64 MiB that every device the
 * library runs on holds from the library's first use there until the
 * process ends; the work lists are copied into it with hipMemcpyAsync on
 * `stream` ahead of the kernels (so the plan must outlive the call's stream
 * work). Runs on the current device (a device plan must be for it) with the
 * plan's context lengths. Every call on a device shares that device's
 * scratch: calls that overlap on one device (on different streams, or from
 * different threads) race and must be serialised by the caller. Nothing in
 * the scratch needs clearing: a call writes every value it reads.
 * Returns PA_E_UNSUPPORTED, before any HIP call, when the plan's work list
 * and partials exceed the scratch (e.g. a 1 Mi-token context cut into
 * 512-key items: use pa_decode_verify or larger items); otherwise the
 * errors of pa_decode_verify, with host-only plans accepted.
 */
pa_status pa_decode_verify_noalloc(const pa_plan_t* plan, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_table,
                                   const float* k_scales, const float* v_scales,
                                   const float* sinks, void* out, void* stream);

/*
 * Paged KV append: write the plan's new tokens (the last q_b positions of
 * every sequence, L_b - q_b .. L_b - 1) into their 16-token slots, the step
 * before verify attention. Source: ATOM #3091 ("High-interactivity
 * monokernel decode for DeepSeek-V4.1-Flash on MI355X", Summary: stores into
 * the paged pool are masked by row liveness, so a padded slot with q_b = 0
 * stores nothing); ATOM #2843 (Motivation: FP8 KV with one fp32 scale per
 * token and KV head, scale = amax / 448 of the token's values).
 *   k_new, v_new  [T][Hkv][D] bf16, T = sum q_b, rows in sequence order (the
 *                 layout of q with Hkv heads)
 *   block_table   [B][max_blocks_per_seq] int32: position p of sequence b
 *                 goes to page block_table[b][p / 16], slot p % 16
 *   k_pool, v_pool [NB][Hkv][16][D] bf16 (copied bit for bit) or e4m3 codes
 *   k_scales, v_scales [NB][Hkv][16] fp32, non-NULL exactly for FP8 KV: per
 *                 (token, KV head) scale = amax / 448 in fp32 (1 when amax is
 *                 0) and code = the e4m3 value nearest to the fp32 quotient
 *                 x / scale clamped to +-448, ties to the even mantissa
 * Only the new tokens' slots are written; a position whose block-table entry
 * lies outside [0, num_blocks) is skipped, so no table can make the call
 * store outside the pool. Enqueued on `stream` of the plan's device;
 * asynchronous, allocation-free and graph-capturable like pa_decode_verify.
 * Served at every (head_dim, KV dtype) pa_plan accepts: 64 and 128 with
 * bf16 or FP8 KV, 256 with FP8 KV. The new tokens' positions come from the
 * plan's context lengths, so the plan must hold the step's actual lengths.
 * Returns PA_E_INVALID for a missing pointer, scales given for bf16 KV or
 * missing for FP8 KV, k_new/v_new/k_pool/v_pool not 4-byte aligned (8-byte
 * at head_dim 256), a plan built with lengths_are_bounds = 1, or a host-only
 * plan; PA_E_UNSUPPORTED for a (head_dim, KV dtype) without an append
 * kernel; PA_E_HIP if the launch fails. Nothing is launched on an error.
 * A plan whose sequences bring no new token returns PA_OK at once.
 */
pa_status pa_kv_append(const pa_plan_t* plan, const void* k_new, const void* v_new,
                       const int32_t* block_table, void* k_pool, void* v_pool,
                       float* k_scales, float* v_scales, void* stream);

/*
 * Greedy verify verdict: the step after the target's head in a verify round.
 * Source: ATOM #3091 ("High-interactivity monokernel decode for
 * DeepSeek-V4.1-Flash on MI355X"): the verify head gives a step's ids and
 * verdict in one launch for greedy rows (Engine hooks), and the next step's
 * input is each request's output id at the verdict's accepted count (the
 * review rounds on the head-served verify).
 * For sequence b with q = q_b verify rows t_b .. t_b + q - 1 (row 0's input
 * is the last committed token, rows 1..q-1 hold the q - 1 draft tokens):
 *   a_i = argmax over v < vocab of logits[t_b + i][v]   (lowest index among
 *         equal maxima; a NaN never wins; no value above -inf gives 0)
 *   n   = the largest n <= q - 1 with input_ids[t_b + 1 + j] == a_j for all
 *         j < n (the leading drafts the target agrees with)
 *   out_ids[t_b + i] = a_i, accepted[b] = n, next_ids[b] = a_n
 * The step emits a_0 .. a_n. A padded slot (q = 0) writes nothing.
 *   logits     [T][row_stride] bf16 or fp32 (logits_dtype), 16-byte aligned,
 *              row_stride >= vocab with a row spanning a multiple of 16 bytes
 *   input_ids  [T] int32, the verify rows' input tokens (layout of q's rows)
 *   out_ids    [T] int32; accepted, next_ids [B] int32
 * Uses the plan's query lengths and its scratch (argmax partials); enqueued
 * on `stream`, allocation-free and graph-capturable. Returns PA_E_INVALID
 * for a missing pointer, vocab < 1, a bad stride or alignment, or a
 * host-only plan, PA_E_UNSUPPORTED for another logits dtype, PA_E_HIP if a
 * launch fails.
 */
pa_status pa_verify_greedy(const pa_plan_t* plan, const void* logits, pa_dtype logits_dtype,
                           int32_t vocab, int64_t row_stride, const int32_t* input_ids,
                           int32_t* out_ids, int32_t* accepted, int32_t* next_ids,
                           void* stream);

/*
 * Measurement call: the streaming floor of a plan. One kernel reads exactly
 * the KV bytes pa_decode_verify's partition kernel reads for this plan
 * (every work item's 16-token pages of K and V through the block table, and
 * for FP8 KV the pages' scales), with the same direct global-to-LDS loads,
 * one workgroup per work item, and computes and writes nothing. Its kernel
 * time is the time the plan's bytes and page pattern take on their own, the
 * floor against which the partition kernel's streaming is judged.
 * Source: ATOM #2843 ("keep MTP-5 decode on FlyDSL pa_decode past the gluon
 * query-length limit", Follow-up in aiter: per-kernel microbenchmarks are
 * how the pages weigh this kernel). Enqueued on `stream`; allocation-free.
 * Returns PA_E_INVALID for a missing pointer, scales given for bf16 KV or
 * missing for FP8 KV, or a host-only plan; PA_E_HIP if the launch fails.
 */
pa_status pa_stream_floor(const pa_plan_t* plan, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const float* k_scales,
                          const float* v_scales, void* stream);

/* Release a plan and its device memory. NULL-safe. The caller makes sure no
 * call that uses the plan is still in flight. */
void pa_free(pa_plan_t* plan);

/* Text of the last non-OK status returned on the calling thread. */
const char* pa_last_error(void);

/*
 * Figures of a plan, each pointer optional:
 *   kv_bytes        algorithmic KV bytes one call reads: for every active
 *                   sequence, Hkv x (visible keys) x (K + V bytes per token,
 *                   plus 8 bytes of FP8 scales)
 *   scratch_bytes   device bytes of the partial results the plan owns
 *                   (with the two-level merge, its first-level partials too,
 *                   and the inner merge nodes' results of the single-launch
 *                   call)
 *   work_items      number of partition work items (workgroups launched)
 *   partition_tokens keys per work item actually used
 */
pa_status pa_plan_info(const pa_plan_t* plan, int64_t* kv_bytes,
                       int64_t* scratch_bytes, int32_t* work_items,
                       int32_t* partition_tokens);

/*
 * Copy the plan's work list to host memory as rows of 7 int32:
 * (sequence, kv head, first key, end key, partial slot or -1 when the item
 * covers all of its (sequence, kv head)'s keys and writes the output
 * directly, first packed row, packed rows). A workgroup carries at most 64
 * packed rows (48 at head_dim 256); a sequence with more is split into row
 * blocks, each an item of its own over the same keys and slot.
 * Writes min(capacity, work_items) rows; returns PA_E_INVALID if items is
 * NULL while capacity > 0.
 */
pa_status pa_plan_items(const pa_plan_t* plan, int32_t* items, int32_t capacity);

/*
 * Optional timing hook: when both are non-NULL (hipEvent_t handles on the
 * plan's device), every later pa_decode_verify launches the partition kernel
 * (and pa_stream_floor its kernel) with the two events attached
 * (hipExtLaunchKernelGGL), so `before` and `after` take that kernel's own
 * start and end timestamps on the call's stream. Pass NULLs to stop (a call
 * to be captured in a graph should run without them). Timing is the only
 * effect; results are unchanged.
 */
pa_status pa_set_partition_events(pa_plan_t* plan, void* before, void* after);

/*
 * Optional diagnostic hook: when `stamps` is non-NULL (a device buffer of
 * `capacity` uint64, owned by the caller, at least 8 x work_items of the
 * plan: PA_E_INVALID otherwise, and the hook is left as it was), every later
 * attention call
 * with this plan (pa_decode_verify, _dev, _fused, _noalloc) has each
 * partition workgroup write, at 8 i + slot for work item i, the device's
 * 100 MHz real-time clock at: 0 its start, 1 every wave past its chunk loop,
 * 2 its outputs issued (for a split item of pa_decode_verify_fused: its
 * partial's stores complete), 3 (fused, split items) its arrival counted,
 * 4 + l (fused, l < 3) its merge of a level-l tree node done when it was the
 * node's last arriver; slot 7 holds the XCC id in the high 32 bits and the
 * HW_ID register (CU, SIMD, shader engine) in the low 32. Slots a
 * workgroup does not reach are left as they were. Pass NULL to stop.
 * Results are unchanged; the stamps cost a few stores per workgroup.
 */
pa_status pa_set_workgroup_stamps(pa_plan_t* plan, void* stamps, int64_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* PA_VERIFY_H */
