/*
 * xqa.h -- batched grouped-query decode attention over a paged FP8-E5M2 KV
 * cache, for one AMD Instinct MI355X (gfx950) GPU.
 *
 * The operation (page "[Kernel][SM70] Pipeline batched E5M2 XQA decode",
 * sections Purpose and Starting bottleneck: batched long-context XQA decode
 * with an FP8 E5M2 KV cache; section Pending work and gates: randomized
 * physical pages, ragged and boundary context lengths). For every sequence b
 * in [0, batch) and query head hq in [0, Hq), with G = Hq / Hkv:
 *
 *     h = hq / G                     (query heads h*G .. h*G+G-1 share KV head h)
 *     n = min(context_lens[b], max_pages_per_seq * page_size)
 *     token t < n lives in page block_table[b][t / page_size], slot t % page_size
 *     z_t = scale * sum_d q[b][hq][d] * dec(k[page][h][slot][d])
 *     out[b][hq][:] = sum_t softmax(z)_t * dec(v[page][h][slot][:])
 *     n <= 0 gives a zero row.
 *
 * dec() is the OCP E5M2 decode: every code widens exactly to binary16 (the
 * code is the high byte of the binary16 word). Scores, softmax and the
 * weighted sum are accumulated in fp32; out is binary16, round to nearest even.
 *
 * Data layout (all device memory, owned by the caller):
 *     q            binary16 [batch][Hq][head_dim], contiguous
 *     k_pages      uint8    [num_pages][Hkv][page_size][head_dim] E5M2 codes
 *     v_pages      uint8    same layout as k_pages
 *     block_table  int32    [batch][max_pages_per_seq], row stride max_pages_per_seq
 *     context_lens int32    [batch]
 *     out          binary16 [batch][Hq][head_dim], contiguous
 * Supported shapes: head_dim 128, page_size 16, 1 <= G <= 16,
 * max_pages_per_seq * page_size <= 2^24.
 *
 * Device-resident values are not validated (that would need a device->host
 * copy and would break graph capture). Contract: block-table entries that a
 * sequence's first ceil(n / page_size) pages use must be valid page ids;
 * entries past them are never read; slots >= n of the last page and pages not
 * referenced never influence out, whatever their bytes (NaN codes included);
 * block tables may alias pages across sequences (read-only sharing).
 *
 * Errors are fail-closed: on any non-XQA_OK status nothing was launched.
 * Streams are passed as void* and must be a hipStream_t (0 = null stream).
 * All entry points are thread-safe except that one handle serves one stream
 * at a time: its workspace is shared between the calls made with it.
 */
#ifndef XQA_H
#define XQA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct xqa_handle_s* xqa_handle_t;

typedef enum {
  XQA_OK = 0,
  XQA_ERR_INVALID_ARG = 1,   /* null / misaligned pointer, out-of-range scalar        */
  XQA_ERR_UNSUPPORTED = 2,   /* shape outside the supported set                       */
  XQA_ERR_OUT_OF_MEMORY = 3, /* workspace allocation failed (xqa_create only)         */
  XQA_ERR_HIP = 4            /* HIP runtime error (no device, launch failure, ...)    */
} xqa_status_t;

/* Format of the cached K/V bytes (xqa_decode_fp8). */
typedef enum {
  XQA_KV_E5M2 = 0,           /* OCP FP8 E5M2: the code is the high byte of binary16      */
  XQA_KV_E4M3 = 1            /* OCP FP8 E4M3 ("E4M3FN"): bias 7, max 448, no infinities  */
} xqa_kv_format_t;

typedef struct {
  int32_t max_batch;         /* >= 1: largest batch a decode call may pass              */
  int32_t num_q_heads;       /* Hq, multiple of num_kv_heads                            */
  int32_t num_kv_heads;      /* Hkv >= 1                                                */
  int32_t head_dim;          /* 128                                                     */
  int32_t page_size;         /* 16                                                      */
  int32_t max_pages_per_seq; /* >= 1: block-table row stride in int32 elements          */
  int32_t max_work_items;    /* 0: sized from the device's occupancy (every CU's        */
                             /* resident slots), capped at the most items the largest   */
                             /* step the handle accepts can use; else the split grid    */
                             /* in workgroups, in [Hkv, Hkv*2048]                       */
  int32_t max_query_tokens;  /* 0 or 1: one query token per sequence; up to M with      */
                             /* G * M <= 16 for xqa_decode_multi                        */
  int32_t max_selected_pages;/* 0: no page-subset decode; else the longest selection    */
                             /* row xqa_decode_pages accepts, <= max_pages_per_seq      */
                             /* (sizes a page table of max_batch rows in the handle)    */
} xqa_config_t;

typedef struct {
  int32_t device;            /* HIP device the handle was created on                    */
  int32_t max_work_items;    /* grid of the split kernel                                */
  int32_t items_per_head;    /* max_work_items / Hkv: work items per KV head (at most)  */
  int32_t token_granule;     /* work items are whole blocks of this many tokens         */
  int32_t threads_per_item;  /* workgroup size of the split kernel                      */
  int32_t item_stride_floats;/* floats per split-state record (two records per item)    */
  int64_t workspace_bytes;   /* device bytes the handle owns                            */
  int32_t kernels_per_step;  /* 2 (split + combine), or 1 when the handle's bounds keep  */
                             /* every sequence in one work item (the split kernel then  */
                             /* also writes the zero rows of empty sequences)           */
} xqa_info_t;

/* Create a handle on the current HIP device. Validates cfg, sizes the split
 * grid from the split kernel's occupancy and allocates the workspace for
 * split states and, when max_selected_pages > 0, the page-subset table (the
 * only allocations the library makes). *out_handle is set
 * only on XQA_OK. Errors: INVALID_ARG (null pointers, non-positive sizes),
 * UNSUPPORTED (head_dim != 128, page_size != 16, Hq % Hkv != 0, G > 16,
 * G * max_query_tokens > 16, max_batch > 65536, more than 2^24 tokens per
 * sequence, max_selected_pages above max_pages_per_seq),
 * OUT_OF_MEMORY, HIP (no device). */
xqa_status_t xqa_create(const xqa_config_t* cfg, xqa_handle_t* out_handle);

/* Free the handle and its workspace. NULL is a no-op. The caller must make
 * sure no work issued with the handle is still running. */
xqa_status_t xqa_destroy(xqa_handle_t handle);

/* Copy the handle's sizes into *info. */
xqa_status_t xqa_get_info(xqa_handle_t handle, xqa_info_t* info);

/* One decode step: the split kernel and the combine kernel, back to back on
 * `stream` (the split kernel alone when the handle's bounds keep every
 * sequence in one work item; xqa_info_t.kernels_per_step). Nothing is allocated and nothing waits on the host, so the call
 * can be captured into a HIP graph and replayed with new contents of q,
 * block_table and context_lens. batch must be in [1, max_batch]; scale must
 * be finite. q, k_pages, v_pages and out must be 16-byte aligned,
 * block_table and context_lens 4-byte aligned. The calling thread's current
 * device must be the handle's device. Calls made with one handle must not
 * overlap in time (they share the handle's workspace); calls on one stream
 * never do. Errors: INVALID_ARG, HIP. */
xqa_status_t xqa_decode(xqa_handle_t handle, const void* q, const uint8_t* k_pages,
                        const uint8_t* v_pages, const int32_t* block_table,
                        const int32_t* context_lens, int32_t batch, float scale,
                        void* out, void* stream);

/* xqa_decode without a handle, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The split-state records and the per-(sequence, KV head)
 * merge records live in a fixed 16 MiB device array inside the library (one
 * per GPU, held until the process ends) instead of a handle's workspace;
 * nothing is allocated, here or later. cfg
 * (host memory) is validated as by xqa_create and sizes the step exactly as
 * a handle made from it would, so the output is bitwise that of xqa_decode
 * on such a handle. The first call on a device looks up the array's address
 * on that device (the calling thread's current device) and keeps it. Every
 * call on one GPU shares that GPU's array: calls on one stream are ordered
 * and safe; calls that overlap in time on one GPU (other streams, other
 * threads) race and give undefined results. Nothing in the array needs to
 * start at zero: every record a call reads, the same call wrote. Limit:
 * 2 * split grid * record floats * 4 bytes plus max_batch * Hkv * 8 bytes
 * must fit 16 MiB (the default grid on one MI355X does for every supported
 * head shape up to max_batch 65536 with 8 KV heads). Arguments,
 * alignment and errors as for xqa_decode, with cfg's max_batch;
 * INVALID_ARG / UNSUPPORTED as for xqa_create; UNSUPPORTED also when the
 * records do not fit the fixed array. */
xqa_status_t xqa_decode_noalloc(const xqa_config_t* cfg, const void* q, const uint8_t* k_pages,
                                const uint8_t* v_pages, const int32_t* block_table,
                                const int32_t* context_lens, int32_t batch, float scale,
                                void* out, void* stream);

/* Several new query tokens per sequence (speculative or multi-token
 * prediction rows, which the page "[Kernel][SM70] Pipeline batched E5M2 XQA
 * decode" lists beside single-token decode in its Purpose), causal among
 * themselves. q and out are binary16 [batch][M][Hq][head_dim], M =
 * num_query_tokens in [1, max_query_tokens]. With n as for xqa_decode (it
 * counts the M new tokens), query token j sits at position n - M + j:
 *     out[b][j][hq][:] = attention of q[b][j][hq] over tokens 0 .. n - M + j
 * and is a zero row when n - M + j < 0. The G * M query rows of a KV head
 * share one pass over its pages (they fill the matrix-core tile that a single
 * token leaves half empty at G = 8), so M = 2 reads the same KV bytes as
 * M = 1. M = 1 is exactly xqa_decode. Other arguments, alignment and errors
 * as for xqa_decode; INVALID_ARG also for num_query_tokens out of range. */
xqa_status_t xqa_decode_multi(xqa_handle_t handle, const void* q, const uint8_t* k_pages,
                              const uint8_t* v_pages, const int32_t* block_table,
                              const int32_t* context_lens, int32_t batch, int32_t num_query_tokens,
                              float scale, void* out, void* stream);

/* The general form: an E5M2 or E4M3 cache with per-tensor dequantisation
 * scales, one or several query tokens. Cached values are k_scale * dec(code)
 * and v_scale * dec(code), dec() the format's exact decode (E4M3 widens to
 * binary16 exactly with the gfx950 conversion instruction). Scores are
 * scale * k_scale * q.k (the product formed in double and rounded once to
 * fp32); outputs are v_scale times the normalised sum. The E4M3 reading
 * follows the page "[Kernel][WIP] Follow up FlashNext batch HC fusion and
 * QSA route audit" (section Test Result), which names E4M3 as a cache format
 * still awaiting quality admission. xqa_decode_multi is kv_format
 * XQA_KV_E5M2 with both scales 1. Errors: as for xqa_decode_multi;
 * INVALID_ARG also for an unknown kv_format or a non-finite k_scale,
 * v_scale or scale * k_scale. */
xqa_status_t xqa_decode_fp8(xqa_handle_t handle, xqa_kv_format_t kv_format, const void* q,
                            const uint8_t* k_pages, const uint8_t* v_pages,
                            const int32_t* block_table, const int32_t* context_lens, int32_t batch,
                            int32_t num_query_tokens, float scale, float k_scale, float v_scale,
                            void* out, void* stream);

/* First stage of xqa_decode alone (device-side plan, page gather, widening,
 * QK, online softmax, PV): rows of sequences that fit one work item and the
 * zero rows of sequences with n <= 0 are written to out; the other
 * sequences leave split states in the workspace, with a per-(sequence, KV
 * head) record of where they are. Same arguments and errors as xqa_decode.
 * xqa_decode_combine must follow on the same stream, with the same batch and
 * out, before the handle is used again. Exposed so the two stages can be
 * timed or scheduled apart. On a handle with kernels_per_step 1 no sequence
 * is split, and the combine finds nothing left to do. */
xqa_status_t xqa_decode_split(xqa_handle_t handle, const void* q, const uint8_t* k_pages,
                              const uint8_t* v_pages, const int32_t* block_table,
                              const int32_t* context_lens, int32_t batch, float scale,
                              void* out, void* stream);

/* Second stage of xqa_decode alone: log-sum-exp merge of the split states of
 * every sequence the split stage left split (fixed order), found through the
 * records the split stage wrote; context_lens is checked but not read.
 * Errors: INVALID_ARG (null or misaligned pointers, batch out of range), HIP. */
xqa_status_t xqa_decode_combine(xqa_handle_t handle, const int32_t* context_lens,
                                int32_t batch, void* out, void* stream);

/* KV append: write each sequence's new token into the paged cache, the step
 * that precedes decode (page "[Kernel][SM70] Pipeline batched E5M2 XQA
 * decode", section Purpose: the deployment keeps K and V as FP8 E5M2).
 *     n = context_lens[b]           length after the append; the new token is n - 1
 *     page = block_table[b][(n - 1) / page_size], slot = (n - 1) % page_size
 *     k_pages[page][h][slot][:] = E5M2(k_new[b][h][:]) for every KV head h; same for V
 * E5M2() rounds each binary16 value to the nearest finite E5M2 value, ties to
 * even: values past 57344 and infinities give +-57344, the sign is kept (a
 * negative value that rounds to zero gives -0), NaN gives 0x7F with its sign.
 * Sequences with n <= 0 or n > max_pages_per_seq * page_size are not written.
 * Layout (device memory, owned by the caller):
 *     k_new, v_new  binary16 [batch][Hkv][head_dim], contiguous, 16-byte aligned
 *     block_table, context_lens  as for xqa_decode
 *     k_pages, v_pages  as for xqa_decode (written), 16-byte aligned
 * The page receiving a token must not be the target of another sequence in
 * the same call. Only the 2 * Hkv * head_dim bytes of each target slot are
 * written. The call allocates nothing and never waits on the host, so it can
 * be captured together with xqa_decode, which must come after it on the same
 * stream. Errors: INVALID_ARG (null or misaligned pointers, batch outside
 * [1, max_batch]), HIP. */
xqa_status_t xqa_append_kv(xqa_handle_t handle, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* context_lens, int32_t batch,
                           uint8_t* k_pages, uint8_t* v_pages, void* stream);

/* One serving step in one call: xqa_append_kv followed by xqa_decode, with
 * the append fused into the decode's split kernel. The wave that will read a
 * sequence's last 32-token block first encodes the new K and V rows
 * (rounding as for xqa_append_kv) and stores them to the page slot, waits
 * until those stores have completed, and only then issues its loads of that
 * block, which read the new rows back like any cached token; no separate
 * launch is needed. Results (out and the page bytes) equal those of the two
 * calls in sequence, bit for bit. E5M2 cache, one query token. k_pages and
 * v_pages are written (the same contract as xqa_append_kv); other arguments
 * and errors as for xqa_decode and xqa_append_kv. */
xqa_status_t xqa_decode_append(xqa_handle_t handle, const void* q, const void* k_new,
                               const void* v_new, uint8_t* k_pages, uint8_t* v_pages,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t batch, float scale, void* out, void* stream);

/* Decode over a selected subset of each sequence's pages: the sparse-decode
 * form the page "[Kernel][WIP] Follow up FlashNext batch HC fusion and QSA
 * route audit" (section Test Result) describes, where a planner picks the KV
 * pages each query attends over. The page does not publish the selection
 * rule, so the selection is an input:
 *     page_select   int32 [batch][select_stride] logical page indices of sequence b
 *                   (index p covers tokens 16p .. 16p + 15), device memory; every
 *                   one of the batch x select_stride entries must be readable,
 *                   whatever the counts (entries past a row's count are read and
 *                   ignored)
 *     select_counts int32 [batch] entries of each row to use (clamped to [0, select_stride])
 * With n as for xqa_decode, an entry p is kept iff 0 <= p < ceil(n / 16) and
 * p is greater than every entry kept before it in its row (callers pass
 * ascending page indices; others are skipped). The query heads of sequence b
 * attend, exactly as in xqa_decode, over the tokens t < n of the kept pages;
 * no kept token gives a zero row. Selecting every page in order gives
 * xqa_decode's result bit for bit.
 * A small kernel first gathers the kept pages' physical ids into the
 * handle's page table (max_batch x max_selected_pages int32) with the
 * matching lengths; the split and combine kernels of xqa_decode then run on
 * it, so KV bytes are read only for the kept pages. E5M2 cache, one query
 * token. Other arguments, alignment and capture rules as for xqa_decode.
 * Errors: UNSUPPORTED when the handle was created with max_selected_pages 0;
 * INVALID_ARG as for xqa_decode, and for null or misaligned page_select /
 * select_counts or select_stride outside [1, max_selected_pages]; HIP. */
xqa_status_t xqa_decode_pages(xqa_handle_t handle, const void* q, const uint8_t* k_pages,
                              const uint8_t* v_pages, const int32_t* block_table,
                              const int32_t* context_lens, const int32_t* page_select,
                              const int32_t* select_counts, int32_t select_stride, int32_t batch,
                              float scale, void* out, void* stream);

/* Host mirror of the device-side plan, for diagnostics and tests:
 * context_lens_host is host memory [batch]. Each KV head's token stream
 * (sequences in batch order, each rounded up to 32-token blocks) is cut into
 * contiguous block ranges, one per work item, of near-equal cost, where a
 * non-empty sequence costs its blocks plus 4 (the price of starting it
 * inside an item). Writes the largest work item in tokens and the number of
 * work items (all heads) the device would use. */
xqa_status_t xqa_plan(xqa_handle_t handle, const int32_t* context_lens_host, int32_t batch,
                      int32_t* split_tokens, int32_t* num_items);

/* Test hook: widen n E5M2 codes with the same device routine the split
 * kernel uses for K. out_f16 receives the binary16 bit patterns, out_f32 the
 * same values as fp32 (either output may be NULL). Device pointers. */
xqa_status_t xqa_debug_widen_e5m2(const uint8_t* in, uint16_t* out_f16, float* out_f32,
                                  int64_t n, void* stream);

/* Test hook: the same for E4M3 codes and the device routine the split
 * kernel uses for E4M3 K. */
xqa_status_t xqa_debug_widen_e4m3(const uint8_t* in, uint16_t* out_f16, float* out_f32,
                                  int64_t n, void* stream);

/* Static name of a status code. */
const char* xqa_status_string(xqa_status_t status);

/* Human-readable detail of the calling thread's most recent error. */
const char* xqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* XQA_H */
