// C-ABI entry points: argument validation, handle and workspace, launches.
// Every check runs before any HIP call, so a rejected call launches nothing
// (fail-closed, as the page "[Kernel][SM70] Fold DeepSeek V4 MXFP4 decode
// exponents" asks of admission code in its audit comments: explicit errors,
// never a silent no-launch, no environment reads in native code).

#include <algorithm>
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include "../../include/xqa.h"
#include "xqa_internal.h"
#include "xqa_noalloc.h"
#include "xqa_select.h"

// Sizes derived from a configuration and the device: the split grid, the
// split-state records and the combine kernel's shape.
struct Geometry {
  int grid;             // split workgroups = work-item capacity
  int per_head;         // grid / Hkv
  int item_stride;      // floats per split-state record
  int max_q;            // query tokens per sequence the records are sized for
  int combine_waves;    // waves per combine workgroup
  bool direct_only;     // no sequence can leave split states: one kernel per step
  size_t partial_bytes; // 2 * grid records
  size_t desc_bytes;    // merge records: max_batch * Hkv int2, after the split states
};

struct xqa_handle_s {
  xqa_config_t cfg;
  int device;
  Geometry geo;
  float* partials;    // workspace: 2 * grid split-state records, then the merge records
  int32_t* vtable;    // page-subset decode: [max_batch][max_selected_pages] page ids, then
  int32_t* vlens;     //   [max_batch] lengths (null when max_selected_pages is 0)
  size_t workspace_bytes;
};

namespace {

thread_local char g_last_error[256] = "";

xqa_status_t fail(xqa_status_t st, const char* fmt, const char* detail = nullptr) {
  if (detail) {
    snprintf(g_last_error, sizeof(g_last_error), fmt, detail);
  } else {
    snprintf(g_last_error, sizeof(g_last_error), "%s", fmt);
  }
  return st;
}

xqa_status_t hip_fail(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
  return XQA_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

xqa_status_t check_decode_args(xqa_handle_t h, const void* q, const uint8_t* k_pages,
                               const uint8_t* v_pages, const int32_t* block_table,
                               const int32_t* context_lens, int32_t batch, float scale,
                               const void* out) {
  if (!h) return fail(XQA_ERR_INVALID_ARG, "null handle");
  if (!q || !k_pages || !v_pages || !block_table || !context_lens || !out)
    return fail(XQA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
    return fail(XQA_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4))
    return fail(XQA_ERR_INVALID_ARG, "block_table and context_lens must be 4-byte aligned");
  if (batch < 1 || batch > h->cfg.max_batch)
    return fail(XQA_ERR_INVALID_ARG, "batch outside [1, max_batch]");
  if (!isfinite(scale)) return fail(XQA_ERR_INVALID_ARG, "scale must be finite");
  return XQA_OK;
}

xqa_status_t check_device(xqa_handle_t h) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != h->device)
    return fail(XQA_ERR_INVALID_ARG, "current device differs from the handle's device");
  return XQA_OK;
}

xqa::AttendArgs attend_args(const xqa_config_t& cfg, const Geometry& geo, void* workspace,
                            const void* q, const uint8_t* k_pages,
                            const uint8_t* v_pages, const int32_t* block_table,
                            const int32_t* context_lens, int32_t batch, float scale, void* out,
                            int32_t q_tokens = 1) {
  xqa::AttendArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.out = static_cast<uint16_t*>(out);
  a.partials = static_cast<float*>(workspace);
  a.merge_desc = reinterpret_cast<int2*>(static_cast<char*>(workspace) + geo.partial_bytes);
  a.batch = batch;
  a.num_kv_heads = cfg.num_kv_heads;
  a.group = cfg.num_q_heads / cfg.num_kv_heads;
  a.q_tokens = q_tokens;
  a.rows = a.group * q_tokens;
  a.max_pages = cfg.max_pages_per_seq;
  a.max_tokens = cfg.max_pages_per_seq * xqa::kPageSize;
  a.per_head = geo.per_head;
  a.item_stride = geo.item_stride;
  a.combine_waves = geo.combine_waves;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.v_scale = 1.0f;
  a.kv_format = xqa::kKvE5M2;
  a.k_new = nullptr;
  a.v_new = nullptr;
  return a;
}

xqa::AttendArgs attend_args(xqa_handle_t h, const void* q, const uint8_t* k_pages,
                            const uint8_t* v_pages, const int32_t* block_table,
                            const int32_t* context_lens, int32_t batch, float scale, void* out,
                            int32_t q_tokens = 1) {
  return attend_args(h->cfg, h->geo, h->partials, q, k_pages, v_pages, block_table, context_lens,
                     batch, scale, out, q_tokens);
}

// Validation shared by xqa_create and xqa_decode_noalloc.
xqa_status_t check_config(const xqa_config_t* cfg) {
  if (cfg->max_batch < 1 || cfg->num_q_heads < 1 || cfg->num_kv_heads < 1 ||
      cfg->max_pages_per_seq < 1 || cfg->max_work_items < 0 || cfg->max_query_tokens < 0 ||
      cfg->max_selected_pages < 0)
    return fail(XQA_ERR_INVALID_ARG, "sizes must be positive");
  if (cfg->max_selected_pages > cfg->max_pages_per_seq)
    return fail(XQA_ERR_UNSUPPORTED, "max_selected_pages above max_pages_per_seq");
  if (cfg->head_dim != xqa::kHeadDim) return fail(XQA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (cfg->page_size != xqa::kPageSize) return fail(XQA_ERR_UNSUPPORTED, "page_size must be 16");
  if (cfg->num_q_heads % cfg->num_kv_heads != 0)
    return fail(XQA_ERR_UNSUPPORTED, "num_q_heads must be a multiple of num_kv_heads");
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  if (G > xqa::kMaxGroup) return fail(XQA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  const int max_q = cfg->max_query_tokens == 0 ? 1 : cfg->max_query_tokens;
  if ((long long)G * max_q > xqa::kMaxGroup)
    return fail(XQA_ERR_UNSUPPORTED,
                "query heads per KV head times max_query_tokens must not exceed 16");
  if (cfg->max_batch > xqa::kMaxBatch) return fail(XQA_ERR_UNSUPPORTED, "max_batch above 65536");
  if ((long long)cfg->max_pages_per_seq * xqa::kPageSize > xqa::kMaxSeqTokens)
    return fail(XQA_ERR_UNSUPPORTED, "max_pages_per_seq * page_size must not exceed 2^24 tokens");
  // Every launch's grid must fit HIP's 2^31 - 1 workgroups: the combine
  // kernel runs up to max_batch * Hkv * 8 workgroups, the split kernel at
  // most Hkv * 2048.
  if ((long long)cfg->max_batch * cfg->num_kv_heads * (xqa::kHeadDim / 16) > INT32_MAX ||
      (long long)cfg->num_kv_heads * xqa::kMaxItemsPerHead > INT32_MAX)
    return fail(XQA_ERR_UNSUPPORTED, "max_batch * num_kv_heads too large for one launch grid");
  const long long min_grid = cfg->num_kv_heads;
  const long long max_grid = (long long)cfg->num_kv_heads * xqa::kMaxItemsPerHead;
  if (cfg->max_work_items > 0 &&
      (cfg->max_work_items < min_grid || cfg->max_work_items > max_grid))
    return fail(XQA_ERR_INVALID_ARG, "max_work_items must lie in [Hkv, Hkv*2048]");
  return XQA_OK;
}

// Sizes of a validated configuration on a device with `cus` compute units
// and `per_cu` resident split workgroups per CU.
Geometry geometry(const xqa_config_t& cfg, int cus, int per_cu) {
  Geometry g;
  const long long min_grid = cfg.num_kv_heads;
  const long long max_grid = (long long)cfg.num_kv_heads * xqa::kMaxItemsPerHead;
  const int32_t max_tokens = (int32_t)((long long)cfg.max_pages_per_seq * xqa::kPageSize);
  long long grid = cfg.max_work_items;
  if (grid == 0) {
    // Every item resident at once: one round of equal-sized items, the same
    // number on every CU.
    grid = (long long)cus * (per_cu < 1 ? 1 : per_cu);
    // A step never has more than max_batch full sequences, so it never plans
    // more than ceil(NB_max / 8) items per head; slots past that would only
    // be dispatched to exit (a few microseconds on small workloads).
    const long long nb_max = (long long)cfg.max_batch * xqa::seq_blocks(max_tokens);
    const long long useful = (long long)cfg.num_kv_heads *
                             ((nb_max + xqa::kMinItemBlocks - 1) / xqa::kMinItemBlocks);
    if (grid > useful) grid = useful;
    if (grid < min_grid) grid = min_grid;
    if (grid > max_grid) grid = max_grid;
  }
  g.per_head = (int)(grid / cfg.num_kv_heads);
  g.grid = g.per_head * cfg.num_kv_heads;
  const int G = cfg.num_q_heads / cfg.num_kv_heads;
  g.max_q = cfg.max_query_tokens == 0 ? 1 : cfg.max_query_tokens;
  // A record holds O, max and sum of every query row: G * max_query_tokens rows.
  g.item_stride = ((G * g.max_q * (xqa::kHeadDim + 2)) + 3) / 4 * 4;
  // Two record slots per work item: its first and its last segment.
  g.partial_bytes = (size_t)2 * g.grid * g.item_stride * sizeof(float);
  g.desc_bytes = (size_t)cfg.max_batch * cfg.num_kv_heads * sizeof(int2);
  // A sequence leaves at most one split state per item and per block, so a
  // handle whose bound stays within one combine round gets the one-wave
  // combine workgroups; a longer one shares the rounds over four waves.
  const int max_states = std::min(g.per_head, xqa::seq_blocks(max_tokens));
  g.combine_waves = max_states > xqa::kCombineRound ? xqa::kCombineMaxWaves : 1;
  // With one state per sequence at most, every sequence is finished in the
  // split kernel, which then also writes the zero rows of empty sequences:
  // a decode step is one kernel.
  g.direct_only = max_states <= 1;
  return g;
}

xqa_status_t device_geometry(const xqa_config_t& cfg, int* dev, Geometry* geo) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, *dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  int per_cu = 0;
  e = xqa::attend_blocks_per_cu(&per_cu);
  if (e != hipSuccess) return hip_fail(e, "occupancy query");
  *geo = geometry(cfg, cus, per_cu);
  return XQA_OK;
}

}  // namespace

extern "C" {

const char* xqa_status_string(xqa_status_t s) {
  switch (s) {
    case XQA_OK: return "XQA_OK";
    case XQA_ERR_INVALID_ARG: return "XQA_ERR_INVALID_ARG";
    case XQA_ERR_UNSUPPORTED: return "XQA_ERR_UNSUPPORTED";
    case XQA_ERR_OUT_OF_MEMORY: return "XQA_ERR_OUT_OF_MEMORY";
    case XQA_ERR_HIP: return "XQA_ERR_HIP";
  }
  return "XQA_ERR_UNKNOWN";
}

const char* xqa_last_error(void) { return g_last_error; }

xqa_status_t xqa_create(const xqa_config_t* cfg, xqa_handle_t* out_handle) {
  if (!cfg || !out_handle) return fail(XQA_ERR_INVALID_ARG, "null cfg or out_handle");
  xqa_status_t st = check_config(cfg);
  if (st != XQA_OK) return st;
  int dev = -1;
  Geometry geo;
  if ((st = device_geometry(*cfg, &dev, &geo)) != XQA_OK) return st;

  xqa_handle_s* h = new (std::nothrow) xqa_handle_s();
  if (!h) return fail(XQA_ERR_OUT_OF_MEMORY, "host allocation failed");
  h->cfg = *cfg;
  h->cfg.max_query_tokens = geo.max_q;
  h->device = dev;
  h->geo = geo;
  // Page-subset decode: a page table of max_batch rows plus their lengths.
  const size_t vt_elems = cfg->max_selected_pages > 0
                              ? (size_t)cfg->max_batch * cfg->max_selected_pages + cfg->max_batch
                              : 0;
  const size_t ws = geo.partial_bytes + geo.desc_bytes;
  h->workspace_bytes = ws + vt_elems * sizeof(int32_t);
  h->partials = nullptr;
  h->vtable = nullptr;
  h->vlens = nullptr;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&h->partials), ws);
  if (e == hipSuccess && vt_elems > 0) {
    e = hipMalloc(reinterpret_cast<void**>(&h->vtable), vt_elems * sizeof(int32_t));
    if (e == hipSuccess) h->vlens = h->vtable + (size_t)cfg->max_batch * cfg->max_selected_pages;
  }
  if (e != hipSuccess) {
    if (h->partials) (void)hipFree(h->partials);
    delete h;
    if (e == hipErrorOutOfMemory) return fail(XQA_ERR_OUT_OF_MEMORY, "workspace allocation failed");
    return hip_fail(e, "workspace allocation");
  }

  *out_handle = h;
  return XQA_OK;
}

xqa_status_t xqa_destroy(xqa_handle_t h) {
  if (!h) return XQA_OK;
  hipError_t e = hipSuccess;
  if (h->partials) e = hipFree(h->partials);
  if (h->vtable) {
    const hipError_t e2 = hipFree(h->vtable);
    if (e == hipSuccess) e = e2;
  }
  delete h;
  if (e != hipSuccess) return hip_fail(e, "hipFree");
  return XQA_OK;
}

xqa_status_t xqa_get_info(xqa_handle_t h, xqa_info_t* info) {
  if (!h || !info) return fail(XQA_ERR_INVALID_ARG, "null handle or info");
  info->device = h->device;
  info->max_work_items = h->geo.grid;
  info->items_per_head = h->geo.per_head;
  info->token_granule = xqa::kBlockTokens;
  info->threads_per_item = xqa::kThreads;
  info->item_stride_floats = h->geo.item_stride;
  info->workspace_bytes = (int64_t)h->workspace_bytes;
  info->kernels_per_step = h->geo.direct_only ? 1 : 2;
  return XQA_OK;
}

xqa_status_t xqa_decode_split(xqa_handle_t h, const void* q, const uint8_t* k_pages,
                              const uint8_t* v_pages, const int32_t* block_table,
                              const int32_t* context_lens, int32_t batch, float scale, void* out,
                              void* stream) {
  xqa_status_t st =
      check_decode_args(h, q, k_pages, v_pages, block_table, context_lens, batch, scale, out);
  if (st != XQA_OK) return st;
  if ((st = check_device(h)) != XQA_OK) return st;
  const xqa::AttendArgs a =
      attend_args(h, q, k_pages, v_pages, block_table, context_lens, batch, scale, out);
  hipError_t e = xqa::launch_split(a, h->geo.grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "split kernel launch");
  return XQA_OK;
}

xqa_status_t xqa_decode_combine(xqa_handle_t h, const int32_t* context_lens, int32_t batch,
                                void* out, void* stream) {
  if (!h) return fail(XQA_ERR_INVALID_ARG, "null handle");
  if (!context_lens || !out) return fail(XQA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(out, 16) || !aligned(context_lens, 4))
    return fail(XQA_ERR_INVALID_ARG, "misaligned pointer");
  if (batch < 1 || batch > h->cfg.max_batch)
    return fail(XQA_ERR_INVALID_ARG, "batch outside [1, max_batch]");
  xqa_status_t st = check_device(h);
  if (st != XQA_OK) return st;
  xqa::AttendArgs a = attend_args(h, nullptr, nullptr, nullptr, nullptr, context_lens, batch, 0.f,
                                  out);
  hipError_t e = xqa::launch_combine(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return XQA_OK;
}

xqa_status_t xqa_decode(xqa_handle_t h, const void* q, const uint8_t* k_pages,
                        const uint8_t* v_pages, const int32_t* block_table,
                        const int32_t* context_lens, int32_t batch, float scale, void* out,
                        void* stream) {
  return xqa_decode_multi(h, q, k_pages, v_pages, block_table, context_lens, batch, 1, scale, out,
                          stream);
}

xqa_status_t xqa_decode_noalloc(const xqa_config_t* cfg, const void* q, const uint8_t* k_pages,
                                const uint8_t* v_pages, const int32_t* block_table,
                                const int32_t* context_lens, int32_t batch, float scale, void* out,
                                void* stream) {
  if (!cfg) return fail(XQA_ERR_INVALID_ARG, "null cfg");
  xqa_status_t st = check_config(cfg);
  if (st != XQA_OK) return st;
  if (!q || !k_pages || !v_pages || !block_table || !context_lens || !out)
    return fail(XQA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
    return fail(XQA_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4))
    return fail(XQA_ERR_INVALID_ARG, "block_table and context_lens must be 4-byte aligned");
  if (batch < 1 || batch > cfg->max_batch)
    return fail(XQA_ERR_INVALID_ARG, "batch outside [1, max_batch]");
  if (!isfinite(scale)) return fail(XQA_ERR_INVALID_ARG, "scale must be finite");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  xqa::NoallocDevice nd;
  e = xqa::noalloc_device(dev, &nd);
  if (e != hipSuccess) return hip_fail(e, "fixed workspace lookup");
  const Geometry geo = geometry(*cfg, nd.cus, nd.per_cu);
  if (geo.partial_bytes + geo.desc_bytes > xqa::kNoallocScratchBytes)
    return fail(XQA_ERR_UNSUPPORTED,
                "the configuration's split states exceed the fixed 16 MiB workspace "
                "(fewer max_work_items, KV heads or query rows)");
  const xqa::AttendArgs a = attend_args(*cfg, geo, nd.scratch, q, k_pages,
                                        v_pages, block_table, context_lens, batch, scale, out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  e = xqa::launch_split(a, geo.grid, s);
  if (e != hipSuccess) return hip_fail(e, "split kernel launch");
  if (geo.direct_only) return XQA_OK;
  e = xqa::launch_combine(a, s);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return XQA_OK;
}

xqa_status_t xqa_decode_multi(xqa_handle_t h, const void* q, const uint8_t* k_pages,
                              const uint8_t* v_pages, const int32_t* block_table,
                              const int32_t* context_lens, int32_t batch, int32_t num_query_tokens,
                              float scale, void* out, void* stream) {
  return xqa_decode_fp8(h, XQA_KV_E5M2, q, k_pages, v_pages, block_table, context_lens, batch,
                        num_query_tokens, scale, 1.0f, 1.0f, out, stream);
}

xqa_status_t xqa_decode_fp8(xqa_handle_t h, xqa_kv_format_t kv_format, const void* q,
                            const uint8_t* k_pages, const uint8_t* v_pages,
                            const int32_t* block_table, const int32_t* context_lens, int32_t batch,
                            int32_t num_query_tokens, float scale, float k_scale, float v_scale,
                            void* out, void* stream) {
  xqa_status_t st =
      check_decode_args(h, q, k_pages, v_pages, block_table, context_lens, batch, scale, out);
  if (st != XQA_OK) return st;
  if (kv_format != XQA_KV_E5M2 && kv_format != XQA_KV_E4M3)
    return fail(XQA_ERR_INVALID_ARG, "kv_format must be XQA_KV_E5M2 or XQA_KV_E4M3");
  if (num_query_tokens < 1 || num_query_tokens > h->cfg.max_query_tokens)
    return fail(XQA_ERR_INVALID_ARG, "num_query_tokens outside [1, max_query_tokens]");
  const double score_scale = (double)scale * (double)k_scale * 1.4426950408889634;
  if (!isfinite(k_scale) || !isfinite(v_scale) || !isfinite((float)score_scale))
    return fail(XQA_ERR_INVALID_ARG, "k_scale, v_scale and scale * k_scale must be finite");
  if ((st = check_device(h)) != XQA_OK) return st;
  xqa::AttendArgs a = attend_args(h, q, k_pages, v_pages, block_table, context_lens, batch, scale,
                                  out, num_query_tokens);
  a.scale_log2e = (float)score_scale;
  a.v_scale = v_scale;
  a.kv_format = kv_format == XQA_KV_E4M3 ? xqa::kKvE4M3 : xqa::kKvE5M2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = xqa::launch_split(a, h->geo.grid, s);
  if (e != hipSuccess) return hip_fail(e, "split kernel launch");
  if (h->geo.direct_only) return XQA_OK;
  e = xqa::launch_combine(a, s);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return XQA_OK;
}

xqa_status_t xqa_append_kv(xqa_handle_t h, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* context_lens, int32_t batch,
                           uint8_t* k_pages, uint8_t* v_pages, void* stream) {
  if (!h) return fail(XQA_ERR_INVALID_ARG, "null handle");
  if (!k_new || !v_new || !block_table || !context_lens || !k_pages || !v_pages)
    return fail(XQA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16))
    return fail(XQA_ERR_INVALID_ARG, "k_new, v_new, k_pages and v_pages must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4))
    return fail(XQA_ERR_INVALID_ARG, "block_table and context_lens must be 4-byte aligned");
  if (batch < 1 || batch > h->cfg.max_batch)
    return fail(XQA_ERR_INVALID_ARG, "batch outside [1, max_batch]");
  xqa_status_t st = check_device(h);
  if (st != XQA_OK) return st;
  xqa::AppendArgs a;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.batch = batch;
  a.num_kv_heads = h->cfg.num_kv_heads;
  a.max_pages = h->cfg.max_pages_per_seq;
  a.max_tokens = h->cfg.max_pages_per_seq * xqa::kPageSize;
  hipError_t e = xqa::launch_append(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append kernel launch");
  return XQA_OK;
}

xqa_status_t xqa_decode_append(xqa_handle_t h, const void* q, const void* k_new, const void* v_new,
                               uint8_t* k_pages, uint8_t* v_pages, const int32_t* block_table,
                               const int32_t* context_lens, int32_t batch, float scale, void* out,
                               void* stream) {
  xqa_status_t st =
      check_decode_args(h, q, k_pages, v_pages, block_table, context_lens, batch, scale, out);
  if (st != XQA_OK) return st;
  if (!k_new || !v_new) return fail(XQA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(XQA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  if ((st = check_device(h)) != XQA_OK) return st;
  xqa::AttendArgs a =
      attend_args(h, q, k_pages, v_pages, block_table, context_lens, batch, scale, out);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = xqa::launch_split(a, h->geo.grid, s);
  if (e != hipSuccess) return hip_fail(e, "split kernel launch");
  if (h->geo.direct_only) return XQA_OK;
  e = xqa::launch_combine(a, s);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return XQA_OK;
}

xqa_status_t xqa_decode_pages(xqa_handle_t h, const void* q, const uint8_t* k_pages,
                              const uint8_t* v_pages, const int32_t* block_table,
                              const int32_t* context_lens, const int32_t* page_select,
                              const int32_t* select_counts, int32_t select_stride, int32_t batch,
                              float scale, void* out, void* stream) {
  xqa_status_t st =
      check_decode_args(h, q, k_pages, v_pages, block_table, context_lens, batch, scale, out);
  if (st != XQA_OK) return st;
  if (h->cfg.max_selected_pages == 0)
    return fail(XQA_ERR_UNSUPPORTED, "handle created with max_selected_pages 0");
  if (!page_select || !select_counts) return fail(XQA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(page_select, 4) || !aligned(select_counts, 4))
    return fail(XQA_ERR_INVALID_ARG, "page_select and select_counts must be 4-byte aligned");
  if (select_stride < 1 || select_stride > h->cfg.max_selected_pages)
    return fail(XQA_ERR_INVALID_ARG, "select_stride outside [1, max_selected_pages]");
  if ((st = check_device(h)) != XQA_OK) return st;
  xqa::SelectArgs sa;
  sa.block_table = block_table;
  sa.context_lens = context_lens;
  sa.page_select = page_select;
  sa.select_counts = select_counts;
  sa.vtable = h->vtable;
  sa.vlens = h->vlens;
  sa.batch = batch;
  sa.max_pages = h->cfg.max_pages_per_seq;
  sa.max_tokens = h->cfg.max_pages_per_seq * xqa::kPageSize;
  sa.select_stride = select_stride;
  sa.vstride = h->cfg.max_selected_pages;
  // The decode runs over the gathered table: its row stride and capacity
  // are the selection's.
  xqa::AttendArgs a = attend_args(h, q, k_pages, v_pages, h->vtable, h->vlens, batch, scale, out);
  a.max_pages = h->cfg.max_selected_pages;
  a.max_tokens = h->cfg.max_selected_pages * xqa::kPageSize;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = xqa::launch_select(sa, s);
  if (e != hipSuccess) return hip_fail(e, "select kernel launch");
  e = xqa::launch_split(a, h->geo.grid, s);
  if (e != hipSuccess) return hip_fail(e, "split kernel launch");
  if (h->geo.direct_only) return XQA_OK;
  e = xqa::launch_combine(a, s);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return XQA_OK;
}

xqa_status_t xqa_plan(xqa_handle_t h, const int32_t* ctx, int32_t batch, int32_t* split_tokens,
                      int32_t* num_items) {
  if (!h || !ctx || !split_tokens || !num_items)
    return fail(XQA_ERR_INVALID_ARG, "null argument");
  if (batch < 1 || batch > h->cfg.max_batch)
    return fail(XQA_ERR_INVALID_ARG, "batch outside [1, max_batch]");
  const int max_tokens = h->cfg.max_pages_per_seq * xqa::kPageSize;
  long long nb_total = 0, cost_total = 0;
  for (int b = 0; b < batch; ++b) nb_total += xqa::seq_blocks(xqa::clamp_len(ctx[b], max_tokens));
  const int P = xqa::items_per_head(nb_total, h->geo.per_head);
  for (int b = 0; b < batch; ++b)
    cost_total += xqa::seq_cost(xqa::seq_blocks(xqa::clamp_len(ctx[b], max_tokens)), nb_total, P);
  // Walk the cost stream once: each item's end, as a block.
  long long largest = 0, lo = 0, coff = 0, off = 0;
  int b = 0;
  for (int i = 1; i <= P; ++i) {
    const long long c = xqa::item_lo(i, cost_total, P);
    long long hi = nb_total;
    if (c < cost_total) {
      for (;; ++b) {
        const int blocks = xqa::seq_blocks(xqa::clamp_len(ctx[b], max_tokens));
        const int cost = xqa::seq_cost(blocks, nb_total, P);
        if (c < coff + cost) {
          const long long local = c - coff - (cost - blocks);
          hi = off + (local > 0 ? local : 0);
          break;
        }
        coff += cost;
        off += blocks;
      }
    }
    largest = std::max(largest, hi - lo);
    lo = hi;
  }
  *split_tokens = (int32_t)(largest * xqa::kBlockTokens);
  *num_items = P * h->cfg.num_kv_heads;
  return XQA_OK;
}

xqa_status_t xqa_debug_widen_e5m2(const uint8_t* in, uint16_t* out_f16, float* out_f32, int64_t n,
                                  void* stream) {
  if (!in || (!out_f16 && !out_f32)) return fail(XQA_ERR_INVALID_ARG, "null pointer");
  if (n < 0) return fail(XQA_ERR_INVALID_ARG, "negative count");
  if ((out_f16 && !aligned(out_f16, 2)) || (out_f32 && !aligned(out_f32, 4)))
    return fail(XQA_ERR_INVALID_ARG, "misaligned output");
  if (n == 0) return XQA_OK;
  hipError_t e =
      xqa::launch_widen(in, out_f16, out_f32, n, xqa::kKvE5M2, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "widen kernel launch");
  return XQA_OK;
}

xqa_status_t xqa_debug_widen_e4m3(const uint8_t* in, uint16_t* out_f16, float* out_f32, int64_t n,
                                  void* stream) {
  if (!in || (!out_f16 && !out_f32)) return fail(XQA_ERR_INVALID_ARG, "null pointer");
  if (n < 0) return fail(XQA_ERR_INVALID_ARG, "negative count");
  if ((out_f16 && !aligned(out_f16, 2)) || (out_f32 && !aligned(out_f32, 4)))
    return fail(XQA_ERR_INVALID_ARG, "misaligned output");
  if (n == 0) return XQA_OK;
  hipError_t e =
      xqa::launch_widen(in, out_f16, out_f32, n, xqa::kKvE4M3, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "widen kernel launch");
  return XQA_OK;
}

}  // extern "C"
