// Host-only check of the C-ABI layer (csrc/xqa_api.cpp): argument validation,
// handle sizing and the arguments each entry point hands to the kernel
// launchers. Built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer, no GPU: the few HIP runtime calls the layer
// makes and the kernel launchers are replaced by host fakes that record what
// they receive. Prints "OK <checks>" or the first failure and exits non-zero.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "xqa.h"
#include "xqa_internal.h"
#include "xqa_noalloc.h"
#include "xqa_select.h"

namespace {

struct Launch {
  char kind;            // 's' split, 'c' combine, 'a' append, 'p' select, 'w' widen
  int grid;
  xqa::AttendArgs a;
  xqa::AppendArgs ap;
  xqa::SelectArgs sel;
};

std::vector<Launch> g_launches;
int g_checks = 0;
int g_fail = 0;

void expect(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok && !g_fail) {
    std::printf("FAIL line %d: %s\n", line, what);
    g_fail = 1;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

}  // namespace

// ---- fakes of the HIP runtime calls the layer makes (host memory only)
extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;   // compute units
  return hipSuccess;
}
hipError_t hipMalloc(void** ptr, size_t size) {
  *ptr = std::malloc(size);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "fake HIP error"; }
}

// ---- fakes of the kernel launchers: record, launch nothing
namespace xqa {
hipError_t launch_split(const AttendArgs& a, int grid, hipStream_t) {
  g_launches.push_back({'s', grid, a, {}, {}});
  return hipSuccess;
}
hipError_t launch_combine(const AttendArgs& a, hipStream_t) {
  g_launches.push_back({'c', 0, a, {}, {}});
  return hipSuccess;
}
hipError_t launch_append(const AppendArgs& a, hipStream_t) {
  g_launches.push_back({'a', 0, {}, a, {}});
  return hipSuccess;
}
hipError_t launch_select(const SelectArgs& a, hipStream_t) {
  g_launches.push_back({'p', 0, {}, {}, a});
  return hipSuccess;
}
hipError_t launch_widen(const uint8_t*, uint16_t*, float*, int64_t, int32_t, hipStream_t) {
  g_launches.push_back({'w', 0, {}, {}, {}});
  return hipSuccess;
}
hipError_t attend_blocks_per_cu(int* blocks) {
  *blocks = 2;
  return hipSuccess;
}
// The fixed workspace: a stand-in address; xqa_decode_noalloc only passes it on.
alignas(256) unsigned char g_fixed[64];
int g_noalloc_lookups = 0;
hipError_t noalloc_device(int device, NoallocDevice* out) {
  ++g_noalloc_lookups;
  out->scratch = g_fixed;
  out->cus = 256;
  out->per_cu = 2;
  return device == 0 ? hipSuccess : hipErrorInvalidDevice;
}
}  // namespace xqa

namespace {

xqa_config_t config(int batch, int hq, int hkv, int pages) {
  xqa_config_t c;
  std::memset(&c, 0, sizeof(c));
  c.max_batch = batch;
  c.num_q_heads = hq;
  c.num_kv_heads = hkv;
  c.head_dim = 128;
  c.page_size = 16;
  c.max_pages_per_seq = pages;
  return c;
}

alignas(16) unsigned char g_buf[1 << 16];

}  // namespace

int main() {
  void* p16 = g_buf;                 // 16-byte aligned stand-ins for device pointers
  void* odd = g_buf + 2;             // 2-byte aligned only
  const uint8_t* kv = g_buf + 32;
  const int32_t* i32 = reinterpret_cast<const int32_t*>(g_buf + 64);
  int32_t host_lens[3] = {100, 0, 5000};

  // Creation: rejected configurations create nothing.
  {
    xqa_handle_t h = nullptr;
    xqa_config_t c = config(16, 32, 4, 64);
    c.head_dim = 64;
    EXPECT(xqa_create(&c, &h) == XQA_ERR_UNSUPPORTED && h == nullptr);
    c = config(16, 32, 4, 64);
    c.max_selected_pages = 65;
    EXPECT(xqa_create(&c, &h) == XQA_ERR_UNSUPPORTED && h == nullptr);
    c.max_selected_pages = -1;
    EXPECT(xqa_create(&c, &h) == XQA_ERR_INVALID_ARG && h == nullptr);
    c = config(16, 34, 4, 64);
    EXPECT(xqa_create(&c, &h) == XQA_ERR_UNSUPPORTED && h == nullptr);
    c = config(1, 8, 1, (1 << 20) + 1);
    EXPECT(xqa_create(&c, &h) == XQA_ERR_UNSUPPORTED && h == nullptr);
    // The combine grid (max_batch * Hkv * 8 workgroups) must fit one launch.
    c = config(65536, 4097, 4097, 1);
    EXPECT(xqa_create(&c, &h) == XQA_ERR_UNSUPPORTED && h == nullptr);
    EXPECT(xqa_create(nullptr, &h) == XQA_ERR_INVALID_ARG);
    EXPECT(std::strlen(xqa_last_error()) > 0);
  }

  // The ragged B16 handle: grid, workspace and the decode launches.
  xqa_handle_t h = nullptr;
  xqa_config_t c = config(16, 32, 4, 16384);
  c.max_selected_pages = 16384;
  EXPECT(xqa_create(&c, &h) == XQA_OK && h != nullptr);
  xqa_info_t info;
  EXPECT(xqa_get_info(h, &info) == XQA_OK);
  EXPECT(info.max_work_items == 512 && info.items_per_head == 128);
  EXPECT(info.kernels_per_step == 2);
  // split-state records, merge descriptors (16 sequences x 4 heads x 8 bytes),
  // then the page-subset table
  EXPECT(info.workspace_bytes == (int64_t)2 * 512 * info.item_stride_floats * 4 + 16 * 4 * 8 +
                                     (int64_t)(16 * 16384 + 16) * 4);
  EXPECT(info.item_stride_floats % 4 == 0 && info.item_stride_floats >= 8 * 130);

  g_launches.clear();
  EXPECT(xqa_decode(h, p16, kv, kv, i32, i32, 16, 0.0883883f, p16, nullptr) == XQA_OK);
  EXPECT(g_launches.size() == 2 && g_launches[0].kind == 's' && g_launches[1].kind == 'c');
  if (g_launches.size() == 2) {
    const xqa::AttendArgs& a = g_launches[0].a;
    EXPECT(g_launches[0].grid == 512);
    EXPECT(a.batch == 16 && a.num_kv_heads == 4 && a.group == 8 && a.rows == 8 && a.q_tokens == 1);
    EXPECT(a.max_pages == 16384 && a.max_tokens == 16384 * 16 && a.per_head == 128);
    EXPECT(a.k_new == nullptr && a.v_new == nullptr && a.kv_format == xqa::kKvE5M2);
    EXPECT(std::fabs(a.scale_log2e - 0.0883883f * 1.4426950408889634f) < 1e-7f);
    EXPECT(a.v_scale == 1.0f);
    EXPECT((const char*)a.merge_desc == (const char*)a.partials + (size_t)2 * 512 * info.item_stride_floats * 4);
  }

  // Rejected calls launch nothing.
  g_launches.clear();
  EXPECT(xqa_decode(h, odd, kv, kv, i32, i32, 16, 0.1f, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode(h, p16, kv, kv, i32, i32, 17, 0.1f, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode(h, p16, kv, kv, i32, i32, 0, 0.1f, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode(h, p16, kv, kv, i32, i32, 4, NAN, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode(h, p16, kv, kv, i32, i32, 4, INFINITY, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode(h, p16, nullptr, kv, i32, i32, 4, 0.1f, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode(nullptr, p16, kv, kv, i32, i32, 4, 0.1f, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode_multi(h, p16, kv, kv, i32, i32, 4, 2, 0.1f, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode_fp8(h, (xqa_kv_format_t)7, p16, kv, kv, i32, i32, 4, 1, 0.1f, 1.f, 1.f, p16,
                        nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode_fp8(h, XQA_KV_E4M3, p16, kv, kv, i32, i32, 4, 1, 0.1f, NAN, 1.f, p16,
                        nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode_fp8(h, XQA_KV_E4M3, p16, kv, kv, i32, i32, 4, 1, 3e38f, 1e10f, 1.f, p16,
                        nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode_pages(h, p16, kv, kv, i32, i32, i32, i32, 16385, 4, 0.1f, p16, nullptr) ==
         XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode_pages(h, p16, kv, kv, i32, i32, nullptr, i32, 8, 4, 0.1f, p16, nullptr) ==
         XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode_append(h, p16, odd, p16, g_buf, g_buf, i32, i32, 4, 0.1f, p16, nullptr) ==
         XQA_ERR_INVALID_ARG);
  EXPECT(xqa_append_kv(h, p16, p16, i32, i32, 17, g_buf, g_buf, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(xqa_decode_combine(h, i32, 0, p16, nullptr) == XQA_ERR_INVALID_ARG);
  EXPECT(g_launches.empty());

  // E4M3 with scales: the score scale folds k_scale, v_scale rides along.
  g_launches.clear();
  EXPECT(xqa_decode_fp8(h, XQA_KV_E4M3, p16, kv, kv, i32, i32, 3, 1, 0.5f, 0.25f, 3.0f, p16,
                        nullptr) == XQA_OK);
  EXPECT(g_launches.size() == 2);
  if (!g_launches.empty()) {
    const xqa::AttendArgs& a = g_launches[0].a;
    EXPECT(a.kv_format == xqa::kKvE4M3 && a.v_scale == 3.0f && a.batch == 3);
    EXPECT(a.scale_log2e == (float)(0.5 * 0.25 * 1.4426950408889634));
  }

  // Page subsets: the selection kernel, then decode over the handle's table.
  g_launches.clear();
  EXPECT(xqa_decode_pages(h, p16, kv, kv, i32, i32, i32 + 4, i32 + 8, 300, 5, 0.1f, p16, nullptr) ==
         XQA_OK);
  EXPECT(g_launches.size() == 3 && g_launches[0].kind == 'p' && g_launches[1].kind == 's' &&
         g_launches[2].kind == 'c');
  if (g_launches.size() == 3) {
    const xqa::SelectArgs& s = g_launches[0].sel;
    const xqa::AttendArgs& a = g_launches[1].a;
    EXPECT(s.batch == 5 && s.select_stride == 300 && s.vstride == 16384);
    EXPECT(s.max_pages == 16384 && s.max_tokens == 16384 * 16);
    EXPECT(s.block_table == i32 && s.page_select == i32 + 4 && s.select_counts == i32 + 8);
    EXPECT(a.block_table == s.vtable && a.context_lens == s.vlens);
    EXPECT(a.max_pages == 16384 && a.max_tokens == 16384 * 16);
    EXPECT(s.vlens == s.vtable + 16 * 16384);
  }

  // Fused append: the split kernel gets the new rows.
  g_launches.clear();
  EXPECT(xqa_decode_append(h, p16, p16, p16, g_buf, g_buf, i32, i32, 2, 0.1f, p16, nullptr) ==
         XQA_OK);
  EXPECT(g_launches.size() == 2 && g_launches[0].a.k_new != nullptr);

  // The host plan mirror.
  int32_t split = 0, items = 0;
  EXPECT(xqa_plan(h, host_lens, 3, &split, &items) == XQA_OK);
  const long long nb = 4 + 0 + 157;   // ceil(100/32) + ceil(5000/32)
  const int P = xqa::items_per_head(nb, 128);   // 21
  // A = 161 / 21 = 7: the 4-block sequence is charged (cost 8), the other
  // is not (157): C = 165, item ends floor(i * 165 / 21) map to blocks 0, 3,
  // 11, 19, ..., 153, 161; the largest items hold 8 blocks.
  EXPECT(items == P * 4 && split == 8 * 32);
  EXPECT(xqa_destroy(h) == XQA_OK);

  // A handle whose bounds never split a sequence: one kernel per step, and
  // the split kernel writes the zero rows.
  c = config(100, 16, 2, 2);
  EXPECT(xqa_create(&c, &h) == XQA_OK);
  EXPECT(xqa_get_info(h, &info) == XQA_OK && info.kernels_per_step == 1);
  g_launches.clear();
  EXPECT(xqa_decode(h, p16, kv, kv, i32, i32, 100, 0.1f, p16, nullptr) == XQA_OK);
  EXPECT(g_launches.size() == 1);
  EXPECT(xqa_decode_pages(h, p16, kv, kv, i32, i32, i32, i32, 1, 4, 0.1f, p16, nullptr) ==
         XQA_ERR_UNSUPPORTED);
  EXPECT(xqa_destroy(h) == XQA_OK);
  EXPECT(xqa_destroy(nullptr) == XQA_OK);

  // The handle-free decode: same grid and launches as a handle from the same
  // configuration, split states in the fixed workspace; rejected calls and
  // steps past the fixed workspace launch nothing.
  {
    xqa_config_t cn = config(16, 32, 4, 16384);
    g_launches.clear();
    EXPECT(xqa_decode_noalloc(&cn, p16, kv, kv, i32, i32, 16, 0.1f, p16, nullptr) == XQA_OK);
    EXPECT(g_launches.size() == 2 && g_launches[0].kind == 's' && g_launches[1].kind == 'c');
    if (g_launches.size() == 2) {
      EXPECT(g_launches[0].grid == 512 && g_launches[0].a.per_head == 128);
      EXPECT((void*)g_launches[0].a.partials == (void*)xqa::g_fixed);
      EXPECT(g_launches[1].a.partials == g_launches[0].a.partials);
      EXPECT(g_launches[0].a.batch == 16 && g_launches[0].a.group == 8);
    }
    g_launches.clear();
    EXPECT(xqa_decode_noalloc(nullptr, p16, kv, kv, i32, i32, 16, 0.1f, p16, nullptr) ==
           XQA_ERR_INVALID_ARG);
    EXPECT(xqa_decode_noalloc(&cn, p16, kv, kv, i32, i32, 17, 0.1f, p16, nullptr) ==
           XQA_ERR_INVALID_ARG);
    EXPECT(xqa_decode_noalloc(&cn, odd, kv, kv, i32, i32, 4, 0.1f, p16, nullptr) ==
           XQA_ERR_INVALID_ARG);
    EXPECT(xqa_decode_noalloc(&cn, p16, kv, kv, i32, i32, 4, NAN, p16, nullptr) ==
           XQA_ERR_INVALID_ARG);
    xqa_config_t bad = cn;
    bad.head_dim = 64;
    EXPECT(xqa_decode_noalloc(&bad, p16, kv, kv, i32, i32, 4, 0.1f, p16, nullptr) ==
           XQA_ERR_UNSUPPORTED);
    // 2048 items per KV head of 16 query rows: 2 * 8192 records of 2080
    // floats, past 16 MiB.
    bad = config(4, 64, 4, 64);
    bad.max_work_items = 4 * 2048;
    EXPECT(xqa_decode_noalloc(&bad, p16, kv, kv, i32, i32, 4, 0.1f, p16, nullptr) ==
           XQA_ERR_UNSUPPORTED);
    EXPECT(std::strstr(xqa_last_error(), "16 MiB") != nullptr);
    EXPECT(g_launches.empty());
    // A handle-free call on a one-kernel configuration launches one kernel.
    xqa_config_t one = config(100, 16, 2, 2);
    EXPECT(xqa_decode_noalloc(&one, p16, kv, kv, i32, i32, 100, 0.1f, p16, nullptr) == XQA_OK);
    EXPECT(g_launches.size() == 1);
    EXPECT(xqa::g_noalloc_lookups > 0);
  }

  if (g_fail) return 1;
  std::printf("OK %d checks\n", g_checks);
  return 0;
}
