// Page-subset decode: per sequence, the pages a selection keeps, gathered
// into a page table of the handle's own (see xqa_select.h).

#include "xqa_select.h"

namespace xqa {
namespace {

// One workgroup of 16 waves per sequence gathers the physical ids of the
// pages its selection keeps into a page table of its own and writes the
// matching length, so the split and combine kernels then run unchanged over
// only those pages. An entry is kept when it names a page the sequence uses
// and exceeds every entry kept before it, i.e. when it is in range and above
// the maximum of the in-range entries before it. Per tile of 1024 entries,
// one per thread: a DPP running maximum inside each wave, the wave maxima
// through LDS, a ballot per wave for the kept entries and their counts
// through LDS for the compaction. A tile's entry loads and its block-table
// gathers are one memory round trip each; the gather is issued before the
// scans, and the first tile's entries are loaded with the length and the
// count, so a row of one tile costs two dependent round trips. A kept page's
// tokens sit at 16 j .. 16 j + 15 of the new table (j its rank); only the
// last kept page can be the sequence's partial last page, so the new length
// is 16 (kept - 1) plus what that page holds below n.
constexpr int kSelectWaves = 16;
constexpr int kSelectThreads = 64 * kSelectWaves;

// Inclusive running maximum over the wave of values >= 0 (lanes with no
// source contribute 0): max with the value 1, 2, 4 and 8 lanes back inside
// each row of 16, then with the last lane of row 0 (into row 1) and of row 2
// (into row 3), then with lane 31 (into rows 2 and 3).
__device__ __forceinline__ int wave_inclusive_max0(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));
  return v;
}

__global__ __launch_bounds__(kSelectThreads) void select_kernel(
    const int32_t* context_lens, const int32_t* select_counts, const int32_t* page_select,
    const int32_t* block_table, int32_t* vtable, int32_t max_tokens, int32_t select_stride,
    int32_t max_pages, int32_t vstride, int32_t* vlens) {
  __shared__ int s_max[kSelectWaves];
  __shared__ int s_cnt[kSelectWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t* sel = page_select + (long long)b * select_stride;
  const int32_t* bt = block_table + (long long)b * max_pages;
  int32_t* vt = vtable + (long long)b * vstride;
  // The length, the count, the first tile's entries (every entry below
  // select_stride is readable, so they need not wait for the count) and
  // vlens, the one argument not preloaded, are loaded together.
  const int n_in = context_lens[b];
  int count = select_counts[b];
  int praw = sel[tid < select_stride ? tid : select_stride - 1];
  asm volatile("" ::"s"(n_in), "s"(count), "v"(praw), "s"(vlens));
  const int n = clamp_len(n_in, max_tokens);
  const int used = (n + kPageSize - 1) / kPageSize;
  count = count < 0 ? 0 : (count > select_stride ? select_stride : count);
  int best1 = 0;   // 1 + the largest page kept so far (0: none yet)
  int kept = 0;
  for (int j0 = 0; j0 < count; j0 += kSelectThreads) {
    const int j = j0 + tid;
    if (j0 > 0) praw = sel[j < count ? j : count - 1];
    const int p = j < count ? praw : -1;
    const bool in = p >= 0 && p < used;
    // The physical id of every in-range entry is gathered before the keep
    // rule is known (p < used <= max_pages; others read entry 0 of the row),
    // so the gather is in flight during the scans below.
    const int pid = bt[in ? p : 0];
    const int run = wave_inclusive_max0(in ? p + 1 : 0);
    if (lane == 63) s_max[wave] = run;
    __syncthreads();
    int before = best1;
    for (int w = 0; w < wave; ++w) before = max(before, s_max[w]);
    const int prev = __shfl_up(run, 1);
    if (lane > 0) before = max(before, prev);
    const bool keep = in && p + 1 > before;
    const unsigned long long mask = __ballot(keep);
    if (lane == 0) s_cnt[wave] = __popcll(mask);
    __syncthreads();
    int off = kept;
    int total = 0;
    int tile_max = best1;
    for (int w = 0; w < kSelectWaves; ++w) {
      const int c = s_cnt[w];
      total += c;
      off += w < wave ? c : 0;
      tile_max = max(tile_max, s_max[w]);
    }
    if (keep) vt[off + __popcll(mask & ((1ull << lane) - 1ull))] = pid;
    kept += total;
    best1 = tile_max;
    __syncthreads();   // s_max and s_cnt are rewritten by the next tile
  }
  if (tid == 0) {
    vlens[b] = kept == 0 ? 0 : kPageSize * (kept - 1) + min(kPageSize, n - kPageSize * (best1 - 1));
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3(a.batch), dim3(kSelectThreads), 0, stream,
                     a.context_lens, a.select_counts, a.page_select, a.block_table, a.vtable,
                     a.max_tokens, a.select_stride, a.max_pages, a.vstride, a.vlens);
  return hipGetLastError();
}

}  // namespace xqa
