// Internal declarations shared by the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xqa {

constexpr int kHeadDim = 128;
constexpr int kPageSize = 16;
constexpr int kPageHeadBytes = kPageSize * kHeadDim;   // one (page, kv head) block: 2 KiB
constexpr int kMaxGroup = 16;                          // query heads per KV head (MFMA N)
constexpr int kWaves = 4;                              // waves per split workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kBlockTokens = 32;                       // tokens per wave iteration (2 pages)
constexpr int kGranule = kWaves * kBlockTokens;        // split lengths are multiples of this
constexpr int kMaxItemsPerHead = 2048;                 // bound on splits per sequence
constexpr int kCombineThreads = 256;
constexpr int kCombineDChunk = 32;                     // head-dim columns per combine workgroup
constexpr int kCombineSplitLanes = 32;                 // split lanes per combine workgroup
constexpr int kCombinePerLane = 4;                     // split states a lane keeps in registers

// ---------------------------------------------------------------------------
// The split plan. Every workgroup of both kernels evaluates it on the device
// from context_lens alone, so the grid never depends on
// device data and a captured graph replays exactly with new lengths.
//
//   n_b    = clamp(context_lens[b], 0, max_tokens)
//   N      = sum_b n_b,  A = #{b : n_b > 0}
//   S      = granule * ceil(ceil(N / max(1, per_head - A)) / granule), S >= granule
//   ns_b   = ceil(n_b / S) splits for sequence b
//   items  = Hkv * sum_b ns_b  <=  Hkv * per_head  <=  grid
// (sum_b ceil(n_b / S) <= N / S + A <= per_head because S >= N / (per_head - A)).
// Work item i: h = i % Hkv, j = i / Hkv; the sequence b with
// prefix_b <= j < prefix_b + ns_b, split s = j - prefix_b, tokens
// [s*S, min(n_b, (s+1)*S)).
// ---------------------------------------------------------------------------
__host__ __device__ inline int32_t clamp_len(int32_t n, int32_t max_tokens) {
  return n <= 0 ? 0 : (n > max_tokens ? max_tokens : n);
}

__host__ __device__ inline int32_t split_tokens(int64_t n_tot, int32_t active, int32_t per_head) {
  int64_t denom = (int64_t)per_head - active;
  if (denom < 1) denom = 1;
  int64_t s = (n_tot + denom - 1) / denom;
  s = (s + kGranule - 1) / kGranule * kGranule;
  if (s < kGranule) s = kGranule;
  return (int32_t)s;
}

__host__ __device__ inline int32_t num_splits(int32_t n, int32_t S) {
  return n <= 0 ? 0 : (n + S - 1) / S;
}

struct AttendArgs {
  const uint16_t* q;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* out;
  float* partials;        // [grid][item_stride] split states
  int32_t batch;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_pages;
  int32_t max_tokens;
  int32_t per_head;       // grid / Hkv
  int32_t item_stride;    // floats per partial record
  float scale_log2e;      // scale * log2(e): scores are kept in base-2 units
};

hipError_t launch_split(const AttendArgs& a, int grid, hipStream_t stream);
hipError_t launch_combine(const AttendArgs& a, hipStream_t stream);
hipError_t launch_widen(const uint8_t* in, uint16_t* out_f16, float* out_f32, int64_t n,
                        hipStream_t stream);
hipError_t attend_blocks_per_cu(int* blocks);

}  // namespace xqa
