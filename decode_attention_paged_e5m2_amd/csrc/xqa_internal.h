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
constexpr int kMinItemBlocks = 8;                      // smallest work item: 8 blocks = 256 tokens
constexpr int kMaxItemsPerHead = 2048;                 // bound on work items per KV head
constexpr int kMaxSeqTokens = 1 << 24;                 // bound on max_pages_per_seq * page_size
constexpr int kMaxBatch = 1 << 16;                     // bound on max_batch
constexpr int kCombineRound = 16;                      // split states per round, one wave per round
constexpr int kCombineSharedRound = 8;                 // per round when a sequence's rounds are shared
                                                       // over the waves of a workgroup
constexpr int kCombineMaxWaves = 4;                    // waves per combine workgroup (1 or 4)

// ---------------------------------------------------------------------------
// The balanced plan. Every workgroup of both kernels evaluates it on the
// device from context_lens alone, so the grid never depends on device data
// and a captured graph replays exactly with new lengths. Each KV head has the
// same token structure; per head:
//
//   n_b   = clamp(context_lens[b], 0, max_tokens)
//   nb_b  = ceil(n_b / 32)              32-token blocks of sequence b
//   off_b = sum_{b' < b} nb_b'          first block of b in the head's block stream
//   NB    = sum_b nb_b
//   P     = min(per_head, ceil(NB / 8))  work items
//
// Items are cut by cost, not by blocks alone. Starting a sequence inside an
// item (its own merge, its partly filled blocks, the waves it leaves idle)
// costs about as much time as kSeqStartCost blocks. A sequence shorter than
// an average item (A = floor(NB / P) blocks) is charged that much more; a
// longer one starts at or near an item boundary anyway and is not:
//
//   s_b   = kSeqStartCost if 0 < nb_b < A, else 0
//   c_b   = nb_b + s_b (0 for an empty sequence)
//   coff_b = sum_{b' < b} c_b', C = sum_b c_b
//   item i covers costs [floor(i C / P), floor((i + 1) C / P)); a cost
//   position c inside sequence b (coff_b <= c < coff_b + c_b) is block
//   off_b + max(0, c - coff_b - s_b) (the charge comes first), and C is
//   block NB. Item i covers the blocks between its two ends, so the items
//   tile [0, NB) in order. Without short sequences this is the plain block
//   plan lo_i = floor(i NB / P); with one, C >= NB + kSeqStartCost and
//   NB > 8 (P - 1) make every item's cost range longer than a charge, so
//   every item holds at least one block.
//
// An item may span several sequences (segments). A sequence lying inside
// one item is finished there; a longer one leaves one split state per item
// it touches, in record slot 2i if it is item i's first segment and 2i + 1
// if it is item i's last (and not first) segment.
// ---------------------------------------------------------------------------
__host__ __device__ inline int32_t clamp_len(int32_t n, int32_t max_tokens) {
  return n <= 0 ? 0 : (n > max_tokens ? max_tokens : n);
}

__host__ __device__ inline int32_t seq_blocks(int32_t n) {
  return (n + kBlockTokens - 1) / kBlockTokens;
}

constexpr int kSeqStartCost = 4;   // plan charge per short sequence, in blocks

// Whether a sequence of `blocks` blocks is charged its start: 0 < blocks <
// A = floor(NB / P), written without a division as (blocks + 1) P <= NB.
__host__ __device__ inline bool seq_charged(int32_t blocks, int64_t nb_total, int32_t items) {
  return blocks > 0 && (int64_t)(blocks + 1) * items <= nb_total;
}

// The sequence's length in the plan's cost stream.
__host__ __device__ inline int32_t seq_cost(int32_t blocks, int64_t nb_total, int32_t items) {
  return blocks + (seq_charged(blocks, nb_total, items) ? kSeqStartCost : 0);
}

__host__ __device__ inline int32_t items_per_head(int64_t nb_total, int32_t per_head) {
  if (nb_total <= 0) return 0;
  const int64_t p = (nb_total + kMinItemBlocks - 1) / kMinItemBlocks;
  return p < per_head ? (int32_t)p : per_head;
}

// Start of item i in a stream of `total` units (blocks or costs) cut into
// `items` near-equal ranges.
__host__ __device__ inline int64_t item_lo(int64_t i, int64_t total, int64_t items) {
  return i * total / items;
}

// The item whose range holds unit x (the inverse of item_lo).
__host__ __device__ inline int32_t item_of_block(int64_t x, int64_t nb_total, int64_t items) {
  return (int32_t)(((x + 1) * items + nb_total - 1) / nb_total - 1);
}

// Format of the cached K/V bytes.
enum KvFormat : int32_t { kKvE5M2 = 0, kKvE4M3 = 1 };

struct AttendArgs {
  const uint16_t* q;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* out;
  float* partials;        // [2 * grid][item_stride] split states
  int2* merge_desc;       // [batch][Hkv] {slot of the first state, work item of the last} per
                          // sequence and KV head ({-1, -1}: no states to merge), written by the
                          // split kernel, read by the combine kernel
  int32_t batch;
  int32_t num_kv_heads;
  int32_t group;
  int32_t q_tokens;       // M new query tokens per sequence (1: single-token decode)
  int32_t rows;           // G * M <= 16: the MFMA N dimension, row r = (token r / G, head r % G)
  int32_t max_pages;
  int32_t max_tokens;
  int32_t per_head;       // grid / Hkv
  int32_t item_stride;    // floats per partial record
  int32_t combine_waves;  // 1: no sequence can leave more than kCombineRound states; else 4
  float scale_log2e;      // scale * k_scale * log2(e): scores are kept in base-2 units
  float v_scale;          // per-tensor V dequantisation scale, applied to the normalised rows
  int32_t kv_format;      // KvFormat
  const uint16_t* k_new;  // fused KV append: new token rows [batch][Hkv][128] binary16,
  const uint16_t* v_new;  //   written into k_pages / v_pages (E5M2); null: no append
};

// KV append: each sequence's new token (binary16 K and V rows for every KV
// head) encoded to E5M2 and written to its page slot.
struct AppendArgs {
  const uint16_t* k_new;         // [batch][Hkv][128] binary16
  const uint16_t* v_new;         // [batch][Hkv][128] binary16
  const int32_t* block_table;
  const int32_t* context_lens;   // lengths after the append
  uint8_t* k_pages;
  uint8_t* v_pages;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t max_pages;
  int32_t max_tokens;
};

hipError_t launch_split(const AttendArgs& a, int grid, hipStream_t stream);
hipError_t launch_combine(const AttendArgs& a, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_widen(const uint8_t* in, uint16_t* out_f16, float* out_f32, int64_t n,
                        int32_t kv_format, hipStream_t stream);
hipError_t attend_blocks_per_cu(int* blocks);

}  // namespace xqa
