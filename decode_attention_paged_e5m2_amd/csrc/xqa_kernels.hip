// Paged FP8 grouped-query decode attention: gfx950 kernels.
//
// What is computed follows the page "[Kernel][SM70] Pipeline batched E5M2
// XQA decode" (Purpose; Pending work and gates): one query token per
// sequence attends over its paged E5M2 K/V cache, query heads sharing KV
// heads. The same kernels also take several new query tokens per sequence
// (causal among themselves), an E4M3 cache with per-tensor K/V scales, and
// a small kernel writes each step's new token into the cache. The phases
// that page lists -- K load + E5M2 conversion, QK, V load + conversion, PV,
// synchronisation -- map onto the code below; the tiling is designed for
// CDNA4 (64-wide waves, MFMA, DPP) rather than taken from it.
//
// A decode step is two kernels. In the split kernel each workgroup is one
// work item = (sequence, KV head, token range); its four waves take
// interleaved 32-token blocks (2 pages):
//
//   Plan: every workgroup derives its own item from context_lens (O(batch)
//      integer work; items are cut evenly by cost, a sequence shorter than
//      an average item being charged for its start), so the grid is fixed
//      and a captured graph replays exactly with new lengths.
//   Gather: a wave fetches the page ids of its next 32 blocks with one
//      vector load and reads them out with v_readlane; K and V of a block are
//      eight 16-byte loads per lane, issued one block ahead (ping-pong). The
//      stream runs on across 32-block chunks and segments: the next chunk's
//      or segment's page ids are fetched when a chunk starts and its first
//      block is issued as soon as a buffer frees, while the segment merges.
//   K: lane l reads token l%16 of the page, head-dim bytes
//      [16q, 16q+16) and [64+16q, 64+16q+16) (q = l/16): each load
//      instruction covers 64 contiguous bytes of all 16 token rows.
//      Widening is one instruction per two codes: v_perm_b32 for E5M2 (the
//      code is the high byte of its binary16 value), the conversion
//      instruction for E4M3 (every E4M3 value is a binary16 value).
//   QK: S^T = K . Q^T with v_mfma_f32_16x16x32_f16, M = the 16 tokens of a
//      page, N = the query rows (the G heads of the group times the M query
//      tokens, padded to 16), four MFMAs over head_dim 128. The contraction
//      index may be permuted freely as long as the K and Q fragments agree,
//      which is what lets K go straight from its load layout into the A
//      operand.
//   Softmax: the accumulator gives lane l the scores of query row l%16 for
//      tokens 4q..4q+3; the block max over a 32-token block is a register
//      max plus two lane-swap steps (16, 32). Scores are kept in base-2
//      units (scale * k_scale * log2 e folded in) and exponentiated with
//      v_exp_f32 against a reference maximum that is raised only when a
//      block passes it by more than 2^8. Tail blocks mask tokens past the
//      segment and, per row, past the row's query position.
//   PV: O^T = V^T . P^T with v_mfma_f32_16x16x32_f16 over the 32 tokens of
//      the block. P^T needs no data movement: the QK accumulator is already
//      the B-operand layout once converted to binary16. V^T does: V's
//      contraction axis (tokens) is strided in memory, so each quad of lanes
//      loads four token rows and transposes the 4x4 byte tile with two DPP
//      quad permutes and three v_perm_b32, the last two of which also widen
//      the bytes to binary16. Row sums come from one more MFMA with an
//      all-ones A operand.
//   Merge: the four waves' (max, sum, O) states merge in LDS. A sequence
//      that fits one item is normalised and written directly; otherwise the
//      item stores its state in the workspace, and the segments at the
//      sequence's two ends write its merge record (where its states are).
//      Empty sequences get zero rows, spread over the grid.
//
// The combine kernel then merges the states of every split sequence, found
// through its merge record, with the exact log-sum-exp rule M = max m_s,
// L = sum l_s 2^(m_s-M), out = v_scale * sum 2^(m_s-M) O_s / L (in rounds of
// loaded states; a long sequence's rounds are shared out over the
// workgroup's four waves, whose partial merges then meet in LDS in a fixed
// order). On a handle whose bounds never split a sequence the step is the
// split kernel alone.
// The kernel boundary makes the split states visible across the chip's
// separately cached dies without any in-kernel cache write-back.
//
// Every reduction runs in a fixed order, so results are bitwise reproducible
// run to run, between eager calls and graph replays, and under any
// permutation of the physical pages.

#include <math.h>

#include "xqa_internal.h"

namespace xqa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ widening
// v_perm_b32 selector bytes 0..3 pick bytes of the second source, 4..7 bytes
// of the first, 0x0C yields 0x00. Each result holds two binary16 values whose
// high bytes are the E5M2 codes and whose low bytes are zero.
__device__ __forceinline__ uint32_t widen_lo(uint32_t x) {   // codes 0, 1 of x
  return __builtin_amdgcn_perm(0u, x, 0x010C000Cu);
}
__device__ __forceinline__ uint32_t widen_hi(uint32_t x) {   // codes 2, 3 of x
  return __builtin_amdgcn_perm(0u, x, 0x030C020Cu);
}

// E5M2 code of a binary16 value. E5M2 is the high byte of binary16 (same
// sign, exponent field and bias), so rounding the 16-bit pattern to its high
// byte, to nearest even, is exact rounding of the value; subnormals and the
// carry into the exponent need no special case. Past the largest finite code
// 0x7B (57344) the nearest finite value is 0x7B: saturation, infinities
// included. NaN gives 0x7F. The sign is kept.
__device__ __forceinline__ uint32_t e5m2_from_f16(uint32_t h) {
  const uint32_t sign = (h >> 8) & 0x80u;
  const uint32_t mag = h & 0x7FFFu;
  uint32_t r = (mag + 0x7Fu + ((mag >> 8) & 1u)) >> 8;
  r = r > 0x7Bu ? 0x7Bu : r;
  r = mag > 0x7C00u ? 0x7Fu : r;
  return sign | r;
}

// E4M3 (OCP, bias 7): two codes of x -> two binary16 values with the gfx950
// conversion instruction at scale 1. Every E4M3 value is a binary16 value,
// so this is exact (checked for all 256 codes through xqa_debug_widen_e4m3).
__device__ __forceinline__ uint32_t e4m3_lo(uint32_t x) {   // codes 0, 1 of x
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
}
__device__ __forceinline__ uint32_t e4m3_hi(uint32_t x) {   // codes 2, 3 of x
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true));
}

template <int F>
__device__ __forceinline__ uint32_t widen_k_lo(uint32_t x) {
  return F == kKvE4M3 ? e4m3_lo(x) : widen_lo(x);
}
template <int F>
__device__ __forceinline__ uint32_t widen_k_hi(uint32_t x) {
  return F == kKvE4M3 ? e4m3_hi(x) : widen_hi(x);
}

// 4x4 byte transpose across a lane quad plus widening. Lane i of the quad
// holds x = row i (4 consecutive head-dim codes of token i); on return it
// holds column i as binary16 pairs: h0 = (row0, row1), h1 = (row2, row3).
// Stage 1 swaps 16-bit halves with lane i^2, stage 2 bytes with lane i^1.
// E5M2: the last two v_perm_b32 also widen (selh0, selh1). E4M3: one v_perm
// puts the column's bytes in row order (selector in selh0) and the
// conversion instruction widens them.
template <int F>
__device__ __forceinline__ void transpose_widen(uint32_t x, uint32_t sel1, uint32_t selh0,
                                                uint32_t selh1, uint32_t& h0, uint32_t& h1) {
  const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  const uint32_t t = __builtin_amdgcn_perm(y, x, sel1);
  const uint32_t z = (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  if constexpr (F == kKvE4M3) {
    const uint32_t c = __builtin_amdgcn_perm(z, t, selh0);
    h0 = e4m3_lo(c);
    h1 = e4m3_hi(c);
  } else {
    h0 = __builtin_amdgcn_perm(z, t, selh0);
    h1 = __builtin_amdgcn_perm(z, t, selh1);
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of v over lane pairs (l, l ^ 16) and (l, l ^ 32). With both
// operands equal, a permlane swap returns, in its two results, the lane's own
// value and its partner's (in either order), so their maximum is the pair's.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Headroom of the reference maximum (base-2 units): weights are at most
// 2^8 = 256, far inside binary16 and fp32 range.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
  half2v h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------- the plan
// Wave-level evaluation of the balanced plan (see xqa_internal.h).
//
// Inclusive prefix sum over the wave with DPP alone (no LDS round trip):
// shifts by 1, 2, 4 and 8 lanes inside each row of 16 (lanes with no source
// add 0) give row prefixes; then the last lane of row 0 is added to row 1 and
// that of row 2 to row 3 (row_bcast:15), and lane 31 to rows 2 and 3
// (row_bcast:31). Sums wrap modulo 2^32, so unsigned totals up to 2^32 - 1
// are exact when read back as unsigned.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
  return v;
}

// A wave-uniform 64-bit value marked uniform for the compiler (it keeps
// what it cannot prove uniform, and everything derived from it, in vector
// registers).
__device__ __forceinline__ long long uniform64(long long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

struct SeqInfo {
  int b;          // sequence index
  int n;          // clamped length
  long long off;  // first block in the head's block stream
};

// The lookups the kernels make. For batch <= 64 one pass over context_lens
// leaves sequence `lane`'s length and block prefix in lane registers, and
// every later lookup is a v_readlane or a ballot with no memory access.
// Larger batches keep, per 64-sequence chunk c, the number of blocks before
// it (off[c], off[nch] = total) and the plan's cost units before it
// (coff[c]), built once per workgroup in LDS (the four waves share out the
// chunks, eight chunk loads in flight per wave; the costs in a second pass,
// once the item count is known). A lookup is then one load of a chunk's
// lengths and a scan; finding the chunk that holds a block or a cost
// position is a ballot over the table, 64 chunks per step.
struct SeqTable {
  const int32_t* ctx;
  int batch, max_tokens;
  bool small;               // batch <= 64
  int n_l;                  // small: clamped length of sequence `lane` (0 past the batch)
  int excl_l;               // small: first block of sequence `lane`
  int cexcl_l;              // small: first cost unit of sequence `lane` (plan cost stream)
  int charge_l;             // small: the plan's charge for sequence `lane` (0 or kSeqStartCost)
  int nch;                  // large: 64-sequence chunks
  const long long* off;     // large: [nch + 1] blocks before each chunk (LDS)
  const long long* coff;    // large: [nch + 1] cost units before each chunk (LDS)
  const int* has_empty;     // large: [nch] nonzero when the chunk holds an empty sequence (LDS)
  long long nb;             // total blocks per head
  int items;                // P: work items per head
  long long ctot;           // total cost units per head (nb when no sequence is charged)
  bool any_empty;           // some sequence of the batch has no token

  // Called by every thread of the workgroup (the large path synchronises the
  // workgroup). lds, lds_cost: room for kMaxBatch / 64 + 1 values each;
  // lds_empty: for kMaxBatch / 64 + 1 flags (the last one: any chunk has one).
  __device__ SeqTable(const int32_t* c, int bt, int mt, int per_head, int lane, int wave,
                      long long* lds, long long* lds_cost, int* lds_empty)
      : ctx(c), batch(bt), max_tokens(mt), small(bt <= 64), n_l(0), excl_l(0), cexcl_l(0),
        charge_l(0), nch(0), off(lds), coff(lds_cost), has_empty(lds_empty), nb(0), items(0),
        ctot(0), any_empty(false) {
    if (small) {
      init_small(lane, per_head);
      return;
    }
    nch = (batch + 63) >> 6;
    for (int c0 = 8 * wave; c0 < nch; c0 += 8 * kWaves) {
      int v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {   // unconditional (clamped) loads: all eight in flight
        const int i = 64 * (c0 + k) + lane;
        const int n = clamp_len(ctx[min(i, batch - 1)], max_tokens);
        v[k] = i < batch ? seq_blocks(n) : -1;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool empty = __ballot(v[k] == 0) != 0;
        const int blocks = v[k] > 0 ? v[k] : 0;
        const unsigned tot = (unsigned)__builtin_amdgcn_readlane(wave_inclusive_scan(blocks), 63);
        if (lane == 0 && c0 + k < nch) {
          lds[c0 + k] = tot;
          lds_empty[c0 + k] = empty;
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      long long run = 0;
      bool any = false;
      for (int c0 = 0; c0 < nch; c0 += 64) {
        const int cc = c0 + lane;
        const unsigned t = cc < nch ? (unsigned)lds[cc] : 0u;
        const bool chunk_any = __ballot(cc < nch && lds_empty[cc] != 0) != 0;
        any = any | chunk_any;
        const unsigned incl = (unsigned)wave_inclusive_scan((int)t);
        if (cc < nch) lds[cc] = run + incl - t;
        run += (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
      }
      if (lane == 0) {
        lds[nch] = run;
        lds_empty[nch] = any;
      }
    }
    __syncthreads();
    nb = lds[nch];
    any_empty = lds_empty[nch] != 0;
    items = items_per_head(nb, per_head);
    // Second pass: the chunks' costs, now that P is known (the lengths are
    // cache hits).
    for (int c0 = 8 * wave; c0 < nch; c0 += 8 * kWaves) {
      int v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = 64 * (c0 + k) + lane;
        const int n = clamp_len(ctx[min(i, batch - 1)], max_tokens);
        v[k] = i < batch ? seq_cost(seq_blocks(n), nb, items) : 0;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const unsigned tot = (unsigned)__builtin_amdgcn_readlane(wave_inclusive_scan(v[k]), 63);
        if (lane == 0 && c0 + k < nch) lds_cost[c0 + k] = tot;
      }
    }
    __syncthreads();
    if (wave == 0) {
      long long crun = 0;
      for (int c0 = 0; c0 < nch; c0 += 64) {
        const int cc = c0 + lane;
        const unsigned tc = cc < nch ? (unsigned)lds_cost[cc] : 0u;
        const unsigned cincl = (unsigned)wave_inclusive_scan((int)tc);
        if (cc < nch) lds_cost[cc] = crun + cincl - tc;
        crun += (unsigned)__builtin_amdgcn_readlane((int)cincl, 63);
      }
      if (lane == 0) lds_cost[nch] = crun;
    }
    __syncthreads();
    ctot = lds_cost[nch];
  }

  // Whether sequence b (this lane's; b < batch when in_batch) has no token.
  // Every lane of the wave calls it. Small: the length is read from lane
  // b's registers by a cross-lane read that every lane executes (a lane
  // left out of it would return no value); large: loaded only when b's
  // chunk holds an empty sequence.
  __device__ bool is_empty(int b, bool in_batch) const {
    if (small) {
      const int n = __shfl(n_l, b & 63);
      return in_batch && n == 0;
    }
    return in_batch && has_empty[b >> 6] && clamp_len(ctx[b], max_tokens) == 0;
  }

  __device__ void init_small(int lane, int per_head) {
    n_l = lane < batch ? clamp_len(ctx[lane], max_tokens) : 0;
    const int b_l = seq_blocks(n_l);
    const int incl = wave_inclusive_scan(b_l);   // <= 64 * 2^19: no overflow
    excl_l = incl - b_l;
    nb = __builtin_amdgcn_readlane(incl, 63);
    items = items_per_head(nb, per_head);
    const bool charged = seq_charged(b_l, nb, items);
    if (__ballot(charged) != 0) {
      charge_l = charged ? kSeqStartCost : 0;
      const int cost = b_l + charge_l;
      const int cincl = wave_inclusive_scan(cost);   // <= 64 * (2^19 + 4): no overflow
      cexcl_l = cincl - cost;
      ctot = __builtin_amdgcn_readlane(cincl, 63);
    } else {   // no charge: the cost stream is the block stream
      cexcl_l = excl_l;
      ctot = nb;
    }
    any_empty = __ballot(lane < batch && n_l == 0) != 0;
  }

  // One 64-sequence chunk: lane's length and its block offset inside the chunk.
  __device__ void load_chunk(int c, int lane, int& n, int& excl, int& blocks) const {
    const int i = 64 * c + lane;
    n = i < batch ? clamp_len(ctx[min(i, batch - 1)], max_tokens) : 0;
    blocks = seq_blocks(n);
    excl = (int)((unsigned)wave_inclusive_scan(blocks) - (unsigned)blocks);
  }

  __device__ SeqInfo at(int b, int lane) const {
    if (small) {
      if (b >= 64) return {b, 0, nb};
      return {b, __builtin_amdgcn_readlane(n_l, b), (long long)__builtin_amdgcn_readlane(excl_l, b)};
    }
    if (b >= batch) return {b, 0, nb};
    const int c = b >> 6;
    int n, excl, blocks;
    load_chunk(c, lane, n, excl, blocks);
    return {b, __builtin_amdgcn_readlane(n, b & 63),
            off[c] + (unsigned)__builtin_amdgcn_readlane(excl, b & 63)};
  }

  // The non-empty sequence whose blocks contain block x (x < nb).
  __device__ SeqInfo containing(long long x, int lane) const {
    if (small) {
      const unsigned long long hit =
          __ballot(n_l > 0 && x >= excl_l && x < excl_l + seq_blocks(n_l));
      if (!hit) return {batch, 0, nb};
      const int src = __ffsll((unsigned long long)hit) - 1;
      return {src, __builtin_amdgcn_readlane(n_l, src), (long long)__builtin_amdgcn_readlane(excl_l, src)};
    }
    // The first chunk whose end passes x.
    int c = nch;
    for (int g = 0; g < nch; g += 64) {
      const unsigned long long hit = __ballot(off[min(g + lane + 1, nch)] > x);
      if (hit) {
        c = g + __ffsll((unsigned long long)hit) - 1;
        break;
      }
    }
    if (c >= nch) return {batch, 0, nb};
    int n, excl, blocks;
    load_chunk(c, lane, n, excl, blocks);
    const long long lo = off[c] + (unsigned)excl;
    const unsigned long long hit = __ballot(blocks > 0 && x >= lo && x < lo + blocks);
    if (!hit) return {batch, 0, nb};
    const int src = __ffsll((unsigned long long)hit) - 1;
    return {64 * c + src, __builtin_amdgcn_readlane(n, src),
            off[c] + (unsigned)__builtin_amdgcn_readlane(excl, src)};
  }

  // Cost position c of the plan: the block it stands for (nb for c >= ctot)
  // and, for c < ctot, the non-empty sequence whose cost range holds it
  // (that sequence also holds the block).
  __device__ long long block_at_cost(long long c, int lane, SeqInfo* seq) const {
    *seq = SeqInfo{batch, 0, nb};
    if (c >= ctot) return nb;
    if (small) {
      const unsigned long long m = __ballot(n_l > 0 && (long long)cexcl_l <= c);
      if (!m) return nb;   // not reached: the first non-empty sequence starts at cost 0
      const int src = 63 - __clzll((long long)m);
      const long long first = (long long)__builtin_amdgcn_readlane(excl_l, src);
      const long long local = c - (long long)__builtin_amdgcn_readlane(cexcl_l, src) -
                              __builtin_amdgcn_readlane(charge_l, src);
      *seq = SeqInfo{src, __builtin_amdgcn_readlane(n_l, src), first};
      return first + (local > 0 ? local : 0);
    }
    // The first chunk whose cost end passes c.
    int k = nch;
    for (int g = 0; g < nch; g += 64) {
      const unsigned long long hit = __ballot(coff[min(g + lane + 1, nch)] > c);
      if (hit) {
        k = g + __ffsll((unsigned long long)hit) - 1;
        break;
      }
    }
    if (k >= nch) return nb;
    int n, excl, blocks;
    load_chunk(k, lane, n, excl, blocks);
    const int cost = seq_cost(blocks, nb, items);
    const int cexcl = wave_inclusive_scan(cost) - cost;
    const long long clo = coff[k] + (unsigned)cexcl;
    const unsigned long long hit = __ballot(blocks > 0 && c >= clo && c < clo + cost);
    if (!hit) return nb;   // not reached
    const int src = __ffsll((unsigned long long)hit) - 1;
    const long long first = off[k] + (unsigned)__builtin_amdgcn_readlane(excl, src);
    const int charge = __builtin_amdgcn_readlane(cost - blocks, src);
    const long long local = c - (coff[k] + (unsigned)__builtin_amdgcn_readlane(cexcl, src)) - charge;
    *seq = SeqInfo{64 * k + src, __builtin_amdgcn_readlane(n, src), first};
    return first + (local > 0 ? local : 0);
  }
};

// ------------------------------------------------------------ split kernel
struct RawBlock {
  u32x4 k[4];   // page a: loads 0, 1; page b: loads 2, 3
  u32x4 v[4];
};

struct WaveState {
  float4v o[8];   // O^T tiles: lane (head l%16, q = l/16) holds d = 64L + 16q + 4k + 0..3
  float4v l;      // running sum of weights of head l%16 (all four entries equal)
  float m;        // running max of the base-2 scores of head l%16
};

__device__ __forceinline__ void load_block(RawBlock& r, const uint8_t* ka, const uint8_t* kb,
                                           const uint8_t* va, const uint8_t* vb, int koff,
                                           int voff) {
  r.k[0] = *(const u32x4*)(ka + koff);
  r.k[1] = *(const u32x4*)(ka + koff + 64);
  r.k[2] = *(const u32x4*)(kb + koff);
  r.k[3] = *(const u32x4*)(kb + koff + 64);
  r.v[0] = *(const u32x4*)(va + voff);
  r.v[1] = *(const u32x4*)(va + voff + 64);
  r.v[2] = *(const u32x4*)(vb + voff);
  r.v[3] = *(const u32x4*)(vb + voff + 64);
}

// kTail: the block may extend past t_end (only a wave's last block of a
// segment can); other blocks skip the masking.
// t_end: end of the segment's tokens (V rows past it are zeroed). row_end:
// this lane's query row sees tokens < row_end (<= t_end; smaller for the
// earlier of several query tokens). t_mask: the smallest row_end of the wave.
template <bool kTail, int F>
__device__ __forceinline__ void process_block(RawBlock& r, const half8 (&qf)[4], WaveState& st,
                                              float scale_log2e, int tok0, int t_end, int row_end,
                                              int t_mask, int lane, uint32_t sel1, uint32_t selh0,
                                              uint32_t selh1) {
  const int q = lane >> 4;
  const bool tail = kTail && tok0 + kBlockTokens > t_mask;   // wave-uniform
  if (tail) {
    // V rows of tokens past the end are zeroed (their bytes may be NaN codes
    // and 0 * NaN would poison the sum). V lane token: 4q + (lane & 3).
    const int tv = tok0 + 4 * q + (lane & 3);
    if (tv >= t_end) {
      r.v[0] = u32x4{0, 0, 0, 0};
      r.v[1] = u32x4{0, 0, 0, 0};
    }
    if (tv + kPageSize >= t_end) {
      r.v[2] = u32x4{0, 0, 0, 0};
      r.v[3] = u32x4{0, 0, 0, 0};
    }
  }

  // QK^T for the group, page a and page b.
  float4v sa = {0.f, 0.f, 0.f, 0.f};
  float4v sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 ka = r.k[i >> 1];
    const u32x4 kb = r.k[2 + (i >> 1)];
    const uint32_t a0 = ka[(i & 1) * 2], a1 = ka[(i & 1) * 2 + 1];
    const uint32_t b0 = kb[(i & 1) * 2], b1 = kb[(i & 1) * 2 + 1];
    const u32x4 fa = {widen_k_lo<F>(a0), widen_k_hi<F>(a0), widen_k_lo<F>(a1), widen_k_hi<F>(a1)};
    const u32x4 fb = {widen_k_lo<F>(b0), widen_k_hi<F>(b0), widen_k_lo<F>(b1), widen_k_hi<F>(b1)};
    sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, fa), qf[i], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, fb), qf[i], sb, 0, 0, 0);
  }

  // Scores in base-2 units are c * s (c = scale * log2 e). A full block
  // takes the extreme raw score and folds c into the exponent's fma; the
  // tail block scales first so that masked tokens are exactly -inf.
  float s8[8];
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    s8[r4] = sa[r4];
    s8[4 + r4] = sb[r4];
  }
  float bm;
  if (tail) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int t = tok0 + 4 * q + r4;
      s8[r4] = t >= row_end ? -INFINITY : s8[r4] * scale_log2e;
      s8[4 + r4] = t + kPageSize >= row_end ? -INFINITY : s8[4 + r4] * scale_log2e;
    }
    bm = fmaxf(fmaxf(fmaxf(s8[0], s8[1]), fmaxf(s8[2], s8[3])),
               fmaxf(fmaxf(s8[4], s8[5]), fmaxf(s8[6], s8[7])));
  } else {
    // max_i(c s_i) = c max_i s_i for c >= 0 and c min_i s_i otherwise,
    // exactly: rounding is monotonic.
    const float hi = fmaxf(fmaxf(fmaxf(s8[0], s8[1]), fmaxf(s8[2], s8[3])),
                           fmaxf(fmaxf(s8[4], s8[5]), fmaxf(s8[6], s8[7])));
    const float lo = fminf(fminf(fminf(s8[0], s8[1]), fminf(s8[2], s8[3])),
                           fminf(fminf(s8[4], s8[5]), fminf(s8[6], s8[7])));
    bm = (scale_log2e >= 0.f ? hi : lo) * scale_log2e;
  }
  bm = max_xor16(bm);   // the four lane quarters of a head agree on the maximum
  bm = max_xor32(bm);
  // st.m is a reference maximum, not the running one: it is raised only when
  // a score exceeds it by more than kRescaleSlack (base-2 units), so weights
  // stay below 2^kRescaleSlack and the state is rescaled on few blocks. Any
  // reference gives the same softmax; the merges below use it as such.
  if (__any(bm > st.m + kRescaleSlack)) {
    const float m_new = fmaxf(st.m, bm);
    // Equal maxima (both -inf for a row that has seen no visible token) keep the state.
    const float alpha = st.m == m_new ? 1.f : exp2_fast(st.m - m_new);
    st.m = m_new;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.o[t] *= alpha;
    st.l *= alpha;
  }
  const float m_ref = st.m;

  u32x4 pf;
  if (tail) {
    // A masked score is -inf; so is m_ref for a row with nothing visible yet.
#pragma unroll
    for (int r2 = 0; r2 < 4; ++r2) {
      const float p0 = s8[2 * r2] == -INFINITY ? 0.f : exp2_fast(s8[2 * r2] - m_ref);
      const float p1 = s8[2 * r2 + 1] == -INFINITY ? 0.f : exp2_fast(s8[2 * r2 + 1] - m_ref);
      pf[r2] = pack_half2(p0, p1);
    }
  } else {
#pragma unroll
    for (int r2 = 0; r2 < 4; ++r2) {
      pf[r2] = pack_half2(exp2_fast(fmaf(s8[2 * r2], scale_log2e, -m_ref)),
                          exp2_fast(fmaf(s8[2 * r2 + 1], scale_log2e, -m_ref)));
    }
  }

  // PV: V^T tiles from the quad transpose, P^T straight from the scores.
  const half8 pfrag = __builtin_bit_cast(half8, pf);
  // Row sums of the same binary16 weights, on the matrix core: an all-ones A
  // operand makes every output row the sum over the block's 32 tokens, so
  // each lane receives its head's total without a cross-lane reduction and
  // the sum is accumulated and rescaled exactly like O.
  const half8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                      (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
  st.l = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pfrag, st.l, 0, 0, 0);
#pragma unroll
  for (int L = 0; L < 2; ++L) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t a0, a1, b0, b1;
      transpose_widen<F>(r.v[L][k], sel1, selh0, selh1, a0, a1);
      transpose_widen<F>(r.v[2 + L][k], sel1, selh0, selh1, b0, b1);
      const u32x4 vf = {a0, a1, b0, b1};
      st.o[L * 4 + k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, vf), pfrag,
                                                             st.o[L * 4 + k], 0, 0, 0);
    }
  }
}

// Sixteen binary16 values (x0: values 0..7, x1: 8..15) -> their sixteen
// E5M2 codes, in memory order.
__device__ __forceinline__ u32x4 e5m2_pack16(const u32x4& x0, const u32x4& x1) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t p0 = w < 2 ? x0[2 * w] : x1[2 * (w - 2)];
    const uint32_t p1 = w < 2 ? x0[2 * w + 1] : x1[2 * (w - 2) + 1];
    r[w] = e5m2_from_f16(p0 & 0xFFFFu) | (e5m2_from_f16(p0 >> 16) << 8) |
           (e5m2_from_f16(p1 & 0xFFFFu) << 16) | (e5m2_from_f16(p1 >> 16) << 24);
  }
  return r;
}

// Fused KV append: writes the new token's E5M2 K and V rows (binary16 rows
// of k_new / v_new for sequence b, KV head h) to slot `row` of page
// page_id. One wave, 16 bytes per lane per row: lane l < 8 encodes K bytes
// [16l, 16l + 16), lanes 8..15 the V bytes. The same wave later reads the
// slot back with its ordinary loads of the page (other lanes than the ones
// that stored), so the caller waits for the stores to complete first; no
// other wave reads the slot.
__device__ __forceinline__ void append_store(const AttendArgs& a, int b, int h, int page_id, int row,
                                             int lane) {
  if (lane >= 16) return;
  const int part = lane & 7;
  const bool is_v = lane >= 8;
  const long long src = ((long long)b * a.num_kv_heads + h) * kHeadDim + 16 * part;
  const uint16_t* x = (is_v ? a.v_new : a.k_new) + src;
  const u32x4 codes = e5m2_pack16(*(const u32x4*)x, *(const u32x4*)(x + 8));
  uint8_t* pages = const_cast<uint8_t*>(is_v ? a.v_pages : a.k_pages);
  *(u32x4*)(pages + ((size_t)page_id * a.num_kv_heads + h) * kPageHeadBytes +
            (size_t)row * kHeadDim + 16 * part) = codes;
}

// Output row of query row r (token r / G, head h * G + r % G) of sequence b:
// out is [batch][M][Hq][head_dim].
__device__ __forceinline__ uint16_t* out_row(const AttendArgs& a, int b, int h, int r) {
  const int G = a.group;
  return a.out + (((long long)b * a.q_tokens + r / G) * a.num_kv_heads * G + (long long)h * G + r % G) *
                     kHeadDim;
}

struct SplitShared {
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  float o[kWaves][kMaxGroup][kHeadDim + 4];
  long long chunk_off[kMaxBatch / 64 + 1];   // batches over 64: blocks before each 64-sequence chunk
  long long chunk_coff[kMaxBatch / 64 + 1];  // batches over 64: plan cost units before each chunk
  int chunk_empty[kMaxBatch / 64 + 1];       // batches over 64: the chunk holds an empty sequence;
                                             // last used entry: any chunk does
};

// One segment of a work item: blocks [jb_lo, jb_hi) of sequence b (n
// tokens) for the workgroup's KV head. `direct`: the segment is the whole
// sequence, so its rows are normalised and written to out; otherwise its
// state goes to record `rec`.
struct Segment {
  int b, n, jb_lo, jb_hi;
  bool direct;
  bool first;       // the item's first segment (state slot 2i; a later one uses 2i + 1)
  long long off;    // the sequence's first block in the head's block stream
  float* rec;
};

// A wave's part of a segment: its blocks are j = wave + 4m, m < my_blocks.
// t_end: end of the segment's tokens (V rows past it are zeroed). row_end:
// this lane's query row sees tokens < row_end (query token j sits at
// position n - M + j and sees tokens <= n - M + j). t_mask: the smallest
// row_end of the wave.
struct WaveSeg {
  int t_begin, t_end, row_end, t_mask, my_blocks, first_page, last_page;
  const int32_t* bt;
};

__device__ __forceinline__ WaveSeg wave_seg(const AttendArgs& a, const Segment& s, int lane,
                                            int wave) {
  WaveSeg w;
  const int G = a.group;
  const int M = a.q_tokens;
  w.t_begin = s.jb_lo * kBlockTokens;
  w.t_end = min(s.n, s.jb_hi * kBlockTokens);
  w.row_end = min(w.t_end, s.n - M + (lane & 15) / G + 1);
  w.t_mask = min(w.t_end, s.n - M + 1);
  const int nblocks = s.jb_hi - s.jb_lo;
  w.my_blocks = nblocks > wave ? (nblocks - wave + kWaves - 1) / kWaves : 0;
  w.first_page = w.t_begin >> 4;
  w.last_page = (w.t_end - 1) >> 4;
  w.bt = a.block_table + (long long)s.b * a.max_pages;
  return w;
}

// Page ids of the wave's blocks c0 .. c0 + 31 of a segment in one vector
// load: lane i holds page (i & 1) of block c0 + i/2 (read out later with
// v_readlane, so address generation never waits on a scalar miss). Blocks
// past the end read a valid page; they are masked in the tail block.
__device__ __forceinline__ int load_ids(const WaveSeg& w, int c0, int lane, int wave) {
  int pg = w.first_page + 2 * (wave + kWaves * (c0 + (lane >> 1))) + (lane & 1);
  pg = min(pg, w.last_page);
  return w.bt[pg];
}

// Q^T fragments: lane (row g, quarter q) holds, for MFMA i, the eight
// head-dim values 64*(i/2) + 16q + 8*(i%2) + 0..7, matching the K bytes.
__device__ __forceinline__ void load_q(const AttendArgs& a, const Segment& s, int h, int lane,
                                       half8 (&qf)[4]) {
  const int G = a.group;
  const int g = lane & 15;
  const int q = lane >> 4;
  if (g < a.rows) {
    const uint16_t* qrow =
        a.q + (((long long)s.b * a.q_tokens + g / G) * a.num_kv_heads * G + (long long)h * G + g % G) *
                  kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[i] = *(const half8*)(qrow + 64 * (i >> 1) + 16 * q + 8 * (i & 1));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[i] = half8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// Fused append: the new token n - 1 lies in a segment's last block unless
// the length was clamped to the table's capacity (then nothing is written).
// The wave that will read that block writes the new rows into the page
// before it issues any K/V load of the segment; its loads then see them.
__device__ __forceinline__ void append_if_owner(const AttendArgs& a, const Segment& s,
                                                const WaveSeg& w, int h, int lane, int wave) {
  if (w.t_end == s.n && (s.n < a.max_tokens || a.context_lens[s.b] == s.n) &&
      ((s.n - 1 - w.t_begin) / kBlockTokens) % kWaves == wave) {
    append_store(a, s.b, h, w.bt[(s.n - 1) / kPageSize], (s.n - 1) % kPageSize, lane);
    // The stores are complete in the L2 cache before the wave issues any K/V
    // load of the segment: those loads miss the CU's L1 (no wave on this CU
    // has read the slot's lines in this launch) and read the new bytes.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  }
}

// The four waves' states of a segment meet in LDS (fixed order); the merged
// (max, sum, O) is normalised and written, or stored as a split state.
// The segments at a sequence's ends also fill in its merge record
// {slot of the first state, item of the last}: the first segment writes the
// slot, the last one its item; a sequence inside one item writes {-1, -1}.
__device__ __forceinline__ void finish_segment(const AttendArgs& a, SplitShared& sh,
                                               const Segment& s, const WaveState& st, int h,
                                               int item, int lane, int wave) {
  if (threadIdx.x == 0) {
    int2* d = a.merge_desc + (long long)s.b * a.num_kv_heads + h;
    if (s.direct) {
      *d = make_int2(-1, -1);
    } else if (s.jb_lo == 0) {
      d->x = 2 * item + (s.first ? 0 : 1);
    } else if (s.jb_hi == seq_blocks(s.n)) {
      d->y = item;
    }
  }
  const int R = a.rows;
  const int g = lane & 15;
  const int q = lane >> 4;
  if (g < R) {
    if (q == 0) {
      sh.m[wave][g] = st.m;
      sh.l[wave][g] = st.l[0];
    }
#pragma unroll
    for (int L = 0; L < 2; ++L) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        *(float4v*)&sh.o[wave][g][64 * L + 16 * q + 4 * k] = st.o[L * 4 + k];
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < R * 32; e += kThreads) {
    const int gg = e >> 5;
    const int d4 = (e & 31) * 4;
    float M = sh.m[0][gg];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh.m[w][gg]);
    float Ls = 0.f;
    float4v o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sh.m[w][gg];
      const float f = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
      Ls += f * sh.l[w][gg];
      o += f * *(const float4v*)&sh.o[w][gg][d4];
    }
    if (s.direct) {
      const float inv = Ls > 0.f ? a.v_scale / Ls : 0.f;   // a row with no visible token is zero
      uint2 packed;
      packed.x = pack_half2(o[0] * inv, o[1] * inv);
      packed.y = pack_half2(o[2] * inv, o[3] * inv);
      *(uint2*)(out_row(a, s.b, h, gg) + d4) = packed;
    } else {
      *(float4v*)(s.rec + gg * kHeadDim + d4) = o;
      if (d4 == 0) {
        s.rec[R * kHeadDim + gg] = M;
        s.rec[R * kHeadDim + R + gg] = Ls;
      }
    }
  }
  __syncthreads();   // the LDS state is reused by the next segment
}

// kAppend: the fused KV append (E5M2 only); a separate instantiation so that
// plain decode carries none of its registers.
//
// A work item is a run of segments. Each wave streams its blocks through two
// buffers (ping-pong): while one block is processed the next is in flight.
// The stream does not stop at a chunk of 32 blocks or at a segment's end:
// the page ids of the next chunk or segment are loaded when the current
// chunk starts, and the first block after the chunk is issued as soon as a
// buffer frees up, so the next segment's first K/V bytes travel while this
// segment is merged. Every load in the steady-state loop is unconditional,
// so the compiler's waits name exactly the buffer about to be used.
//
// This kernel and the combine kernel take the three values the plan needs
// first (context_lens, batch, max_tokens) as leading scalar arguments ahead
// of the argument block: the build preloads them into SGPRs
// (amdgpu-kernarg-preload-count=4), so the first load of context_lens is
// issued without waiting for the argument block to arrive from memory.
template <int F, bool kAppend>
__global__ __launch_bounds__(kThreads) void split_kernel(const int32_t* context_lens, int32_t batch,
                                                         int32_t max_tokens, AttendArgs a) {
  __shared__ SplitShared sh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int Hkv = a.num_kv_heads;

  const SeqTable seqs(context_lens, batch, max_tokens, a.per_head, lane, wave, sh.chunk_off,
                      sh.chunk_coff, sh.chunk_empty);
  const int P = seqs.items;
  const int item = blockIdx.x / Hkv;
  const int h = blockIdx.x % Hkv;
  // Empty sequences: zero rows and a merge record with no states, written
  // once the workgroup's own work is done. Sequence b belongs to item
  // b % per_head, wave (b / per_head) % 4, so the writes spread over the
  // grid; each empty sequence's R rows are written by its whole wave, 16
  // bytes per lane per store.
  auto finish_empty = [&]() {
    if (!seqs.any_empty) return;
    const int R = a.rows;
    const long long ph = a.per_head;
    // Lane l of wave w looks at k = w + 4 (l + 64 j), sequence item + k per_head.
    for (long long kb = wave; item + kb * ph < a.batch; kb += kWaves * 64) {
      const long long bl = item + (kb + kWaves * lane) * ph;
      const bool empty = seqs.is_empty((int)min(bl, (long long)a.batch - 1), bl < a.batch);
      unsigned long long mask = __ballot(empty);
      if (empty) a.merge_desc[bl * Hkv + h] = make_int2(-1, -1);
      while (mask) {
        const int bz = (int)(item + (kb + kWaves * (__ffsll(mask) - 1)) * ph);
        mask &= mask - 1;
        for (int e = lane; e < R * (kHeadDim / 8); e += 64) {
          *(uint4*)(out_row(a, bz, h, e / (kHeadDim / 8)) + (e % (kHeadDim / 8)) * 8) =
              make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  if (item >= P) {   // no work item: the whole workgroup leaves
    finish_empty();
    return;
  }
  // The item's block range, from its two ends in the plan's cost stream (the
  // block stream itself when no sequence is charged); the sequence holding
  // its first block comes with it.
  long long lo, hi;
  SeqInfo sq;
  if (seqs.ctot == seqs.nb) {
    lo = item_lo(item, seqs.nb, P);
    hi = item_lo(item + 1, seqs.nb, P);
    sq = seqs.containing(lo, lane);
  } else {
    SeqInfo sq_end;
    lo = seqs.block_at_cost(item_lo(item, seqs.ctot, P), lane, &sq);
    hi = seqs.block_at_cost(item_lo(item + 1, seqs.ctot, P), lane, &sq_end);
  }
  // The same on every lane; marked so for the compiler, which does not see
  // it through the lookups.
  lo = uniform64(lo);
  hi = uniform64(hi);
  sq.b = __builtin_amdgcn_readfirstlane(sq.b);
  sq.n = __builtin_amdgcn_readfirstlane(sq.n);
  sq.off = uniform64(sq.off);
  if (lo >= hi || sq.b >= batch) {   // not reached: every item holds a block
    finish_empty();
    return;
  }

  const int g = lane & 15;
  const int q = lane >> 4;
  const int koff = g * kHeadDim + 16 * q;
  const int voff = (4 * q + (lane & 3)) * kHeadDim + 16 * ((lane >> 2) & 3);
  const uint32_t sel1 = (lane & 2) ? 0x03020706u : 0x05040100u;
  // E4M3 uses selh0 for the row-order byte selector of the transpose.
  const uint32_t selh0 = F == kKvE4M3 ? ((lane & 1) ? 0x03070105u : 0x06020400u)
                                      : ((lane & 1) ? 0x010C050Cu : 0x040C000Cu);
  const uint32_t selh1 = (lane & 1) ? 0x030C070Cu : 0x060C020Cu;
  const size_t page_stride = (size_t)Hkv * kPageHeadBytes;
  const uint8_t* kbase = a.k_pages + (size_t)h * kPageHeadBytes;
  const uint8_t* vbase = a.v_pages + (size_t)h * kPageHeadBytes;

  auto issue = [&](RawBlock& r, int ids, int mm) {
    const int pa = __builtin_amdgcn_readlane(ids, 2 * mm);
    const int pb = __builtin_amdgcn_readlane(ids, 2 * mm + 1);
    load_block(r, kbase + (size_t)pa * page_stride, kbase + (size_t)pb * page_stride,
               vbase + (size_t)pa * page_stride, vbase + (size_t)pb * page_stride, koff, voff);
  };
  // Item i's first segment keeps its state in record slot 2i, a later one
  // (the last, when it is not whole) in slot 2i + 1.
  auto make_segment = [&](const SeqInfo& sq, bool first) {
    const int nb = seq_blocks(sq.n);
    const long long seg_lo = lo > sq.off ? lo : sq.off;
    const long long seg_hi = hi < sq.off + nb ? hi : sq.off + nb;
    Segment s;
    s.b = sq.b;
    s.n = sq.n;
    s.jb_lo = (int)(seg_lo - sq.off);
    s.jb_hi = (int)(seg_hi - sq.off);
    // Items are contiguous block ranges, so the sequence lies in one item
    // exactly when all its blocks fall in this item's range [lo, hi).
    s.direct = sq.off >= lo && sq.off + nb <= hi;
    s.first = first;
    s.off = sq.off;
    s.rec = a.partials + ((long long)(2 * item + (first ? 0 : 1)) * Hkv + h) * a.item_stride;
    return s;
  };

  Segment cur = make_segment(sq, true);
  WaveSeg cw = wave_seg(a, cur, lane, wave);
  half8 qf[4];
  load_q(a, cur, h, lane, qf);
  RawBlock A, B;
  int ids = 0;
  if (cw.my_blocks > 0) ids = load_ids(cw, 0, lane, wave);
  // The append's loads travel with the page-id and Q loads; its store still
  // precedes every K/V load of the segment.
  if constexpr (kAppend) append_if_owner(a, cur, cw, h, lane, wave);
  if (cw.my_blocks > 0) issue(A, ids, 0);

  while (true) {
    // The next segment of the item: the next non-empty sequence (one exists
    // while the item has blocks left).
    const bool has_next = sq.off + seq_blocks(sq.n) < hi;
    SeqInfo nq = sq;
    if (has_next) {
      do {
        nq = seqs.at(nq.b + 1, lane);
      } while (nq.n == 0);
    }
    const Segment nxt = make_segment(nq, false);
    const WaveSeg nw = wave_seg(a, nxt, lane, wave);
    const bool next_blocks = has_next && nw.my_blocks > 0;

    WaveState st;
    st.m = -INFINITY;
    st.l = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) st.o[t] = float4v{0.f, 0.f, 0.f, 0.f};

    // Precondition of each chunk: A holds (or is loading) its first block.
    for (int c0 = 0; c0 < cw.my_blocks; c0 += 32) {
      const int cnt = min(32, cw.my_blocks - c0);
      const bool more_here = c0 + 32 < cw.my_blocks;
      int ids_next = 0;
      if (more_here) {
        ids_next = load_ids(cw, c0 + 32, lane, wave);
      } else if (next_blocks) {
        ids_next = load_ids(nw, 0, lane, wave);
        if constexpr (kAppend) append_if_owner(a, nxt, nw, h, lane, wave);
      }
      const bool follow = more_here || next_blocks;
      auto tok0 = [&](int mm) { return cw.t_begin + (wave + kWaves * (c0 + mm)) * kBlockTokens; };
      int mm = 0;
      for (; mm + 2 < cnt; mm += 2) {
        issue(B, ids, mm + 1);
        process_block<false, F>(A, qf, st, a.scale_log2e, tok0(mm), cw.t_end, cw.row_end,
                                cw.t_mask, lane, sel1, selh0, selh1);
        issue(A, ids, mm + 2);
        process_block<false, F>(B, qf, st, a.scale_log2e, tok0(mm + 1), cw.t_end, cw.row_end,
                                cw.t_mask, lane, sel1, selh0, selh1);
      }
      if (cnt - mm == 2) {
        issue(B, ids, mm + 1);
        process_block<false, F>(A, qf, st, a.scale_log2e, tok0(mm), cw.t_end, cw.row_end,
                                cw.t_mask, lane, sel1, selh0, selh1);
        if (follow) issue(A, ids_next, 0);
        process_block<true, F>(B, qf, st, a.scale_log2e, tok0(mm + 1), cw.t_end, cw.row_end,
                               cw.t_mask, lane, sel1, selh0, selh1);
      } else {
        process_block<true, F>(A, qf, st, a.scale_log2e, tok0(mm), cw.t_end, cw.row_end,
                               cw.t_mask, lane, sel1, selh0, selh1);
        if (follow) issue(A, ids_next, 0);
      }
      ids = ids_next;
    }
    if (cw.my_blocks == 0 && next_blocks) {   // idle in this segment: start the next one now
      ids = load_ids(nw, 0, lane, wave);
      if constexpr (kAppend) append_if_owner(a, nxt, nw, h, lane, wave);
      issue(A, ids, 0);
    }
    finish_segment(a, sh, cur, st, h, item, lane, wave);
    if (!has_next) break;
    sq = nq;
    cur = nxt;
    cw = nw;
    load_q(a, cur, h, lane, qf);
  }
  finish_empty();
}

// ----------------------------------------------------------- combine kernel
// The combine kernel needs neither the lengths nor the plan: it reads the
// merge record the split kernel wrote for its (sequence, KV head).
// Workgroups of W waves (W = 1, or 4 when a sequence can leave more states
// than one round holds) merge each sequence's split states with the
// log-sum-exp rule, reading states in rounds of kCombineRound with every load
// of a round issued before any is used. A workgroup covers 16 W columns of
// one (sequence, KV head); 128 / (16 W) workgroups cover the head.
//
// Up to one round of states (most sequences), or W = 1: wave w owns 16
// columns, lane t the columns 2(t%8), 2(t%8)+1 of query row t/8; one memory
// round trip per round and no cross-lane step.
//
// More states with W = 4 (a long sequence split over many items): the four
// waves split rounds of kCombineSharedRound states (wave w takes rounds w,
// w+4, ...), lane t owning 8 columns of row t/8 across the workgroup's 64;
// the four partial merges then meet in LDS in wave order. The split depends
// on the state count only, so the result is the same on every run. Rounds
// of 8 rather than 16 here keep the kernel at ~100 VGPRs instead of ~155,
// which measured faster for both paths.
//
// The kernel's path is short, so its set-up counts:
// - Every value it reads besides the records and states comes as a leading
//   scalar argument. All 13 dwords are preloaded into SGPRs, so nothing
//   waits for the argument block, which arrives ~1 us after launch.
// - State addresses come from one running pointer, since states after the
//   first are a fixed stride apart, not from a 64-bit product per state.
//   The scalar unit a CU's waves share spent ~0.3 us more on those
//   products than the states take to arrive.

// Merges one round of split states (cnt valid entries) into (M, L, o[0..N)).
// A state of a query row that saw no token has m = -inf and weight 0; equal
// maxima keep the sums unscaled.
template <int K, int N>
__device__ __forceinline__ void merge_round(const float (&mv)[K], const float (&lv)[K],
                                            const float (&ov)[K][N], int cnt, float& M, float& L,
                                            float (&o)[N]) {
  float mr = M;
#pragma unroll
  for (int k = 0; k < K; ++k) mr = fmaxf(mr, k < cnt ? mv[k] : -INFINITY);
  const float fa = M == mr ? 1.f : exp2_fast(M - mr);   // 0 on the first round
  L *= fa;
#pragma unroll
  for (int c = 0; c < N; ++c) o[c] *= fa;
  M = mr;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float w = (k < cnt && mv[k] != -INFINITY) ? exp2_fast(mv[k] - M) : 0.f;
    L += w * lv[k];
#pragma unroll
    for (int c = 0; c < N; ++c) o[c] += w * ov[k][c];
  }
}

struct CombineShared {
  float m[kCombineMaxWaves][kMaxGroup * 8];
  float l[kCombineMaxWaves][kMaxGroup * 8];
  float4v o[kCombineMaxWaves][kMaxGroup * 8][2];
};

template <int W>
__global__ __launch_bounds__(64 * W) void combine_kernel(const int2* merge_desc, int32_t hkv,
                                                         int32_t per_head, const float* partials,
                                                         int32_t item_stride, int32_t rows,
                                                         uint16_t* out, int32_t group,
                                                         int32_t q_tokens, float v_scale) {
  constexpr int kWgCols = 16 * W;
  constexpr int kChunks = kHeadDim / kWgCols;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int R = rows;
  const int Hkv = hkv;
  const int chunk = blockIdx.x % kChunks;
  auto orow = [&](int bb, int hh, int r) {
    return out + (((long long)bb * q_tokens + r / group) * Hkv * group + (long long)hh * group +
                  r % group) * kHeadDim;
  };
  const int bh = blockIdx.x / kChunks;
  const int b = bh / Hkv;
  const int h = bh % Hkv;

  // The split kernel's record of this (sequence, KV head): the slot of its
  // first state and the work item of its last. Empty sequences and
  // sequences finished in one work item (slot -1) were written by the split
  // kernel.
  const int2 desc = merge_desc[bh];
  const int slot0 = desc.x;
  // The first state is in slot 2 i0 (the sequence starts item i0's block
  // range) or 2 i0 + 1; later items i hold it in slot 2 i. A record that
  // does not describe at least two states inside the grid's slots is not
  // read (a valid one always does).
  const int i0 = slot0 >> 1;
  if (slot0 < 0 || desc.y <= i0 || desc.y >= per_head) return;
  const int nsb = desc.y - i0 + 1;
  const int mo = R * kHeadDim;
  // State s > 0 sits in slot 2 (i0 + s): consecutive states are `step` floats apart.
  const long long step = 2LL * Hkv * item_stride;
  const float* first = partials + ((long long)slot0 * Hkv + h) * item_stride;
  const float* second = partials + ((long long)(2 * (i0 + 1)) * Hkv + h) * item_stride;

  if (__builtin_expect(W == 1 || nsb <= kCombineRound, 1)) {
    // With W = 1 the handle bounds the state count by kCombineRound, so
    // every instantiation merges a single round here.
    for (int e = lane; e < R * 8; e += 64) {
      const int gg = e >> 3;
      const int c = chunk * kWgCols + 16 * wave + (e & 7) * 2;
      float mv[kCombineRound], lv[kCombineRound], ov[kCombineRound][2];
      // Unconditional loads (slots past the last state re-read it and are
      // masked in the merge), so the whole round is in flight at once.
      const float* rk = second;
      const float* last = first;
#pragma unroll
      for (int k = 0; k < kCombineRound; ++k) {
        if (k > 0 && k < nsb) last = rk;
        if (k > 0) rk += step;
        const float* r = k == 0 ? first : last;
        const float2 v = *(const float2*)(r + gg * kHeadDim + c);
        ov[k][0] = v.x;
        ov[k][1] = v.y;
        mv[k] = r[mo + gg];
        lv[k] = r[mo + R + gg];
      }
      float M = -INFINITY, L = 0.f, o[2] = {0.f, 0.f};
      merge_round<kCombineRound, 2>(mv, lv, ov, min(nsb, kCombineRound), M, L, o);
      const float inv = L > 0.f ? v_scale / L : 0.f;   // a row with no visible token is zero
      *(uint32_t*)(orow(b, h, gg) + c) = pack_half2(o[0] * inv, o[1] * inv);
    }
    return;
  }

  if constexpr (W > 1) {
    __shared__ CombineShared sh;
    // Wave w merges rounds w, w + W, ...; lane entry e: row e/8, columns
    // 64 chunk + 8(e%8) .. +8.
    for (int e = lane; e < R * 8; e += 64) {
      const int gg = e >> 3;
      const int c = chunk * kWgCols + (e & 7) * 8;
      float M = -INFINITY, L = 0.f;
      float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const float* lastp = second + (long long)(nsb - 2) * step;   // nsb > 16 here
      for (int s0 = kCombineSharedRound * wave; s0 < nsb; s0 += kCombineSharedRound * W) {
        float mv[kCombineSharedRound], lv[kCombineSharedRound], ov[kCombineSharedRound][8];
        const float* rk = second + (long long)(s0 > 0 ? s0 - 1 : 0) * step;   // state max(s0, 1)
#pragma unroll
        for (int k = 0; k < kCombineSharedRound; ++k) {
          const float* r = s0 + k == 0 ? first : (s0 + k < nsb ? rk : lastp);
          if (s0 + k > 0) rk += step;
          const float4v v0 = *(const float4v*)(r + gg * kHeadDim + c);
          const float4v v1 = *(const float4v*)(r + gg * kHeadDim + c + 4);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            ov[k][x] = v0[x];
            ov[k][4 + x] = v1[x];
          }
          mv[k] = r[mo + gg];
          lv[k] = r[mo + R + gg];
        }
        merge_round<kCombineSharedRound, 8>(mv, lv, ov, min(kCombineSharedRound, nsb - s0), M, L,
                                            o);
      }
      sh.m[wave][e] = M;   // -inf and 0 for a wave with no rounds
      sh.l[wave][e] = L;
      sh.o[wave][e][0] = float4v{o[0], o[1], o[2], o[3]};
      sh.o[wave][e][1] = float4v{o[4], o[5], o[6], o[7]};
    }
    __syncthreads();
    for (int e = threadIdx.x; e < R * 8; e += 64 * W) {
      float M = sh.m[0][e];
#pragma unroll
      for (int w = 1; w < W; ++w) M = fmaxf(M, sh.m[w][e]);
      float L = 0.f;
      float4v o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = sh.m[w][e];
        const float f = mw == -INFINITY ? 0.f : exp2_fast(mw - M);
        L += f * sh.l[w][e];
        o0 += f * sh.o[w][e][0];
        o1 += f * sh.o[w][e][1];
      }
      const float inv = L > 0.f ? v_scale / L : 0.f;
      uint4 packed;
      packed.x = pack_half2(o0[0] * inv, o0[1] * inv);
      packed.y = pack_half2(o0[2] * inv, o0[3] * inv);
      packed.z = pack_half2(o1[0] * inv, o1[1] * inv);
      packed.w = pack_half2(o1[2] * inv, o1[3] * inv);
      *(uint4*)(orow(b, h, e >> 3) + chunk * kWgCols + (e & 7) * 8) = packed;
    }
  }
}

// ---------------------------------------------------------------- KV append
// One thread per (sequence, KV head, K or V, 8 head-dim values): a 16-byte
// read of the new row, an 8-byte write into the page slot. 16 consecutive
// threads cover one 128-value row, so reads and writes are contiguous.
constexpr int kAppendThreads = 256;

// The grid holds batch * Hkv * 32 threads, which can pass 2^32, so the
// thread index is 64-bit; b * Hkv + h stays below 2^28 (creation bounds
// max_batch * Hkv * 8 below 2^31), so the division by Hkv is 32-bit. All
// arguments but v_pages arrive preloaded in SGPRs; v_pages, the length and
// the new row are loaded together.
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const int32_t* context_lens, const int32_t* block_table, const uint16_t* k_new,
    const uint16_t* v_new, uint8_t* k_pages, int32_t batch, int32_t num_kv_heads,
    int32_t max_pages, uint8_t* v_pages) {
  const unsigned long long gid = (unsigned long long)blockIdx.x * kAppendThreads + threadIdx.x;
  if (gid >= (unsigned long long)batch * num_kv_heads * 32u) return;
  const int j = (int)(gid & 15);
  const int is_v = (int)((gid >> 4) & 1);
  const unsigned bh = (unsigned)(gid >> 5);   // b * Hkv + h
  const int h = (int)(bh % (unsigned)num_kv_heads);
  const int b = (int)(bh / (unsigned)num_kv_heads);
  const int n = context_lens[b];
  const uint16_t* src = (is_v ? v_new : k_new) + (size_t)bh * kHeadDim + 8 * j;
  const u32x4 x = *(const u32x4*)src;
  asm volatile("" ::"v"(n), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "s"(v_pages));
  if (n <= 0 || n > max_pages * kPageSize) return;   // no slot for this sequence
  const int t = n - 1;
  const int page = block_table[(long long)b * max_pages + t / kPageSize];
  uint32_t packed[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t p0 = x[2 * w], p1 = x[2 * w + 1];
    packed[w] = e5m2_from_f16(p0 & 0xFFFFu) | (e5m2_from_f16(p0 >> 16) << 8) |
                (e5m2_from_f16(p1 & 0xFFFFu) << 16) | (e5m2_from_f16(p1 >> 16) << 24);
  }
  uint8_t* dst = (is_v ? v_pages : k_pages) +
                 (((size_t)page * num_kv_heads + h) * kPageSize + t % kPageSize) * kHeadDim + 8 * j;
  *(uint2*)dst = make_uint2(packed[0], packed[1]);
}

// ------------------------------------------------------------ widen (test)
// Each thread widens one group of four codes with the same helpers the K
// path uses, so every byte position of both selectors is exercised.
template <int F>
__global__ void widen_kernel(const uint8_t* in, uint16_t* out16, float* out32, long long n) {
  const long long grp = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long i0 = grp * 4;
  if (i0 >= n) return;
  uint32_t x = 0;
  for (int k = 0; k < 4; ++k) {
    if (i0 + k < n) x |= (uint32_t)in[i0 + k] << (8 * k);
  }
  const uint32_t lo = widen_k_lo<F>(x), hi = widen_k_hi<F>(x);
  const uint16_t bits[4] = {(uint16_t)(lo & 0xFFFFu), (uint16_t)(lo >> 16), (uint16_t)(hi & 0xFFFFu),
                            (uint16_t)(hi >> 16)};
  for (int k = 0; k < 4; ++k) {
    if (i0 + k >= n) break;
    if (out16) out16[i0 + k] = bits[k];
    if (out32) out32[i0 + k] = (float)__builtin_bit_cast(_Float16, bits[k]);
  }
}

}  // namespace

hipError_t launch_split(const AttendArgs& a, int grid, hipStream_t stream) {
  if (a.k_new != nullptr) {
    hipLaunchKernelGGL((split_kernel<kKvE5M2, true>), dim3(grid), dim3(kThreads), 0, stream,
                       a.context_lens, a.batch, a.max_tokens, a);
  } else if (a.kv_format == kKvE4M3) {
    hipLaunchKernelGGL((split_kernel<kKvE4M3, false>), dim3(grid), dim3(kThreads), 0, stream,
                       a.context_lens, a.batch, a.max_tokens, a);
  } else {
    hipLaunchKernelGGL((split_kernel<kKvE5M2, false>), dim3(grid), dim3(kThreads), 0, stream,
                       a.context_lens, a.batch, a.max_tokens, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const AttendArgs& a, hipStream_t stream) {
  if (a.combine_waves == kCombineMaxWaves) {
    constexpr int W = kCombineMaxWaves;
    const int grid = a.batch * a.num_kv_heads * (kHeadDim / (16 * W));
    hipLaunchKernelGGL(combine_kernel<W>, dim3(grid), dim3(64 * W), 0, stream, a.merge_desc,
                       a.num_kv_heads, a.per_head, a.partials, a.item_stride, a.rows, a.out,
                       a.group, a.q_tokens, a.v_scale);
  } else {
    const int grid = a.batch * a.num_kv_heads * (kHeadDim / 16);
    hipLaunchKernelGGL(combine_kernel<1>, dim3(grid), dim3(64), 0, stream, a.merge_desc,
                       a.num_kv_heads, a.per_head, a.partials, a.item_stride, a.rows, a.out,
                       a.group, a.q_tokens, a.v_scale);
  }
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const long long total = (long long)a.batch * a.num_kv_heads * 32;
  const long long blocks = (total + kAppendThreads - 1) / kAppendThreads;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream,
                     a.context_lens, a.block_table, a.k_new, a.v_new, a.k_pages, a.batch,
                     a.num_kv_heads, a.max_pages, a.v_pages);
  return hipGetLastError();
}

hipError_t launch_widen(const uint8_t* in, uint16_t* out_f16, float* out_f32, int64_t n,
                        int32_t kv_format, hipStream_t stream) {
  const long long groups = (n + 3) / 4;
  const int threads = 256;
  const long long blocks = (groups + threads - 1) / threads;
  if (kv_format == kKvE4M3) {
    hipLaunchKernelGGL(widen_kernel<kKvE4M3>, dim3((unsigned)blocks), dim3(threads), 0, stream, in,
                       out_f16, out_f32, (long long)n);
  } else {
    hipLaunchKernelGGL(widen_kernel<kKvE5M2>, dim3((unsigned)blocks), dim3(threads), 0, stream, in,
                       out_f16, out_f32, (long long)n);
  }
  return hipGetLastError();
}

// Resident split workgroups per CU: the smallest figure of the three
// instantiations, so one grid serves all of them.
hipError_t attend_blocks_per_cu(int* blocks) {
  int a = 0, b = 0, c = 0;
  hipError_t e =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, split_kernel<kKvE5M2, false>, kThreads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, split_kernel<kKvE4M3, false>, kThreads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, split_kernel<kKvE5M2, true>, kThreads, 0);
  if (e != hipSuccess) return e;
  *blocks = a < b ? a : b;
  if (c < *blocks) *blocks = c;
  return e;
}

}  // namespace xqa
