// Page-subset decode (xqa_decode_pages): the kernel that gathers each
// sequence's kept pages into a page table of its own. Kept apart from the
// attention kernels, which then run unchanged over that table.
#pragma once

#include "xqa_internal.h"

namespace xqa {

struct SelectArgs {
  const int32_t* block_table;     // [batch][max_pages]
  const int32_t* context_lens;    // [batch]
  const int32_t* page_select;     // [batch][select_stride] logical page indices
  const int32_t* select_counts;   // [batch]
  int32_t* vtable;                // [batch][vstride] physical ids of the kept pages
  int32_t* vlens;                 // [batch] tokens of the kept pages below n
  int32_t batch;
  int32_t max_pages;
  int32_t max_tokens;             // max_pages * page size
  int32_t select_stride;          // <= vstride
  int32_t vstride;
};

hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

}  // namespace xqa
