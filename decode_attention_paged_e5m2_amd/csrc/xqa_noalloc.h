// The fixed device workspace of xqa_decode_noalloc.
#pragma once

#include "xqa_internal.h"

namespace xqa {

// Size of the fixed workspace on each device: split-state records, then the
// per-(sequence, KV head) merge records.
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;

struct NoallocDevice {
  void* scratch;   // device address of the workspace on this device
  int cus;         // compute units
  int per_cu;      // resident split workgroups per CU
};

// The workspace address and the split grid's inputs for `device`, which must
// be the current device. Looked up on the first call per device and kept.
hipError_t noalloc_device(int device, NoallocDevice* out);

}  // namespace xqa
