// Workspace for xqa_decode_noalloc: a fixed device array instead of memory
// the library allocates, for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// Host code never passes the array's name to a kernel: its address on each
// device is looked up once, with that device current, and kept.

#include <mutex>

#include "xqa_noalloc.h"

namespace xqa {
namespace {

// Split-state and merge records of one decode call at a time (each call
// writes every record it reads, so no contents carry over between calls).
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceSlot {
  bool ready;
  NoallocDevice dev;
};

std::mutex g_mutex;
DeviceSlot g_slots[kMaxDevices];

}  // namespace

hipError_t noalloc_device(int device, NoallocDevice* out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceSlot& s = g_slots[device];
  if (!s.ready) {
    NoallocDevice d;
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return e;
    e = attend_blocks_per_cu(&d.per_cu);
    if (e != hipSuccess) return e;
    d.scratch = ptr;
    s.dev = d;
    s.ready = true;
  }
  *out = s.dev;
  return hipSuccess;
}

}  // namespace xqa
