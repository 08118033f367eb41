// mlaq_scratch.hip -- the library-owned device scratch of the allocation-free
// attention entry point (mlaq_attn_run_noalloc), for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// The array is a zero-initialised file-scope device variable: the loader
// places one copy on every device the code object is loaded on, and it lives
// until the process ends. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address of each device's copy is looked up once with hipGetSymbolAddress,
// with that device current, and cached here.
#include <mutex>

#include "mlaq_internal.h"

namespace mlaq {
namespace {

static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

} // namespace

hipError_t scratch_address(int device, void** ptr) {
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

} // namespace mlaq
