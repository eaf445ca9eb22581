// scratch.hip -- the library's static device scratch, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc): dsa_decode_noalloc carves the decode
// workspace from this array instead of a caller's buffer.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy, from the first use until the process ends.  In
// host code its name is only a host-side stand-in for the symbol, never a
// device address: the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device; every
// kernel argument uses that address.
//
// Nothing in the scratch needs to start at zero: the decode kernels write
// every element they later read (score rows up to each context, the
// selection, every split's partial output and softmax pair).  Calls that use
// it on one GPU share it, so two such calls that overlap in time on that GPU
// (different streams, different threads) race.
#include <mutex>

#include "dsa_common.h"
#include "dsa_launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;  // 128 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch`, per device (null until looked up)

}  // namespace

namespace dsa {

size_t static_scratch_bytes() { return kScratchBytes; }

hipError_t static_scratch(hipStream_t stream, void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;  // the lookup is made on the current device
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace dsa
