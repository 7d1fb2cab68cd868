// The grouped fused matmul for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the SPLIT decode path with
// its workspace (activation layouts, partial slots, counters, statistics) in a scratch array the
// library owns, one per device.
//
// The array is a file-scope __device__ variable: every device the library runs on holds one
// copy, at its own address, until the process ends.  Its device address is looked up once per
// device (with that device current) and kept; host code passes that address to the kernels,
// never the array's name (which, in host code, is only a host-side stand-in).  All calls on one
// device share its copy, so calls that overlap in time on one device race; the split counters
// are cleared by the prologue kernel of each launch, and the statistics word only accumulates.
#include <mutex>

#include "../../include/bitdelta.h"
#include "bd_internal.h"

namespace bd {
bitdelta_status status_of_hip(hipError_t e);
bitdelta_status matmul_grouped_split(const bitdelta_problem* problems, int32_t num_problems,
                                     int64_t M, const int32_t* seg_offsets,
                                     const int32_t* seg_variant, int32_t num_segments,
                                     int32_t y_dtype, int32_t path, void* workspace,
                                     size_t ws_bytes, hipStream_t stream);
}  // namespace bd

namespace {

__device__ __align__(256) unsigned char scratch[BITDELTA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // per device: the device address of `scratch`, null until found

// The current device's copy of `scratch` (looked up on the first call on each device).
hipError_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" bitdelta_status bitdelta_matmul_grouped_noalloc(
    const bitdelta_problem* problems, int32_t num_problems, int64_t M, const int32_t* seg_offsets,
    const int32_t* seg_variant, int32_t num_segments, int32_t y_dtype, int32_t path,
    bitdelta_stream stream) {
  void* ws = nullptr;
  const hipError_t e = device_scratch(&ws);
  if (e != hipSuccess) return bd::status_of_hip(e);
  return bd::matmul_grouped_split(problems, num_problems, M, seg_offsets, seg_variant,
                                  num_segments, y_dtype, path, ws, BITDELTA_NOALLOC_SCRATCH_BYTES,
                                  static_cast<hipStream_t>(stream));
}
