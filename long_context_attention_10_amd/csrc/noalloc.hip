// Entry points that allocate nothing: the library-owned scratch they run in.
//
// csa_index_topk_decode needs B * n_entries * 20 bytes of scratch (scores,
// chunk lists, tie lists) plus its histograms, which must be zero when a call
// starts.  Callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc) use the
// variant here, which takes that scratch from a file-scope device array of a
// fixed size instead of a caller workspace.
//
// The array is one per GPU (each device holds its own copy at its own
// address).  In host code its name is only a host-side stand-in, so its
// device address is looked up once per device with hipGetSymbolAddress and
// that pointer alone is handed to kernels.  Every call on a GPU shares the
// array, so calls that overlap on one GPU (unordered streams) race.
#include <mutex>

#include "csa_launch.h"

namespace csa {
namespace {

constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;  // 32 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

struct DeviceScratch {
  void* ptr = nullptr;     // device address of `scratch` on this device
  size_t zero_prefix = 0;  // leading bytes the last call left zero
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

__global__ void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The calling thread's current device's scratch record, with its address
// looked up on first use (that device is current during the lookup).
int device_scratch(DeviceScratch** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_ERR_HIP;
  DeviceScratch& s = g_dev[dev];
  if (!s.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA_ERR_HIP;
    s.ptr = p;
    s.zero_prefix = 0;
  }
  *out = &s;
  return CSA_OK;
}

}  // namespace

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

int index_topk_decode_noalloc(const csa_index_desc& d, const void* qI, const void* wI,
                              const void* KI, const int64_t* pos, int32_t* idx_out,
                              hipStream_t st) {
  const size_t need = index_decode_ws_bytes(d);
  const size_t zero = index_decode_zero_bytes(d);  // a multiple of 256
  if (need > kNoallocScratchBytes) return CSA_ERR_WORKSPACE;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch* s = nullptr;
  int rc = device_scratch(&s);
  if (rc) return rc;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess) return CSA_ERR_HIP;
  if (zero > s->zero_prefix) {
    // the histogram region grew past what the last call left zero: clear it
    // with a kernel (no memset node, so the call can be captured)
    const size_t n16 = zero / 16;
    const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    zero_fill_kernel<<<blocks, 256, 0, st>>>((uint4*)s->ptr, n16);
    if (hipGetLastError() != hipSuccess) return CSA_ERR_HIP;
  }
  const hipError_t e = launch_index_topk_decode(d, qI, wI, KI, pos, idx_out, s->ptr, st);
  if (e != hipSuccess) {
    s->zero_prefix = 0;
    return CSA_ERR_HIP;
  }
  // An eager call leaves exactly its histogram region zero.  A captured call
  // has not run yet, and its replays will leave only that region zero, so
  // the record may only shrink.
  s->zero_prefix = cap == hipStreamCaptureStatusNone
                       ? zero
                       : (zero < s->zero_prefix ? zero : s->zero_prefix);
  return CSA_OK;
}

}  // namespace csa
