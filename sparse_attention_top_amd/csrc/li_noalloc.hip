// li_indexer_noalloc: li_indexer with the library's own device scratch as its
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace (the head-reduced scores of every visible pair and the
// candidate lists of split rows) is a file-scope device array of
// kScratchBytes, which every GPU the library runs on holds until the process
// ends. Its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// ever handed to kernels: in host code the array's name stands for a host-side
// shadow, not for device memory.
//
// Nothing in the workspace needs clearing between calls: the score kernel
// writes every score the top-k kernels read, and the first top-k pass writes
// every candidate the second reads. Every call on one GPU shares that GPU's
// array, so calls that may overlap on one GPU (two streams, two threads) race
// on it; calls ordered on one stream do not.
#include <mutex>

#include "li_internal.h"

namespace {

// 256 MiB: the workspace of an 8K x 8K causal prefill (8192 rows of 8192
// floats), the largest single problem the allocation-free path serves.
constexpr size_t kScratchBytes = size_t(256) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

extern "C" {

size_t li_noalloc_capacity(void) { return kScratchBytes; }

li_status li_indexer_noalloc(const li_problem* p, const li_inputs* in, const void* meta_host,
                             const void* meta_dev, int32_t* sparse_indices,
                             float* sparse_values, void* stream) {
  // Problem, table and size first: an oversized problem is rejected before any
  // HIP call.
  size_t need = 0;
  li_status st = li_workspace_size(p, meta_host, &need);
  if (st != LI_OK) return st;
  if (need > kScratchBytes)
    return li::set_error(LI_ERR_WORKSPACE_TOO_SMALL,
                         "li_indexer_noalloc: the problem needs a %zu-byte workspace, the "
                         "library's scratch holds %zu bytes; use li_indexer with a caller "
                         "workspace",
                         need, kScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return li::set_error(LI_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return li::set_error(LI_ERR_UNSUPPORTED, "device %d is beyond the %d devices served", dev,
                         kMaxDevices);
  std::call_once(g_once[dev], [dev] {
    void* ptr = nullptr;
    g_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_err[dev] != hipSuccess || g_ptr[dev] == nullptr)
    return li::set_error(LI_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                         hipGetErrorString(g_err[dev]));
  return li_indexer(p, in, meta_host, meta_dev, g_ptr[dev], kScratchBytes, sparse_indices,
                    sparse_values, stream);
}

}  // extern "C"
