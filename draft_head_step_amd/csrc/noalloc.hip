// Allocation-free variant of the Markov-head draft for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The draft's only scratch is its packed per-step results (gamma * R words of
// up to 16 x 8 bytes), which dspark_markov_draft takes from a caller
// workspace.  This variant takes them from `scratch`, a file-scope device
// array of a fixed size, instead.  Every GPU the library runs on holds its own
// copy until the process ends.  Its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept; host code
// never passes the array's own name to a kernel or a copy, since on the host
// that name is only a stand-in for the symbol, not a device address.
//
// Calls on one GPU share that GPU's array: two calls that overlap in time on
// one device (different streams, or host threads) race on it and must be
// ordered by the caller.  The kernels clear the words they use at the start of
// every call (a fill kernel, no memset node), so stale contents from an
// earlier call do not matter.
#include <mutex>

#include "dspark_internal.h"

namespace dspark {
namespace {

constexpr size_t kScratchBytes = DSPARK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
dspark_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DSPARK_EDEVICE, "markov_draft_noalloc: no usable current device");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DSPARK_EDEVICE, "markov_draft_noalloc: hipGetSymbolAddress failed: %s",
                  hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return DSPARK_OK;
}

}  // namespace
}  // namespace dspark

extern "C" dspark_status dspark_markov_draft_noalloc(
    const uint16_t* W1, const uint16_t* W2, const float* base, const int32_t* anchors, int R,
    int gamma, int V, int r, int layout, int mode, float temperature, const float* uniforms,
    int32_t* tokens, void* stream) {
  dspark_status st = dspark::check_markov_args(W1, W2, base, anchors, R, gamma, V, r, layout, mode,
                                               temperature, uniforms, tokens, nullptr);
  if (st != DSPARK_OK) return st;
  const size_t need = dspark_markov_draft_workspace(R, gamma, V, r);
  if (need > dspark::kScratchBytes)
    return dspark::fail(DSPARK_EUNSUPPORTED,
                        "markov_draft_noalloc: needs %zu bytes of scratch but the static array "
                        "holds %zu (R * gamma at most %zu)",
                        need, dspark::kScratchBytes, dspark::kScratchBytes / 128);
  void* ws = nullptr;
  st = dspark::scratch_ptr(&ws);
  if (st != DSPARK_OK) return st;
  return dspark::launch_markov_draft(W1, W2, base, anchors, R, gamma, V, r, layout, mode,
                                     temperature, uniforms, tokens, nullptr, ws, nullptr,
                                     reinterpret_cast<hipStream_t>(stream));
}
