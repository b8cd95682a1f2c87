// moe_grouped_ffn for callers that cannot allocate device memory: the SwiGLU
// activations between the gate/up and the down GEMM go to a fixed scratch
// array that the library keeps in each GPU's memory, instead of a
// caller-provided workspace.  Everything else is moe_grouped_ffn: the same
// validation, the same kernels, the same bits.
#include <mutex>

#include "launch.h"

namespace moev {
namespace {

constexpr size_t kScratchBytes = MOEV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// One copy per GPU, alive until the process ends.  Host code must not take
// this name as a device address: the address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, looked up on its first call

// The device address of the current device's scratch array (NULL after
// recording the reason).  Called with the caller's device current.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("moe_grouped_ffn_noalloc: no usable current device (%d)", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("moe_grouped_ffn_noalloc: hipGetSymbolAddress failed on device %d: %s", dev,
                hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace moev

extern "C" moev_status moe_grouped_ffn_noalloc(const void* x, const int32_t* sorted_src,
                                               const int32_t* group_offsets, const float* topk_w,
                                               const void* w_gate, const void* w_up, const void* w_down,
                                               int T, int H, int I, int E, int k, int ns, int dt,
                                               float* y_slots, void* stream) {
  // the size limit first, so an oversized call is rejected before any HIP call
  if (T > 0 && I > 0 && k >= 0 && ns >= 0 && (dt == MOEV_F32 || dt == MOEV_BF16)) {
    const size_t need = moev::grouped_ffn_ws_bytes(T, I, k, ns, dt);
    MOEV_REQUIRE(need <= moev::kScratchBytes, MOEV_ERR_WORKSPACE,
                 "moe_grouped_ffn_noalloc: T=%d needs %zu bytes of activations; the static scratch holds %zu",
                 T, need, moev::kScratchBytes);
  }
  // the checks of moe_grouped_ffn, with the scratch array as the workspace
  // (any 16-byte aligned non-NULL address stands in for it here)
  if (moev_status st = moev::validate_grouped_ffn(x, sorted_src, group_offsets, topk_w, w_gate, w_up, w_down,
                                                  T, H, I, E, k, ns, dt, y_slots,
                                                  reinterpret_cast<const void*>(uintptr_t{256}),
                                                  moev::kScratchBytes))
    return st;
  if (T == 0) return MOEV_OK;
  void* ws = moev::scratch_address();
  if (ws == nullptr) return MOEV_ERR_HIP;
  moev::launch_grouped_ffn(x, sorted_src, group_offsets, topk_w, w_gate, w_up, w_down, T, H, I, E, k, ns, dt,
                           y_slots, ws, moev::as_stream(stream));
  return moev::launch_status("moe_grouped_ffn_noalloc");
}
