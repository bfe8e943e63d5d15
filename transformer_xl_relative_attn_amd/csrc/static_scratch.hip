// txl_rel_attn_fwd_static: txl_rel_attn_fwd for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The temporaries that txl_rel_attn_fwd keeps in the
// caller's workspace (projected q, K, V^T, position keys, key-range split
// partials) live instead in `scratch`, a file-scope device array that each GPU
// the library runs on holds until the process ends.
//
// `scratch` is a device symbol: in host code its name is not a device address.
// Its address on the current device is taken once per device with
// hipGetSymbolAddress and only that pointer is used afterwards.  Every call on
// one GPU shares that GPU's array and leaves its contents behind; nothing in
// it has to start at zero (every region is written before it is read, as with
// a caller workspace).  Calls that overlap on one GPU (two streams, two
// threads) race on the array.
#include <mutex>

#include "dev_common.h"

namespace txl {
namespace {

constexpr size_t kScratchBytes = (size_t)TXL_STATIC_SCRATCH_BYTES;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The array's address on the current device (looked up once per device).
txl_status_t scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(TXL_ERR_HIP, "txl_rel_attn_fwd_static: no current HIP device");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(TXL_ERR_HIP, "txl_rel_attn_fwd_static: hipGetSymbolAddress(scratch) failed");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return TXL_OK;
}

}  // namespace
}  // namespace txl

extern "C" txl_status_t txl_rel_attn_fwd_static(const txl_attn_shape_t* shape, const void* h,
                                                const void* mem, int32_t mem_start,
                                                const void* W_q, const void* W_kE,
                                                const void* W_kR, const void* W_v, const void* u,
                                                const void* v, const void* R, const void* Rk,
                                                void* out, void* stream) {
  // An invalid shape needs no scratch: txl_rel_attn_fwd reports it.
  const size_t need = txl_rel_attn_workspace_bytes(shape);
  if (need > txl::kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg,
             "txl_rel_attn_fwd_static: this shape needs %zu bytes of scratch, above the "
             "static maximum of %zu",
             need, txl::kScratchBytes);
    return txl::set_error(TXL_ERR_WORKSPACE_TOO_SMALL, msg);
  }
  void* ws = nullptr;
  if (need > 0) {
    const txl_status_t st = txl::scratch_ptr(&ws);
    if (st != TXL_OK) return st;
  }
  txl::suppress_timing(true);
  const txl_status_t st = txl_rel_attn_fwd(shape, h, mem, mem_start, W_q, W_kE, W_kR, W_v, u, v,
                                           R, Rk, out, ws, need > 0 ? txl::kScratchBytes : 0,
                                           stream);
  txl::suppress_timing(false);
  return st;
}
