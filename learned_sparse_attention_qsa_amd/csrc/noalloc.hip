// qsa_forward_noalloc: qsa_forward with its scratch memory in a file-scope
// device array instead of a caller workspace, for callers that cannot
// allocate (code under stream capture, serving loops that forbid
// allocation).  The kernels are qsa_forward's; they receive this array's
// device address where qsa_forward passes the caller's workspace.
//
// The array exists once per GPU the library runs on (the runtime places it
// with the code object, for the life of the process), at a different address
// on each GPU: the address is taken once per device, with that device
// current, by hipGetSymbolAddress, and only that address is ever handed to
// kernels.  (In host code the array's name is a host-side stand-in, not a
// device address.)  Every call on one GPU shares the array, so calls that
// overlap in time on one GPU race; every word the kernels read from it is
// written earlier in the same call, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/qsa.h"
#include "internal.h"

namespace {

constexpr size_t kScratchBytes = QSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once taken

qsa_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QSA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QSA_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return QSA_OK;
}

}  // namespace

extern "C" {

qsa_status qsa_forward_noalloc(const qsa_shape* shape, const uint16_t* q_idx,
                               const uint16_t* k_idx, uint16_t* k_cmp,
                               const int32_t* first_block, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* lens, uint16_t* out, float* lse,
                               int32_t* sel_out, int32_t* n_sel_out, void* stream) {
  if (!shape) return QSA_ERR_NULL;
  // (an invalid shape needs 0 bytes here and is rejected by qsa_forward)
  const size_t need = qsa_workspace_bytes(shape, QSA_OP_FORWARD);
  if (need > kScratchBytes) return QSA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const qsa_status st = scratch_address(&ws);
    if (st != QSA_OK) return st;
  }
  return qsa_forward(shape, q_idx, k_idx, k_cmp, first_block, q, k, v, lens, out, lse, sel_out,
                     n_sel_out, ws, need, stream);
}

}  // extern "C"
