// tb_ternary_gemv_noalloc: tb_ternary_gemv for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The workspace tb_ternary_gemv takes from
// its caller -- the K slices' partial rows of the decode-batch path, or the
// prepared activation of the prepare/run path -- lives instead in `scratch`,
// a file-scope device array of TB_NOALLOC_SCRATCH_BYTES that every GPU the
// library runs on holds until the process ends.  The kernels are those of
// tb_ternary_gemv; only the workspace differs.
//
// `scratch` names a host-side stand-in in host code, not the device array:
// its device address is looked up once per device with hipGetSymbolAddress
// (each GPU has its own copy at its own address) and only that address is
// ever handed to a kernel.
#include <atomic>

#include "tb_gemv.h"

namespace tb {

static __device__ __align__(256) char scratch[TB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (nullptr and an error
// message on failure).  Looked up on the first call on each device, with
// that device current; two threads racing store the same address.
static void* scratch_on_current_device(const char* who) {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("%s: no usable current HIP device", who);
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    set_error("%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", who, dev,
              hipGetErrorString(e));
    return nullptr;
  }
  addr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace tb

using namespace tb;

extern "C" int tb_ternary_gemv_noalloc(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs,
                                       int block, const uint32_t* codes, const uint16_t* scales,
                                       const uint16_t* biases, int64_t N, float* y, void* stream) {
  const char* who = "tb_ternary_gemv_noalloc";
  TB_TRY(gemv_checked_args(x, x_dtype, B, K, signs, block, codes, scales, biases, N, y, who));
  if (B == 0 || N == 0) return TB_OK;
  // The decode-batch path when its partial rows fit the scratch array, else
  // the path that needs only the prepared activation; a call that needs more
  // than the array holds is refused before anything is enqueued.
  const size_t need = tb_ternary_gemv_workspace_size(B, K);
  if (need > TB_NOALLOC_SCRATCH_BYTES) {
    set_error("%s: B=%lld K=%lld needs %zu bytes of scratch; this entry point holds %zu (use tb_ternary_gemv "
              "with a workspace)", who, (long long)B, (long long)K, need, (size_t)TB_NOALLOC_SCRATCH_BYTES);
    return TB_ERR_WORKSPACE;
  }
  void* ws = scratch_on_current_device(who);
  if (!ws) return TB_ERR_HIP;
  return gemv_dispatch(x, x_dtype, B, K, signs, block, codes, scales, biases, N, y, ws, TB_NOALLOC_SCRATCH_BYTES,
                       static_cast<hipStream_t>(stream), who);
}
