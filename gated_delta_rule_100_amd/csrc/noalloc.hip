// noalloc.hip -- gdr_chunk_prefill_noalloc: the chunked prefill with the
// library's own static device scratch in place of a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is a file-scope device array, so each GPU that runs the library
// holds its own copy (in the memory of this file's code object on that
// device) from the first call until the process ends.  Host code never uses
// the array's name as an address: at the first call on a device, with that
// device current, hipGetSymbolAddress yields the device address of that
// device's copy, which is kept per device and passed to the kernels like a
// workspace.  Nothing here allocates or frees.  No scratch word is read
// before the same call has written it, so leftovers of an earlier call do not
// matter and nothing is cleared.  Calls that overlap on one device (two
// streams, two threads) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(128) << 20;  // 128 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[gdr::kMaxDevices];

}  // namespace

namespace gdr {

gdr_status static_scratch_address(int device, void** ptr) {
  DeviceScratch& d = g_scratch[device];
  std::call_once(d.once, [&d] {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess) d.ptr = p;
  });
  if (d.err != hipSuccess) return hip_status(d.err, "hipGetSymbolAddress(scratch)");
  *ptr = d.ptr;
  return GDR_OK;
}

}  // namespace gdr

extern "C" gdr_status gdr_chunk_prefill_noalloc(
    const void* q, const void* k, const void* v, const float* g, const float* beta,
    const int32_t* cu_seqlens, int N, const float* state_in, float* state_out, void* o,
    float* L_out, float* M_out, float* fixed_out, int T_total, int H, int dk, int dv, int chunk,
    gdr_dtype in_dtype, gdr_dtype out_dtype, gdr_stream_t stream) {
  return gdr::chunk_prefill("gdr_chunk_prefill_noalloc", q, k, v, g, beta, cu_seqlens, N,
                            state_in, state_out, o, L_out, M_out, fixed_out, T_total, H, dk, dv,
                            chunk, in_dtype, out_dtype, nullptr, kScratchBytes, true, stream);
}
