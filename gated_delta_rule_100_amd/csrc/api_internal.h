// api_internal.h -- host-side pieces of the C ABI shared between its source
// files (internal to libgdr).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/gdr.h"

namespace gdr {

constexpr int kMaxDevices = 64;

// Records a message for gdr_last_error() on the calling thread and returns s.
gdr_status fail(gdr_status s, const char* fmt, ...);
// Clears the calling thread's message and returns GDR_OK.
gdr_status ok();
// GDR_OK for hipSuccess, else GDR_ERR_HIP with "<what>: <HIP error>".
gdr_status hip_status(hipError_t e, const char* what);
// Checks that the current device is a gfx950 (properties cached per device)
// and, when `device` is given, stores its id there.
gdr_status check_device(int* device = nullptr);

// The device address of the library's static scratch (noalloc.hip) on device
// `device` (the current device), looked up once per device.
gdr_status static_scratch_address(int device, void** ptr);

// Validation and dispatch of gdr_chunk_prefill (arguments as in gdr.h).  `who`
// names the entry point in error messages.  With static_scratch the workspace
// is the library's own scratch array of workspace_bytes bytes, and a call that
// needs more is refused with GDR_ERR_UNSUPPORTED before anything is launched.
gdr_status chunk_prefill(const char* who, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const int32_t* cu_seqlens, int N,
                         const float* state_in, float* state_out, void* o, float* L_out,
                         float* M_out, float* fixed_out, int T_total, int H, int dk, int dv,
                         int chunk, gdr_dtype in_dtype, gdr_dtype out_dtype, void* workspace,
                         size_t workspace_bytes, bool static_scratch, gdr_stream_t stream);

}  // namespace gdr
