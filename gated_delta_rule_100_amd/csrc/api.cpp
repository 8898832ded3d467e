// api.cpp -- the C ABI of libgdr: host-side validation and dispatch.
//
// Every entry point validates its arguments on the host, records a message
// for gdr_last_error() on failure and launches nothing in that case.  Nothing
// here allocates, frees or synchronises; all work is enqueued on the caller's
// stream.  The only global state is a per-device property cache (the
// per-device attribute caching of the host launcher on the FlashInfer PR #4593
// page, code analysis 1, follows the same pattern).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string_view>

#include "../../include/gdr.h"
#include "api_internal.h"
#include "launch.h"

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

namespace gdr {

gdr_status fail(gdr_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

gdr_status ok() {
  g_last_error[0] = '\0';
  return GDR_OK;
}

gdr_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GDR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

namespace {

// Per-device properties, filled once per device.
struct DeviceProps {
  bool filled = false;
  bool gfx950 = false;
  char arch[64] = "";
};
DeviceProps g_props[kMaxDevices];
std::mutex g_props_mu;

}  // namespace

gdr_status check_device(int* device) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(GDR_ERR_UNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_props_mu);
  DeviceProps& p = g_props[dev];
  if (!p.filled) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
    snprintf(p.arch, sizeof p.arch, "%s", prop.gcnArchName);
    p.gfx950 = std::string_view(prop.gcnArchName).substr(0, 6) == "gfx950";
    p.filled = true;
  }
  if (!p.gfx950) return fail(GDR_ERR_UNSUPPORTED, "device %d is %s; libgdr is built for gfx950", dev, p.arch);
  if (device) *device = dev;
  return GDR_OK;
}

}  // namespace gdr

namespace {

using gdr::check_device;
using gdr::fail;
using gdr::hip_status;
using gdr::ok;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dims(int dk, int dv) { return (dk == 64 && dv == 64) || (dk == 128 && dv == 128); }

bool valid_dtype(int d) { return d == GDR_BF16 || d == GDR_FP32; }

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Segment size (in chunks) of the two-level fixup, or 0 for the single-level
// scan.  Two levels pay off when sequences are long and there are too few
// (sequence, head) pairs to fill the GPU: a chain of n chunks becomes about
// 2*seg + n/seg dependent steps for three times the work.  Only host-side
// sizes are known here, so the average sequence length decides.
int fixup_segment(int T_total, int N, int H, int chunk) {
  const int64_t avg_chunks = (static_cast<int64_t>(T_total) + static_cast<int64_t>(N) * chunk - 1) /
                             (static_cast<int64_t>(N) * chunk);
  if (avg_chunks < 256 || static_cast<int64_t>(N) * H > 64) return 0;
  int seg = 16;
  while (seg < 64 && static_cast<int64_t>(seg) * seg * 4 <= avg_chunks) seg *= 2;
  return seg;
}

struct SegSizes {
  int seg = 0, max_segs = 0;
  size_t state_bytes = 0;  // bytes of one [max_segs, H, d, d] fp32 buffer
};

SegSizes seg_sizes(int T_total, int N, int H, int d, int chunk, int max_chunks) {
  SegSizes z;
  z.seg = fixup_segment(T_total, N, H, chunk);
  if (z.seg > 0) {
    z.max_segs = max_chunks / z.seg + N;
    z.state_bytes = static_cast<size_t>(z.max_segs) * H * d * d * sizeof(float);
  }
  return z;
}

size_t seg_workspace(const SegSizes& z, int N) {
  if (z.seg == 0) return 0;
  return align_up(sizeof(int32_t) * (static_cast<size_t>(N) + 1)) +
         align_up(sizeof(int32_t) * 2 * static_cast<size_t>(z.max_segs)) + 3 * align_up(z.state_bytes);
}

size_t layout_workspace(int N, int mc) {
  return align_up(sizeof(int32_t) * (static_cast<size_t>(N) + 1)) +
         align_up(sizeof(int32_t) * 2 * static_cast<size_t>(mc));
}

size_t scan_workspace(int mc, int H, int chunk) {
  const gdr::ChunkFactorSizes z = gdr::chunk_factor_sizes(mc, H, chunk);
  return align_up(z.t) + align_up(z.p) + align_up(z.gate);
}

// Schedule of gdr_chunk_prefill.  The sequential scan (scan.hip) keeps every
// state in registers for a whole sequence and forms neither L, M nor the
// per-chunk states; it takes bf16 inputs and chunk 64.  For long sequences at
// low parallelism, where one dependent chain per (sequence, head) would leave
// the GPU idle, the segmented scan cuts every sequence into segments of whole
// chunks and runs two scan passes over all segments at once -- one carrying
// two state chains per segment (its local end state from zero, and its
// transfer matrix from the identity with v = 0), and the final pass from the
// true segment starts -- with the segment-level fixup of the chunk-parallel
// form between them.  When the caller asks for L or M, the
// chunk-local kernel writes them into the caller's buffers in parallel and
// the chain still runs in factored form (reading 25.6 KB of factors per
// chunk-head instead of L_c and M_c, 128 KiB).  The chunk-parallel form
// (chunk-local L and M, dense fixup, chunk outputs) serves fp32 inputs and
// chunk 16.
enum Schedule { kChunkParallel = 0, kScan = 1, kSegmentedScan = 2 };

Schedule schedule(int T_total, int N, int H, int chunk, int in_dtype) {
  if (in_dtype != GDR_BF16 || chunk != 64) return kChunkParallel;
  return fixup_segment(T_total, N, H, chunk) == 0 ? kScan : kSegmentedScan;
}

// Segment length (chunks) of the segmented scan: about 128 / (N H) segments
// per sequence, so that a pass runs about 256 workgroups (two per (segment,
// head)), and at least 16 chunks per segment.
int scan_segment(int T_total, int N, int H, int chunk) {
  const int64_t pairs = static_cast<int64_t>(N) * H;
  const int64_t avg_chunks = (static_cast<int64_t>(T_total) + static_cast<int64_t>(N) * chunk - 1) /
                             (static_cast<int64_t>(N) * chunk);
  int64_t per_seq = 128 / (pairs > 0 ? pairs : 1);
  if (per_seq < 2) per_seq = 2;
  int64_t seg = (avg_chunks + per_seq - 1) / per_seq;
  if (seg < 16) seg = 16;
  return static_cast<int>(seg);
}

struct SegScanSizes {
  int seg = 0, max_segs = 0;
  size_t state_bytes = 0;  // bytes of one [max_segs, H, d, d] fp32 buffer
};

SegScanSizes segscan_sizes(int T_total, int N, int H, int d, int chunk, int max_chunks) {
  SegScanSizes z;
  if (fixup_segment(T_total, N, H, chunk) == 0) return z;
  z.seg = scan_segment(T_total, N, H, chunk);
  z.max_segs = max_chunks / z.seg + N;
  z.state_bytes = static_cast<size_t>(z.max_segs) * H * d * d * sizeof(float);
  return z;
}

// segment offsets | segment indices | cu_seg | offs_seg | L | M | end | start
size_t segscan_workspace(const SegScanSizes& z, int N) {
  if (z.seg == 0) return 0;
  return align_up(sizeof(int32_t) * (static_cast<size_t>(N) + 1)) +
         align_up(sizeof(int32_t) * 2 * static_cast<size_t>(z.max_segs)) +
         2 * align_up(sizeof(int32_t) * (static_cast<size_t>(z.max_segs) + 1)) +
         4 * align_up(z.state_bytes);
}

// A failed launch, reported as "<entry point>: <phase>: <HIP error>".
gdr_status hip_fail(hipError_t e, const char* who, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GDR_ERR_HIP, "%s: %s: %s", who, what, hipGetErrorString(e));
}

}  // namespace

namespace gdr {

// Validation and dispatch of gdr_chunk_prefill.  `who` names the entry point
// in error messages; with static_scratch the workspace is the library's own
// scratch array, and a call that needs more than it holds is refused as
// unsupported.
gdr_status chunk_prefill(const char* who, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const int32_t* cu_seqlens, int N,
                         const float* state_in, float* state_out, void* o, float* L_out,
                         float* M_out, float* fixed_out, int T_total, int H, int dk, int dv,
                         int chunk, gdr_dtype in_dtype, gdr_dtype out_dtype, void* workspace,
                         size_t workspace_bytes, bool static_scratch, gdr_stream_t stream) {
  if (!cu_seqlens || !state_out) return fail(GDR_ERR_INVALID_ARG, "%s: NULL cu_seqlens/state_out", who);
  if (T_total > 0 && (!q || !k || !v || !g || !beta || !o))
    return fail(GDR_ERR_INVALID_ARG, "%s: NULL tensor pointer", who);
  if (T_total < 0 || N <= 0 || H <= 0)
    return fail(GDR_ERR_INVALID_ARG, "%s: T_total=%d N=%d H=%d", who, T_total, N, H);
  if (N > 65536 || H > 65535) return fail(GDR_ERR_INVALID_ARG, "%s: N or H too large", who);
  if (!supported_dims(dk, dv))
    return fail(GDR_ERR_UNSUPPORTED, "%s: (dk, dv) = (%d, %d) not in {(64,64), (128,128)}", who, dk, dv);
  if (chunk != 16 && chunk != 64)
    return fail(GDR_ERR_UNSUPPORTED, "%s: chunk=%d not in {16, 64}", who, chunk);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(GDR_ERR_UNSUPPORTED, "%s: dtype codes must be GDR_BF16 or GDR_FP32", who);
  const void* ptrs[] = {q, k, v, g, beta, state_in, state_out, o, L_out, M_out, fixed_out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", who);
  const int mc = gdr_max_chunks(T_total, N, chunk);
  if (mc < 0) return fail(GDR_ERR_INVALID_ARG, "%s: too many chunks", who);
  if (static_cast<int64_t>(T_total) * H > INT32_MAX || static_cast<int64_t>(mc) * H > INT32_MAX)
    return fail(GDR_ERR_INVALID_ARG, "%s: T_total*H too large", who);

  // workspace carve-up: offsets | indices | factors [| segments] (sequential
  // scan), or offsets | indices | [L] | [M] | [fixed] | [segments]
  // (chunk-parallel form)
  const Schedule sched = schedule(T_total, N, H, chunk, in_dtype);
  const bool scan = sched != kChunkParallel;
  const size_t per = static_cast<size_t>(mc) * H * sizeof(float);
  size_t need = layout_workspace(N, mc);
  SegSizes segz;
  SegScanSizes ssz;
  if (scan) {
    need += scan_workspace(mc, H, chunk);
    if (sched == kSegmentedScan) {
      ssz = segscan_sizes(T_total, N, H, dk, chunk, mc);
      need += segscan_workspace(ssz, N);
    }
  } else {
    if (!L_out) need += align_up(per * dv * dk);
    if (!M_out) need += align_up(per * dk * dk);
    if (!fixed_out) need += align_up(per * dv * dk);
    segz = seg_sizes(T_total, N, H, dk, chunk, mc);
    need += seg_workspace(segz, N);
  }
  if (static_scratch && need > workspace_bytes)
    return fail(GDR_ERR_UNSUPPORTED,
                "%s: this call needs %zu bytes of scratch and the library's static scratch holds "
                "%zu; call gdr_chunk_prefill with a workspace instead", who, need, workspace_bytes);
  if (!static_scratch && (workspace_bytes < need || (!workspace && need > 0)))
    return fail(GDR_ERR_INVALID_ARG, "%s: workspace of %zu bytes, need %zu", who, workspace_bytes, need);
  int dev = 0;
  gdr_status s = check_device(&dev);
  if (s != GDR_OK) return s;
  if (static_scratch) {
    s = static_scratch_address(dev, &workspace);
    if (s != GDR_OK) return s;
  }

  char* ws = static_cast<char*>(workspace);
  int32_t* offs = reinterpret_cast<int32_t*>(ws);
  ws += align_up(sizeof(int32_t) * (static_cast<size_t>(N) + 1));
  int32_t* cidx = reinterpret_cast<int32_t*>(ws);
  ws += align_up(sizeof(int32_t) * 2 * static_cast<size_t>(mc));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = gdr::launch_layout(cu_seqlens, N, chunk, offs, cidx, mc, st);
  if (e != hipSuccess) return hip_fail(e, who, "layout");

  if (scan) {
    const gdr::ChunkFactorSizes z = gdr::chunk_factor_sizes(mc, H, chunk);
    gdr::ChunkFactors f;
    f.t = reinterpret_cast<uint16_t*>(ws);
    ws += align_up(z.t);
    f.p = reinterpret_cast<uint16_t*>(ws);
    ws += align_up(z.p);
    f.gate = reinterpret_cast<float*>(ws);
    if (T_total > 0) {
      if (L_out || M_out) {  // requested local states and transfer matrices
        e = gdr::launch_chunk_local(k, v, g, beta, cu_seqlens, cidx, L_out, M_out, mc, T_total, H,
                                    dk, dv, chunk, in_dtype, st);
        if (e != hipSuccess) return hip_fail(e, who, "chunk_local");
      }
      e = gdr::launch_chunk_factors(q, k, g, beta, cu_seqlens, cidx, f, mc, T_total, H, dk, chunk,
                                    st);
      if (e != hipSuccess) return hip_fail(e, who, "chunk factors");
    }
    ws += align_up(z.gate);
    if (sched == kScan) {
      e = gdr::launch_chunk_scan(q, k, v, cu_seqlens, offs, f, state_in, state_out, fixed_out, o,
                                 N, H, dk, chunk, mc, T_total, out_dtype, st);
      return hip_fail(e, who, "chunk scan");
    }
    // segmented scan
    const int ms = ssz.max_segs;
    int32_t* seg_offs = reinterpret_cast<int32_t*>(ws);
    ws += align_up(sizeof(int32_t) * (static_cast<size_t>(N) + 1));
    int32_t* seg_idx = reinterpret_cast<int32_t*>(ws);
    ws += align_up(sizeof(int32_t) * 2 * static_cast<size_t>(ms));
    int32_t* cu_seg = reinterpret_cast<int32_t*>(ws);
    ws += align_up(sizeof(int32_t) * (static_cast<size_t>(ms) + 1));
    int32_t* offs_seg = reinterpret_cast<int32_t*>(ws);
    ws += align_up(sizeof(int32_t) * (static_cast<size_t>(ms) + 1));
    float* seg_L = reinterpret_cast<float*>(ws);
    ws += align_up(ssz.state_bytes);
    float* seg_M = reinterpret_cast<float*>(ws);
    ws += align_up(ssz.state_bytes);
    float* seg_end = reinterpret_cast<float*>(ws);
    ws += align_up(ssz.state_bytes);
    float* seg_start = reinterpret_cast<float*>(ws);
    e = gdr::launch_layout(offs, N, ssz.seg, seg_offs, seg_idx, ms, st);
    if (e == hipSuccess)
      e = gdr::launch_segment_ranges(cu_seqlens, offs, seg_idx, N, ssz.seg, chunk, ms, cu_seg,
                                     offs_seg, st);
    // local end state (from zero) and transfer matrix (identity start, v = 0)
    // of every segment, both chains in one pass
    if (e == hipSuccess)
      e = gdr::launch_chunk_scan_pair(k, v, cu_seg, offs_seg, f, nullptr, seg_L, seg_M, ms, H, dk,
                                      chunk, mc, T_total, st);
    // segment-level fixup: the end state of every segment
    if (e == hipSuccess)
      e = gdr::launch_fixup_mode(0, seg_L, seg_M, state_in, seg_offs, nullptr, 0, nullptr,
                                 seg_end, nullptr, ms, H, N, dk, 2, st);
    if (e == hipSuccess)
      e = gdr::launch_segment_starts(state_in, seg_end, seg_idx, ms, H, dk, seg_start, st);
    // outputs (and chunk-end states) from the true segment starts
    if (e == hipSuccess)
      e = gdr::launch_chunk_scan(q, k, v, cu_seg, offs_seg, f, seg_start, nullptr, fixed_out, o,
                                 ms, H, dk, chunk, mc, T_total, out_dtype, st);
    if (e != hipSuccess) return hip_fail(e, who, "segmented scan");
    e = gdr::launch_final_state(state_in, seg_end, seg_offs, N, H, dk, dv, ms, state_out, st);
    return hip_fail(e, who, "final state");
  }

  float* L = L_out;
  if (!L) { L = reinterpret_cast<float*>(ws); ws += align_up(per * dv * dk); }
  float* M = M_out;
  if (!M) { M = reinterpret_cast<float*>(ws); ws += align_up(per * dk * dk); }
  float* fixed = fixed_out;
  if (!fixed) { fixed = reinterpret_cast<float*>(ws); ws += align_up(per * dv * dk); }
  int32_t* seg_offs = nullptr;
  int32_t* seg_idx = nullptr;
  float *seg_L = nullptr, *seg_M = nullptr, *seg_fixed = nullptr;
  if (segz.seg > 0) {
    seg_offs = reinterpret_cast<int32_t*>(ws);
    ws += align_up(sizeof(int32_t) * (static_cast<size_t>(N) + 1));
    seg_idx = reinterpret_cast<int32_t*>(ws);
    ws += align_up(sizeof(int32_t) * 2 * static_cast<size_t>(segz.max_segs));
    seg_L = reinterpret_cast<float*>(ws);
    ws += align_up(segz.state_bytes);
    seg_M = reinterpret_cast<float*>(ws);
    ws += align_up(segz.state_bytes);
    seg_fixed = reinterpret_cast<float*>(ws);
    ws += align_up(segz.state_bytes);
  }

  if (T_total > 0) {
    e = gdr::launch_chunk_local(k, v, g, beta, cu_seqlens, cidx, L, M, mc, T_total, H, dk, dv,
                                chunk, in_dtype, st);
    if (e != hipSuccess) return hip_fail(e, who, "chunk_local");
    const int planes = in_dtype == GDR_BF16 ? 2 : 3;
    if (segz.seg == 0) {
      e = gdr::launch_fixup(L, M, state_in, offs, N, fixed, mc, H, dk, dv, planes, st);
      if (e != hipSuccess) return hip_fail(e, who, "fixup");
    } else {
      // two-level scan: segments of segz.seg chunks
      e = gdr::launch_layout(offs, N, segz.seg, seg_offs, seg_idx, segz.max_segs, st);
      if (e == hipSuccess)
        e = gdr::launch_fixup_mode(1, L, M, nullptr, offs, seg_idx, segz.seg, nullptr, seg_L,
                                   seg_M, mc, H, segz.max_segs, dk, planes, st);
      if (e == hipSuccess)
        e = gdr::launch_fixup_mode(0, seg_L, seg_M, state_in, seg_offs, nullptr, 0, nullptr,
                                   seg_fixed, nullptr, segz.max_segs, H, N, dk, planes, st);
      if (e == hipSuccess)
        e = gdr::launch_fixup_mode(2, L, M, state_in, offs, seg_idx, segz.seg, seg_fixed, fixed,
                                   nullptr, mc, H, segz.max_segs, dk, planes, st);
      if (e != hipSuccess) return hip_fail(e, who, "segmented fixup");
    }
    e = gdr::launch_chunk_out(q, k, v, g, beta, cu_seqlens, cidx, state_in, fixed, o, mc, T_total,
                              H, dk, dv, chunk, in_dtype, out_dtype, st);
    if (e != hipSuccess) return hip_fail(e, who, "chunk_out");
  }
  e = gdr::launch_final_state(state_in, fixed, offs, N, H, dk, dv, mc, state_out, st);
  return hip_fail(e, who, "final state");
}

}  // namespace gdr

extern "C" {

const char* gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
  }
  return "unknown gdr_status";
}

const char* gdr_last_error(void) { return g_last_error; }

gdr_status gdr_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, void* o, int N, int H, int dk, int dv,
                           gdr_dtype in_dtype, gdr_dtype out_dtype, gdr_stream_t stream) {
  if (!q || !k || !v || !g || !beta || !state || !o)
    return fail(GDR_ERR_INVALID_ARG, "gdr_decode_step: NULL tensor pointer");
  if (N <= 0 || H <= 0) return fail(GDR_ERR_INVALID_ARG, "gdr_decode_step: N=%d H=%d must be > 0", N, H);
  if (static_cast<int64_t>(N) * H > INT32_MAX)
    return fail(GDR_ERR_INVALID_ARG, "gdr_decode_step: N*H too large");
  if (!supported_dims(dk, dv))
    return fail(GDR_ERR_UNSUPPORTED, "gdr_decode_step: (dk, dv) = (%d, %d) not in {(64,64), (128,128)}", dk, dv);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(GDR_ERR_UNSUPPORTED, "gdr_decode_step: dtype codes must be GDR_BF16 or GDR_FP32");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) || !aligned16(o) ||
      !aligned16(g) || !aligned16(beta))
    return fail(GDR_ERR_INVALID_ARG, "gdr_decode_step: pointers must be 16-byte aligned");
  gdr_status s = check_device();
  if (s != GDR_OK) return s;
  return hip_status(gdr::launch_decode(q, k, v, g, beta, state, o, N * H, dk, dv, in_dtype,
                                       out_dtype, static_cast<hipStream_t>(stream)),
                    "gdr_decode_step launch");
}

gdr_status gdr_decode_mtp(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* state_in, float* state_out, void* o,
                          float* inter, int N, int T, int H, int dk, int dv, gdr_dtype in_dtype,
                          gdr_dtype out_dtype, gdr_stream_t stream) {
  if (!q || !k || !v || !g || !beta || !state_in || !o)
    return fail(GDR_ERR_INVALID_ARG, "gdr_decode_mtp: NULL tensor pointer");
  if (N <= 0 || H <= 0) return fail(GDR_ERR_INVALID_ARG, "gdr_decode_mtp: N=%d H=%d must be > 0", N, H);
  if (T < 1 || T > 64) return fail(GDR_ERR_INVALID_ARG, "gdr_decode_mtp: T=%d not in [1, 64]", T);
  if (static_cast<int64_t>(N) * H > INT32_MAX || static_cast<int64_t>(N) * T * H > INT32_MAX)
    return fail(GDR_ERR_INVALID_ARG, "gdr_decode_mtp: N*T*H too large");
  if (!supported_dims(dk, dv))
    return fail(GDR_ERR_UNSUPPORTED, "gdr_decode_mtp: (dk, dv) = (%d, %d) not in {(64,64), (128,128)}", dk, dv);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(GDR_ERR_UNSUPPORTED, "gdr_decode_mtp: dtype codes must be GDR_BF16 or GDR_FP32");
  const void* ptrs[] = {q, k, v, g, beta, state_in, state_out, o, inter};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "gdr_decode_mtp: pointers must be 16-byte aligned");
  gdr_status s = check_device();
  if (s != GDR_OK) return s;
  return hip_status(gdr::launch_mtp(q, k, v, g, beta, state_in, state_out, o, inter, N, T, H, dk,
                                    dv, in_dtype, out_dtype, static_cast<hipStream_t>(stream)),
                    "gdr_decode_mtp launch");
}

int gdr_max_chunks(int T_total, int N, int chunk) {
  if (T_total < 0 || N <= 0 || chunk <= 0) return -1;
  const int64_t m = static_cast<int64_t>(T_total) / chunk + N;
  return m > INT32_MAX ? -1 : static_cast<int>(m);
}

gdr_status gdr_chunk_layout(const int32_t* cu_seqlens, int N, int chunk, int32_t* chunk_offsets,
                            int32_t* chunk_indices, int max_chunks, gdr_stream_t stream) {
  if (!cu_seqlens || !chunk_offsets || (!chunk_indices && max_chunks > 0))
    return fail(GDR_ERR_INVALID_ARG, "gdr_chunk_layout: NULL pointer");
  if (N <= 0 || N > 65536) return fail(GDR_ERR_INVALID_ARG, "gdr_chunk_layout: N=%d not in [1, 65536]", N);
  if (chunk <= 0) return fail(GDR_ERR_INVALID_ARG, "gdr_chunk_layout: chunk=%d must be > 0", chunk);
  if (max_chunks < 0) return fail(GDR_ERR_INVALID_ARG, "gdr_chunk_layout: max_chunks < 0");
  gdr_status s = check_device();
  if (s != GDR_OK) return s;
  return hip_status(gdr::launch_layout(cu_seqlens, N, chunk, chunk_offsets, chunk_indices,
                                       max_chunks, static_cast<hipStream_t>(stream)),
                    "gdr_chunk_layout launch");
}

size_t gdr_chunk_prefill_workspace_bytes(int T_total, int N, int H, int dk, int dv, int chunk,
                                         gdr_dtype in_dtype) {
  const int mc = gdr_max_chunks(T_total, N, chunk);
  if (mc < 0 || H <= 0 || !supported_dims(dk, dv) || (chunk != 16 && chunk != 64) ||
      !valid_dtype(in_dtype))
    return 0;
  size_t cp = 0;
  const size_t per = static_cast<size_t>(mc) * H * sizeof(float);
  cp += align_up(per * dv * dk);  // L
  cp += align_up(per * dk * dk);  // M
  cp += align_up(per * dv * dk);  // fixed
  cp += seg_workspace(seg_sizes(T_total, N, H, dk, chunk, mc), N);
  // bf16 inputs at chunk 64 always take a scan schedule, the others the
  // chunk-parallel form
  if (schedule(T_total, N, H, chunk, in_dtype) != kChunkParallel)
    return layout_workspace(N, mc) + scan_workspace(mc, H, chunk) +
           segscan_workspace(segscan_sizes(T_total, N, H, dk, chunk, mc), N);
  return layout_workspace(N, mc) + cp;
}

gdr_status gdr_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int32_t* cu_seqlens, int N,
                             const float* state_in, float* state_out, void* o, float* L_out,
                             float* M_out, float* fixed_out, int T_total, int H, int dk, int dv,
                             int chunk, gdr_dtype in_dtype, gdr_dtype out_dtype, void* workspace,
                             size_t workspace_bytes, gdr_stream_t stream) {
  return gdr::chunk_prefill("gdr_chunk_prefill", q, k, v, g, beta, cu_seqlens, N, state_in,
                            state_out, o, L_out, M_out, fixed_out, T_total, H, dk, dv, chunk,
                            in_dtype, out_dtype, workspace, workspace_bytes, false, stream);
}

gdr_status gdr_state_fixup(const float* L, const float* M, const float* state_in,
                           const int32_t* chunk_offsets, int N, float* fixed, int n_chunks, int H,
                           int dk, int dv, gdr_stream_t stream) {
  if (!L || !M || !chunk_offsets || !fixed)
    return fail(GDR_ERR_INVALID_ARG, "gdr_state_fixup: NULL pointer");
  if (N <= 0 || N > 65536 || H <= 0 || H > 65535 || n_chunks < 0)
    return fail(GDR_ERR_INVALID_ARG, "gdr_state_fixup: N=%d H=%d n_chunks=%d", N, H, n_chunks);
  if (!supported_dims(dk, dv))
    return fail(GDR_ERR_UNSUPPORTED, "gdr_state_fixup: (dk, dv) = (%d, %d) not in {(64,64), (128,128)}", dk, dv);
  if (!aligned16(L) || !aligned16(M) || !aligned16(fixed) || (state_in && !aligned16(state_in)))
    return fail(GDR_ERR_INVALID_ARG, "gdr_state_fixup: pointers must be 16-byte aligned");
  gdr_status s = check_device();
  if (s != GDR_OK) return s;
  if (n_chunks == 0) return ok();
  return hip_status(gdr::launch_fixup(L, M, state_in, chunk_offsets, N, fixed, n_chunks, H, dk,
                                      dv, 3, static_cast<hipStream_t>(stream)),
                    "gdr_state_fixup launch");
}

}  // extern "C"
