// layout.hip -- varlen chunk layout (integer work, bit-exact).
//
// chunk_offsets[n+1] = chunk_offsets[n] + ceil(len_n / chunk) is a prefix sum
// over sequences; the chunk -> (sequence, index) table is filled in parallel,
// one thread per chunk slot, by a binary search in chunk_offsets.  Up to 1024
// sequences both happen in one launch (every workgroup scans in LDS); beyond
// that one workgroup scans in tiles of 1024 sequences and a second launch
// fills the table.  Slots past the real chunk
// count get (-1, -1).  Lengths are clamped to >= 0 and every derived index to
// the buffer sizes, so malformed cu_seqlens cannot cause out-of-bounds writes.
#include "gdr_device.h"
#include "launch.h"

namespace gdr {
namespace {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void chunk_offsets_kernel(
    const int32_t* __restrict__ cu, int N, int chunk, int32_t* __restrict__ offs) {
  __shared__ int32_t buf[kScanThreads];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry = 0;
    offs[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < N; base += kScanThreads) {
    const int n = base + tid;
    int cnt = 0;
    if (n < N) {
      const int len = cu[n + 1] - cu[n];
      cnt = len > 0 ? (len + chunk - 1) / chunk : 0;
    }
    buf[tid] = cnt;
    __syncthreads();
    // Hillis-Steele inclusive scan
    for (int d = 1; d < kScanThreads; d <<= 1) {
      const int add = tid >= d ? buf[tid - d] : 0;
      __syncthreads();
      buf[tid] += add;
      __syncthreads();
    }
    if (n < N) offs[n + 1] = carry + buf[tid];
    __syncthreads();
    if (tid == kScanThreads - 1) carry += buf[tid];
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void chunk_indices_kernel(const int32_t* __restrict__ offs,
                                                            int N, int32_t* __restrict__ idx,
                                                            int max_chunks) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= max_chunks) return;
  const int total = offs[N];
  int n = -1, j = -1;
  if (c < total) {
    // largest n in [0, N) with offs[n] <= c
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offs[mid] <= c) lo = mid; else hi = mid - 1;
    }
    n = lo;
    j = c - offs[lo];
  }
  idx[2 * c + 0] = n;
  idx[2 * c + 1] = j;
}

// Both tables in one launch for N <= kFusedMaxN sequences: every workgroup
// loads cu_seqlens into LDS, forms the chunk counts and their prefix sum there
// (four entries per thread, then a scan of the 256 partial sums), and fills its
// 256 chunk slots by a binary search in LDS; workgroup 0 also writes
// chunk_offsets.  Saves a launch and the dependent global reads of the search.
constexpr int kFusedThreads = 256;
constexpr int kFusedMaxN = 4 * kFusedThreads;

__global__ __launch_bounds__(kFusedThreads) void chunk_layout_kernel(
    const int32_t* __restrict__ cu, int N, int chunk, int32_t* __restrict__ offs,
    int32_t* __restrict__ idx, int max_chunks) {
  __shared__ int32_t so[kFusedMaxN + 1];
  __shared__ int32_t part[kFusedThreads];
  const int tid = threadIdx.x;
  // chunk counts of this thread's four sequences, and their running sums
  int local[4], run = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int n = 4 * tid + e;
    int cnt = 0;
    if (n < N) {
      const int len = cu[n + 1] - cu[n];
      cnt = len > 0 ? (len + chunk - 1) / chunk : 0;
    }
    run += cnt;
    local[e] = run;
  }
  part[tid] = run;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread totals
  for (int d = 1; d < kFusedThreads; d <<= 1) {
    const int add = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const int before = tid > 0 ? part[tid - 1] : 0;
  if (tid == 0) so[0] = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int n = 4 * tid + e;
    if (n < N) so[n + 1] = before + local[e];
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int n = tid; n <= N; n += kFusedThreads) offs[n] = so[n];
  const int c = blockIdx.x * kFusedThreads + tid;
  if (c >= max_chunks) return;
  const int total = so[N];
  int n = -1, j = -1;
  if (c < total) {
    // largest n in [0, N) with so[n] <= c
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (so[mid] <= c) lo = mid; else hi = mid - 1;
    }
    n = lo;
    j = c - so[lo];
  }
  idx[2 * c + 0] = n;
  idx[2 * c + 1] = j;
}

}  // namespace

hipError_t launch_layout(const int32_t* cu_seqlens, int N, int chunk, int32_t* chunk_offsets,
                         int32_t* chunk_indices, int max_chunks, hipStream_t stream) {
  if (N <= kFusedMaxN && max_chunks > 0) {
    hipLaunchKernelGGL(chunk_layout_kernel, dim3((max_chunks + kFusedThreads - 1) / kFusedThreads),
                       dim3(kFusedThreads), 0, stream, cu_seqlens, N, chunk, chunk_offsets,
                       chunk_indices, max_chunks);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(kScanThreads), 0, stream, cu_seqlens, N,
                     chunk, chunk_offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_chunks <= 0) return e;
  hipLaunchKernelGGL(chunk_indices_kernel, dim3((max_chunks + 255) / 256), dim3(256), 0, stream,
                     chunk_offsets, N, chunk_indices, max_chunks);
  return hipGetLastError();
}

}  // namespace gdr
