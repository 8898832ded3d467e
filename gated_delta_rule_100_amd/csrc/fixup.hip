// fixup.hip -- inter-chunk state fixup and final-state copy on gfx950.
//
// fixed[c] = fixed[c-1] M_c + L_c is a chain of dependent matrix products per
// (sequence, head) (the fixup of the FlashInfer PR #3866 page, "CP delta-rule
// precompute optimisation for ultra-low parallelism", code changes 2: the
// state multiplies M_c from the left, accumulate_state_fragment).  Row i of
// the new state only needs row i of the previous one, so the work is split
// over workgroups of state rows; each walks its sequence's chunks in order.
#include "launch.h"
#include "mfma_planes.h"

namespace gdr {
namespace {

// Matrix-core fixup: ROWS state rows per workgroup (16, 32 or 64: one to four
// 16-row MFMA tiles) and one wave per 16-wide output column tile (8 waves at
// d = 128).  Per chunk:
// S' = S M_c + L_c with S as bf16 planes in LDS (double-buffered, so one
// barrier per chunk).  Lane (c, g) of the B operand holds
// M[32kb + 8g .. 8g+7][16w + c]: eight loads, each of which reads 64
// contiguous bytes of a row of M_c across the 16 lanes of a group, issued
// while the previous chunk is multiplied.  L is loaded in the output layout.
// Workgroups of one unit (and head) are placed on one XCD (dispatch is
// round-robin over the 8 XCDs by workgroup id), so M_c is fetched from HBM
// once and served to all of them from L2.
//
// Each chunk costs every workgroup a full M_c from L2, so a long chain is
// bound by that per-step transfer; long sequences therefore use a two-level
// scan over segments of `seg` chunks (the segment-size heuristic plays the
// role of the CP chunking heuristic on the FlashInfer PR #3866 page, code
// changes 3):
//   kSeq      units are sequences; fixed[c] for every chunk;
//   kCompose  units are segments; rows 0..D-1 run from a zero state and give
//             the segment's local state L_s (written once), rows D..2D-1 start
//             from the identity without L and give the segment's transfer
//             M_s = M_c0 M_c1 ... (its rows are the rows of that state);
//   kApply    units are segments; the start state is the previous segment's
//             scanned state (or the sequence's initial state) and fixed[c] is
//             written for every chunk.
// The scan over segments is kSeq on (L_s, M_s).
constexpr int kXcds = 8;
enum FixMode { kSeq = 0, kCompose = 1, kApply = 2 };

template <int D, int P, int MODE, int ROWS>
__global__ __launch_bounds__(D * 4) void fixup_mfma_kernel(
    const float* __restrict__ L, const float* __restrict__ M, const float* __restrict__ state_in,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ seg_idx, int seg,
    const float* __restrict__ seg_start, float* __restrict__ out, float* __restrict__ out_m,
    int n_chunks, int H, int n_units) {
  constexpr int NTHR = D * 4;       // one wave per 16 output columns
  constexpr int RT = ROWS / 16;     // 16-row MFMA tiles per workgroup
  constexpr int RB = D / ROWS;      // row blocks (workgroups) per state
  constexpr int RBU = MODE == kCompose ? 2 * RB : RB;  // row blocks per unit
  constexpr int KB = D / 32;        // 32-deep contraction blocks
  constexpr int LDS_LD = D + 8;     // row stride of the state planes (bf16 elements)
  constexpr int PS = ROWS * LDS_LD; // plane stride
  __shared__ __align__(16) uint16_t s_planes[2][P * PS];

  // XCD-aware placement of (unit x head, row block)
  const int b = blockIdx.x;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int pair = xcd + kXcds * (slot / RBU);
  const int rbu = slot % RBU;
  if (pair >= n_units * H) return;
  const int u = pair / H, h = pair % H;
  const bool trans_rows = MODE == kCompose && rbu >= RB;  // transfer-product rows
  const int row0 = (rbu % RB) * ROWS;

  int n, c_begin, c_end, sidx = 0;
  if (MODE == kSeq) {
    n = u;
    c_begin = offs[n];
    c_end = offs[n + 1];
  } else {
    n = seg_idx[2 * u];
    sidx = seg_idx[2 * u + 1];
    if (n < 0 || sidx < 0) return;
    c_begin = offs[n] + sidx * seg;
    c_end = offs[n + 1];
    c_end = c_end < c_begin + seg ? c_end : c_begin + seg;
  }
  c_end = c_end < n_chunks ? c_end : n_chunks;
  c_begin = c_begin < 0 ? 0 : c_begin;
  if (c_begin >= c_end) return;

  const int tid = threadIdx.x, wave = tid >> 6;
  const int c16 = tid & 15, g4 = (tid & 63) >> 4;
  const int col = 16 * wave + c16;
  auto st_at = [&](int c, int i, int cc) -> size_t {  // element (row0+i, cc) of a state slot
    return ((static_cast<size_t>(c) * H + h) * D + row0 + i) * D + cc;
  };

  // Start rows -> planes (buffer 0).
  const float* init = nullptr;  // start state rows, or nullptr for "first local state"
  if (MODE == kSeq) {
    if (state_in != nullptr) init = state_in + (static_cast<size_t>(n) * H + h) * D * D;
  } else if (MODE == kApply) {
    if (sidx > 0) init = seg_start + (static_cast<size_t>(u - 1) * H + h) * D * D;
    else if (state_in != nullptr) init = state_in + (static_cast<size_t>(n) * H + h) * D * D;
  }
  const bool from_L = !trans_rows && init == nullptr;
  int start = from_L ? c_begin + 1 : c_begin;
  for (int idx = tid; idx < ROWS * D; idx += NTHR) {
    const int i = idx / D, cc = idx % D;
    float x;
    if (trans_rows) {
      x = (row0 + i == cc) ? 1.f : 0.f;
    } else if (init != nullptr) {
      x = init[static_cast<size_t>(row0 + i) * D + cc];
    } else {
      x = L[st_at(c_begin, i, cc)];
      if (MODE != kCompose) out[st_at(c_begin, i, cc)] = x;
    }
    uint16_t sp[P];
    split_planes<P>(x, sp);
#pragma unroll
    for (int p = 0; p < P; ++p) s_planes[0][p * PS + i * LDS_LD + cc] = sp[p];
  }
  __syncthreads();

  typedef float MRaw[KB][8];
  typedef float LRaw[RT][4];
  // Loads are unconditional (a chunk past the end re-reads the last one).
  auto fetch = [&](int c, MRaw& m, LRaw& l) {
    c = c < c_end ? c : c_end - 1;
    const float* src = M + (static_cast<size_t>(c) * H + h) * D * D +
                       static_cast<size_t>(8 * g4) * D + col;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) m[kb][j] = src[static_cast<size_t>(32 * kb + j) * D];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        l[r][e] = trans_rows ? 0.f : L[st_at(c, 16 * r + 4 * g4 + e, col)];
  };

  // Raw operands run two chunks ahead: the loads of chunk c+2 are issued at
  // the top of step c (into the registers chunk c's operands were loaded into,
  // already converted), and chunk c+1's, loaded during step c-1, become
  // planes at the end of step c, after the barrier.  Loaded registers never
  // cross a loop back-edge unconverted, so nothing waits for a load early.
  MRaw ma, mb_raw;
  LRaw la, lb;
  bf16x8 mb[KB][P];
  float lc[RT][4];
  auto convert = [&](const MRaw& m, const LRaw& l) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) split8<P>(m[kb], mb[kb]);
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) lc[r][e] = l[r][e];
  };
  fetch(start, ma, la);
  fetch(start + 1, mb_raw, lb);
  convert(ma, la);
  int buf = 0;
  float last[RT][4] = {};
  // One chunk step: S' = S M_c + L_c from the planes of buffer `buf`; mf, lf
  // receive chunk c+2's operands, mc, lcr (chunk c+1's) are converted last.
  auto step = [&](int c, MRaw& mf, LRaw& lf, const MRaw& mc, const LRaw& lcr) {
    fetch(c + 2, mf, lf);

    // S' tiles = S M_c: two accumulators per tile (even / odd k blocks) keep
    // the dependent MFMA chains short.
    floatx4 acc[RT][2];
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r][0] = acc[r][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* cur = s_planes[buf];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        bf16x8 sa[P];
        load_lds8<P>(cur + (16 * r + c16) * LDS_LD + 32 * kb + 8 * g4, PS, sa);
        mma_planes<P, P>(acc[r][kb & 1], sa, mb[kb]);
      }
    }
    uint16_t* nxt = s_planes[buf ^ 1];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * r + 4 * g4 + e;
        const float x = (acc[r][0][e] + acc[r][1][e]) + lc[r][e];
        last[r][e] = x;
        if (MODE != kCompose) out[st_at(c, row, col)] = x;
        uint16_t sp[P];
        split_planes<P>(x, sp);
#pragma unroll
        for (int p = 0; p < P; ++p) nxt[p * PS + row * LDS_LD + col] = sp[p];
      }
    }
    buf ^= 1;
    // The new rows are in LDS for every wave; global loads (the next chunks'
    // operands) and stores (fixed[c]) stay in flight: __syncthreads() would
    // drain them and expose a memory round trip per chunk.
    lds_barrier();
    convert(mc, lcr);
  };
  for (int c = start; c < c_end; c += 2) {
    step(c, ma, la, mb_raw, lb);
    if (c + 1 < c_end) step(c + 1, mb_raw, lb, ma, la);
  }

  if (MODE == kCompose) {
    // Final rows of the segment: L_s or M_s, both in state layout.
    if (start >= c_end) {  // a one-chunk segment without transfer rows: L_s = L of that chunk
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) last[r][e] = L[st_at(c_begin, 16 * r + 4 * g4 + e, col)];
    }
    float* dst = (trans_rows ? out_m : out) + (static_cast<size_t>(u) * H + h) * D * D;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = row0 + 16 * r + 4 * g4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[static_cast<size_t>(row + e) * D + col] = last[r][e];
    }
  }
}

// One state per (blockIdx.x, all blockIdx.y): blockIdx.y picks a slice of
// kFinalSlices of the state, so that a few states still spread over many
// compute units.
constexpr int kFinalSlices = 16;

__global__ __launch_bounds__(256) void final_state_kernel(const float* __restrict__ state_in,
                                                          const float* __restrict__ fixed,
                                                          const int32_t* __restrict__ offs,
                                                          int H, int elems, int n_chunks,
                                                          float* state_out) {
  const int pair = blockIdx.x;  // n * H + h
  const int n = pair / H;
  const int h = pair % H;
  int c_end = offs[n + 1];
  int c_begin = offs[n];
  c_end = c_end < n_chunks ? c_end : n_chunks;
  c_begin = c_begin < 0 ? 0 : c_begin;
  const float* src = nullptr;
  if (c_begin < c_end) {
    src = fixed + (static_cast<size_t>(c_end - 1) * H + h) * elems;
  } else if (state_in != nullptr) {
    src = state_in + static_cast<size_t>(pair) * elems;
  }
  float4* dst = reinterpret_cast<float4*>(state_out + static_cast<size_t>(pair) * elems);
  if (src == reinterpret_cast<const float*>(dst)) return;  // in place, nothing to move
  const int per = elems / 4 / kFinalSlices;  // float4 per slice (elems is a multiple of 4096)
  for (int e = blockIdx.y * per + threadIdx.x; e < (blockIdx.y + 1) * per; e += blockDim.x)
    dst[e] = src ? reinterpret_cast<const float4*>(src)[e] : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_fixup_mode(int mode, const float* L, const float* M, const float* state_in,
                             const int32_t* offs, const int32_t* seg_idx, int seg,
                             const float* seg_start, float* out, float* out_m, int n_chunks,
                             int H, int n_units, int dk, int planes, hipStream_t stream) {
  if (n_units <= 0) return hipSuccess;
  const int pairs = n_units * H;
  // Every workgroup moves a whole M_c from L2 into its CU per chunk, so more
  // rows per workgroup means less traffic per row; take the most rows that
  // still give every CU a workgroup.
  const int copies = mode == kCompose ? 2 : 1;
  int rows = 16;
  while (rows < 64 && rows < dk && static_cast<int64_t>(pairs) * copies * (dk / (2 * rows)) >= 256)
    rows *= 2;
  const int rbu = (dk / rows) * copies;
  const dim3 grid(kXcds * ((pairs + kXcds - 1) / kXcds) * rbu);
#define GDR_FIX_R(D_, P_, M_, R_)                                                               \
  hipLaunchKernelGGL((fixup_mfma_kernel<D_, P_, M_, R_>), grid, dim3(D_ * 4), 0, stream, L, M,   \
                     state_in, offs, seg_idx, seg, seg_start, out, out_m, n_chunks, H, n_units)
#define GDR_FIX(D_, P_, M_)                                                                     \
  do {                                                                                          \
    if (rows == 64) GDR_FIX_R(D_, P_, M_, 64);                                                  \
    else if (rows == 32) GDR_FIX_R(D_, P_, M_, 32);                                             \
    else GDR_FIX_R(D_, P_, M_, 16);                                                             \
  } while (0)
#define GDR_FIX_P(D_, M_)                                                                       \
  do {                                                                                          \
    if (planes == 2) GDR_FIX(D_, 2, M_); else GDR_FIX(D_, 3, M_);                               \
  } while (0)
#define GDR_FIX_M(D_)                                                                           \
  do {                                                                                          \
    if (mode == kSeq) GDR_FIX_P(D_, kSeq);                                                      \
    else if (mode == kCompose) GDR_FIX_P(D_, kCompose);                                         \
    else GDR_FIX_P(D_, kApply);                                                                 \
  } while (0)
  if (dk == 128) GDR_FIX_M(128); else GDR_FIX_M(64);
#undef GDR_FIX_M
#undef GDR_FIX_P
#undef GDR_FIX
#undef GDR_FIX_R
  return hipGetLastError();
}

hipError_t launch_fixup(const float* L, const float* M, const float* state_in,
                        const int32_t* chunk_offsets, int N, float* fixed, int n_chunks, int H,
                        int dk, int dv, int planes, hipStream_t stream) {
  (void)dv;
  return launch_fixup_mode(kSeq, L, M, state_in, chunk_offsets, nullptr, 0, nullptr, fixed,
                           nullptr, n_chunks, H, N, dk, planes, stream);
}

hipError_t launch_final_state(const float* state_in, const float* fixed,
                              const int32_t* chunk_offsets, int N, int H, int dk, int dv,
                              int n_chunks, float* state_out, hipStream_t stream) {
  hipLaunchKernelGGL(final_state_kernel, dim3(N * H, kFinalSlices), dim3(256), 0, stream,
                     state_in, fixed, chunk_offsets, H, dk * dv, n_chunks, state_out);
  return hipGetLastError();
}

}  // namespace gdr
