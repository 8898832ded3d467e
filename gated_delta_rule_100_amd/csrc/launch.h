// launch.h -- host-side launchers of the gfx950 kernels (internal to libgdr).
// Every launcher assumes its arguments were validated by the C ABI layer and
// returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

// One decode token for NH = N*H states, in place.
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float* state, void* o, int NH, int dk, int dv,
                         int in_dtype, int out_dtype, hipStream_t stream);

// T decode tokens per (sequence, head): state_in read once, state_out (may be
// state_in, or NULL) written once, `inter` (or NULL) gets the state after every
// token.
hipError_t launch_mtp(const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* state_in, float* state_out, void* o,
                      float* inter, int N, int T, int H, int dk, int dv, int in_dtype,
                      int out_dtype, hipStream_t stream);

// Varlen layout: chunk_offsets [N+1], chunk_indices [max_chunks, 2].
hipError_t launch_layout(const int32_t* cu_seqlens, int N, int chunk, int32_t* chunk_offsets,
                         int32_t* chunk_indices, int max_chunks, hipStream_t stream);

// Inter-chunk fixup: fixed[c] = fixed[c-1] M_c + L_c per (sequence, head),
// with M_c[a][b] at row a, column b of its slot.  planes = 2 or 3: the state
// and M are carried as that many bf16 planes on the matrix cores (3 keeps fp32
// precision).
hipError_t launch_fixup(const float* L, const float* M, const float* state_in,
                        const int32_t* chunk_offsets, int N, float* fixed, int n_chunks, int H,
                        int dk, int dv, int planes, hipStream_t stream);

// Fixup variants over units (sequences or segments of `seg` chunks); see
// fixup.hip.  mode 0: per-sequence scan writing every chunk state to `out`;
// mode 1: per-segment local state (out) and transfer product (out_m); mode 2:
// per-segment scan from the scanned segment starts (seg_start) writing every
// chunk state to `out`.
hipError_t launch_fixup_mode(int mode, const float* L, const float* M, const float* state_in,
                             const int32_t* offs, const int32_t* seg_idx, int seg,
                             const float* seg_start, float* out, float* out_m, int n_chunks,
                             int H, int n_units, int dk, int planes, hipStream_t stream);

// Chunk-local precompute: L_c and M_c for every chunk slot < max_chunks (L or
// M may be NULL: not stored).
hipError_t launch_chunk_local(const void* k, const void* v, const float* g, const float* beta,
                              const int32_t* cu_seqlens, const int32_t* chunk_indices,
                              float* L, float* M, int max_chunks, int T_total, int H, int dk,
                              int dv, int chunk, int in_dtype, hipStream_t stream);

// Chunk outputs from the fixed states (start state of chunk j of sequence n is
// fixed[c-1] for j > 0 and state_in[n] (or zero) for j = 0).
hipError_t launch_chunk_out(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens,
                            const int32_t* chunk_indices, const float* state_in,
                            const float* fixed, void* o, int max_chunks, int T_total, int H,
                            int dk, int dv, int chunk, int in_dtype, int out_dtype,
                            hipStream_t stream);

// Final states: state_out[n] = fixed[last chunk of n], or state_in[n] (zero
// without one) for an empty sequence.
hipError_t launch_final_state(const float* state_in, const float* fixed,
                              const int32_t* chunk_offsets, int N, int H, int dk, int dv,
                              int n_chunks, float* state_out, hipStream_t stream);

// Per-chunk factors of the sequential schedule, one slot per (chunk slot,
// head) (C = chunk = 64).  T and P are lower triangular and stored compactly:
// rows t < C/2 keep their first C/2 columns, rows t >= C/2 all C (TL = 3 C^2 / 4
// elements per plane); P rows store their contraction index in operand-slot
// order (chunk.hip):
//   t     [slots][H][TL]      kTScale T, T = (I + A)^{-1}, as one fp16 plane
//   p     [slots][H][TL]      kPScale P, P = (Q K^T) (.) Gamma (s <= t), as one
//                             fp16 plane
//   gate  [slots][H][4][C]    gamma_t, D_t, beta_t / kTScale and zeros, fp32
// The scan forms U = T diag(beta) R as (kTScale T)(diag(beta / kTScale) R)
// and P U as (kPScale P)(U / kPScale), exactly the same products: the
// power-of-two scales move the fp16 range of the R and U planes up by 16
// (fp16 holds T with its unit diagonal exactly and its other entries, and P,
// to 11 bits).
constexpr float kTScale = 16.f;
constexpr float kPScale = 16.f;
struct ChunkFactors {
  uint16_t* t;
  uint16_t* p;
  float* gate;
};

// Bytes of each ChunkFactors array for `slots` chunk slots (host helper).
struct ChunkFactorSizes {
  size_t t, p, gate;
};
inline ChunkFactorSizes chunk_factor_sizes(int slots, int H, int chunk) {
  const size_t n = static_cast<size_t>(slots) * H;
  const size_t c = static_cast<size_t>(chunk);
  const size_t tl = 3 * c * c / 4;
  return {n * tl * 2, n * tl * 2, n * 4 * c * 4};
}

// Factors of every chunk slot < max_chunks (bf16 inputs, chunk 64).
hipError_t launch_chunk_factors(const void* q, const void* k, const float* g, const float* beta,
                                const int32_t* cu_seqlens, const int32_t* chunk_indices,
                                const ChunkFactors& f, int max_chunks, int T_total, int H, int d,
                                int chunk, hipStream_t stream);

// Sequential scan over the chunks of every sequence from the factors and the
// q, k, v inputs: outputs o (skipped when o is NULL), final states (skipped
// when state_out is NULL), and (when fixed != NULL) the state at every chunk
// end.
hipError_t launch_chunk_scan(const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, const int32_t* chunk_offsets,
                             const ChunkFactors& f, const float* state_in, float* state_out,
                             float* fixed, void* o, int N, int H, int d, int chunk, int n_slots,
                             int T_total, int out_dtype, hipStream_t stream);

// The scan without outputs carrying two state chains per (sequence, head):
// the first from state_in (zero when NULL) with v, whose end state goes to
// state_out, and one from the identity with v = 0, whose end state -- the
// transfer matrix of the sequence's chunks -- goes to transfer_out (d = dk =
// dv).  Both read the same chunk data once.
hipError_t launch_chunk_scan_pair(const void* k, const void* v, const int32_t* cu_seqlens,
                                  const int32_t* chunk_offsets, const ChunkFactors& f,
                                  const float* state_in, float* state_out, float* transfer_out,
                                  int N, int H, int d, int chunk, int n_slots, int T_total,
                                  hipStream_t stream);

// Segments of a chunk-parallel layout as pseudo-sequences for the scan: for
// every segment slot m < max_segs with seg_idx[m] = (n, j), tokens
// [cu_seg[m], cu_seg[m+1]) and chunk slots [offs_seg[m], offs_seg[m+1]) are
// chunks j*seg .. of sequence n; slots past the real count are empty.
hipError_t launch_segment_ranges(const int32_t* cu_seqlens, const int32_t* chunk_offsets,
                                 const int32_t* seg_idx, int N, int seg, int chunk, int max_segs,
                                 int32_t* cu_seg, int32_t* offs_seg, hipStream_t stream);

// Start state of every segment: the sequence's state_in (zero when NULL) for
// its first segment, else the end state of the previous segment.
hipError_t launch_segment_starts(const float* state_in, const float* seg_end,
                                 const int32_t* seg_idx, int max_segs, int H, int d,
                                 float* seg_start, hipStream_t stream);

}  // namespace gdr
