/*
 * gdr.h -- C ABI of libgdr: the gated delta rule on AMD Instinct MI355X (gfx950).
 *
 * The method.  For each sequence and head a state S (dv rows x dk columns,
 * fp32, dk contiguous) evolves token by token as
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t                      (the state after the update)
 *     alpha_t = exp(g_t)
 *
 * (the gated delta rule of GDN-style linear attention).  Two forms are
 * provided: a one-token decode step that updates the state in place, and a
 * chunked ("CP", chunk-parallel) prefill over packed variable-length
 * sequences.  The chunked form follows the structure described on the
 * FlashInfer PR #3866 page ("CP delta-rule precompute optimisation for
 * ultra-low parallelism"): every chunk c gets a local state L_c and a
 * transfer matrix M_c in parallel, then a sequential fixup
 *     fixed[c] = fixed[c-1] * M_c + L_c
 * produces the state at the end of each chunk (section "code changes 2",
 * accumulate_state_fragment: the state multiplies M from the left;
 * init_state_tile: with an initial state the scan starts at chunk 0, without
 * one the first fixed state is L_0 and the scan starts at chunk 1), and the
 * outputs of chunk c are computed from fixed[c-1].
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller, dense
 *     row-major (C order), 16-byte aligned.  The library never allocates,
 *     frees or synchronises; work is enqueued on `stream` (a hipStream_t,
 *     NULL = the default stream) and buffers must stay alive until the stream
 *     has passed the call.  No call reads a host copy of device data, so every
 *     call may be captured in a HIP graph.
 *   - Validation happens on the host before any launch.  A failing check
 *     returns GDR_ERR_INVALID_ARG or GDR_ERR_UNSUPPORTED, launches nothing and
 *     writes nothing; gdr_last_error() then holds a message (per thread).
 *     A failed launch returns GDR_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Device-side integer inputs (cu_seqlens, chunk_offsets) are not
 *     inspected on the host (that would need a synchronisation).  They must be
 *     non-decreasing, start at 0 and end at T_total (resp. the chunk count);
 *     kernels clamp every index they derive from them to the buffer sizes
 *     given, so bad values give wrong results but no out-of-bounds access.
 *   - Supported shapes: (dk, dv) in {(64, 64), (128, 128)}; chunk in {16, 64}.
 *   - Dtypes: q, k, v are bf16 or fp32 (in_dtype); o is bf16 or fp32
 *     (out_dtype; bf16 is round-to-nearest-even of the fp32 result).  g, beta,
 *     states, L, M and fixed states are always fp32.
 *   - Calls are thread-safe.  The only global state is a per-device property
 *     cache filled on first use.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = 1, /* NULL pointer, misalignment, bad size */
  GDR_ERR_UNSUPPORTED = 2, /* shape or dtype outside the supported set */
  GDR_ERR_HIP = 3          /* a HIP runtime call or launch failed */
} gdr_status;

typedef enum { GDR_BF16 = 0, GDR_FP32 = 1 } gdr_dtype;

/* hipStream_t, kept opaque so that this header needs no HIP headers. */
typedef void* gdr_stream_t;

/*
 * gdr_decode_step -- one token of the recurrence for N independent
 * (sequence, head) states, updated IN PLACE.
 *
 * The decode step is the recurrence above with T = 1.  Its kernel streams
 * each fp32 state row straight from HBM into registers with 16-byte loads and
 * back, with no LDS staging: the state has no reuse (the FlashInfer PR #7156
 * page, "Cake GDP kernel optimisation: less shared memory, direct register
 * loads", code analysis 1, describes the same change for a split-V T=1 step).
 *
 *   q, k      [N, H, dk]      in_dtype
 *   v         [N, H, dv]      in_dtype
 *   g, beta   [N, H]          fp32; alpha = exp(g); g and beta are used as
 *                             given (no clamping)
 *   state     [N, H, dv, dk]  fp32, read and overwritten with S_t
 *   o         [N, H, dv]      out_dtype, o = S_t q
 *   N, H      > 0
 * q, k, v, g, beta and o must not overlap `state`.
 */
gdr_status gdr_decode_step(const void* q, const void* k, const void* v,
                           const float* g, const float* beta,
                           float* state, void* o,
                           int N, int H, int dk, int dv,
                           gdr_dtype in_dtype, gdr_dtype out_dtype,
                           gdr_stream_t stream);

/*
 * gdr_decode_mtp -- T decode tokens for each of N x H (sequence, head) states
 * (multi-token decode, e.g. verifying T draft tokens).
 *
 * The FlashInfer PR #7156 page ("Cake GDP kernel optimisation: less shared
 * memory, direct register loads", introduction) optimises the T = 1 variant of
 * a multi-token ("MTP") decode kernel; this entry point is the general T.
 * Token t of sequence n applies the recurrence to the state after token t-1
 * (state_in for t = 0), and its output uses the updated state.  The result is
 * that of gdr_chunk_prefill over N packed sequences of T tokens, and T = 1 is
 * gdr_decode_step (bit for bit).  The state is read once and written once
 * whatever T is.  Without `inter`, T >= 2 tokens are applied in chunks of 8
 * (the last may be shorter) of the chunked form on the matrix cores, other T
 * token by token; the two agree to rounding (1e-3 for bf16 inputs, 1e-5 for
 * fp32 inputs, against the token-by-token recurrence), and each is
 * deterministic.
 *
 *   q, k       [N, T, H, dk]     in_dtype (row n*T + t is token t of sequence n)
 *   v          [N, T, H, dv]     in_dtype
 *   g, beta    [N, T, H]         fp32; alpha = exp(g), used as given
 *   state_in   [N, H, dv, dk]    fp32 input states
 *   state_out  [N, H, dv, dk]    fp32 final states; may equal state_in (updated
 *                                in place); NULL: no final state is written
 *   o          [N, T, H, dv]     out_dtype
 *   inter      [N, T, H, dv, dk] fp32 or NULL: the state after every token
 *                                (inter[n][T-1] is the final state), e.g. to
 *                                restart from the last accepted draft token
 *   N, H > 0; 1 <= T <= 64
 * q, k, v, g, beta, o and inter must not overlap state_in or state_out.
 */
gdr_status gdr_decode_mtp(const void* q, const void* k, const void* v,
                          const float* g, const float* beta,
                          const float* state_in, float* state_out, void* o,
                          float* inter, int N, int T, int H, int dk, int dv,
                          gdr_dtype in_dtype, gdr_dtype out_dtype,
                          gdr_stream_t stream);

/*
 * gdr_max_chunks -- host-only upper bound on the number of chunks of a packed
 * batch of N sequences with T_total tokens: T_total / chunk + N (every
 * sequence adds at most one partial chunk).  Returns -1 on bad arguments.
 * Chunk-indexed buffers (L, M, fixed, chunk_indices) hold this many slots.
 */
int gdr_max_chunks(int T_total, int N, int chunk);

/*
 * gdr_chunk_layout -- varlen chunk layout, device to device (bit-exact).
 *
 *   cu_seqlens     [N+1] int32   token offsets of the packed sequences
 *   chunk_offsets  [N+1] int32   out: chunk_offsets[0] = 0,
 *                  chunk_offsets[n+1] = chunk_offsets[n] + ceil(len_n / chunk)
 *   chunk_indices  [max_chunks, 2] int32  out: row chunk_offsets[n] + j holds
 *                  (n, j); rows past the real chunk count hold (-1, -1)
 *   max_chunks     rows of chunk_indices (>= gdr_max_chunks(T_total, N, chunk))
 * Chunk j of sequence n covers tokens [cu[n] + j*chunk, min(cu[n] + (j+1)*chunk, cu[n+1])).
 * Chunks never straddle a sequence boundary (the FlashInfer PR #3866 page
 * handles variable-length batches with per-sequence chunk counts and zeroes
 * the slots past a sequence's valid chunks, zero_invalid_slots; here chunks
 * are packed, so there are no invalid slots inside the range).
 */
gdr_status gdr_chunk_layout(const int32_t* cu_seqlens, int N, int chunk,
                            int32_t* chunk_offsets, int32_t* chunk_indices,
                            int max_chunks, gdr_stream_t stream);

/*
 * gdr_chunk_prefill_workspace_bytes -- device workspace that gdr_chunk_prefill
 * needs for inputs of in_dtype when L_out, M_out and fixed_out are all NULL,
 * for whichever schedule the call takes (an upper bound for every other case).
 * Returns 0 on bad arguments (also for a shape or dtype gdr_chunk_prefill
 * refuses).
 */
size_t gdr_chunk_prefill_workspace_bytes(int T_total, int N, int H, int dk, int dv,
                                         int chunk, gdr_dtype in_dtype);

/*
 * gdr_chunk_prefill -- chunked prefill over packed variable-length sequences.
 *
 *   q, k        [T_total, H, dk]  in_dtype
 *   v           [T_total, H, dv]  in_dtype
 *   g, beta     [T_total, H]      fp32
 *   cu_seqlens  [N+1] int32       device; sequence n is tokens [cu[n], cu[n+1])
 *   state_in    [N, H, dv, dk]    fp32 initial states, or NULL for zero states
 *   state_out   [N, H, dv, dk]    fp32 final states (may equal state_in)
 *   o           [T_total, H, dv]  out_dtype
 *   L_out       [max_chunks, H, dv, dk] fp32 or NULL: local state of every chunk
 *               (the chunk run from a zero state): L_out[c][h][i][j] = L_c[i][j]
 *   M_out       [max_chunks, H, dk, dk] fp32 or NULL: transfer matrix of every
 *               chunk, M_out[c][h][a][b] = M_c[a][b], in the orientation of
 *               the recurrence: S_end = S_start M_c + L_c, i.e.
 *               S_end[i][b] = sum_a S_start[i][a] M_c[a][b] + L_c[i][b]
 *               (M_c = gamma_c I - W^T diag(D) K, the product of the chunk's
 *               per-token maps alpha_t (I - beta_t k_t k_t^T) in token order)
 *   fixed_out   [max_chunks, H, dv, dk] fp32 or NULL: state at the end of every
 *               chunk
 *   (max_chunks = gdr_max_chunks(T_total, N, chunk); chunk slot
 *    chunk_offsets[n] + j belongs to chunk j of sequence n; slots past the real
 *    chunk count are not written)
 *   T_total >= 0, N > 0, H > 0; chunk in {16, 64}; in_dtype bf16 or fp32 at
 *   either chunk size
 *   workspace   device scratch of workspace_bytes bytes (see
 *               gdr_chunk_prefill_workspace_bytes); may be NULL only when the
 *               bound is 0; its contents on entry do not matter
 * Sequences of length 0 are allowed: their final state is the initial state
 * (or zero).  q, k, v, g, beta and o must not overlap each other or the
 * state/L/M/fixed buffers.  All work is enqueued on `stream`, in one of the
 * following schedules, with the same results up to rounding order:
 *   - chunk-parallel: layout, chunk-local L/M, fixup over the chunks of each
 *     sequence (two-level for long sequences with few heads), chunk outputs,
 *     final states.  Taken for fp32 inputs or chunk 16 (fp32 inputs keep
 *     every product at fp32 precision);
 *   - sequential scan: layout, per-chunk factors T = (I + A)^{-1} and
 *     P = (Q K^T) (.) Gamma, then one pass per (sequence, head, block of state
 *     rows) that applies the UT transform and the fixup in factored form
 *     (S M_c + L_c = gamma_C S + (diag(D) T diag(beta) (V - diag(gamma) K S^T))^T K,
 *     without forming M, L, W or Ut) and writes the outputs, the final states
 *     and, when given, fixed_out.  Taken for bf16 inputs at chunk 64; for long
 *     sequences at low parallelism as a segmented scan: one pass over
 *     segments of whole chunks carrying two chains per segment, from zero
 *     (segment local states) and from the identity with v = 0 (segment
 *     transfer matrices), the segment-level fixup, and a final pass from every
 *     segment's true start.  When L_out or
 *     M_out is given, the chunk-local kernel of the chunk-parallel form writes
 *     them in parallel, before the scan.  The scan holds T and P as one fp16
 *     plane each (scaled by 16), and beta (V - diag(gamma) K S^T) / 16 and
 *     U / 16 as two fp16 planes each: entries of beta (v - gamma S k) or of U
 *     beyond about 1e6 in magnitude overflow to non-finite results (keys are
 *     expected L2-normalised, as the method assumes).
 */
gdr_status gdr_chunk_prefill(const void* q, const void* k, const void* v,
                             const float* g, const float* beta,
                             const int32_t* cu_seqlens, int N,
                             const float* state_in, float* state_out, void* o,
                             float* L_out, float* M_out, float* fixed_out,
                             int T_total, int H, int dk, int dv, int chunk,
                             gdr_dtype in_dtype, gdr_dtype out_dtype,
                             void* workspace, size_t workspace_bytes,
                             gdr_stream_t stream);

/*
 * gdr_chunk_prefill_noalloc -- gdr_chunk_prefill without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, layouts, schedules and results are those of gdr_chunk_prefill
 * (bit for bit: the same kernels run), minus workspace and workspace_bytes.
 * The workspace is instead a static device array of the library, 128 MiB
 * (134,217,728 bytes) on each GPU it runs on, held from the first call on that
 * GPU until the process ends.  A call that needs more than that (see
 * gdr_chunk_prefill_workspace_bytes; e.g. 4 sequences x 4096 tokens x 16 heads
 * at d = 128 needs about 55 MB) returns GDR_ERR_UNSUPPORTED with a message
 * and launches nothing.  Nothing is allocated or freed, here or on later
 * calls.  All calls on one GPU share its array, which keeps the last call's
 * contents (no call depends on them): calls that may overlap on one GPU, from
 * two streams or two threads, race and must be serialised by the caller.
 */
gdr_status gdr_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                                     const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int N,
                                     const float* state_in, float* state_out, void* o,
                                     float* L_out, float* M_out, float* fixed_out,
                                     int T_total, int H, int dk, int dv, int chunk,
                                     gdr_dtype in_dtype, gdr_dtype out_dtype,
                                     gdr_stream_t stream);

/*
 * gdr_state_fixup -- the inter-chunk fixup alone.
 *
 *   L             [n_chunks, H, dv, dk] fp32 local states, L[c][h][i][j] = L_c[i][j]
 *   M             [n_chunks, H, dk, dk] fp32 transfer matrices in the
 *                 orientation of the recurrence, M[c][h][a][b] = M_c[a][b]
 *                 (the same layout as gdr_chunk_prefill's M_out)
 *   state_in      [N, H, dv, dk] fp32, or NULL (no initial state)
 *   chunk_offsets [N+1] int32 device: sequence n owns chunk slots
 *                 [chunk_offsets[n], chunk_offsets[n+1])
 *   fixed         [n_chunks, H, dv, dk] fp32 out:
 *                 fixed[c0] = state_in[n] M_c0 + L_c0   (c0 = first chunk of n)
 *                           = L_c0                      (state_in == NULL)
 *                 fixed[c]  = fixed[c-1] M_c + L_c      (later chunks of n)
 *   n_chunks      slots in L, M and fixed; chunk ids at or past it are ignored
 * The FlashInfer PR #3866 page ("CP delta-rule precompute optimisation for
 * ultra-low parallelism", code changes 2) describes this scan: the state
 * multiplies M_c from the left, and without an initial state the first chunk's
 * state is its local state.  Here it runs one workgroup per (sequence, head,
 * block of state rows) on the matrix cores with the state and M_c split into
 * three bf16 planes each (fp32 precision), and loads chunk c+1's M and L while
 * chunk c is multiplied.  fixed must not overlap L, M or state_in.
 */
gdr_status gdr_state_fixup(const float* L, const float* M, const float* state_in,
                           const int32_t* chunk_offsets, int N, float* fixed,
                           int n_chunks, int H, int dk, int dv, gdr_stream_t stream);

/* Static text for a status code. */
const char* gdr_status_string(gdr_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* gdr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
