// scan.hip -- sequential chunk scan of the chunked gated delta rule on gfx950:
// the schedule for batches with many (sequence, head) pairs.
//
// One workgroup per (sequence, head, block of 64 state rows) walks the chunks
// of its sequence in order and keeps its rows of the state in registers for
// the whole sequence.  For a chunk with start state S (this workgroup's rows
// v), its q, k, v rows and the chunk factors T = (I + A)^{-1}, P, gamma, D,
// beta (chunk.hip):
//   Z = K S^T,   Y^T = S Q^T                        (contractions over dk)
//   U = T diag(beta) (V - diag(gamma) Z)            (the UT transform)
//   O^T = Y^T diag(gamma) + U^T P^T                 (the chunk's outputs)
//   S <- gamma_C S + (diag(D) U)^T K                (the state at the chunk end)
// The last line is the inter-chunk fixup S_end = S M + L of the FlashInfer
// PR #3866 page ("CP delta-rule precompute optimisation for ultra-low
// parallelism") with M = gamma_C I - W^T diag(D) K, L = Ut^T diag(D) K and
// W = T diag(beta gamma) K, Ut = T diag(beta) V, applied in factored form: no
// dk x dk matrix and neither W nor Ut is formed or stored, and the outputs
// come out of the same pass.  The re-association is derived from the
// recurrence.
//
// Compute waves.  Four waves (one per SIMD) each own one 16-row tile of state
// rows, held as
// D tiles of S^T: lane (c, g) holds S[v = 16 vt + c][16 jt + 4 g + e], e = 0..3.
// That is the accumulator layout of the state update (A = K^T, B = diag(D) U).
// For the contractions over dk the state is split into bf16 hi/lo planes and
// regrouped into natural fragments with permlane swaps, which serve as B (rows
// of S^T) in K S^T and as A (rows of S) in S Q^T.  Z, R and U are D tiles with
// tokens as rows; two of them stacked are an operand fragment in slot order,
// which is how R meets T (whose rows are stored in slot order) and U meets P
// and K^T.  k, q, v are exact bf16; fp32 operands are hi/lo planes: bf16
// planes, except in U = T R, where T is one fp16 plane and R two, and in
// P U, where P is one fp16 plane and U two (fp16's 11-bit significand holds
// T and P well enough for the 1e-3 budget, one bf16 plane would not).  The
// compute waves read only LDS and write their outputs and states straight to
// global memory.
//
// Copy waves.  Four more waves move each chunk's k, q, v rows, T, P and gates
// into LDS with direct global-to-LDS loads, one chunk ahead: LDS holds two
// chunk buffers, and one barrier per chunk separates the compute waves'
// reading of one buffer from the copy waves' filling of the other.
//
// LDS layout.  Rows are stored densely and the 16-byte chunks of a row are
// permuted (physical chunk = logical chunk XOR a function of the row) so that
// the rows one fragment read touches fall into distinct banks; the permutation
// is applied on the global side of the copies (each lane of a global-to-LDS
// load names its own source address), so every copy instruction fills a dense
// 1 KiB block.
#include <type_traits>

#include "launch.h"
#include "mfma_planes.h"

namespace gdr {
namespace {

constexpr int kXcds = 8;
constexpr int kCopyWaves = 4;
constexpr int kComputeWaves = 4;  // 16 state rows each
constexpr int kThreads = 64 * (kComputeWaves + kCopyWaves);

template <int D, int C, int NH>
struct ScanCfg {
  static constexpr int NT = C / 16;    // 16-token tiles
  static constexpr int ND = D / 16;    // 16-wide tiles of state columns
  static constexpr int KB = D / 32;    // 32-deep blocks over state columns
  static constexpr int KH = KB / 2;    // blocks per column half
  static constexpr int CB = C / 32;    // 32-deep blocks over tokens
  static constexpr int CHD = D / 8;    // 16-byte chunks per row of D bf16
  static constexpr int CHC = C / 8;    // 16-byte chunks per row of C bf16
  // NH compute waves share one 16-row state tile, each holding 1/NH of its
  // columns (NH = 2: the column halves sit on two SIMDs and exchange their
  // partial contractions over dk through LDS once per chunk).
  static constexpr int ROWS = 16 * kComputeWaves / NH;  // state rows per workgroup
  static constexpr int NVB = D / ROWS;                  // workgroups per (sequence, head)
  static constexpr int JT = ND / NH;                    // 16-wide column tiles per wave
  static constexpr int NO = NT / NH;                    // output token tiles per wave
  // T and P planes: rows t < C/2 keep their first C/2 columns (the rest is
  // above the diagonal), rows t >= C/2 keep all C.  T and P are one fp16
  // plane each.
  static constexpr int TL_LO = (C / 2) * (C / 2);
  static constexpr int TL = TL_LO + (C / 2) * C;
  // regions of one chunk buffer (bytes); each a whole number of 1 KiB blocks
  static constexpr int K_BYTES = C * D * 2;
  static constexpr int Q_BYTES = C * D * 2;
  static constexpr int T_BYTES = TL * 2;
  static constexpr int P_BYTES = TL * 2;
  static constexpr int V_BYTES = C * ROWS * 2;
  static constexpr int G_BYTES = 4 * C * 4;  // gamma, D, beta, zeros
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = OFF_K + K_BYTES;
  static constexpr int OFF_T = OFF_Q + Q_BYTES;
  static constexpr int OFF_P = OFF_T + T_BYTES;
  static constexpr int OFF_V = OFF_P + P_BYTES;
  static constexpr int OFF_G = OFF_V + V_BYTES;
  static constexpr int BUF = OFF_G + G_BYTES;
  // exchange region (NH = 2): per compute wave and lane, its partial K S^T
  // (NT tiles) and its partial S Q^T for the partner's output tiles (NO)
  static constexpr int X_SLOTS = NH > 1 ? NT + NO : 0;
  static constexpr int OFF_X = 2 * BUF;
  static constexpr int BYTES = 2 * BUF + X_SLOTS * kComputeWaves * 64 * 16;
  // copy instructions (1 KiB each) per region, and each copy wave's share
  // (T and P: the first NTT % kCopyWaves copy waves issue one more)
  static constexpr int NK = K_BYTES / 1024, NQ = Q_BYTES / 1024, NTT = T_BYTES / 1024;
  static constexpr int NP = P_BYTES / 1024, NV = V_BYTES / 1024;
  static constexpr int SK = NK / kCopyWaves, SQ = NQ / kCopyWaves;
  static constexpr int STT = (NTT + kCopyWaves - 1) / kCopyWaves, SP = STT;
  static constexpr int SV = NV / kCopyWaves;
  static_assert(C == 64 && (D == 64 || D == 128) && (NH == 1 || NH == 2), "shape");
  static_assert(K_BYTES % (1024 * kCopyWaves) == 0 && P_BYTES == T_BYTES &&
                    T_BYTES % 1024 == 0 && V_BYTES % (1024 * kCopyWaves) == 0 &&
                    G_BYTES == 1024,
                "copy tiling");
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// Chunk permutation of a dense row of `ch` 16-byte chunks (ch = 4, 8 or 16):
// rows that share a 256-byte bank line get different permutations.
__device__ __forceinline__ int swz(int row, int ch) { return (row * ch / 16) & (ch - 1); }

// Row offset (elements) of row t in a compact lower-triangular plane.
template <int C>
__device__ __forceinline__ int tl_row(int t) {
  return t < C / 2 ? t * (C / 2) : (C / 2) * (C / 2) + (t - C / 2) * C;
}

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// A fragment in slot order (two stacked D tiles: lane group g holds columns
// 4g..4g+3 of the first tile in slots 0-3 and of the second in slots 4-7) to
// natural order (lane group g holds columns 8g..8g+7).  Dwords 0-1 carry the
// first tile, 2-3 the second; a 32-lane swap then a 16-lane swap (gfx950
// v_permlane32_swap, v_permlane16_swap) route each pair of 16-lane groups.
__device__ __forceinline__ bf16x8 slot_to_natural(bf16x8 x) {
  const u32x4v w = __builtin_bit_cast(u32x4v, x);
  const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
  const auto c = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(c[0], c[1], false, false);
  return __builtin_bit_cast(bf16x8, u32x4v{b[0], d[0], b[1], d[1]});
}

// Four consecutive outputs to global memory (8 bytes bf16, round to nearest
// even; 16 bytes fp32).
template <Dt OUTD>
__device__ __forceinline__ void store4(void* o, size_t idx, const floatx4& x) {
  if constexpr (OUTD == Dt::F32) {
    *reinterpret_cast<floatx4*>(static_cast<float*>(o) + idx) = x;
  } else {
    uint32_t lo[1], hi[1];
    split2<1>(x[0], x[1], lo);
    split2<1>(x[2], x[3], hi);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o) + idx) = make_uint2(lo[0], hi[0]);
  }
}

// Workgroup barrier without a memory fence.  __syncthreads() would also wait
// for every global access still in flight (its release fence covers global
// memory and the LDS writes of global-to-LDS loads); here the copy waves wait
// for exactly their own loads and the compute waves only read LDS, so a bare
// s_barrier is enough.  The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte lane of a global-to-LDS copy: the 64 lanes of the wave fill the
// 1 KiB at `lds` in lane order.
__device__ __forceinline__ void copy16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}

// Scheduling pattern for a region of R LDS reads and R matrix products (masks
// of sched_group_barrier: 0x100 LDS read, 0x008 matrix product): L reads
// first, then pairs of one read and one product, then the remaining L
// products.  A wave issues in order, so the reads run L ahead of their use.
template <int L, int R, int I = 0>
__device__ __forceinline__ void lead_interleave() {
  if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(0x100, L, 0);
  if constexpr (I < R - L) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    lead_interleave<L, R, I + 1>();
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, L, 0);
  }
}

// NS = 2 (no outputs, whole tiles) carries a second state chain beside the
// first: it starts from the identity and sees v = 0, so its end state is the
// transfer matrix of the chunks walked (the map S -> S M of the recurrence
// without its v k^T terms), written to state_out2, while the first chain (from
// state_in, or zero) gives the local end state.  Both chains read the same K, T
// and gate fragments from LDS, and the two independent chains fill each
// other's latency in the compute waves.
// The LDS of a scan kernel, one array per kernel (Tag names the kernel and
// holds its size): both forms in the mixed kernel share one.  The body below
// names the array directly rather than through a pointer variable, which
// keeps its addresses compile-time constants.
template <class Tag>
__shared__ __align__(1024) unsigned char scan_lds[Tag::BYTES];

template <int D, int C, Dt OUTD, bool OUT, int NH, int NS, bool MIXED>
struct ScanLds {
  static constexpr int BYTES = MIXED ? (ScanCfg<D, C, 1>::BYTES > ScanCfg<D, C, 2>::BYTES
                                            ? ScanCfg<D, C, 1>::BYTES
                                            : ScanCfg<D, C, 2>::BYTES)
                                     : ScanCfg<D, C, NH>::BYTES;
};

// The work of one workgroup: state rows ROWS vb .. ROWS vb + ROWS - 1 of
// (sequence n, head h), in the LDS array scan_lds<Lds>.
template <int D, int C, Dt OUTD, bool OUT, int NH, int NS, class Lds>
__device__ __forceinline__ void scan_workgroup(
    int n, int h, int vb, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offs, const ChunkFactors& f,
    const float* state_in, float* state_out, float* state_out2, float* __restrict__ fixed,
    void* __restrict__ o, int H, int n_slots, int T_total) {
  static_assert(NS == 1 || (NS == 2 && !OUT && NH == 1), "two chains: no outputs, whole tiles");
  using Cfg = ScanCfg<D, C, NH>;
  constexpr int NT = Cfg::NT, KB = Cfg::KB, KH = Cfg::KH, CB = Cfg::CB, JT = Cfg::JT;
  constexpr int NO = Cfg::NO;
  constexpr int CHD = Cfg::CHD, CHC = Cfg::CHC, TL = Cfg::TL;
  constexpr int CHV = Cfg::ROWS / 8;  // 16-byte chunks per staged v row
  static_assert(Lds::BYTES >= Cfg::BYTES, "LDS");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;

  int c0 = offs[n], c1 = offs[n + 1];
  c0 = c0 < 0 ? 0 : (c0 > n_slots ? n_slots : c0);
  c1 = c1 < c0 ? c0 : (c1 > n_slots ? n_slots : c1);
  if (T_total <= 0) c1 = c0;  // no token to read, whatever the offsets claim
  int tb = cu[n], te = cu[n + 1];
  tb = tb < 0 ? 0 : (tb > T_total ? T_total : tb);
  te = te < tb ? tb : (te > T_total ? T_total : te);

  // Token range of chunk slot s (length 0 when the offsets disagree with cu).
  auto chunk_range = [&](int s, int& tok0) {
    tok0 = tb + (s - c0) * C;
    const int end = tok0 + C < te ? tok0 + C : te;
    return end > tok0 ? end - tok0 : 0;
  };

  if (wave >= kComputeWaves) {
    // ---- copy waves: each issues a quarter of every region's copies (the
    // gates are one copy, issued by the first wave).  Without outputs, q and
    // P are not needed.
    if (c1 <= c0) return;
    // wave-uniform, so that LDS destinations (and M0) stay scalar
    const int cw = __builtin_amdgcn_readfirstlane(wave - kComputeWaves);
    const uint32_t row_bytes = 2u * static_cast<uint32_t>(H) * D;  // one token row of q, k, v
    // per-lane source offsets of this wave's copies: chunk row and byte offset
    // inside the row (k, q, v), the two combined for a full chunk, and the
    // byte offset in a T or P slot (the same compact layout)
    int krow[Cfg::SK], qrow[Cfg::SQ], vrow[Cfg::SV];
    uint32_t kcol[Cfg::SK], qcol[Cfg::SQ], vcol[Cfg::SV];
    uint32_t kfull[Cfg::SK], qfull[Cfg::SQ], vfull[Cfg::SV];
    uint32_t toff[Cfg::STT];
#pragma unroll
    for (int x = 0; x < Cfg::SK; ++x) {
      const int p = 64 * (cw + kCopyWaves * x) + lane, t = p / CHD, pc = p % CHD;
      krow[x] = t;
      kcol[x] = 16u * (pc ^ swz_tr(t, CHD));
      kfull[x] = static_cast<uint32_t>(t) * row_bytes + kcol[x];
    }
#pragma unroll
    for (int x = 0; x < Cfg::SQ; ++x) {
      const int p = 64 * (cw + kCopyWaves * x) + lane, t = p / CHD, pc = p % CHD;
      qrow[x] = t;
      qcol[x] = 16u * (pc ^ swz(t, CHD));
      qfull[x] = static_cast<uint32_t>(t) * row_bytes + qcol[x];
    }
#pragma unroll
    for (int x = 0; x < Cfg::SV; ++x) {
      const int p = 64 * (cw + kCopyWaves * x) + lane, t = p / CHV, pc = p % CHV;
      vrow[x] = t;
      vcol[x] = 2u * (Cfg::ROWS * vb) + 16u * (pc ^ swz_tr(t, CHV));
      vfull[x] = static_cast<uint32_t>(t) * row_bytes + vcol[x];
    }
    // byte offset of the 16-byte piece p of a compact plane sequence
    auto tl_piece = [&](int p) {
      const int pl = p / (TL / 8), rr = p % (TL / 8);
      int t, pc, ch;
      if (rr < Cfg::TL_LO / 8) {
        t = rr / (CHC / 2);
        pc = rr % (CHC / 2);
        ch = CHC / 2;
      } else {
        t = C / 2 + (rr - Cfg::TL_LO / 8) / CHC;
        pc = (rr - Cfg::TL_LO / 8) % CHC;
        ch = CHC;
      }
      return 2u * (pl * TL + tl_row<C>(t) + 8 * (pc ^ swz(t, ch)));
    };
#pragma unroll
    for (int x = 0; x < Cfg::STT; ++x) {
      const int i = cw + kCopyWaves * x;
      toff[x] = tl_piece(64 * (i < Cfg::NTT ? i : 0) + lane);
    }
    const uint32_t goff = 16u * lane;
    // Chunk s into buffer (s - c0) & 1.  In a chunk shorter than C, rows past
    // its end repeat its last token (their beta is zero, so they leave U, O
    // and the state alone), and every row read stays inside the inputs.
    auto copy_chunk = [&](int s) {
      int tok;
      const int cl = chunk_range(s, tok);
      tok = tok < T_total ? tok : T_total - 1;
      int last = cl > 0 ? cl - 1 : 0;
      last = tok + last < T_total ? last : T_total - 1 - tok;
      const size_t tbase = (static_cast<size_t>(tok) * H + h) * D;
      const char* ks = reinterpret_cast<const char*>(k + tbase);
      const char* qs = reinterpret_cast<const char*>(q + tbase);
      const char* vs = reinterpret_cast<const char*>(v + tbase);
      const size_t slot = static_cast<size_t>(s) * H + h;
      const char* ts = reinterpret_cast<const char*>(f.t + slot * TL);
      const char* ps = reinterpret_cast<const char*>(f.p + slot * TL);
      unsigned char* buf = scan_lds<Lds> + ((s - c0) & 1) * Cfg::BUF;
      if (last == C - 1) {
#pragma unroll
        for (int x = 0; x < Cfg::SK; ++x) copy16(ks + kfull[x], buf + Cfg::OFF_K + 1024 * (cw + kCopyWaves * x));
        if constexpr (OUT) {
#pragma unroll
          for (int x = 0; x < Cfg::SQ; ++x) copy16(qs + qfull[x], buf + Cfg::OFF_Q + 1024 * (cw + kCopyWaves * x));
        }
#pragma unroll
        for (int x = 0; x < Cfg::SV; ++x) copy16(vs + vfull[x], buf + Cfg::OFF_V + 1024 * (cw + kCopyWaves * x));
      } else {
#pragma unroll
        for (int x = 0; x < Cfg::SK; ++x)
          copy16(ks + static_cast<uint32_t>(krow[x] < last ? krow[x] : last) * row_bytes + kcol[x],
                 buf + Cfg::OFF_K + 1024 * (cw + kCopyWaves * x));
        if constexpr (OUT) {
#pragma unroll
          for (int x = 0; x < Cfg::SQ; ++x)
            copy16(qs + static_cast<uint32_t>(qrow[x] < last ? qrow[x] : last) * row_bytes + qcol[x],
                   buf + Cfg::OFF_Q + 1024 * (cw + kCopyWaves * x));
        }
#pragma unroll
        for (int x = 0; x < Cfg::SV; ++x)
          copy16(vs + static_cast<uint32_t>(vrow[x] < last ? vrow[x] : last) * row_bytes + vcol[x],
                 buf + Cfg::OFF_V + 1024 * (cw + kCopyWaves * x));
      }
#pragma unroll
      for (int x = 0; x < Cfg::STT; ++x)
        if (cw + kCopyWaves * x < Cfg::NTT)  // wave-uniform
          copy16(ts + toff[x], buf + Cfg::OFF_T + 1024 * (cw + kCopyWaves * x));
      if constexpr (OUT) {
#pragma unroll
        for (int x = 0; x < Cfg::SP; ++x)
          if (cw + kCopyWaves * x < Cfg::NP)  // wave-uniform
            copy16(ps + toff[x], buf + Cfg::OFF_P + 1024 * (cw + kCopyWaves * x));
      }
      if (cw == 0) copy16(reinterpret_cast<const char*>(f.gate + slot * 4 * C) + goff, buf + Cfg::OFF_G);
    };

    copy_chunk(c0);
    __builtin_amdgcn_s_waitcnt(0);  // every count, vmcnt included, to zero
    bare_barrier();                 // B0: chunk c0 is in LDS
    for (int s = c0; s < c1; ++s) {
      if (s + 1 < c1) copy_chunk(s + 1);  // into the buffer chunk s - 1 released
      if constexpr (NH > 1) bare_barrier();  // the compute waves' exchange barrier
      __builtin_amdgcn_s_waitcnt(0);
      bare_barrier();  // chunk s is done; chunk s + 1 is in LDS
    }
    return;
  }

  // ---- compute waves ----
  // The column half hp is a compile-time constant of each instantiation, so
  // that the choice of output tiles and exchange slots costs no instructions.
  auto compute_waves = [&](auto hpc) {
    // Wave (rt, hp): state rows 16 rt .. 16 rt + 15 of this workgroup's
    // block, column tiles hp JT .. hp JT + JT - 1.
    constexpr int hp = decltype(hpc)::value;
    const int rt = wave / NH;
    const int vrow = Cfg::ROWS * vb + 16 * rt + c16;  // state row held by this lane
    const int jt0 = hp * JT;                          // first column tile held
    const size_t sbase = (static_cast<size_t>(n) * H + h) * D * D + static_cast<size_t>(vrow) * D;
    floatx4 S[NS][JT];
#pragma unroll
    for (int jl = 0; jl < JT; ++jl) {
      const int jt = jt0 + jl;
#pragma unroll
      for (int ch = 0; ch < NS; ++ch) {
        if (ch == 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) S[ch][jl][e] = vrow == 16 * jt + 4 * g4 + e ? 1.f : 0.f;
        } else {
          S[ch][jl] = state_in
                          ? *reinterpret_cast<const floatx4*>(state_in + sbase + 16 * jt + 4 * g4)
                          : floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    // Output token tiles of this wave: all of them when NH = 1; with NH = 2 the
    // column halves split them so that each does three 32-deep blocks of
    // U^T P^T: half 0 takes tiles 0 and 3, half 1 tiles 1 and 2 (tile a needs
    // blocks kb <= a / 2; four token tiles, C = 64).  Tile u of half x (NH = 2):
    auto otile = [](int x, int u) { return u == 0 ? x : 3 - x; };
    float* xch = reinterpret_cast<float*>(scan_lds<Lds> + Cfg::OFF_X);
    auto xslot = [&](int w, int x) {
      return reinterpret_cast<floatx4*>(xch) + (x * kComputeWaves + w) * 64 + lane;
    };

    if (c1 > c0) {
      // The state registers are carried through the loop: drain their loads
      // here, or a wait for them inside the loop would also wait for later
      // stores on every iteration.
      __builtin_amdgcn_s_waitcnt(0);
      bare_barrier();  // B0: chunk c0 is in LDS

      // One chunk step; the chunk buffer is a compile-time constant (chunk s of
      // the sequence sits in buffer (s - c0) & 1), so that each of the two
      // copies of the step below reads LDS at loop-invariant addresses.
      auto step = [&](int s, auto bsel) {
        using B = decltype(bsel);
        const unsigned char* buf = scan_lds<Lds> + B::value * Cfg::BUF;
        const uint16_t* Kl = reinterpret_cast<const uint16_t*>(buf + Cfg::OFF_K);
        const uint16_t* Ql = reinterpret_cast<const uint16_t*>(buf + Cfg::OFF_Q);
        const uint16_t* Tl = reinterpret_cast<const uint16_t*>(buf + Cfg::OFF_T);
        const uint16_t* Pl = reinterpret_cast<const uint16_t*>(buf + Cfg::OFF_P);
        const uint16_t* Vl = reinterpret_cast<const uint16_t*>(buf + Cfg::OFF_V);
        const float* Gl = reinterpret_cast<const float*>(buf + Cfg::OFF_G);

        // Z = K S^T (rows: tokens) and Y^T = S Q^T (rows: state rows), as the
        // sum of two partial contractions over the column halves of S (the
        // 32-deep blocks kb < KH, then kb >= KH), which are added last.  S^T
        // enters as operand planes in natural order (lane group g holds columns
        // 32 kb + 8 g .. +7): the two stacked D tiles are split, then regrouped
        // with permlane swaps.  The 16x16x32 A and B fragments have the same
        // lane layout, so these registers serve as B (rows of S^T) in K S^T and
        // as A (rows of S) in S Q^T.
        constexpr int NCH = 2 / NH;  // column halves contracted by this wave
        floatx4 Zh[NS][NCH][NT], Yh[NCH][NT];
#pragma unroll
        for (int hc = 0; hc < NCH; ++hc) {
#pragma unroll
          for (int a = 0; a < NT; ++a) {
#pragma unroll
            for (int ch = 0; ch < NS; ++ch) Zh[ch][hc][a] = floatx4{0.f, 0.f, 0.f, 0.f};
            if constexpr (OUT) Yh[hc][a] = floatx4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int kl = 0; kl < KH; ++kl) {
            const int kbl = hc * KH + kl;  // block among this wave's columns
            const int kb = hp * (KB / NH) + kbl;
            bf16x8 sbk[NS][2];
#pragma unroll
            for (int ch = 0; ch < NS; ++ch) {
              float x[8];
#pragma unroll
              for (int e2 = 0; e2 < 8; ++e2) x[e2] = S[ch][2 * kbl + e2 / 4][e2 & 3];
              split8<2>(x, sbk[ch]);
#pragma unroll
              for (int p = 0; p < 2; ++p) sbk[ch][p] = slot_to_natural(sbk[ch][p]);
            }
            bf16x8 ka[NT], qa[NT];
#pragma unroll
            for (int a = 0; a < NT; ++a) {
              const int t = 16 * a + c16, n8 = 4 * kb + g4;
              ka[a] = *reinterpret_cast<const bf16x8*>(Kl + t * D + 8 * (n8 ^ swz_tr(t, CHD)));
              if constexpr (OUT)
                qa[a] = *reinterpret_cast<const bf16x8*>(Ql + t * D + 8 * (n8 ^ swz(t, CHD)));
            }
            // plane pairs, smallest terms first; the four token tiles (and the
            // chains) are interleaved so that consecutive products are
            // independent
#pragma unroll
            for (int a = 0; a < NT; ++a)
#pragma unroll
              for (int ch = 0; ch < NS; ++ch)
                Zh[ch][hc][a] = mfma16x16x32(ka[a], sbk[ch][1], Zh[ch][hc][a]);
#pragma unroll
            for (int a = 0; a < NT; ++a)
#pragma unroll
              for (int ch = 0; ch < NS; ++ch)
                Zh[ch][hc][a] = mfma16x16x32(ka[a], sbk[ch][0], Zh[ch][hc][a]);
            if constexpr (OUT) {
#pragma unroll
              for (int a = 0; a < NT; ++a) Yh[hc][a] = mfma16x16x32(sbk[0][1], qa[a], Yh[hc][a]);
#pragma unroll
              for (int a = 0; a < NT; ++a) Yh[hc][a] = mfma16x16x32(sbk[0][0], qa[a], Yh[hc][a]);
            }
          }
        }
        floatx4 Z[NS][NT], Yo[NO];  // Yo: Y^T of this wave's output tiles
        if constexpr (NH == 1) {
#pragma unroll
          for (int a = 0; a < NT; ++a) {
#pragma unroll
            for (int ch = 0; ch < NS; ++ch) Z[ch][a] = Zh[ch][0][a] + Zh[ch][1][a];
            if constexpr (OUT) Yo[a] = Yh[0][a] + Yh[1][a];
          }
        } else {
          // exchange with the wave holding the other column half (wave ^ 1):
          // all of its partial Z, and its partial Y^T of this wave's tiles
#pragma unroll
          for (int a = 0; a < NT; ++a) *xslot(wave, a) = Zh[0][0][a];
          if constexpr (OUT) {
#pragma unroll
            for (int u = 0; u < NO; ++u) {
              const int ap = otile(1 - hp, u);  // the partner's tile u
              floatx4 y = Yh[0][0];
#pragma unroll
              for (int a = 1; a < NT; ++a) y = ap == a ? Yh[0][a] : y;
              *xslot(wave, NT + u) = y;
            }
          }
          // the LDS writes above must be complete before the barrier (gfx950
          // does not wait for them at s_barrier)
          lds_barrier();  // exchange written
#pragma unroll
          for (int a = 0; a < NT; ++a) Z[0][a] = Zh[0][0][a] + *xslot(wave ^ 1, a);
          if constexpr (OUT) {
#pragma unroll
            for (int u = 0; u < NO; ++u) {
              const int am = otile(hp, u);
              floatx4 y = Yh[0][0];
#pragma unroll
              for (int a = 1; a < NT; ++a) y = am == a ? Yh[0][a] : y;
              Yo[u] = y + *xslot(wave ^ 1, NT + u);
            }
          }
        }

        // R = diag(beta / kTScale) (V - diag(gamma) Z) (v rows 16 a + 4 g + e
        // at this lane's state row: a transpose read), as two fp16 operand
        // planes of 32 tokens (two stacked D tiles, slot order), then
        // U = (kTScale T) R over the lower blocks: T rows are stored in slot
        // order, so the T fragment of row 16 i + c and 32-block m is one
        // 16-byte read.  Both column halves form the same R and U.
        // (the second chain has v = 0)
        floatx4 R[NS][NT];
#pragma unroll
        for (int a = 0; a < NT; ++a) {
          const floatx4 gam = *reinterpret_cast<const floatx4*>(Gl + 16 * a + 4 * g4);
          const floatx4 bet = *reinterpret_cast<const floatx4*>(Gl + 2 * C + 16 * a + 4 * g4);
          const shortx4 vv = read_tr4(Vl, Cfg::ROWS, CHV, 16 * a, 16 * rt, c16, g4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            R[0][a][e] =
                bet[e] * (bf16_bits_to_f32(static_cast<uint16_t>(vv[e])) - gam[e] * Z[0][a][e]);
            if constexpr (NS == 2) R[1][a][e] = bet[e] * (0.f - gam[e] * Z[1][a][e]);
          }
        }
        halfx8 rb[NS][CB][2];
#pragma unroll
        for (int ch = 0; ch < NS; ++ch)
#pragma unroll
          for (int m = 0; m < CB; ++m) {
            float x[8];
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) x[e2] = R[ch][2 * m + e2 / 4][e2 & 3];
            split8_h<2>(x, rb[ch][m]);
          }
        floatx4 U[NS][NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const int t = 16 * i + c16, cw16 = t < C / 2 ? CHC / 2 : CHC;
#pragma unroll
          for (int ch = 0; ch < NS; ++ch) U[ch][i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m <= i / 2; ++m) {
            const halfx8 tf = *reinterpret_cast<const halfx8*>(Tl + tl_row<C>(t) +
                                                               8 * ((4 * m + g4) ^ swz(t, cw16)));
#pragma unroll
            for (int ch = 0; ch < NS; ++ch) {
              U[ch][i] = mfma16x16x32(tf, rb[ch][m][1], U[ch][i]);
              U[ch][i] = mfma16x16x32(tf, rb[ch][m][0], U[ch][i]);
            }
          }
        }

        // U as operand planes (32 tokens per block, slot order): U / kPScale
        // as two fp16 planes against the fp16 plane of kPScale P, and
        // diag(D) U as two bf16 planes against the exact K.
        halfx8 ub[CB][2];
        bf16x8 udb[NS][CB][2];
#pragma unroll
        for (int kb = 0; kb < CB; ++kb) {
#pragma unroll
          for (int ch = 0; ch < NS; ++ch) {
            float x[8], xd[8];
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
              const int a0 = 2 * kb + e2 / 4, e = e2 & 3;
              x[e2] = U[ch][a0][e] * (1.f / kPScale);  // exact: a power of two
              xd[e2] = Gl[C + 16 * a0 + 4 * g4 + e] * U[ch][a0][e];
            }
            if constexpr (OUT) split8_h<2>(x, ub[kb]);
            split8<2>(xd, udb[ch][kb]);
          }
        }

        if constexpr (OUT) {
          // O^T = Y^T diag(gamma) + U^T P^T for this wave's token tiles: lane
          // (c, g) ends up with token 16 a + c and state rows 4 g .. 4 g + 3 of
          // its row tile.  P is zero above the diagonal, so token tile a needs
          // the 32-blocks kb <= a / 2.
          floatx4 oa[NO];
          int at[NO];
#pragma unroll
          for (int u = 0; u < NO; ++u) {
            at[u] = NH == 1 ? u : otile(hp, u);
            oa[u] = Yo[u] * Gl[16 * at[u] + c16];
          }
#pragma unroll
          for (int kb = 0; kb < CB; ++kb) {
            // tiles with a / 2 >= kb: NH = 1: a >= 2 kb; NH = 2: u >= kb
            halfx8 pa[NO];
#pragma unroll
            for (int u = 0; u < NO; ++u) {
              if (NH == 1 ? u < 2 * kb : u < kb) continue;
              const int t = 16 * at[u] + c16;
              const int ch = (NH == 1 ? u < NT / 2 : u == 0) ? CHC / 2 : CHC;
              pa[u] = *reinterpret_cast<const halfx8*>(Pl + tl_row<C>(t) +
                                                       8 * ((4 * kb + g4) ^ swz(t, ch)));
            }
#pragma unroll
            for (int u = 0; u < NO; ++u)
              if (NH == 1 ? u >= 2 * kb : u >= kb) oa[u] = mfma16x16x32(ub[kb][1], pa[u], oa[u]);
#pragma unroll
            for (int u = 0; u < NO; ++u)
              if (NH == 1 ? u >= 2 * kb : u >= kb) oa[u] = mfma16x16x32(ub[kb][0], pa[u], oa[u]);
          }
          int tok0;
          const int cl = chunk_range(s, tok0);
#pragma unroll
          for (int u = 0; u < NO; ++u) {
            const int t = 16 * at[u] + c16;
            if (t < cl)
              store4<OUTD>(o, (static_cast<size_t>(tok0 + t) * H + h) * D + Cfg::ROWS * vb + 16 * rt + 4 * g4,
                           oa[u]);
          }
        }

        __builtin_amdgcn_sched_barrier(0);
        // S <- gamma_C S + (diag(D) U)^T K, as S^T = gamma_C S^T + K^T diag(D) U,
        // on this wave's column tiles.  K^T fragments (features 16 jt + c16;
        // slots = tokens 32 kb + 4 g4 + e and 32 kb + 16 + 4 g4 + e) come from
        // transpose reads of the K rows, running ahead of the products that
        // consume them.
        bf16x8 kt[CB][JT];
#pragma unroll
        for (int kb = 0; kb < CB; ++kb)
#pragma unroll
          for (int jl = 0; jl < JT; ++jl) {
            const shortx4 lo = read_tr4(Kl, D, CHD, 32 * kb, 16 * (jt0 + jl), c16, g4);
            const shortx4 hi = read_tr4(Kl, D, CHD, 32 * kb + 16, 16 * (jt0 + jl), c16, g4);
            kt[kb][jl] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        const float gam_end = Gl[C - 1];
#pragma unroll
        for (int ch = 0; ch < NS; ++ch)
#pragma unroll
          for (int jl = 0; jl < JT; ++jl) S[ch][jl] *= gam_end;
#pragma unroll
        for (int kb = 0; kb < CB; ++kb)
#pragma unroll
          for (int jl = 0; jl < JT; ++jl) {
            bf16x8 kk[1] = {kt[kb][jl]};
#pragma unroll
            for (int ch = 0; ch < NS; ++ch) mma_planes<1, 2>(S[ch][jl], kk, udb[ch][kb]);
          }
        lead_interleave<8, 2 * CB * JT * NS>();
        __builtin_amdgcn_sched_barrier(0);
        if (fixed) {
          float* fx = fixed + (static_cast<size_t>(s) * H + h) * D * D + static_cast<size_t>(vrow) * D;
#pragma unroll
          for (int jl = 0; jl < JT; ++jl)
            *reinterpret_cast<floatx4*>(fx + 16 * (jt0 + jl) + 4 * g4) = S[0][jl];
        }
        bare_barrier();  // chunk s is done with its buffer; chunk s + 1 is in LDS
      };
      for (int s = c0; s < c1; s += 2) {
        step(s, std::integral_constant<int, 0>{});
        if (s + 1 < c1) step(s + 1, std::integral_constant<int, 1>{});
      }
    }

    if (state_out) {
#pragma unroll
      for (int jl = 0; jl < JT; ++jl)
        *reinterpret_cast<floatx4*>(state_out + sbase + 16 * (jt0 + jl) + 4 * g4) = S[0][jl];
    }
    if constexpr (NS == 2) {
      if (state_out2) {
#pragma unroll
        for (int jl = 0; jl < JT; ++jl)
          *reinterpret_cast<floatx4*>(state_out2 + sbase + 16 * (jt0 + jl) + 4 * g4) = S[1][jl];
      }
    }
  };
  if constexpr (NH == 1) {
    compute_waves(std::integral_constant<int, 0>{});
  } else if (wave % NH == 0) {
    compute_waves(std::integral_constant<int, 0>{});
  } else {
    compute_waves(std::integral_constant<int, 1>{});
  }
}

template <int D, int C, Dt OUTD, bool OUT, int NH, int NS = 1>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ offs, ChunkFactors f, const float* state_in, float* state_out,
    float* state_out2, float* __restrict__ fixed, void* __restrict__ o, int N, int H,
    int n_slots, int T_total) {
  using Cfg = ScanCfg<D, C, NH>;
  // XCD-aware placement: linear ids with the same residue mod 8 share an XCD,
  // so the workgroups of one (sequence, head) share its L2.
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds, r = lin / kXcds;
  const int vb = r % Cfg::NVB;
  const int pair = (r / Cfg::NVB) * kXcds + xcd;
  if (pair >= N * H) return;
  scan_workgroup<D, C, OUTD, OUT, NH, NS, ScanLds<D, C, OUTD, OUT, NH, NS, false>>(
      pair / H, pair % H, vb, q, k, v, cu, offs, f, state_in, state_out, state_out2, fixed, o, H,
      n_slots, T_total);
}

// MI355X has 256 compute units and one scan workgroup fills one (its LDS).
constexpr int kCus = 256;
// Workgroups of the column-split form (NH = 2) that fit the GPU at once.
constexpr int64_t kSplitMaxGroups = kCus;

// Mixed launch: when the column split of every sequence does not fit the GPU
// at once, the sequence with the most chunks may still take it while the
// others run in whole tiles.  A chunk step of the split form takes about
// 0.887 of the whole-tile step on a busy GPU (2.27 against 2.56 us at
// d = 128, both measured with every compute unit running a scan workgroup).
constexpr int64_t kStepSplit = 887, kStepWhole = 1000;
constexpr int kMixedMaxN = 63;  // one lane per chunk offset

// The sequence that the mixed launch runs in the split form, or -1 for none.
// Every wave of every workgroup reaches the same answer from the chunk
// offsets.  The candidate is the sequence with the most chunks (the first of
// equal ones).  It is split when the modelled time of the launch falls:
//   whole tiles: max(its chain, all workgroup-steps / compute units),
//   mixed:       max(its chain at the split step, the longest other chain,
//                    the other workgroup-steps / the compute units left).
template <int NVB1, int NVB2>
__device__ __forceinline__ int mixed_split_choice(const int32_t* __restrict__ offs, int N, int H,
                                                  int n_slots) {
  const int lane = threadIdx.x & 63;
  int a = lane <= N ? offs[lane] : 0;
  a = a < 0 ? 0 : (a > n_slots ? n_slots : a);
  const int b = __shfl_down(a, 1);
  const int cnt = lane < N && b > a ? b - a : 0;  // < 2^25 chunks: the key fits 31 bits
  int key = (cnt << 6) | (63 - lane), sum = cnt;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const int ok = __shfl_xor(key, m);
    key = ok > key ? ok : key;
    sum += __shfl_xor(sum, m);
  }
  const int star = 63 - (key & 63);
  const int64_t lmax = key >> 6;
  int other = lane != star ? cnt : 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const int oo = __shfl_xor(other, m);
    other = oo > other ? oo : other;
  }
  const int64_t all_steps = static_cast<int64_t>(sum) * H * NVB1;
  const int64_t rest_steps = (sum - lmax) * H * NVB1;
  const int64_t free_cus = kCus - static_cast<int64_t>(H) * NVB2;
  const int64_t spread_all = (all_steps + kCus - 1) / kCus;
  const int64_t spread_rest = (rest_steps + free_cus - 1) / free_cus;
  const int64_t t_whole = kStepWhole * (lmax > spread_all ? lmax : spread_all);
  const int64_t t_rest = kStepWhole * (other > spread_rest ? other : spread_rest);
  const int64_t t_mixed = kStepSplit * lmax > t_rest ? kStepSplit * lmax : t_rest;
  return __builtin_amdgcn_readfirstlane(lmax > 0 && t_mixed < t_whole ? star : -1);
}

// Linear ids [0, split_groups) are the split form's workgroups of the chosen
// sequence (XCD-aware as above, over its heads); the rest are the whole-tile
// workgroups of every (sequence, head) pair, of which the chosen sequence's
// exit at once.  When no sequence is chosen, the first part exits instead.
// Both forms give identical bits, so the choice changes no result.
template <int D, int C, Dt OUTD, bool OUT>
__global__ __launch_bounds__(kThreads) void chunk_scan_mixed_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ offs, ChunkFactors f, const float* state_in, float* state_out,
    float* __restrict__ fixed, void* __restrict__ o, int N, int H, int n_slots, int T_total,
    int split_groups) {
  using C1 = ScanCfg<D, C, 1>;
  using C2 = ScanCfg<D, C, 2>;
  using Lds = ScanLds<D, C, OUTD, OUT, 1, 1, true>;
  const int star = mixed_split_choice<C1::NVB, C2::NVB>(offs, N, H, n_slots);
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds;
  if (lin < split_groups) {
    if (star < 0) return;
    const int r = lin / kXcds, vb = r % C2::NVB;
    const int h = (r / C2::NVB) * kXcds + xcd;
    if (h >= H) return;
    scan_workgroup<D, C, OUTD, OUT, 2, 1, Lds>(star, h, vb, q, k, v, cu, offs, f, state_in,
                                                state_out, nullptr, fixed, o, H, n_slots, T_total);
    return;
  }
  const int r = (lin - split_groups) / kXcds, vb = r % C1::NVB;
  const int pair = (r / C1::NVB) * kXcds + xcd;
  if (pair >= N * H || pair / H == star) return;
  scan_workgroup<D, C, OUTD, OUT, 1, 1, Lds>(pair / H, pair % H, vb, q, k, v, cu, offs, f,
                                              state_in, state_out, nullptr, fixed, o, H, n_slots,
                                              T_total);
}

template <int D, int C, Dt OUTD, bool OUT, int NH, int NS = 1>
hipError_t scan_launch(const void* q, const void* k, const void* v, const int32_t* cu,
                       const int32_t* offs, const ChunkFactors& f, const float* state_in,
                       float* state_out, float* state_out2, float* fixed, void* o, int N, int H,
                       int n_slots, int T_total, hipStream_t stream) {
  const int64_t pairs = static_cast<int64_t>(N) * H;
  const int64_t groups = (pairs + kXcds - 1) / kXcds * kXcds * ScanCfg<D, C, NH>::NVB;
  if (groups > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((chunk_scan_kernel<D, C, OUTD, OUT, NH, NS>),
                     dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), cu, offs, f, state_in, state_out, state_out2,
                     fixed, o, N, H, n_slots, T_total);
  return hipGetLastError();
}

// The scan is a chain of dependent chunk steps per (sequence, head), so its
// time is the step latency times the chunks of the longest sequence as long
// as the workgroups fit the GPU at once.  Splitting every 16-row state tile
// over two SIMDs (NH = 2) cuts a step's matrix products per wave from 132 to
// 75 for twice the workgroups; it is taken when those still fit at once.
// Both forms add the two column halves' contractions in the same order, so
// their results are identical bit for bit.
template <int D, int C, Dt OUTD>
hipError_t scan_t(const void* q, const void* k, const void* v, const int32_t* cu,
                  const int32_t* offs, const ChunkFactors& f, const float* state_in,
                  float* state_out, float* fixed, void* o, int N, int H, int n_slots, int T_total,
                  hipStream_t stream) {
  constexpr int NVB1 = ScanCfg<D, C, 1>::NVB, NVB2 = ScanCfg<D, C, 2>::NVB;
  const int64_t split_groups = (static_cast<int64_t>(N) * H + kXcds - 1) / kXcds * kXcds * NVB2;
  const bool split = split_groups <= kSplitMaxGroups;
  if (!split && N <= kMixedMaxN && static_cast<int64_t>(H) * NVB2 <= kCus / 2) {
    // the split part covers the heads of one sequence
    const int64_t head_groups = (static_cast<int64_t>(H) + kXcds - 1) / kXcds * kXcds * NVB2;
    const int64_t groups =
        head_groups + (static_cast<int64_t>(N) * H + kXcds - 1) / kXcds * kXcds * NVB1;
    if (groups > INT32_MAX) return hipErrorInvalidConfiguration;
#define GDR_SCAN_M(OUT_)                                                                        \
  hipLaunchKernelGGL((chunk_scan_mixed_kernel<D, C, OUTD, OUT_>),                               \
                     dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0, stream,            \
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),          \
                     static_cast<const uint16_t*>(v), cu, offs, f, state_in, state_out, fixed, o, \
                     N, H, n_slots, T_total, static_cast<int>(head_groups))
    if (o) GDR_SCAN_M(true);
    else GDR_SCAN_M(false);
#undef GDR_SCAN_M
    return hipGetLastError();
  }
#define GDR_SCAN_L(OUT_, NH_)                                                                   \
  return scan_launch<D, C, OUTD, OUT_, NH_>(q, k, v, cu, offs, f, state_in, state_out, nullptr, \
                                            fixed, o, N, H, n_slots, T_total, stream)
  if (o) {
    if (split) GDR_SCAN_L(true, 2);
    GDR_SCAN_L(true, 1);
  }
  if (split) GDR_SCAN_L(false, 2);
  GDR_SCAN_L(false, 1);
#undef GDR_SCAN_L
}

__global__ __launch_bounds__(256) void segment_ranges_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ seg_idx, int N, int seg, int chunk, int max_segs,
    int32_t* __restrict__ cu_seg, int32_t* __restrict__ offs_seg) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m > max_segs) return;
  int tok = cu[N], c = offs[N];  // end sentinel and slots past the real count
  if (m < max_segs) {
    const int n = seg_idx[2 * m], j = seg_idx[2 * m + 1];
    if (n >= 0 && n < N && j >= 0) {
      const int64_t t = cu[n] + static_cast<int64_t>(j) * seg * chunk;
      const int64_t cc = offs[n] + static_cast<int64_t>(j) * seg;
      tok = static_cast<int>(t < cu[n + 1] ? t : cu[n + 1]);
      c = static_cast<int>(cc < offs[n + 1] ? cc : offs[n + 1]);
    }
  }
  cu_seg[m] = tok;
  offs_seg[m] = c;
}

// blockIdx.z picks one of kStartSlices slices of the state, so that the few
// segment starts of a long sequence still spread over many compute units.
constexpr int kStartSlices = 16;

template <int D>
__global__ __launch_bounds__(256) void segment_starts_kernel(const float* state_in,
                                                             const float* __restrict__ seg_end,
                                                             const int32_t* __restrict__ seg_idx,
                                                             int H, float* __restrict__ seg_start) {
  const int m = blockIdx.x, h = blockIdx.y;
  const int n = seg_idx[2 * m], j = seg_idx[2 * m + 1];
  if (n < 0 || j < 0) return;  // no segment: the scan never reads this slot
  const floatx4* src = nullptr;
  if (j > 0)
    src = reinterpret_cast<const floatx4*>(seg_end + (static_cast<size_t>(m - 1) * H + h) * D * D);
  else if (state_in)
    src = reinterpret_cast<const floatx4*>(state_in + (static_cast<size_t>(n) * H + h) * D * D);
  floatx4* dst = reinterpret_cast<floatx4*>(seg_start + (static_cast<size_t>(m) * H + h) * D * D);
  constexpr int per = D * D / 4 / kStartSlices;
  static_assert(per % 256 == 0 || per < 256, "slice");
  for (int i = blockIdx.z * per + threadIdx.x; i < (blockIdx.z + 1) * per; i += blockDim.x)
    dst[i] = src ? src[i] : floatx4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace

hipError_t launch_segment_ranges(const int32_t* cu_seqlens, const int32_t* chunk_offsets,
                                 const int32_t* seg_idx, int N, int seg, int chunk, int max_segs,
                                 int32_t* cu_seg, int32_t* offs_seg, hipStream_t stream) {
  hipLaunchKernelGGL(segment_ranges_kernel, dim3((max_segs + 1 + 255) / 256), dim3(256), 0, stream,
                     cu_seqlens, chunk_offsets, seg_idx, N, seg, chunk, max_segs, cu_seg, offs_seg);
  return hipGetLastError();
}

hipError_t launch_segment_starts(const float* state_in, const float* seg_end,
                                 const int32_t* seg_idx, int max_segs, int H, int d,
                                 float* seg_start, hipStream_t stream) {
  if (max_segs <= 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL(segment_starts_kernel<128>, dim3(max_segs, H, kStartSlices), dim3(256), 0,
                       stream, state_in, seg_end, seg_idx, H, seg_start);
  else
    hipLaunchKernelGGL(segment_starts_kernel<64>, dim3(max_segs, H, kStartSlices), dim3(256), 0,
                       stream, state_in, seg_end, seg_idx, H, seg_start);
  return hipGetLastError();
}

hipError_t launch_chunk_scan_pair(const void* k, const void* v, const int32_t* cu_seqlens,
                                  const int32_t* chunk_offsets, const ChunkFactors& f,
                                  const float* state_in, float* state_out, float* transfer_out,
                                  int N, int H, int d, int chunk, int n_slots, int T_total,
                                  hipStream_t stream) {
  if (chunk != 64) return hipErrorInvalidValue;
  if (d == 128)
    return scan_launch<128, 64, Dt::F32, false, 1, 2>(nullptr, k, v, cu_seqlens, chunk_offsets, f,
                                                      state_in, state_out, transfer_out, nullptr,
                                                      nullptr, N, H, n_slots, T_total, stream);
  return scan_launch<64, 64, Dt::F32, false, 1, 2>(nullptr, k, v, cu_seqlens, chunk_offsets, f,
                                                   state_in, state_out, transfer_out, nullptr,
                                                   nullptr, N, H, n_slots, T_total, stream);
}

hipError_t launch_chunk_scan(const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, const int32_t* chunk_offsets,
                             const ChunkFactors& f, const float* state_in, float* state_out,
                             float* fixed, void* o, int N, int H, int d, int chunk, int n_slots,
                             int T_total, int out_dtype, hipStream_t stream) {
  if (chunk != 64) return hipErrorInvalidValue;
#define GDR_SCAN(D_, OUT_)                                                                         \
  return scan_t<D_, 64, OUT_>(q, k, v, cu_seqlens, chunk_offsets, f, state_in, state_out, fixed, o, \
                              N, H, n_slots, T_total, stream)
  if (d == 128) {
    if (out_dtype == 0) GDR_SCAN(128, Dt::BF16);
    GDR_SCAN(128, Dt::F32);
  }
  if (out_dtype == 0) GDR_SCAN(64, Dt::BF16);
  GDR_SCAN(64, Dt::F32);
#undef GDR_SCAN
}

}  // namespace gdr
