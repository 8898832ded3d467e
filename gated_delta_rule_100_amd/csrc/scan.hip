// scan.hip -- sequential chunk scan of the chunked gated delta rule on gfx950:
// the schedule for batches with many (sequence, head) pairs.
//
// One workgroup per (sequence, head, block of 64 state rows) walks the chunks
// of its sequence in order and keeps its rows of the state in registers for
// the whole sequence.  For a chunk with start state S (this workgroup's rows v)
// and the chunk factors W, Ut, P, K, gamma, D (chunk.hip):
//   X = W S^T,   Y^T = S Q^T                (contractions over dk)
//   U = Ut - X
//   O^T = Y^T diag(gamma) + U^T P^T         (the chunk's outputs, transposed)
//   S <- gamma_C S + (diag(D) U)^T K        (the state at the chunk end)
// The last line is the inter-chunk fixup S_end = S M + L of the FlashInfer
// PR #3866 page ("CP delta-rule precompute optimisation for ultra-low
// parallelism") with M = gamma_C I - W^T diag(D) K and L = Ut^T diag(D) K
// applied in factored form: no dk x dk matrix is formed or stored, and the
// outputs come out of the same pass, so neither M, L nor the per-chunk states
// travel through HBM.  The re-association is derived from the recurrence.
//
// Compute waves.  Four waves each own one 16-row tile of state rows, held as
// D tiles of S^T: lane (c, g) holds S[v = 16 vt + c][16 jt + 4 g + e], e = 0..3.
// That is the accumulator layout of the state update (A = K^T, B = diag(D) U)
// and, two tiles stacked, an operand fragment of the 16x16x32 products with the
// slot-permuted contraction order (mfma_planes.h): B (rows of S^T) in W S^T and
// A (rows of S) in S Q^T, whose D tiles give each lane four consecutive outputs
// of one token.  fp32 operands are bf16 hi/lo planes (three plane products); K
// and Q are exact bf16.  The compute waves touch only LDS and registers: every
// operand arrives in LDS, and outputs leave through an LDS staging tile.
//
// Copy waves.  Four more waves move data with direct global-to-LDS loads and
// write the staged outputs.  A single wave keeps too few loads in flight to
// stream from L2 at more than ~16 GB/s, so every region's copies are spread
// over the four.  An LDS region is refilled for a later chunk as soon as the
// compute waves are done with it; three barriers per chunk mark the phases:
//     compute:  [W S^T, S Q^T] B1 [U, O] B2 [state update] B3
//     copy:     B1: W, Q of c+2 (double-buffered);  B2: Ut^T, P, gates of c+1;
//               B3: write O of c, K of c+1
// A copy is waited for just before the barrier that precedes its first use;
// loads complete in order, so the loads issued after it stay in flight.
// (Touching the lines of later chunks to warm L2 was measured to slow this
// down: those loads occupy the same miss capacity the copies need.)
//
// LDS layout.  Rows are stored densely and the 16-byte chunks of a row are
// permuted (physical chunk = logical chunk XOR a function of the row) so that
// the rows one fragment read touches fall into distinct banks; the permutation
// is applied on the global side of the copies (each lane of a global-to-LDS
// load names its own source address), so every copy instruction fills a dense
// 1 KiB block.  Workgroups of one (sequence, head) are placed on the same XCD
// so that they share its L2.
#include "launch.h"
#include "mfma_planes.h"

namespace gdr {
namespace {

constexpr int kXcds = 8;
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt_hi[15:14]); only vmcnt is constrained.
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kComputeWaves = 4;
constexpr int kCopyWaves = 4;
constexpr int kThreads = 64 * (kComputeWaves + kCopyWaves);

template <int D, int C, int OB>  // OB: bytes per output element
struct ScanCfg {
  static constexpr int NT = C / 16;    // 16-token tiles
  static constexpr int ND = D / 16;    // 16-wide tiles of state columns
  static constexpr int KB = D / 32;    // 32-deep blocks over state columns
  static constexpr int CB = C / 32;    // 32-deep blocks over tokens
  static constexpr int CHD = D / 8;    // 16-byte chunks per row of D bf16
  static constexpr int CHC = C / 8;    // 16-byte chunks per row of C bf16
  static constexpr int CHU = C / 4;    // 16-byte chunks per row of C fp32
  static constexpr int ROWS = 16 * kComputeWaves;  // state rows per workgroup
  // P plane: rows t < C/2 keep their first C/2 columns only (the rest is above
  // the diagonal), rows t >= C/2 keep all C.
  static constexpr int P_LO = (C / 2) * (C / 2);
  static constexpr int P_PLANE = P_LO + (C / 2) * C;
  // LDS regions (bytes); every copied region is a whole number of 1 KiB blocks
  static constexpr int W_BYTES = 2 * C * D * 2;
  static constexpr int Q_BYTES = C * D * 2;
  static constexpr int K_BYTES = D * C * 2;
  static constexpr int P_BYTES = 2 * P_PLANE * 2;
  static constexpr int U_BYTES = ROWS * C * 4;
  static constexpr int G_BYTES = 2 * C * 4;   // gamma_t, D_t; two buffers
  static constexpr int O_LD = ROWS * OB + 16;  // staged output row (tokens x state rows)
  // W and Q are double-buffered (buffer (c - first chunk) & 1 holds chunk c),
  // the other regions hold one chunk
  static constexpr int WQ_BYTES = W_BYTES + Q_BYTES;
  static constexpr int OFF_W = 0;  // + buffer * WQ_BYTES
  static constexpr int OFF_Q = OFF_W + W_BYTES;
  static constexpr int OFF_K = 2 * WQ_BYTES;
  static constexpr int OFF_P = OFF_K + K_BYTES;
  static constexpr int OFF_U = OFF_P + P_BYTES;
  static constexpr int OFF_G = OFF_U + U_BYTES;
  static constexpr int OFF_O = OFF_G + 2 * G_BYTES;
  static constexpr int BYTES = OFF_O + C * O_LD;
  // copy instructions (1 KiB each) per region
  static constexpr int NW = W_BYTES / 1024, NQ = Q_BYTES / 1024, NK = K_BYTES / 1024;
  static constexpr int NP = P_BYTES / 1024, NU = U_BYTES / 1024;
  // output rows are written in 16-byte pieces
  static constexpr int OPR = ROWS * OB / 16, NO = C * OPR / 64;
  // each copy wave's share of the copy instructions of a region
  static constexpr int share(int n) { return (n + kCopyWaves - 1) / kCopyWaves; }
  static constexpr int SW = share(NW), SQ = share(NQ), SK = share(NK), SU = share(NU), SP = share(NP);
  static constexpr int SO = NO / kCopyWaves;
  static_assert(C == 64 && (D == 64 || D == 128) && (OB == 2 || OB == 4), "shape");
  static_assert(W_BYTES % 1024 == 0 && Q_BYTES % 1024 == 0 && K_BYTES % 1024 == 0 &&
                    P_BYTES % 1024 == 0 && U_BYTES % 1024 == 0 && G_BYTES == 512 &&
                    C * OPR % 64 == 0,
                "copy tiling");
  static_assert(NO % kCopyWaves == 0, "copy shares");
  static_assert(SW + SQ + SU + SP + SK + SO + 2 <= 63, "vmcnt range");
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// Chunk permutation of a dense row of `ch` 16-byte chunks (ch = 4, 8 or 16):
// rows that share a 256-byte bank line get different permutations.
__device__ __forceinline__ int swz(int row, int ch) { return (row * ch / 16) & (ch - 1); }

// Fragment of an operand row stored in slot order (chunk.hip): 16-byte chunk
// n8 = 4 kb + g of the row holds lane group g's eight contraction slots of the
// 32-block kb; chunks are permuted per row as above.
template <int PL>
__device__ __forceinline__ void read_slots(const uint16_t* row0, int plane_stride, int row,
                                           int ch, int n8, bf16x8 (&out)[PL]) {
  const int off = 8 * (n8 ^ swz(row, ch));
#pragma unroll
  for (int p = 0; p < PL; ++p)
    out[p] = *reinterpret_cast<const bf16x8*>(row0 + p * plane_stride + off);
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

// Four consecutive outputs into LDS (8 bytes bf16, round to nearest even; 16
// bytes fp32).
template <Dt OUTD>
__device__ __forceinline__ void stage4(unsigned char* dst, const floatx4& x) {
  if constexpr (OUTD == Dt::F32) {
    *reinterpret_cast<floatx4*>(dst) = x;
  } else {
    const uint32_t lo = f32_to_bf16_bits(x[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(x[1])) << 16);
    const uint32_t hi = f32_to_bf16_bits(x[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(x[3])) << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  }
}

// Barrier of the copy waves.  A plain s_barrier: __syncthreads() would first
// wait for every load still in flight (its release fence covers the LDS writes
// of global-to-LDS loads), which would make each barrier wait for the refills
// just issued.  The copy waves instead wait, before each barrier, for exactly
// the copies the next phase reads.
__device__ __forceinline__ void copy_barrier() { __builtin_amdgcn_s_barrier(); }

// One 16-byte lane of a global-to-LDS copy: the 64 lanes of the wave fill the
// 1 KiB at `lds` in lane order.
__device__ __forceinline__ void copy16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}

template <int D, int C, Dt OUTD>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ offs, ChunkFactors f,
    const float* state_in, float* state_out, float* __restrict__ fixed, void* __restrict__ o,
    int N, int H, int n_slots, int T_total) {
  constexpr int OB = OUTD == Dt::F32 ? 4 : 2;
  using Cfg = ScanCfg<D, C, OB>;
  constexpr int NT = Cfg::NT, ND = Cfg::ND, KB = Cfg::KB, CB = Cfg::CB;
  constexpr int CHD = Cfg::CHD, CHC = Cfg::CHC, CHU = Cfg::CHU;
  constexpr int NVB = D / Cfg::ROWS;  // workgroups per (sequence, head)
  __shared__ __align__(1024) unsigned char smem[Cfg::BYTES];

  // XCD-aware placement: linear ids with the same residue mod 8 share an XCD.
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds, r = lin / kXcds;
  const int vb = r % NVB;
  const int pair = (r / NVB) * kXcds + xcd;
  if (pair >= N * H) return;
  const int n = pair / H, h = pair % H;
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
  // Factor slot of chunk s; past the sequence the last chunk is used again
  // (copies into a region after its last use are harmless).
  auto slot_of = [&](int s) { return static_cast<size_t>(s < c1 ? s : c1 - 1) * H + h; };

  if (wave >= kComputeWaves) {
    // ---- copy waves: each issues a quarter of every region's copies (the
    // last share is padded with repeats of the region's last copy, which
    // rewrite the same bytes), so that every wave's wait counts are the same
    // constants.  Loads complete in order, so each wait below names how many
    // younger loads may still be in flight.
    if (c1 <= c0) return;
    const int cw = wave - kComputeWaves;
    auto pick = [&](int k, int n) { const int i = cw + kCopyWaves * k; return i < n ? i : n - 1; };
    // per-lane source offsets of this wave's copies (bytes from the chunk's base)
    uint32_t woff[Cfg::SW], qoff[Cfg::SQ], koff[Cfg::SK], uoff[Cfg::SU], poff[Cfg::SP];
    int wdst[Cfg::SW], qdst[Cfg::SQ], kdst[Cfg::SK], udst[Cfg::SU], pdst[Cfg::SP];
    int qrow[Cfg::SQ], krow[Cfg::SK];  // chunk row each Q / K copy lane reads
#pragma unroll
    for (int k = 0; k < Cfg::SW; ++k) {
      const int i = pick(k, Cfg::NW), p = 64 * i + lane, row = p / CHD, pc = p % CHD;
      woff[k] = 2u * (row * D + 8 * (pc ^ swz(row % C, CHD)));
      wdst[k] = Cfg::OFF_W + 1024 * i;
    }
#pragma unroll
    for (int x = 0; x < Cfg::SQ; ++x) {
      const int i = pick(x, Cfg::NQ), p = 64 * i + lane, t = p / CHD, pc = p % CHD;
      qrow[x] = t;
      qoff[x] = 16u * (pc ^ swz(t, CHD));
      qdst[x] = Cfg::OFF_Q + 1024 * i;
    }
#pragma unroll
    for (int x = 0; x < Cfg::SK; ++x) {
      const int i = pick(x, Cfg::NK), p = 64 * i + lane, t = p / CHD, pc = p % CHD;
      krow[x] = t;
      koff[x] = 16u * (pc ^ swz_tr(t, CHD));
      kdst[x] = Cfg::OFF_K + 1024 * i;
    }
    const uint32_t row_bytes = 2u * static_cast<uint32_t>(H) * D;  // one token row of q or k
#pragma unroll
    for (int k = 0; k < Cfg::SU; ++k) {
      const int i = pick(k, Cfg::NU), p = 64 * i + lane, vl = p / CHU, pc = p % CHU;
      uoff[k] = 4u * ((Cfg::ROWS * vb + vl) * C + 4 * (pc ^ swz(vl, CHU)));
      udst[k] = Cfg::OFF_U + 1024 * i;
    }
#pragma unroll
    for (int k = 0; k < Cfg::SP; ++k) {
      const int i = pick(k, Cfg::NP), p = 64 * i + lane;
      const int pl = p / (Cfg::P_PLANE / 8), rr = p % (Cfg::P_PLANE / 8);
      int t, pc, ch;
      if (rr < Cfg::P_LO / 8) {
        t = rr / (CHC / 2);
        pc = rr % (CHC / 2);
        ch = CHC / 2;
      } else {
        t = C / 2 + (rr - Cfg::P_LO / 8) / CHC;
        pc = (rr - Cfg::P_LO / 8) % CHC;
        ch = CHC;
      }
      poff[k] = 2u * ((pl * C + t) * C + 8 * (pc ^ swz(t, ch)));
      pdst[k] = Cfg::OFF_P + 1024 * i;
    }
    // First token of chunk s and the last row a copy may read: rows past the
    // chunk repeat its last token (their outputs are never stored, and their
    // K rows meet zero rows of U), and the row stays inside the input.
    auto token_rows = [&](int s, int& tok, int& last) {
      const int sc = s < c1 ? s : c1 - 1;
      const int cl = chunk_range(sc, tok);
      tok = tok < T_total ? tok : T_total - 1;
      last = cl > 0 ? cl - 1 : 0;
      last = tok + last < T_total ? last : T_total - 1 - tok;
    };
    auto copy_wq = [&](int s) {
      const size_t slot = slot_of(s);
      const char* w = reinterpret_cast<const char*>(f.w + slot * 2 * C * D);
      int tok, last;
      token_rows(s, tok, last);
      const char* qs = reinterpret_cast<const char*>(q + (static_cast<size_t>(tok) * H + h) * D);
      unsigned char* buf = smem + ((s - c0) & 1) * Cfg::WQ_BYTES;
#pragma unroll
      for (int x = 0; x < Cfg::SW; ++x) copy16(w + woff[x], buf + wdst[x]);
#pragma unroll
      for (int x = 0; x < Cfg::SQ; ++x)
        copy16(qs + static_cast<uint32_t>(qrow[x] < last ? qrow[x] : last) * row_bytes + qoff[x],
               buf + qdst[x]);
    };
    auto copy_k = [&](int s) {
      int tok, last;
      token_rows(s, tok, last);
      const char* ks = reinterpret_cast<const char*>(k + (static_cast<size_t>(tok) * H + h) * D);
#pragma unroll
      for (int x = 0; x < Cfg::SK; ++x)
        copy16(ks + static_cast<uint32_t>(krow[x] < last ? krow[x] : last) * row_bytes + koff[x],
               smem + kdst[x]);
    };
    auto copy_upg = [&](int s) {
      const size_t slot = slot_of(s);
      const char* u = reinterpret_cast<const char*>(f.ut + slot * D * C);
      const char* p = reinterpret_cast<const char*>(f.p + slot * 2 * C * C);
#pragma unroll
      for (int k = 0; k < Cfg::SU; ++k) copy16(u + uoff[k], smem + udst[k]);
#pragma unroll
      for (int k = 0; k < Cfg::SP; ++k) copy16(p + poff[k], smem + pdst[k]);
      // gates: 512 bytes from lanes 0..31 (every wave writes the same bytes)
      if (lane < Cfg::G_BYTES / 16)
        copy16(f.gate + slot * 2 * C + 4 * lane, smem + Cfg::OFF_G + ((s - c0) & 1) * Cfg::G_BYTES);
    };
    // outputs of chunk s: this wave's share of the staged 16-byte pieces.
    // Every lane stores (rows past the chunk go to the sink), so that the
    // number of loads and stores in flight, and with it every wait count
    // below, is the same on every path.
    auto write_out = [&](int s) {
      int tok0;
      const int cl = chunk_range(s, tok0);
#pragma unroll
      for (int x = 0; x < Cfg::SO; ++x) {
        const int p = 64 * (cw + kCopyWaves * x) + lane, t = p / Cfg::OPR, pc = p % Cfg::OPR;
        const uint4 v = *reinterpret_cast<const uint4*>(smem + Cfg::OFF_O + t * Cfg::O_LD + 16 * pc);
        char* dst = t < cl ? static_cast<char*>(o) +
                                 ((static_cast<size_t>(tok0 + t) * H + h) * D + Cfg::ROWS * vb) * OB +
                                 16 * pc
                           : reinterpret_cast<char*>(f.sink) + 16 * lane;
        *reinterpret_cast<uint4*>(dst) = v;
      }
    };

    copy_wq(c0);
    copy_wq(c0 + 1);
    copy_k(c0);
    copy_upg(c0);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    copy_barrier();  // B0: chunk c0 is in LDS
    for (int s = c0; s < c1; ++s) {
      copy_barrier();  // B1: W S^T and S Q^T of chunk s are done
      copy_wq(s + 2);  // into the buffer chunk s has just released
      // K of chunk s (issued after B3 of chunk s-1) has landed, and with it
      // everything older: W, Q of chunk s+1 (issued after B1 of chunk s-1)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(Cfg::SW + Cfg::SQ));
      copy_barrier();  // B2: U and the outputs of chunk s are done and staged
      copy_upg(s + 1);
      copy_barrier();  // B3: the state update of chunk s is done
      write_out(s);    // the staging tile is rewritten only after B1 of chunk s+1
      copy_k(s + 1);
      // Ut^T, P, gates of chunk s+1 have landed (and the older W, Q of s+2)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(Cfg::SO + Cfg::SK));
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // nothing may land after the workgroup ends
    return;
  }

  // ---- compute waves ----
  const int vl = 16 * wave + c16;               // local state row of this lane
  const int vrow = Cfg::ROWS * vb + vl;         // state row held by this lane
  const size_t sbase = (static_cast<size_t>(n) * H + h) * D * D + static_cast<size_t>(vrow) * D;
  floatx4 S[ND];
#pragma unroll
  for (int jt = 0; jt < ND; ++jt)
    S[jt] = state_in ? *reinterpret_cast<const floatx4*>(state_in + sbase + 16 * jt + 4 * g4)
                     : floatx4{0.f, 0.f, 0.f, 0.f};

  if (c1 > c0) {
    const uint16_t* Kl = reinterpret_cast<const uint16_t*>(smem + Cfg::OFF_K);
    const uint16_t* Pl = reinterpret_cast<const uint16_t*>(smem + Cfg::OFF_P);
    const float* Ul = reinterpret_cast<const float*>(smem + Cfg::OFF_U) + vl * C;
    unsigned char* Ol = smem + Cfg::OFF_O + (16 * wave + 4 * g4) * OB;
    // The state registers are carried through the loop: drain their loads
    // here, or a wait for them inside the loop would also wait for later
    // stores on every iteration.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __syncthreads();  // B0: chunk c0 is in LDS

    for (int s = c0; s < c1; ++s) {
      const float* Gl = reinterpret_cast<const float*>(smem + Cfg::OFF_G + ((s - c0) & 1) * Cfg::G_BYTES);
      const unsigned char* wq = smem + ((s - c0) & 1) * Cfg::WQ_BYTES;
      const uint16_t* Wl = reinterpret_cast<const uint16_t*>(wq + Cfg::OFF_W);
      const uint16_t* Ql = reinterpret_cast<const uint16_t*>(wq + Cfg::OFF_Q);

      // S^T as operand planes, 32 state columns per block, in natural order
      // (lane group g holds columns 32 kb + 8 g .. +7): split the two stacked D
      // tiles, then regroup with permlane swaps.  The 16x16x32 A and B
      // fragments have the same lane layout, so these registers serve as B
      // (rows of S^T) in W S^T and as A (rows of S) in S Q^T.
      bf16x8 sb[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float x[8];
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) x[e2] = S[2 * kb + e2 / 4][e2 & 3];
        split8<2>(x, sb[kb]);
#pragma unroll
        for (int p = 0; p < 2; ++p) sb[kb][p] = slot_to_natural(sb[kb][p]);
      }
      // X = W S^T (rows: tokens) and Y^T = S Q^T (rows: state rows); the four
      // token tiles are interleaved so that consecutive products are
      // independent.
      floatx4 X[NT], Yt[NT];
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        X[a] = floatx4{0.f, 0.f, 0.f, 0.f};
        Yt[a] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        bf16x8 wa[NT][2], qa[NT][1];
#pragma unroll
        for (int a = 0; a < NT; ++a) {
          const int t = 16 * a + c16;
          read_slots<2>(Wl + t * D, C * D, t, CHD, 4 * kb + g4, wa[a]);
          read_slots<1>(Ql + t * D, 0, t, CHD, 4 * kb + g4, qa[a]);
        }
        // plane pairs, smallest terms first
#pragma unroll
        for (int a = 0; a < NT; ++a) X[a] = mfma16x16x32(wa[a][1], sb[kb][0], X[a]);
#pragma unroll
        for (int a = 0; a < NT; ++a) X[a] = mfma16x16x32(wa[a][0], sb[kb][1], X[a]);
#pragma unroll
        for (int a = 0; a < NT; ++a) X[a] = mfma16x16x32(wa[a][0], sb[kb][0], X[a]);
#pragma unroll
        for (int a = 0; a < NT; ++a) Yt[a] = mfma16x16x32(sb[kb][1], qa[a][0], Yt[a]);
#pragma unroll
        for (int a = 0; a < NT; ++a) Yt[a] = mfma16x16x32(sb[kb][0], qa[a][0], Yt[a]);
      }
      __syncthreads();  // B1: W and Q may be refilled

      // U = Ut - X as operand planes (32 tokens per block, slot-permuted),
      // plain and scaled by D.  Ut^T row vl, tokens 16 a + 4 g .. +3.
      bf16x8 ub[CB][2], udb[CB][2];
#pragma unroll
      for (int kb = 0; kb < CB; ++kb) {
        floatx4 u2[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          u2[h2] = *reinterpret_cast<const floatx4*>(Ul + 4 * ((4 * (2 * kb + h2) + g4) ^ swz(vl, CHU)));
        float x[8], xd[8];
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          const int a0 = 2 * kb + e2 / 4, e = e2 & 3;
          const float u = u2[e2 / 4][e] - X[a0][e];
          x[e2] = u;
          xd[e2] = Gl[C + 16 * a0 + 4 * g4 + e] * u;
        }
        split8<2>(x, ub[kb]);
        split8<2>(xd, udb[kb]);
      }
      // O^T = Y^T diag(gamma) + U^T P^T, one 16-token tile at a time: lane
      // (c, g) ends up with token 16 a + c and state rows 4 g .. 4 g + 3 of its
      // wave's tile, staged with one write.  P is zero above the diagonal, so
      // token tile a needs the 32-blocks kb <= a / 2.
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        const int t = 16 * a + c16;
        floatx4 oa = Yt[a] * Gl[t];
        const uint16_t* prow = t < C / 2 ? Pl + t * (C / 2) : Pl + Cfg::P_LO + (t - C / 2) * C;
        const int pch = t < C / 2 ? CHC / 2 : CHC;
#pragma unroll
        for (int kb = 0; kb <= a / 2; ++kb) {
          bf16x8 pa[2];
          read_slots<2>(prow, Cfg::P_PLANE, t, pch, 4 * kb + g4, pa);
          oa = mfma16x16x32(ub[kb][1], pa[0], oa);
          oa = mfma16x16x32(ub[kb][0], pa[1], oa);
          oa = mfma16x16x32(ub[kb][0], pa[0], oa);
        }
        stage4<OUTD>(Ol + t * Cfg::O_LD, oa);
      }
      __syncthreads();  // B2: outputs staged; Ut^T and P may be refilled

      // S <- gamma_C S + (diag(D) U)^T K, as S^T = gamma_C S^T + K^T diag(D) U
      const float gam_end = Gl[C - 1];
#pragma unroll
      for (int jt = 0; jt < ND; ++jt) {
        S[jt] *= gam_end;
#pragma unroll
        for (int kb = 0; kb < CB; ++kb) {
          // K^T fragment: features 16 jt + c16, slots = tokens 32 kb + 4 g4 + e
          // and 32 kb + 16 + 4 g4 + e (transpose reads of the K rows)
          const shortx4 lo = read_tr4(Kl, D, CHD, 32 * kb, 16 * jt, c16, g4);
          const shortx4 hi = read_tr4(Kl, D, CHD, 32 * kb + 16, 16 * jt, c16, g4);
          bf16x8 ka[1] = {__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7))};
          mma_planes<1, 2>(S[jt], ka, udb[kb]);
        }
      }
      if (fixed) {
        float* fx = fixed + (static_cast<size_t>(s) * H + h) * D * D + static_cast<size_t>(vrow) * D;
#pragma unroll
        for (int jt = 0; jt < ND; ++jt)
          *reinterpret_cast<floatx4*>(fx + 16 * jt + 4 * g4) = S[jt];
      }
      __syncthreads();  // B3: K^T may be refilled
    }
  }

#pragma unroll
  for (int jt = 0; jt < ND; ++jt)
    *reinterpret_cast<floatx4*>(state_out + sbase + 16 * jt + 4 * g4) = S[jt];
}

template <int D, int C, Dt OUTD>
hipError_t scan_t(const void* q, const void* k, const int32_t* cu, const int32_t* offs,
                  const ChunkFactors& f,
                  const float* state_in, float* state_out, float* fixed, void* o, int N, int H,
                  int n_slots, int T_total, hipStream_t stream) {
  constexpr int NVB = D / (16 * kComputeWaves);
  const int64_t pairs = static_cast<int64_t>(N) * H;
  const int64_t groups = (pairs + kXcds - 1) / kXcds * kXcds * NVB;
  if (groups > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((chunk_scan_kernel<D, C, OUTD>), dim3(static_cast<unsigned>(groups)),
                     dim3(kThreads), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), cu, offs, f, state_in, state_out, fixed, o,
                     N, H, n_slots, T_total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_scan(const void* q, const void* k, const int32_t* cu_seqlens,
                             const int32_t* chunk_offsets,
                             const ChunkFactors& f, const float* state_in, float* state_out,
                             float* fixed, void* o, int N, int H, int d, int chunk, int n_slots,
                             int T_total, int out_dtype, hipStream_t stream) {
  if (chunk != 64) return hipErrorInvalidValue;
#define GDR_SCAN(D_, OUT_)                                                                      \
  return scan_t<D_, 64, OUT_>(q, k, cu_seqlens, chunk_offsets, f, state_in, state_out, fixed, o, N, \
                              H, n_slots, T_total, stream)
  if (d == 128) {
    if (out_dtype == 0) GDR_SCAN(128, Dt::BF16);
    GDR_SCAN(128, Dt::F32);
  }
  if (out_dtype == 0) GDR_SCAN(64, Dt::BF16);
  GDR_SCAN(64, Dt::F32);
#undef GDR_SCAN
}

}  // namespace gdr
