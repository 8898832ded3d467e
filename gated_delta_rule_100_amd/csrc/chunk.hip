// chunk.hip -- chunk-local precompute and chunk outputs of the chunked
// gated delta rule on gfx950.
//
// One 256-thread workgroup (4 waves) per (chunk slot, head).  For a chunk of
// c <= C tokens starting from state S0 (dv x dk):
//   G_t = sum_{s<=t} g_s,  gamma_t = exp(G_t),  Gamma_ts = exp(G_t - G_s) (s <= t),
//   D_s = exp(G_C - G_s)                         (every exponent <= 0)
//   A_ts = beta_t Gamma_ts (k_t . k_s)  (s < t)
//   (I + A) W = diag(beta gamma) K,   (I + A) Ut = diag(beta) V
//   L = Ut^T diag(D) K,   M = gamma_C I - W^T diag(D) K      (S_end = S0 M + L)
//   U = Ut - W S0^T,   O = diag(gamma) Q S0^T + (Q K^T (.) Gamma) U
// This is the recurrence S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T
// re-associated over a chunk: u_t = beta_t (v_t - alpha_t S_{t-1} k_t) obeys
// (I + A) U = diag(beta) V - diag(beta gamma) K S0^T.  The chunk-parallel split
// into local states, transfer matrices and a fixup follows the FlashInfer
// PR #3866 page ("CP delta-rule precompute optimisation for ultra-low
// parallelism"); the intra-chunk algebra is derived from the recurrence.
//
// The unit lower triangular systems are solved by block forward substitution
// over 16-row blocks: the diagonal blocks are inverted by substitution (one
// wave each, fp32), then every wave runs X_i = T_ii (B_i - sum_{j<i} A_ij X_j)
// for its own feature columns on the matrix cores.  X_j comes out of one
// 16x16x16 product in exactly the layout the next product takes as its B
// operand, so the whole solve stays in registers; only A and the T_ii are
// read from LDS.
//
// Padding: positions t >= c get g = 0, beta = 0 and zero k, v, q, which makes
// them identity steps (no effect on L, M) -- masking in the kernel instead of
// padded copies on the host (the out-of-bounds-fill idea on the FlashInfer
// PR #6291 page, "Mamba-2 SSD optimisation, round 4", code analysis 3).
//
// Products run on v_mfma_f32_16x16x{16,32}_bf16 with fp32 operands split into
// bf16 planes (mfma_planes.h).  L and M are written in the orientation of the
// recurrence: slot c holds M_c[a][b] at row a, column b (S_end = S0 M_c + L_c).
#include "launch.h"
#include "mfma_planes.h"

namespace gdr {
namespace {

template <int D, int C, Dt IN, bool OUT, bool TF = false>
struct ChunkCfg {
  static constexpr int Cp = C < 32 ? 32 : C;              // contraction extent over the chunk
  static constexpr int PI = IN == Dt::BF16 ? 1 : 3;       // planes of q, k, v
  static constexpr int PT = IN == Dt::BF16 ? 2 : 3;       // planes of fp32 intermediates
  static constexpr int NT = C / 16;                       // 16-row blocks along the chunk
  static constexpr int ND = D / 16;                       // 16-wide tiles along features
  static constexpr int DPW = ND / 4;                      // feature tiles per wave
  static constexpr int KB = D / 32;                       // 32-deep blocks along features
  static constexpr int CB = Cp / 32;                      // 32-deep blocks along the chunk
  static constexpr int NOFF = NT * (NT - 1) / 2;          // strictly lower 16x16 blocks
  static constexpr int LDP = Cp + 8;                      // row stride of P planes
  static constexpr int LDD = D + 8;                       // row stride of W planes (16-byte reads)
  static constexpr int LDB = 24;                          // row stride of 16x16 block planes
  static constexpr int CHD = D / 8;                       // 16-byte chunks per K/V row
  static constexpr int KR_PS = Cp * D;                    // K, V rows per plane (dense, swz_tr)
  static constexpr int P_PS = C * LDP;
  static constexpr int W_PS = C * LDD;
  static constexpr int BLK_PS = 16 * LDB;
  static constexpr int r16(int x) { return (x + 15) / 16 * 16; }
  static constexpr int mx(int a, int b) { return a > b ? a : b; }
  static constexpr int KT_BYTES = TF ? 0 : r16(PI * KR_PS * 2);
  static constexpr int KV_BYTES = 2 * KT_BYTES;
  static constexpr int W_BYTES = r16(PT * W_PS * 2);
  // lower-triangular C x C matrix, compact: rows t < C/2 keep C/2 columns
  static constexpr int TL_PLANE = (C / 2) * (C / 2) + (C / 2) * C;
  static constexpr int TL_BYTES = TF ? r16(PT * TL_PLANE * 2) : 0;
  static constexpr int KVW_BYTES = TF ? TL_BYTES : OUT ? mx(KV_BYTES, W_BYTES) : KV_BYTES;
  static constexpr int AOFF_BYTES = r16(mx(NOFF, 1) * PT * BLK_PS * 2);
  static constexpr int LDA = 20;                          // row stride of A_ii (16-byte rows)
  static constexpr int DIAG_BLK = r16(mx(16 * LDA * 4, PT * BLK_PS * 2));  // A_ii fp32, then T_ii planes
  static constexpr int P_BYTES = TF ? r16(TL_PLANE * 2) : OUT ? r16(PT * P_PS * 2) : 0;
  static constexpr int GATE_BYTES = (6 * C + 4) * 4;  // six vectors and a spare slot
  static constexpr int OFF_KR = 0;
  static constexpr int OFF_VR = KT_BYTES;
  static constexpr int OFF_W = 0;                         // W planes overlay K/V (outputs)
  static constexpr int OFF_TL = 0;                        // T planes (factors of the scan)
  static constexpr int OFF_AOFF = KVW_BYTES;
  static constexpr int OFF_DIAG = OFF_AOFF + AOFF_BYTES;
  static constexpr int OFF_P = OFF_DIAG + NT * DIAG_BLK;
  // the chunk-local kernel also solves the undecayed system (I + A') W' =
  // diag(beta) K for M: a second set of A blocks and diagonal inverses
  static constexpr bool TWO_A = !OUT && !TF;
  static constexpr int OFF_A2 = OFF_P + P_BYTES;            // A' strictly lower blocks
  static constexpr int OFF_DIAG2 = OFF_A2 + (TWO_A ? AOFF_BYTES : 0);
  static constexpr int OFF_GATE = OFF_DIAG2 + (TWO_A ? NT * DIAG_BLK : 0);
  static constexpr int BYTES = OFF_GATE + GATE_BYTES;
  static_assert(D % 64 == 0 && (C == 16 || C == 64), "shape");
};

struct ChunkTokens {
  int tok0;  // first token of the chunk
  int c;     // real length (0 = nothing to do)
  int n, j;  // sequence, chunk index within it
};

__device__ __forceinline__ ChunkTokens chunk_tokens(const int32_t* cu, const int32_t* idx,
                                                    int cid, int C, int T_total) {
  ChunkTokens r{0, 0, -1, -1};
  const int n = idx[2 * cid], j = idx[2 * cid + 1];
  if (n < 0 || j < 0) return r;
  const int a = cu[n] + j * C;
  int b = cu[n + 1];
  b = b < a + C ? b : a + C;
  if (a < 0 || b > T_total || b <= a) return r;
  r.tok0 = a;
  r.c = b - a;
  r.n = n;
  r.j = j;
  return r;
}

template <int D, int C, Dt IN, bool OUT, bool TF = false>
struct ChunkWork {
  using Cfg = ChunkCfg<D, C, IN, OUT, TF>;
  static constexpr int PI = Cfg::PI, PT = Cfg::PT, NT = Cfg::NT, DPW = Cfg::DPW, KB = Cfg::KB;

  unsigned char* smem;
  int tok0, c, h, H;
  int tid, wave, c16, g4;
  float *sg, *sb, *sG, *sgam, *sD, *sbg;

  __device__ uint16_t* Kr() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_KR); }
  __device__ uint16_t* Vr() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_VR); }
  __device__ uint16_t* Wp() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_W); }
  __device__ uint16_t* Tl() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_TL); }
  // Set 0: A (decayed) and its diagonal inverses; set 1 (chunk-local kernel
  // only): A'_ts = beta_t (k_t . k_s) without the decay and its inverses.
  __device__ uint16_t* Aoff(int blk, int set = 0) const {
    return reinterpret_cast<uint16_t*>(smem + (set ? Cfg::OFF_A2 : Cfg::OFF_AOFF)) +
           blk * PT * Cfg::BLK_PS;
  }
  __device__ float* Adiag(int i, int set = 0) const {
    return reinterpret_cast<float*>(smem + (set ? Cfg::OFF_DIAG2 : Cfg::OFF_DIAG) + i * Cfg::DIAG_BLK);
  }
  __device__ uint16_t* Tdiag(int i, int set = 0) const {
    return reinterpret_cast<uint16_t*>(smem + (set ? Cfg::OFF_DIAG2 : Cfg::OFF_DIAG) +
                                       i * Cfg::DIAG_BLK);
  }
  __device__ uint16_t* Pp() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_P); }

  __device__ void init(unsigned char* s, int tok0_, int c_, int h_, int H_) {
    smem = s;
    tok0 = tok0_;
    c = c_;
    h = h_;
    H = H_;
    tid = threadIdx.x;
    wave = tid >> 6;
    c16 = tid & 15;
    g4 = (tid & 63) >> 4;
    float* gate = reinterpret_cast<float*>(s + Cfg::OFF_GATE);
    sg = gate;
    sb = gate + C;
    sG = gate + 2 * C;
    sgam = gate + 3 * C;
    sD = gate + 4 * C;
    sbg = gate + 5 * C;
  }

  __device__ size_t tok_off(int t) const { return (static_cast<size_t>(tok0 + t) * H + h) * D; }

  // 8 consecutive features of token row t (zeros past the chunk) as planes.
  __device__ void row_frag(const void* base, int t, int k0, bf16x8 (&out)[PI]) const {
    const bool ok = t < c;
    load_global8<IN, PI>(base, ok ? tok_off(t) + k0 : 0, ok, out);
  }

  // Row fragments (8 consecutive features of one token row) of every chunk
  // row, for the Gram products; zeros past the chunk.
  __device__ void rows_frags(const void* base, bf16x8 (&f)[NT][KB][PI]) const {
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int t = 16 * ti + c16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        load_global8<IN, PI>(base, t < c ? tok_off(t) + 32 * kb + 8 * g4 : 0, t < c, f[ti][kb]);
    }
  }

  // Row fragments of K for the Gram products from the planes load() staged in
  // LDS (the same values rows_frags would load, without a second, scattered
  // read of K from global memory).  Call after load().
  __device__ void k_frags_lds(bf16x8 (&f)[NT][KB][PI]) const {
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int t = 16 * ti + c16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int off = t * D + 8 * ((4 * kb + g4) ^ swz_tr(t, Cfg::CHD));
#pragma unroll
        for (int p = 0; p < PI; ++p)
          f[ti][kb][p] = *reinterpret_cast<const bf16x8*>(Kr() + p * Cfg::KR_PS + off);
      }
    }
  }

  // K and V rows as planes (row-major, zero for t >= c, 16-byte chunks
  // permuted by swz_tr for the transpose reads), gates and their prefix
  // quantities.  Every global load is issued before the first LDS write; a
  // 16-byte load becomes one 16-byte LDS write per plane, and bf16 inputs are
  // stored bit for bit.
  __device__ void load(const void* k, const void* v, const float* g, const float* beta) {
    constexpr int G8 = D / 8;
    constexpr int ITER = Cfg::Cp * G8 / 256;
    static_assert(Cfg::Cp * G8 % 256 == 0, "load tiling");
    constexpr int NW = IN == Dt::BF16 ? 1 : 2;  // 16-byte words per 8 elements
    constexpr int ESZ = IN == Dt::BF16 ? 2 : 4;
    uint4 rk[ITER][NW], rv[ITER][NW];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int idx = tid + 256 * it;
      const int t = idx / G8, d0 = (idx % G8) * 8;
      const bool ok = t < c;
      const size_t off = ok ? tok_off(t) + d0 : 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        rk[it][w] = ok ? reinterpret_cast<const uint4*>(static_cast<const char*>(k) + off * ESZ)[w]
                       : make_uint4(0, 0, 0, 0);
        rv[it][w] = ok ? reinterpret_cast<const uint4*>(static_cast<const char*>(v) + off * ESZ)[w]
                       : make_uint4(0, 0, 0, 0);
      }
    }
    float gv, bv;
    read_gates(g, beta, gv, bv);
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int idx = tid + 256 * it;
      const int t = idx / G8, ch = idx % G8;
      const int dst = t * D + 8 * (ch ^ swz_tr(t, G8));
      if constexpr (IN == Dt::BF16) {
        *reinterpret_cast<uint4*>(Kr() + dst) = rk[it][0];
        *reinterpret_cast<uint4*>(Vr() + dst) = rv[it][0];
      } else {
        float xk[8], xv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xk[e] = __uint_as_float((&rk[it][e / 4].x)[e % 4]);
          xv[e] = __uint_as_float((&rv[it][e / 4].x)[e % 4]);
        }
        bf16x8 pk[PI], pv[PI];
        split8<PI>(xk, pk);
        split8<PI>(xv, pv);
#pragma unroll
        for (int p = 0; p < PI; ++p) {
          *reinterpret_cast<bf16x8*>(Kr() + p * Cfg::KR_PS + dst) = pk[p];
          *reinterpret_cast<bf16x8*>(Vr() + p * Cfg::KR_PS + dst) = pv[p];
        }
      }
    }
    finish_gates(gv, bv);
  }

  // g_t and beta_t of this thread's token (the chunk's last token past it), as
  // load() reads them; finish_gates() zeroes the padding.  Every thread loads,
  // with no branch, so the wait counts for these and later loads stay exact.
  __device__ void read_gates(const float* g, const float* beta, float& gv, float& bv) const {
    const size_t i = static_cast<size_t>(tok0 + (tid < c ? tid : c - 1)) * H + h;
    gv = g[i];
    bv = beta[i];
  }

  // Gates into LDS (zero past the chunk) and their prefix quantities G, gamma,
  // D, beta gamma.  The padding is zeroed by a multiplication, not a select on
  // the loaded value (which the compiler would turn back into a conditional
  // load), and every thread writes (threads past C to the spare slot), so no
  // branch sits between the loads of gv, bv and their use.
  __device__ void finish_gates(float gv, float bv) {
    const float keep = tid < c && tid < C ? 1.f : 0.f;
    float* spare = sg + 6 * C;
    *(tid < C ? sg + tid : spare) = gv * keep;
    *(tid < C ? sb + tid : spare + 1) = bv * keep;
    lds_barrier();  // row loads may stay in flight
    if (tid < C) {
      // Inclusive prefix over the chunk's lanes (one wave; a fixed shuffle
      // tree, so the result is deterministic), accumulated in fp64: the decays
      // e^{G} have a relative error equal to the absolute error of G, and an
      // fp32 prefix over 64 gates carries about |G| 2^-24 per step (about 1e-5
      // at G = -55), which would show in gamma_C and so in M.  Every lane takes
      // G_C from the last lane.  gamma and D come from the fp64 sums, rounded
      // once.
      double Gt = static_cast<double>(sg[tid]);
#pragma unroll
      for (int off = 1; off < C; off <<= 1) {
        const double y = __shfl_up(Gt, off, C);
        if ((tid & (C - 1)) >= off) Gt += y;
      }
      const double G = __shfl(Gt, C - 1, C);
      const float gam = static_cast<float>(exp(Gt));
      sG[tid] = static_cast<float>(Gt);
      sgam[tid] = gam;
      sD[tid] = static_cast<float>(exp(G - Gt));
      sbg[tid] = sb[tid] * gam;
    }
    lds_barrier();
  }

  // A_ts = beta_t Gamma_ts (k_t . k_s), s < t: diagonal blocks in fp32
  // (zero on and above the diagonal), strictly lower blocks as planes; in the
  // chunk-local kernel also A'_ts = beta_t (k_t . k_s) (set 1).
  __device__ void gram_kk(const bf16x8 (&kf)[NT][KB][PI]) {
    int tcount = 0;
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
#pragma unroll
      for (int tj = 0; tj <= ti; ++tj, ++tcount) {
        if ((tcount & 3) != wave) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma_planes<PI, PI>(acc, kf[ti][kb], kf[tj][kb]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          const int t = 16 * ti + r, s = 16 * tj + c16;
          const float a1 = s < t ? sb[t] * acc[e] : 0.f;
          const float a = s < t ? a1 * expf(sG[t] - sG[s]) : 0.f;
#pragma unroll
          for (int set = 0; set < (Cfg::TWO_A ? 2 : 1); ++set) {
            const float x = set ? a1 : a;
            if (ti == tj) {
              Adiag(ti, set)[r * Cfg::LDA + c16] = x;
            } else {
              uint16_t sp[PT];
              split_planes<PT>(x, sp);
              uint16_t* blk = Aoff(ti * (ti - 1) / 2 + tj, set);
#pragma unroll
              for (int p = 0; p < PT; ++p) blk[p * Cfg::BLK_PS + r * Cfg::LDB + c16] = sp[p];
            }
          }
        }
      }
    }
  }

  // P = (Q K^T) (.) Gamma (s <= t, zero elsewhere and in padding columns), planes.
  __device__ void gram_qk(const bf16x8 (&qf)[NT][KB][PI], const bf16x8 (&kf)[NT][KB][PI]) {
#pragma unroll
    for (int tile = 0; tile < NT * NT; ++tile) {
      if ((tile & 3) != wave) continue;
      const int ti = tile / NT, tj = tile % NT;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      if (tj <= ti) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma_planes<PI, PI>(acc, qf[ti][kb], kf[tj][kb]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ti + 4 * g4 + e, s = 16 * tj + c16;
        const float x = s <= t ? acc[e] * expf(sG[t] - sG[s]) : 0.f;
        uint16_t sp[PT];
        split_planes<PT>(x, sp);
#pragma unroll
        for (int p = 0; p < PT; ++p) Pp()[p * Cfg::P_PS + t * Cfg::LDP + s] = sp[p];
      }
    }
    if constexpr (Cfg::Cp > C) {
      for (int idx = tid; idx < C * (Cfg::Cp - C); idx += 256) {
        const int t = idx / (Cfg::Cp - C), s = C + idx % (Cfg::Cp - C);
#pragma unroll
        for (int p = 0; p < PT; ++p) Pp()[p * Cfg::P_PS + t * Cfg::LDP + s] = 0;
      }
    }
  }

  // Gamma_ts = e^{G_t - G_s} on the hardware base-2 exponential: with the
  // difference scaled by log2(e) in fp32 the relative error is about
  // |G_t - G_s| * 2^-24 (a few 1e-6 at the largest in-chunk decays), far below
  // the bf16 plane split that follows.  Evaluated for every element, with the
  // triangle applied by a select, so that no branch separates the LDS reads
  // from their use.
  static __device__ __forceinline__ float decay(float Gt, float Gs) {
    return __builtin_amdgcn_exp2f((Gt - Gs) * 1.4426950408889634f);
  }

  // Both Gram products of the scan factors, with the operands swapped so that
  // a lane holds four consecutive columns of one row (row 16 ti + c, columns
  // 16 tj + 4 g .. +3), which go to LDS as one 8-byte write per plane:
  //   A_ts = beta_t Gamma_ts (k_t . k_s), s < t: diagonal blocks fp32 (zero on
  //     and above the diagonal), strictly lower blocks as planes;
  //   P = (Q K^T) (.) Gamma (s <= t, zero elsewhere) as one fp16 plane of
  //     kPScale P (round to nearest even) in the compact lower layout (rows
  //     t < C/2 keep C/2 columns), each row in operand-slot
  //     order: column 16 tj + c of 32-block tj/2 sits at slot
  //     8 (c/4) + 4 (tj % 2) + c % 4; in LDS the 16-byte pieces of a row are
  //     permuted (tl_piece).
  __device__ void gram_t(const bf16x8 (&kf)[NT][KB][PI], const bf16x8 (&qf)[NT][KB][PI]) {
    static_assert(TF, "factors layout");
    int tcount = 0;
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
#pragma unroll
      for (int tj = 0; tj <= ti; ++tj, ++tcount) {
        if ((tcount & 3) != wave) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma_planes<PI, PI>(acc, kf[tj][kb], kf[ti][kb]);
        const int t = 16 * ti + c16;
        const float bt = sb[t], Gt = sG[t];
        const floatx4 Gs = *reinterpret_cast<const floatx4*>(sG + 16 * tj + 4 * g4);
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = 16 * tj + 4 * g4 + e;
          const float x = bt * decay(Gt, Gs[e]) * acc[e];
          a[e] = s < t ? x : 0.f;
        }
        if (ti == tj) {
          *reinterpret_cast<floatx4*>(Adiag(ti) + c16 * Cfg::LDA + 4 * g4) = floatx4{a[0], a[1], a[2], a[3]};
        } else {
          uint32_t lo[PT], hi[PT];
          split2<PT>(a[0], a[1], lo);
          split2<PT>(a[2], a[3], hi);
          uint16_t* blk = Aoff(ti * (ti - 1) / 2 + tj) + c16 * Cfg::LDB + 4 * g4;
#pragma unroll
          for (int p = 0; p < PT; ++p)
            *reinterpret_cast<uint2*>(blk + p * Cfg::BLK_PS) = make_uint2(lo[p], hi[p]);
        }
      }
    }
    int pcount = 0;
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) {
        if (ti < NT / 2 && tj >= NT / 2) continue;  // not stored
        if ((pcount++ & 3) != wave) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if (tj <= ti) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mma_planes<PI, PI>(acc, kf[tj][kb], qf[ti][kb]);
        }
        const int t = 16 * ti + c16;
        const float Gt = sG[t];
        const floatx4 Gs = *reinterpret_cast<const floatx4*>(sG + 16 * tj + 4 * g4);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = 16 * tj + 4 * g4 + e;
          const float y = acc[e] * decay(Gt, Gs[e]);
          x[e] = s <= t ? y : 0.f;
        }
        uint32_t lo[1], hi[1];
        split2_h<1>(kPScale * x[0], kPScale * x[1], lo);
        split2_h<1>(kPScale * x[2], kPScale * x[3], hi);
        uint16_t* dst = Pp() + tl_piece(t, 4 * (tj >> 1) + g4) + 4 * (tj & 1);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo[0], hi[0]);
      }
    }
  }

  // T_ii = (I + A_ii)^{-1} for every diagonal block, by substitution in fp32
  // (wave i, lane j computes column j; lanes 16 + j do the same for A' in the
  // chunk-local kernel), stored as planes over A_ii.
  __device__ void invert_diagonal() {
    const int lane = tid & 63;
    if (wave < NT && lane < (Cfg::TWO_A ? 32 : 16)) {
      const int j = lane & 15, set = lane >> 4;
      const float* A = Adiag(wave, set);
      float a[16][16];
#pragma unroll
      for (int t = 1; t < 16; ++t)
#pragma unroll
        for (int s4 = 0; s4 < t; s4 += 4) {
          const floatx4 r = *reinterpret_cast<const floatx4*>(A + t * Cfg::LDA + s4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (s4 + e < t) a[t][s4 + e] = r[e];
        }
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) x[t] = t == j ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
#pragma unroll
        for (int t = s + 1; t < 16; ++t) x[t] = fmaf(-a[t][s], x[s], x[t]);
      }
      uint16_t* T = Tdiag(wave, set);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        uint16_t sp[PT];
        split_planes<PT>(x[t], sp);
#pragma unroll
        for (int p = 0; p < PT; ++p) T[p * Cfg::BLK_PS + t * Cfg::LDB + j] = sp[p];
      }
    }
    __syncthreads();
  }

  // Right-hand side of block row i for feature tile b in D-tile layout:
  // rows t = 16 i + 4 g4 + e, column 16 b + c16, scaled by w_t (a transpose
  // read of the K or V rows per plane).
  __device__ floatx4 rhs(const uint16_t* Xr, const float* w, int i, int b) const {
    float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PI; ++p) {
      const shortx4 v = read_tr4(Xr + p * Cfg::KR_PS, D, Cfg::CHD, 16 * i, 16 * b, c16, g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += bf16_bits_to_f32(static_cast<uint16_t>(v[e]));
    }
    floatx4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = w[16 * i + 4 * g4 + e] * x[e];
    return r;
  }

  // Slot-permuted K^T fragment (rows: features 16 bj + c16; contraction slots:
  // chunk rows 32 kb + 4 g4 + e and 32 kb + 16 + 4 g4 + e), two transpose reads
  // per plane.
  __device__ void kt_frag(int kb, int bj, bf16x8 (&out)[PI]) const {
#pragma unroll
    for (int p = 0; p < PI; ++p) {
      const uint16_t* base = Kr() + p * Cfg::KR_PS;
      const shortx4 lo = read_tr4(base, D, Cfg::CHD, 32 * kb, 16 * bj, c16, g4);
      const shortx4 hi = read_tr4(base, D, Cfg::CHD, 32 * kb + 16, 16 * bj, c16, g4);
      out[p] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }

  // Block forward substitution, all in this wave's registers, for the wave's
  // feature tiles:
  //   Ut = (I + A)^{-1} diag(beta) V, and
  //   W  = (I + A)^{-1} diag(beta gamma) K      (PRIME = false), or
  //   W' = (I + A')^{-1} diag(beta) K           (PRIME = true; A' undecayed, set 1)
  // where W = diag(gamma) W'.
  template <bool PRIME>
  __device__ void solve_wy(floatx4 (&Wacc)[NT][DPW], floatx4 (&Uacc)[NT][DPW]) const {
    constexpr int WS = PRIME ? 1 : 0;  // block set of the W system
    static_assert(!PRIME || Cfg::TWO_A, "the undecayed system needs the second block set");
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      shortx4 tii[PT], tiw[PT];
      load_lds4<PT>(Tdiag(i) + c16 * Cfg::LDB + 4 * g4, Cfg::BLK_PS, tii);
      load_lds4<PT>(Tdiag(i, WS) + c16 * Cfg::LDB + 4 * g4, Cfg::BLK_PS, tiw);
#pragma unroll
      for (int bb = 0; bb < DPW; ++bb) {
        const int b = wave + 4 * bb;
        floatx4 rw = rhs(Kr(), PRIME ? sb : sbg, i, b);
        floatx4 ru = rhs(Vr(), sb, i, b);
        floatx4 sw = {0.f, 0.f, 0.f, 0.f}, su = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < i; ++j) {
          shortx4 aij[PT], awj[PT], xw[PT], xu[PT];
          load_lds4<PT>(Aoff(i * (i - 1) / 2 + j) + c16 * Cfg::LDB + 4 * g4, Cfg::BLK_PS, aij);
          load_lds4<PT>(Aoff(i * (i - 1) / 2 + j, WS) + c16 * Cfg::LDB + 4 * g4, Cfg::BLK_PS, awj);
          split4<PT>(Wacc[j][bb], xw);
          split4<PT>(Uacc[j][bb], xu);
          mma16_planes<PT, PT>(sw, awj, xw);
          mma16_planes<PT, PT>(su, aij, xu);
        }
        rw -= sw;
        ru -= su;
        shortx4 pw[PT], pu[PT];
        split4<PT>(rw, pw);
        split4<PT>(ru, pu);
        floatx4 w = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
        mma16_planes<PT, PT>(w, tiw, pw);
        mma16_planes<PT, PT>(u, tii, pu);
        Wacc[i][bb] = w;
        Uacc[i][bb] = u;
      }
    }
  }

  // Offset of row t in the compact lower-triangular layout of a C x C plane
  // (rows t < C/2 keep their first C/2 columns, the others all C).
  static __device__ __forceinline__ int tl_row(int t) {
    return t < C / 2 ? t * (C / 2) : (C / 2) * (C / 2) + (t - C / 2) * C;
  }
  // LDS position of 16-byte piece pc of row t in the factors kernel's compact
  // planes: pieces permuted by row so that the 16 rows one write touches fall
  // into distinct banks (rows of 64 bytes: XOR (t/4) % 4; of 128: (t/2) % 8).
  static __device__ __forceinline__ int tl_piece(int t, int pc) {
    const int sw = t < C / 2 ? (t >> 2) & (C / 16 - 1) : (t >> 1) & (C / 8 - 1);
    return tl_row(t) + 8 * (pc ^ sw);
  }

  // T = (I + A)^{-1}, lower triangular, into the compact plane at Tl() (rows
  // in operand-slot order, as P): wave j forms column block j by block
  // forward substitution,
  //   T_jj from the diagonal inversion,  T_ij = -T_ii sum_{j <= m < i} A_im T_mj,
  // every block in D-tile layout, which is the B operand of the next product.
  // T is stored as one fp16 plane of kTScale T (round to nearest even; the
  // unit diagonal is exact), the operand of the scan's U = T R with R / kTScale
  // in two fp16 planes.  The blocks of the compact layout above the diagonal
  // are zeroed.
  __device__ void solve_t() {
    static_assert(NT <= 4, "one column block per wave");
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j != wave) continue;
      floatx4 X[NT];
      {
        // T_jj in D-tile layout: its planes times the identity
        shortx4 tjj[PT], id[1];
        load_lds4<PT>(Tdiag(j) + c16 * Cfg::LDB + 4 * g4, Cfg::BLK_PS, tjj);
#pragma unroll
        for (int e = 0; e < 4; ++e) id[0][e] = 4 * g4 + e == c16 ? short(0x3F80) : short(0);
        X[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        mma16_planes<PT, 1>(X[j], tjj, id);
      }
#pragma unroll
      for (int i = j + 1; i < NT; ++i) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = j; m < i; ++m) {
          shortx4 aim[PT], xm[PT];
          load_lds4<PT>(Aoff(i * (i - 1) / 2 + m) + c16 * Cfg::LDB + 4 * g4, Cfg::BLK_PS, aim);
          split4<PT>(X[m], xm);
          mma16_planes<PT, PT>(acc, aim, xm);
        }
        shortx4 tii[PT], ap[PT];
        load_lds4<PT>(Tdiag(i) + c16 * Cfg::LDB + 4 * g4, Cfg::BLK_PS, tii);
        split4<PT>(acc, ap);
        floatx4 x = {0.f, 0.f, 0.f, 0.f};
        mma16_planes<PT, PT>(x, tii, ap);
        X[i] = -x;
      }
      // column 16 j + c of 32-block j/2 sits at slot 8 (c/4) + 4 (j % 2) + c % 4
      const int col = 32 * (j >> 1) + 8 * (c16 >> 2) + 4 * (j & 1) + (c16 & 3);
#pragma unroll
      for (int i = j; i < NT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * i + 4 * g4 + e;
          Tl()[tl_piece(t, col >> 3) + (col & 7)] = f16_bits(kTScale * X[i][e]);
        }
      // blocks above the diagonal that the compact layout stores: zeros
#pragma unroll
      for (int i = 0; i < j; ++i) {
        if (i < NT / 2 && j >= NT / 2) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) Tl()[tl_piece(16 * i + 4 * g4 + e, col >> 3) + (col & 7)] = 0;
      }
    }
  }

  // Operand fragment built from D tiles: slot e' of 32-block kb is chunk row
  // 16 (2kb + e'/4) + 4 g4 + e'%4 of feature tile bb, optionally scaled by D.
  template <bool SCALE_D>
  __device__ void tile_frag(const floatx4 (&acc)[NT][DPW], int bb, int kb,
                            bf16x8 (&out)[PT]) const {
    float x[8];
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) {
      const int a0 = 2 * kb + e2 / 4;
      const int t = 16 * a0 + 4 * g4 + (e2 & 3);
      float val = 0.f;
      if (a0 < NT) {
        val = acc[a0 < NT ? a0 : 0][bb][e2 & 3];
        if (SCALE_D) val *= sD[t];
      }
      x[e2] = val;
    }
    split8<PT>(x, out);
  }
};

template <int D, int C, Dt IN>
__global__ __launch_bounds__(256) void chunk_local_kernel(
    const void* __restrict__ k, const void* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cidx, float* __restrict__ Lout, float* __restrict__ Mout, int H,
    int T_total) {
  using W_ = ChunkWork<D, C, IN, false>;
  using Cfg = typename W_::Cfg;
  __shared__ __align__(16) unsigned char smem[Cfg::BYTES];
  const int cid = blockIdx.x, h = blockIdx.y;
  const ChunkTokens ct = chunk_tokens(cu, cidx, cid, C, T_total);
  if (ct.c <= 0) return;

  W_ w;
  w.init(smem, ct.tok0, ct.c, h, H);
  {
    w.load(k, v, g, beta);
    bf16x8 kf[Cfg::NT][Cfg::KB][Cfg::PI];
    w.k_frags_lds(kf);
    w.gram_kk(kf);
  }
  __syncthreads();
  w.invert_diagonal();

  floatx4 Wacc[Cfg::NT][Cfg::DPW], Uacc[Cfg::NT][Cfg::DPW];
  w.template solve_wy<true>(Wacc, Uacc);

  // L = Ut^T diag(D) K and M = gamma_C I - W^T diag(D) K = gamma_C (I - W'^T K)
  // (W^T diag(D) = W'^T diag(gamma_t D_t) and gamma_t D_t = gamma_C: the decays
  // are scalars and factor out of the transfer matrix, which is
  // gamma_C prod_t (I - beta_t k_t k_t^T)).  Forming M from the undecayed W'
  // keeps every operand of order one, so M keeps fp32 precision when gamma_C
  // is near the bottom of the fp32 range (operands of that size would have
  // their last bf16 plane below the normal range, where the matrix cores
  // flush it).  Rows of this wave's feature tiles.
  //
  // The tiles leave in 256-byte row pieces: a wave stages four column tiles
  // (16 rows x 64 columns of L and of M) in LDS that the V rows and the A
  // blocks no longer need, and each store instruction then covers 4 rows x
  // 256 B instead of the D-tile layout's 4 rows x 64 B (which writes at about
  // 60% of the rate in an in-place copy of the same bytes).  Each wave owns
  // its staging rows and LDS accesses of a wave complete in order, so only the
  // barrier that retires V and A is needed.
  constexpr int SLD = 68;                      // padded staging row (floats)
  constexpr int STAGE = 2 * 16 * SLD;          // floats per wave: L, then M
  constexpr bool STAGED = Cfg::OFF_GATE - Cfg::OFF_VR >= 4 * STAGE * 4 && Cfg::ND % 4 == 0;
  const float gam_end = w.sgam[C - 1];
  const size_t base = (static_cast<size_t>(cid) * H + h) * D * D;
  if constexpr (STAGED) __syncthreads();  // V rows and A blocks are dead
  float* stg = reinterpret_cast<float*>(smem + Cfg::OFF_VR) + w.wave * STAGE;
#pragma unroll
  for (int bb = 0; bb < Cfg::DPW; ++bb) {
    const int b = w.wave + 4 * bb;
    bf16x8 AU[Cfg::CB][Cfg::PT], AW[Cfg::CB][Cfg::PT];
#pragma unroll
    for (int kb = 0; kb < Cfg::CB; ++kb) {
      w.template tile_frag<true>(Uacc, bb, kb, AU[kb]);
      w.template tile_frag<false>(Wacc, bb, kb, AW[kb]);
    }
    for (int bj = 0; bj < Cfg::ND; ++bj) {
      floatx4 l = {0.f, 0.f, 0.f, 0.f}, m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < Cfg::CB; ++kb) {
        bf16x8 kf[Cfg::PI];
        w.kt_frag(kb, bj, kf);
        mma_planes<Cfg::PT, Cfg::PI>(l, AU[kb], kf);
        mma_planes<Cfg::PT, Cfg::PI>(m, AW[kb], kf);
      }
      const int i0 = 16 * b + 4 * w.g4, j = 16 * bj + w.c16;
      if constexpr (STAGED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * w.g4 + e, cc = 16 * (bj & 3) + w.c16;
          stg[r * SLD + cc] = l[e];
          stg[16 * SLD + r * SLD + cc] = gam_end * ((i0 + e == j ? 1.f : 0.f) - m[e]);
        }
        if ((bj & 3) == 3) {  // four column tiles staged: 16 rows x 256 B of each
          const int lane = w.tid & 63;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + (lane >> 4), cc = 4 * (lane & 15);
            const size_t at = base + static_cast<size_t>(16 * b + r) * D + 64 * (bj >> 2) + cc;
            if (Lout)
              *reinterpret_cast<floatx4*>(Lout + at) = *reinterpret_cast<const floatx4*>(stg + r * SLD + cc);
            if (Mout)
              *reinterpret_cast<floatx4*>(Mout + at) =
                  *reinterpret_cast<const floatx4*>(stg + 16 * SLD + r * SLD + cc);
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const size_t at = base + static_cast<size_t>(i0 + e) * D + j;
          if (Lout) Lout[at] = l[e];
          if (Mout) Mout[at] = gam_end * ((i0 + e == j ? 1.f : 0.f) - m[e]);
        }
      }
    }
  }
}

template <int D, int C, Dt IN, Dt OUTD>
__global__ __launch_bounds__(256, 2) void chunk_out_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cidx, const float* __restrict__ state_in,
    const float* __restrict__ fixed, void* __restrict__ o, int H, int T_total) {
  using W_ = ChunkWork<D, C, IN, true>;
  using Cfg = typename W_::Cfg;
  constexpr int PI = Cfg::PI, PT = Cfg::PT, NT = Cfg::NT, DPW = Cfg::DPW, KB = Cfg::KB;
  __shared__ __align__(16) unsigned char smem[Cfg::BYTES];
  const int cid = blockIdx.x, h = blockIdx.y;
  const ChunkTokens ct = chunk_tokens(cu, cidx, cid, C, T_total);
  if (ct.c <= 0) return;

  W_ w;
  w.init(smem, ct.tok0, ct.c, h, H);
  {
    bf16x8 kf[NT][KB][PI], qf[NT][KB][PI];
    w.rows_frags(q, qf);
    w.load(k, v, g, beta);
    w.k_frags_lds(kf);
    w.gram_kk(kf);
    w.gram_qk(qf, kf);
  }

  // Start-state rows of this wave's feature tiles as planes, loaded early
  // (nothing before this point depends on them).
  const float* S0 = nullptr;
  if (ct.j > 0) {
    S0 = fixed + (static_cast<size_t>(cid - 1) * H + h) * D * D;
  } else if (state_in != nullptr) {
    S0 = state_in + (static_cast<size_t>(ct.n) * H + h) * D * D;
  }
  bf16x8 SB[DPW][KB][PT];
#pragma unroll
  for (int bb = 0; bb < DPW; ++bb) {
    const int i = 16 * (w.wave + 4 * bb) + w.c16;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      load_global8<Dt::F32, PT>(S0, S0 ? static_cast<size_t>(i) * D + 32 * kb + 8 * w.g4 : 0,
                                S0 != nullptr, SB[bb][kb]);
  }
  __syncthreads();
  w.invert_diagonal();

  floatx4 Wacc[NT][DPW], Uacc[NT][DPW];
  w.template solve_wy<false>(Wacc, Uacc);
  __syncthreads();  // K and V are consumed; W planes take their place

#pragma unroll
  for (int a = 0; a < NT; ++a) {
#pragma unroll
    for (int bb = 0; bb < DPW; ++bb) {
      const int b = w.wave + 4 * bb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * a + 4 * w.g4 + e, d = 16 * b + w.c16;
        uint16_t sp[PT];
        split_planes<PT>(Wacc[a][bb][e], sp);
#pragma unroll
        for (int p = 0; p < PT; ++p) w.Wp()[p * Cfg::W_PS + t * Cfg::LDD + d] = sp[p];
      }
    }
  }
  __syncthreads();  // W planes visible

  // U = Ut - W S0^T
#pragma unroll
  for (int a = 0; a < NT; ++a) {
#pragma unroll
    for (int bb = 0; bb < DPW; ++bb) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        bf16x8 wa[PT];
        load_lds8<PT>(w.Wp() + (16 * a + w.c16) * Cfg::LDD + 32 * kb + 8 * w.g4, Cfg::W_PS, wa);
        mma_planes<PT, PT>(acc, wa, SB[bb][kb]);
      }
      Uacc[a][bb] -= acc;
    }
  }

  // O = diag(gamma) Q S0^T + P U  (Q fragments re-read: cheaper than holding them)
  floatx4 Oacc[NT][DPW];
#pragma unroll
  for (int a = 0; a < NT; ++a) {
    bf16x8 qa[KB][PI];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) w.row_frag(q, 16 * a + w.c16, 32 * kb + 8 * w.g4, qa[kb]);
#pragma unroll
    for (int bb = 0; bb < DPW; ++bb) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) mma_planes<PI, PT>(acc, qa[kb], SB[bb][kb]);
#pragma unroll
      for (int e = 0; e < 4; ++e) Oacc[a][bb][e] = w.sgam[16 * a + 4 * w.g4 + e] * acc[e];
    }
  }
#pragma unroll
  for (int bb = 0; bb < DPW; ++bb) {
    bf16x8 UB[Cfg::CB][PT];
#pragma unroll
    for (int kb = 0; kb < Cfg::CB; ++kb) w.template tile_frag<false>(Uacc, bb, kb, UB[kb]);
#pragma unroll
    for (int a = 0; a < NT; ++a) {
#pragma unroll
      for (int kb = 0; kb < Cfg::CB; ++kb) {
        bf16x8 pa[PT];
        load_lds8_perm<PT>(w.Pp() + (16 * a + w.c16) * Cfg::LDP + 32 * kb + 4 * w.g4, Cfg::P_PS,
                           pa);
        mma_planes<PT, PT>(Oacc[a][bb], pa, UB[kb]);
      }
    }
  }

#pragma unroll
  for (int a = 0; a < NT; ++a) {
#pragma unroll
    for (int bb = 0; bb < DPW; ++bb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * a + 4 * w.g4 + e;
        if (t < ct.c)
          store_scalar<OUTD>(o, w.tok_off(t) + 16 * (w.wave + 4 * bb) + w.c16, Oacc[a][bb][e]);
      }
    }
  }
}

// Per-chunk factors of the sequential schedule (bf16 inputs, C = 64): the
// matrices of the chunk that do not depend on the state,
//   T = (I + A)^{-1}  and  P = (Q K^T) (.) Gamma  (both lower triangular in
//   compact rows; 16 T and 16 P as one fp16 plane each),  gamma_t,
//   D_t, beta_t / 16,
// laid out the way the scan kernel stages them.  The scan takes q, k, v
// straight from the inputs and applies the UT transform itself:
//   U = T diag(beta) (V - diag(gamma) K S0^T),
// which is (I + A) U = diag(beta) V - diag(beta gamma) K S0^T solved with the
// inverse instead of forming W and Ut here.
//
// T and P rows (operands of products whose other operand comes from D tiles)
// store their contraction index in operand-slot order: inside every 32-wide block, lane group g's eight slots
// (elements 4g..4g+3 and 16+4g..16+4g+3, the order in which D tiles stack,
// mfma_planes.h) are adjacent, so that the scan reads each fragment with one
// 16-byte load.
// Chunk rows of q and k staged in LDS for the factors kernel: dense rows of D
// bf16 whose 16-byte chunks are permuted by row (physical chunk = logical
// chunk XOR rows_swz(row)), so that the 16 rows one fragment read touches fall
// into distinct banks.
template <int CH>
__device__ __forceinline__ int rows_swz(int row) { return (row * CH / 16) & (CH - 1); }

// One 16-byte lane of a global-to-LDS copy: the 64 lanes of the wave fill the
// 1 KiB at `lds` in lane order (the LDS address must be wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}

template <int D, int C>
__global__ __launch_bounds__(256, 2) void chunk_factors_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu, const int32_t* __restrict__ cidx,
    ChunkFactors f, int H, int T_total, int max_chunks) {
  using W_ = ChunkWork<D, C, Dt::BF16, false, true>;
  using Cfg = typename W_::Cfg;
  constexpr int PT = Cfg::PT, NT = Cfg::NT, KB = Cfg::KB, TLP = Cfg::TL_PLANE, CHD = Cfg::CHD;
  static_assert(PT == 2 && Cfg::Cp == C && C == 64, "factors of the scan: bf16 inputs, C = 64");
  // The chunk's k rows then q rows are copied into LDS with whole-row copies
  // (each 1 KiB copy instruction reads 1024 / (2 D) rows in full) and read
  // back as MFMA fragments.  They occupy the start of LDS, which the T, A and
  // P planes reuse once the fragments are in registers.
  constexpr int RB_BYTES = 2 * C * D * 2;
  constexpr int NCP = RB_BYTES / 1024, CPW = NCP / 4;
  static_assert(RB_BYTES <= Cfg::OFF_GATE && NCP % 8 == 0, "row staging");
  __shared__ __align__(1024) unsigned char smem[Cfg::BYTES];
  // Heads vary fastest in dispatch order, so the workgroups in flight at once
  // read whole token rows of q and k (all heads of a chunk) rather than one
  // head's 256-byte slice of rows H * 256 bytes apart.  Chunks are produced
  // last-first: the scan reads them first-first, so the earliest chunks are
  // the most recently written (and still cache-resident) when it starts.
  const int h = blockIdx.x % H, cid = max_chunks - 1 - static_cast<int>(blockIdx.x / H);
  const ChunkTokens ct = chunk_tokens(cu, cidx, cid, C, T_total);
  if (ct.c <= 0) return;

  W_ w;
  w.init(smem, ct.tok0, ct.c, h, H);
  {
    // the gates first: loads complete in order, so their prefix overlaps the
    // row copies
    float gv, bv;
    w.read_gates(g, beta, gv, bv);
    __builtin_amdgcn_sched_barrier(0);
    // Rows past the chunk repeat its last token (their beta is zero, so they
    // leave A alone, and the P rows they produce belong to outputs that are
    // never stored).
    const int wave = __builtin_amdgcn_readfirstlane(w.wave), lane = w.tid & 63;
#pragma unroll
    for (int x = 0; x < CPW; ++x) {
      const int i = wave + 4 * x;  // copy index: k rows first, then q rows
      const int p = 64 * (i % (NCP / 2)) + lane, t = p / CHD, pc = p % CHD;
      const int tt = t < ct.c ? t : ct.c - 1;
      const uint16_t* src = static_cast<const uint16_t*>(x < CPW / 2 ? k : q) + w.tok_off(tt) +
                            8 * (pc ^ rows_swz<CHD>(t));
      dma16(src, smem + 1024 * i);
    }
    w.finish_gates(gv, bv);  // LDS-only barriers: the copies stay in flight
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies (vmcnt) and LDS ops
    lds_barrier();                  // every wave's copies have landed
    const uint16_t* rows = reinterpret_cast<const uint16_t*>(smem);
    bf16x8 kf[NT][KB][1], qf[NT][KB][1];
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int t = 16 * ti + w.c16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int off = t * D + 8 * ((4 * kb + w.g4) ^ rows_swz<CHD>(t));
        kf[ti][kb][0] = *reinterpret_cast<const bf16x8*>(rows + off);
        qf[ti][kb][0] = *reinterpret_cast<const bf16x8*>(rows + C * D + off);
      }
    }
    lds_barrier();  // the staged rows are in registers: the planes may overwrite them
    w.gram_t(kf, qf);
  }
  __syncthreads();
  w.invert_diagonal();
  w.solve_t();

  const size_t slot = static_cast<size_t>(cid) * H + h;
  if (w.tid < C) {
    float* gt = f.gate + slot * 4 * C;
    gt[w.tid] = w.sgam[w.tid];
    gt[C + w.tid] = w.sD[w.tid];
    gt[2 * C + w.tid] = w.sb[w.tid] * (1.f / kTScale);  // beta / kTScale (exact)
    gt[3 * C + w.tid] = 0.f;
  }
  __syncthreads();  // T and P planes complete
  uint16_t* tg = f.t + slot * TLP;
  uint16_t* pg = f.p + slot * TLP;
  // global piece idx (the compact layout, unpermuted) from its LDS position
  for (int idx = w.tid; idx < TLP / 8; idx += 256) {
    constexpr int LO = (C / 2) * (C / 2) / 8;  // pieces of the rows t < C/2
    const int t = idx < LO ? idx / (C / 16) : C / 2 + (idx - LO) / (C / 8);
    const int pc = idx < LO ? idx % (C / 16) : (idx - LO) % (C / 8);
    const int src = W_::tl_piece(t, pc);
    *reinterpret_cast<uint4*>(tg + 8 * idx) = *reinterpret_cast<const uint4*>(w.Tl() + src);
    *reinterpret_cast<uint4*>(pg + 8 * idx) = *reinterpret_cast<const uint4*>(w.Pp() + src);
  }
}

template <int D, int C>
hipError_t factors_t(const void* q, const void* k, const float* g, const float* beta,
                     const int32_t* cu, const int32_t* cidx, const ChunkFactors& f,
                     int max_chunks, int T_total, int H, hipStream_t stream) {
  const int64_t groups = static_cast<int64_t>(max_chunks) * H;
  if (groups > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((chunk_factors_kernel<D, C>), dim3(static_cast<unsigned>(groups)), dim3(256), 0,
                     stream, q, k, g, beta, cu, cidx, f, H, T_total, max_chunks);
  return hipGetLastError();
}

template <int D, int C, Dt IN>
hipError_t local_t(const void* k, const void* v, const float* g, const float* beta,
                   const int32_t* cu, const int32_t* cidx, float* L, float* M, int max_chunks,
                   int T_total, int H, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_local_kernel<D, C, IN>), dim3(max_chunks, H), dim3(256), 0, stream, k,
                     v, g, beta, cu, cidx, L, M, H, T_total);
  return hipGetLastError();
}

template <int D, int C, Dt IN, Dt OUTD>
hipError_t out_t(const void* q, const void* k, const void* v, const float* g, const float* beta,
                 const int32_t* cu, const int32_t* cidx, const float* state_in,
                 const float* fixed, void* o, int max_chunks, int T_total, int H,
                 hipStream_t stream) {
  hipLaunchKernelGGL((chunk_out_kernel<D, C, IN, OUTD>), dim3(max_chunks, H), dim3(256), 0,
                     stream, q, k, v, g, beta, cu, cidx, state_in, fixed, o, H, T_total);
  return hipGetLastError();
}

template <int D, int C, Dt IN>
hipError_t out_dispatch_out(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu, const int32_t* cidx,
                            const float* state_in, const float* fixed, void* o, int max_chunks,
                            int T_total, int H, int out_dtype, hipStream_t stream) {
  if (out_dtype == 0)
    return out_t<D, C, IN, Dt::BF16>(q, k, v, g, beta, cu, cidx, state_in, fixed, o, max_chunks,
                                     T_total, H, stream);
  return out_t<D, C, IN, Dt::F32>(q, k, v, g, beta, cu, cidx, state_in, fixed, o, max_chunks,
                                  T_total, H, stream);
}

}  // namespace

hipError_t launch_chunk_local(const void* k, const void* v, const float* g, const float* beta,
                              const int32_t* cu_seqlens, const int32_t* chunk_indices,
                              float* L, float* M, int max_chunks, int T_total, int H, int dk,
                              int dv, int chunk, int in_dtype, hipStream_t stream) {
  (void)dv;
  if (max_chunks <= 0) return hipSuccess;
#define GDR_LOCAL(D_, C_, IN_)                                                                  \
  return local_t<D_, C_, IN_>(k, v, g, beta, cu_seqlens, chunk_indices, L, M, max_chunks,       \
                              T_total, H, stream)
  if (in_dtype == 0) {
    if (dk == 128) {
      if (chunk == 64) GDR_LOCAL(128, 64, Dt::BF16);
      GDR_LOCAL(128, 16, Dt::BF16);
    }
    if (chunk == 64) GDR_LOCAL(64, 64, Dt::BF16);
    GDR_LOCAL(64, 16, Dt::BF16);
  }
  if (dk == 128) {
    if (chunk == 64) GDR_LOCAL(128, 64, Dt::F32);
    GDR_LOCAL(128, 16, Dt::F32);
  }
  if (chunk == 64) GDR_LOCAL(64, 64, Dt::F32);
  GDR_LOCAL(64, 16, Dt::F32);
#undef GDR_LOCAL
}

hipError_t launch_chunk_out(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens,
                            const int32_t* chunk_indices, const float* state_in,
                            const float* fixed, void* o, int max_chunks, int T_total, int H,
                            int dk, int dv, int chunk, int in_dtype, int out_dtype,
                            hipStream_t stream) {
  (void)dv;
  if (max_chunks <= 0) return hipSuccess;
#define GDR_OUT(D_, C_, IN_)                                                                    \
  return out_dispatch_out<D_, C_, IN_>(q, k, v, g, beta, cu_seqlens, chunk_indices, state_in,   \
                                       fixed, o, max_chunks, T_total, H, out_dtype, stream)
  if (in_dtype == 0) {
    if (dk == 128) {
      if (chunk == 64) GDR_OUT(128, 64, Dt::BF16);
      GDR_OUT(128, 16, Dt::BF16);
    }
    if (chunk == 64) GDR_OUT(64, 64, Dt::BF16);
    GDR_OUT(64, 16, Dt::BF16);
  }
  if (dk == 128) {
    if (chunk == 64) GDR_OUT(128, 64, Dt::F32);
    GDR_OUT(128, 16, Dt::F32);
  }
  if (chunk == 64) GDR_OUT(64, 64, Dt::F32);
  GDR_OUT(64, 16, Dt::F32);
#undef GDR_OUT
}

hipError_t launch_chunk_factors(const void* q, const void* k, const float* g, const float* beta,
                                const int32_t* cu_seqlens, const int32_t* chunk_indices,
                                const ChunkFactors& f, int max_chunks, int T_total, int H, int d,
                                int chunk, hipStream_t stream) {
  if (max_chunks <= 0) return hipSuccess;
  if (chunk != 64) return hipErrorInvalidValue;
  if (d == 128)
    return factors_t<128, 64>(q, k, g, beta, cu_seqlens, chunk_indices, f, max_chunks, T_total, H,
                              stream);
  return factors_t<64, 64>(q, k, g, beta, cu_seqlens, chunk_indices, f, max_chunks, T_total, H,
                           stream);
}

}  // namespace gdr
