// chunk.hip -- chunk-local precompute and chunk outputs of the chunked
// gated delta rule on gfx950.
//
// One 256-thread workgroup (4 waves) per (chunk slot, head).  For a chunk of
// c <= C tokens starting from state S0 (dv x dk):
//   G_t = sum_{s<=t} g_s,  gamma_t = exp(G_t),  Gamma_ts = exp(G_t - G_s) (s <= t),
//   D_s = exp(G_C - G_s)                         (every exponent <= 0)
//   A_ts = beta_t Gamma_ts (k_t . k_s)  (s < t),  T = (I + A)^{-1}
//   W = T diag(beta gamma) K,  Ut = T diag(beta) V
//   L = Ut^T diag(D) K,  M = gamma_C I - W^T diag(D) K    (S_end = S0 M + L)
//   U = Ut - W S0^T,  O = diag(gamma) Q S0^T + (Q K^T (.) Gamma) U
// This is the recurrence S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T
// re-associated over a chunk (u_t = beta_t (v_t - alpha_t S_{t-1} k_t) obeys
// (I + A) U = diag(beta) V - diag(beta gamma) K S0^T).  The chunk-parallel
// split into local states, transfer matrices and a fixup follows the
// FlashInfer PR #3866 page ("CP delta-rule precompute optimisation for ultra-
// low parallelism"); the intra-chunk algebra is derived from the recurrence.
//
// Padding: positions t >= c get g = 0, beta = 0 and zero k, v, q, which makes
// them identity steps (no effect on L, M) -- masking in the kernel instead of
// padded copies on the host (the out-of-bounds-fill idea on the FlashInfer
// PR #6291 page, "Mamba-2 SSD optimisation, round 4", code analysis 3).
//
// Matrix products run on v_mfma_f32_16x16x32_bf16 with fp32 operands split
// into bf16 planes (mfma_planes.h).  LDS holds K^T and V^T (chunk index
// contiguous), A/T in fp32, T diag(beta gamma) and T diag(beta) as planes,
// and, for the outputs, the masked decay-weighted Q K^T and W.  Outputs of
// one product that feed the next stay in registers: the W/Ut tiles of a wave
// are the A operand of L and M, and the U tiles the B operand of P U.
#include "launch.h"
#include "mfma_planes.h"

namespace gdr {
namespace {

template <int D, int C, Dt IN>
struct ChunkCfg {
  static constexpr int Cp = C < 32 ? 32 : C;              // contraction extent over the chunk
  static constexpr int PI = IN == Dt::BF16 ? 1 : 3;       // planes of q, k, v
  static constexpr int PT = IN == Dt::BF16 ? 2 : 3;       // planes of fp32 intermediates
  static constexpr int NT = C / 16;                       // 16-row tiles along the chunk
  static constexpr int ND = D / 16;                       // 16-wide tiles along features
  static constexpr int DPW = ND / 4;                      // feature tiles per wave
  static constexpr int KB = D / 32;                       // 32-deep blocks along features
  static constexpr int CB = Cp / 32;                      // 32-deep blocks along the chunk
  static constexpr int LDC = Cp + 8;                      // row stride of chunk-indexed planes
  static constexpr int LDD = D + 8;                       // row stride of W planes
  static constexpr int LDA = C + 1;                       // row stride of fp32 A / T
  static constexpr int KT_PS = D * LDC;                   // plane stride of K^T, V^T
  static constexpr int TT_PS = C * LDC;                   // plane stride of T', T'', P
  static constexpr int W_PS = C * LDD;                    // plane stride of W
  static constexpr int KT_BYTES = PI * KT_PS * 2;
  static constexpr int AF_BYTES = C * LDA * 4;
  static constexpr int TT_BYTES = PT * TT_PS * 2;
  static constexpr int RA_BYTES = ((AF_BYTES > TT_BYTES ? AF_BYTES : TT_BYTES) + 15) / 16 * 16;
  static constexpr int W_BYTES = PT * W_PS * 2;
  static constexpr int RAT_BYTES = 2 * RA_BYTES > W_BYTES ? 2 * RA_BYTES : (W_BYTES + 15) / 16 * 16;
  static constexpr int GATE_BYTES = 5 * C * 4;
  static constexpr int X_BYTES = NT > 1 ? 4 * 256 * 4 : 16;
  // layout: Kt | Vt | RA (A, then T') | RT (T, then T'') [W overlays RA+RT] | P | gates | X
  static constexpr int OFF_KT = 0;
  static constexpr int OFF_VT = OFF_KT + KT_BYTES;
  static constexpr int OFF_RA = OFF_VT + KT_BYTES;
  static constexpr int OFF_RT = OFF_RA + RA_BYTES;
  static constexpr int OFF_P = OFF_RA + RAT_BYTES;
  static constexpr int OFF_GATE_LOCAL = OFF_P;  // chunk_local has no P
  static constexpr int LOCAL_BYTES = OFF_GATE_LOCAL + GATE_BYTES + X_BYTES;
  static constexpr int OFF_GATE_OUT = OFF_P + TT_BYTES;
  static constexpr int OUT_BYTES = OFF_GATE_OUT + GATE_BYTES + X_BYTES;
  static_assert(KT_BYTES % 16 == 0 && TT_BYTES % 16 == 0, "alignment");
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

template <int D, int C, Dt IN>
struct ChunkWork {
  using Cfg = ChunkCfg<D, C, IN>;
  static constexpr int PI = Cfg::PI, PT = Cfg::PT, NT = Cfg::NT, DPW = Cfg::DPW;

  unsigned char* smem;
  int tok0, c, h, H;
  int tid, wave, c16, g4;

  __device__ uint16_t* Kt() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_KT); }
  __device__ uint16_t* Vt() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_VT); }
  __device__ float* Af() const { return reinterpret_cast<float*>(smem + Cfg::OFF_RA); }
  __device__ float* Tf() const { return reinterpret_cast<float*>(smem + Cfg::OFF_RT); }
  __device__ uint16_t* Tp() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_RA); }
  __device__ uint16_t* Tpp() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_RT); }
  __device__ uint16_t* Wp() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_RA); }
  __device__ uint16_t* Pp() const { return reinterpret_cast<uint16_t*>(smem + Cfg::OFF_P); }

  float *sg, *sb, *sG, *sgam, *sD, *X;

  __device__ void init(unsigned char* s, int gate_off, int tok0_, int c_, int h_, int H_) {
    smem = s;
    tok0 = tok0_;
    c = c_;
    h = h_;
    H = H_;
    tid = threadIdx.x;
    wave = tid >> 6;
    c16 = tid & 15;
    g4 = (tid & 63) >> 4;
    float* gate = reinterpret_cast<float*>(s + gate_off);
    sg = gate;
    sb = gate + C;
    sG = gate + 2 * C;
    sgam = gate + 3 * C;
    sD = gate + 4 * C;
    X = gate + 5 * C;
  }

  __device__ size_t tok_off(int t) const { return (static_cast<size_t>(tok0 + t) * H + h) * D; }

  // K^T, V^T planes (chunk index contiguous, zero for t >= c and t >= C),
  // gates and their prefix quantities.
  __device__ void load(const void* k, const void* v, const float* g, const float* beta) {
    constexpr int G8 = D / 8;
    for (int idx = tid; idx < Cfg::Cp * G8; idx += 256) {
      const int t = idx / G8;
      const int d0 = (idx % G8) * 8;
      float xk[8], xv[8];
      if (t < c) {
        load_vec<IN, 8>(k, tok_off(t) + d0, xk);
        load_vec<IN, 8>(v, tok_off(t) + d0, xv);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xk[e] = xv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t sk[PI], sv[PI];
        split_planes<PI>(xk[e], sk);
        split_planes<PI>(xv[e], sv);
#pragma unroll
        for (int p = 0; p < PI; ++p) {
          Kt()[p * Cfg::KT_PS + (d0 + e) * Cfg::LDC + t] = sk[p];
          Vt()[p * Cfg::KT_PS + (d0 + e) * Cfg::LDC + t] = sv[p];
        }
      }
    }
    if (tid < C) {
      const bool ok = tid < c;
      sg[tid] = ok ? g[static_cast<size_t>(tok0 + tid) * H + h] : 0.f;
      sb[tid] = ok ? beta[static_cast<size_t>(tok0 + tid) * H + h] : 0.f;
    }
    __syncthreads();
    if (tid < C) {
      // Sequential prefix in a fixed order: every thread forms the same G_C.
      float G = 0.f, Gt = 0.f;
      for (int s = 0; s < C; ++s) {
        G += sg[s];
        if (s == tid) Gt = G;
      }
      sG[tid] = Gt;
      sgam[tid] = expf(Gt);
      sD[tid] = expf(G - Gt);
    }
    __syncthreads();
  }

  // 8 consecutive features of token row t (zeros past the chunk) as planes.
  __device__ void row_frag(const void* base, int t, int k0, bf16x8 (&out)[PI]) const {
    const bool ok = t < c;
    load_global8<IN, PI>(base, ok ? tok_off(t) + k0 : 0, ok, out);
  }

  // A = strictly lower beta_t Gamma_ts (k_t . k_s), fp32, into Af.
  __device__ void gram_kk(const void* k) {
    int tcount = 0;
    for (int ti = 0; ti < NT; ++ti) {
      for (int tj = 0; tj <= ti; ++tj, ++tcount) {
        if ((tcount & 3) != wave) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < Cfg::KB; ++kb) {
          bf16x8 a[PI], b[PI];
          row_frag(k, 16 * ti + c16, 32 * kb + 8 * g4, a);
          row_frag(k, 16 * tj + c16, 32 * kb + 8 * g4, b);
          mma_planes<PI, PI>(acc, a, b);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * ti + 4 * g4 + e, s = 16 * tj + c16;
          Af()[t * Cfg::LDA + s] = s < t ? sb[t] * expf(sG[t] - sG[s]) * acc[e] : 0.f;
        }
      }
    }
  }

  // P = (Q K^T) (.) Gamma (s <= t, zero elsewhere and in padding columns), planes.
  __device__ void gram_qk(const void* q, const void* k) {
    for (int tile = wave; tile < NT * NT; tile += 4) {
      const int ti = tile / NT, tj = tile % NT;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      if (tj <= ti) {
#pragma unroll
        for (int kb = 0; kb < Cfg::KB; ++kb) {
          bf16x8 a[PI], b[PI];
          row_frag(q, 16 * ti + c16, 32 * kb + 8 * g4, a);
          row_frag(k, 16 * tj + c16, 32 * kb + 8 * g4, b);
          mma_planes<PI, PI>(acc, a, b);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ti + 4 * g4 + e, s = 16 * tj + c16;
        const float x = s <= t ? acc[e] * expf(sG[t] - sG[s]) : 0.f;
        uint16_t sp[PT];
        split_planes<PT>(x, sp);
#pragma unroll
        for (int p = 0; p < PT; ++p) Pp()[p * Cfg::TT_PS + t * Cfg::LDC + s] = sp[p];
      }
    }
    if constexpr (Cfg::Cp > C) {
      for (int idx = tid; idx < C * (Cfg::Cp - C); idx += 256) {
        const int t = idx / (Cfg::Cp - C), s = C + idx % (Cfg::Cp - C);
#pragma unroll
        for (int p = 0; p < PT; ++p) Pp()[p * Cfg::TT_PS + t * Cfg::LDC + s] = 0;
      }
    }
  }

  // T = (I + A)^{-1} (unit lower triangular), fp32, blockwise over 16x16 blocks:
  // diagonal blocks by substitution, then T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  // one block diagonal at a time.  Reads Af, writes Tf (lower blocks only).
  __device__ void solve() {
    if (wave < NT && (tid & 63) < 16) {
      const int j = tid & 15, base = 16 * wave;
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) x[t] = t == j ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
#pragma unroll
        for (int t = s + 1; t < 16; ++t)
          x[t] = fmaf(-Af()[(base + t) * Cfg::LDA + base + s], x[s], x[t]);
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) Tf()[(base + t) * Cfg::LDA + base + j] = x[t];
    }
    __syncthreads();
    for (int d = 1; d < NT; ++d) {
      const int jb = wave, ib = wave + d;
      const bool active = ib < NT;
      if (active) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float acc = 0.f;
          for (int kb = jb; kb < ib; ++kb) {
#pragma unroll
            for (int m = 0; m < 16; ++m)
              acc = fmaf(Af()[(16 * ib + r) * Cfg::LDA + 16 * kb + m],
                         Tf()[(16 * kb + m) * Cfg::LDA + 16 * jb + c16], acc);
          }
          X[wave * 256 + r * 16 + c16] = acc;
        }
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float acc = 0.f;
#pragma unroll
          for (int m = 0; m < 16; ++m)
            acc = fmaf(Tf()[(16 * ib + r) * Cfg::LDA + 16 * ib + m], X[wave * 256 + m * 16 + c16],
                       acc);
          Tf()[(16 * ib + r) * Cfg::LDA + 16 * jb + c16] = -acc;
        }
      }
      __syncthreads();
    }
  }

  // T' = T diag(beta gamma) and T'' = T diag(beta) as planes over C x Cp.
  __device__ void scale_t() {
    constexpr int NE = C * Cfg::Cp;
    constexpr int PER = (NE + 255) / 256;
    float tv[PER];
#pragma unroll
    for (int qq = 0; qq < PER; ++qq) {
      const int idx = tid + 256 * qq;
      const int t = idx / Cfg::Cp, s = idx % Cfg::Cp;
      tv[qq] = (idx < NE && s < C && s <= t) ? Tf()[t * Cfg::LDA + s] : 0.f;
    }
    __syncthreads();  // T is fully read before T'' overwrites it
#pragma unroll
    for (int qq = 0; qq < PER; ++qq) {
      const int idx = tid + 256 * qq;
      if (idx >= NE) break;
      const int t = idx / Cfg::Cp, s = idx % Cfg::Cp;
      const float bs = s < C ? sb[s] : 0.f;
      const float gs = s < C ? sgam[s] : 0.f;
      uint16_t a[PT], b[PT];
      split_planes<PT>(tv[qq] * (bs * gs), a);
      split_planes<PT>(tv[qq] * bs, b);
#pragma unroll
      for (int p = 0; p < PT; ++p) {
        Tp()[p * Cfg::TT_PS + t * Cfg::LDC + s] = a[p];
        Tpp()[p * Cfg::TT_PS + t * Cfg::LDC + s] = b[p];
      }
    }
    __syncthreads();
  }

  // W = T' K and Ut = T'' V for this wave's feature tiles (all chunk rows).
  __device__ void wy(floatx4 (&Wacc)[NT][DPW], floatx4 (&Uacc)[NT][DPW]) const {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
#pragma unroll
      for (int bb = 0; bb < DPW; ++bb) {
        const int b = wave + 4 * bb;
        floatx4 w = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < Cfg::CB; ++kb) {
          bf16x8 ta[PT], tb[PT], kf[PI], vf[PI];
          const int arow = (16 * a + c16) * Cfg::LDC + 32 * kb + 8 * g4;
          const int brow = (16 * b + c16) * Cfg::LDC + 32 * kb + 8 * g4;
          load_lds8<PT>(Tp() + arow, Cfg::TT_PS, ta);
          load_lds8<PT>(Tpp() + arow, Cfg::TT_PS, tb);
          load_lds8<PI>(Kt() + brow, Cfg::KT_PS, kf);
          load_lds8<PI>(Vt() + brow, Cfg::KT_PS, vf);
          mma_planes<PT, PI>(w, ta, kf);
          mma_planes<PT, PI>(u, tb, vf);
        }
        Wacc[a][bb] = w;
        Uacc[a][bb] = u;
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
  using Cfg = ChunkCfg<D, C, IN>;
  __shared__ __align__(16) unsigned char smem[Cfg::LOCAL_BYTES];
  const int cid = blockIdx.x, h = blockIdx.y;
  const ChunkTokens ct = chunk_tokens(cu, cidx, cid, C, T_total);
  if (ct.c <= 0) return;

  ChunkWork<D, C, IN> w;
  w.init(smem, Cfg::OFF_GATE_LOCAL, ct.tok0, ct.c, h, H);
  w.load(k, v, g, beta);
  w.gram_kk(k);
  __syncthreads();
  w.solve();
  w.scale_t();

  floatx4 Wacc[Cfg::NT][Cfg::DPW], Uacc[Cfg::NT][Cfg::DPW];
  w.wy(Wacc, Uacc);

  const float gam_end = w.sgam[C - 1];
  const size_t base = (static_cast<size_t>(cid) * H + h) * D * D;
#pragma unroll
  for (int bb = 0; bb < Cfg::DPW; ++bb) {
    const int b = w.wave + 4 * bb;
    bf16x8 AU[Cfg::CB][Cfg::PT], AW[Cfg::CB][Cfg::PT];
#pragma unroll
    for (int kb = 0; kb < Cfg::CB; ++kb) {
      w.template tile_frag<true>(Uacc, bb, kb, AU[kb]);
      w.template tile_frag<true>(Wacc, bb, kb, AW[kb]);
    }
    for (int bj = 0; bj < Cfg::ND; ++bj) {
      floatx4 l = {0.f, 0.f, 0.f, 0.f}, m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < Cfg::CB; ++kb) {
        bf16x8 kf[Cfg::PI];
        load_lds8_perm<Cfg::PI>(w.Kt() + (16 * bj + w.c16) * Cfg::LDC + 32 * kb + 4 * w.g4,
                                Cfg::KT_PS, kf);
        mma_planes<Cfg::PT, Cfg::PI>(l, AU[kb], kf);
        mma_planes<Cfg::PT, Cfg::PI>(m, AW[kb], kf);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * b + 4 * w.g4 + e, j = 16 * bj + w.c16;
        Lout[base + static_cast<size_t>(i) * D + j] = l[e];
        Mout[base + static_cast<size_t>(i) * D + j] = (i == j ? gam_end : 0.f) - m[e];
      }
    }
  }
}

template <int D, int C, Dt IN, Dt OUT>
__global__ __launch_bounds__(256) void chunk_out_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cidx, const float* __restrict__ state_in,
    const float* __restrict__ fixed, void* __restrict__ o, int H, int T_total) {
  using Cfg = ChunkCfg<D, C, IN>;
  constexpr int PI = Cfg::PI, PT = Cfg::PT, NT = Cfg::NT, DPW = Cfg::DPW;
  __shared__ __align__(16) unsigned char smem[Cfg::OUT_BYTES];
  const int cid = blockIdx.x, h = blockIdx.y;
  const ChunkTokens ct = chunk_tokens(cu, cidx, cid, C, T_total);
  if (ct.c <= 0) return;

  ChunkWork<D, C, IN> w;
  w.init(smem, Cfg::OFF_GATE_OUT, ct.tok0, ct.c, h, H);
  w.load(k, v, g, beta);
  w.gram_kk(k);
  w.gram_qk(q, k);
  __syncthreads();
  w.solve();
  w.scale_t();

  floatx4 Wacc[NT][DPW], Uacc[NT][DPW];
  w.wy(Wacc, Uacc);
  __syncthreads();  // T' and T'' are consumed; W planes take their place

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

  // Start state rows of this wave's feature tiles, as planes.
  const float* S0 = nullptr;
  if (ct.j > 0) {
    S0 = fixed + (static_cast<size_t>(cid - 1) * H + h) * D * D;
  } else if (state_in != nullptr) {
    S0 = state_in + (static_cast<size_t>(ct.n) * H + h) * D * D;
  }
  bf16x8 SB[DPW][Cfg::KB][PT];
#pragma unroll
  for (int bb = 0; bb < DPW; ++bb) {
    const int i = 16 * (w.wave + 4 * bb) + w.c16;
#pragma unroll
    for (int kb = 0; kb < Cfg::KB; ++kb)
      load_global8<Dt::F32, PT>(S0, static_cast<size_t>(i) * D + 32 * kb + 8 * w.g4,
                                S0 != nullptr, SB[bb][kb]);
  }
  __syncthreads();  // W planes visible

  // U = Ut - W S0^T
#pragma unroll
  for (int a = 0; a < NT; ++a) {
#pragma unroll
    for (int bb = 0; bb < DPW; ++bb) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < Cfg::KB; ++kb) {
        bf16x8 wa[PT];
        load_lds8<PT>(w.Wp() + (16 * a + w.c16) * Cfg::LDD + 32 * kb + 8 * w.g4, Cfg::W_PS, wa);
        mma_planes<PT, PT>(acc, wa, SB[bb][kb]);
      }
      Uacc[a][bb] -= acc;
    }
  }

  // O = diag(gamma) Q S0^T + P U
  floatx4 Oacc[NT][DPW];
#pragma unroll
  for (int a = 0; a < NT; ++a) {
#pragma unroll
    for (int bb = 0; bb < DPW; ++bb) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < Cfg::KB; ++kb) {
        bf16x8 qa[PI];
        w.row_frag(q, 16 * a + w.c16, 32 * kb + 8 * w.g4, qa);
        mma_planes<PI, PT>(acc, qa, SB[bb][kb]);
      }
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
        load_lds8_perm<PT>(w.Pp() + (16 * a + w.c16) * Cfg::LDC + 32 * kb + 4 * w.g4, Cfg::TT_PS,
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
          store_scalar<OUT>(o, w.tok_off(t) + 16 * (w.wave + 4 * bb) + w.c16, Oacc[a][bb][e]);
      }
    }
  }
}

template <int D, int C, Dt IN>
hipError_t local_t(const void* k, const void* v, const float* g, const float* beta,
                   const int32_t* cu, const int32_t* cidx, float* L, float* M, int max_chunks,
                   int T_total, int H, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_local_kernel<D, C, IN>), dim3(max_chunks, H), dim3(256), 0, stream, k,
                     v, g, beta, cu, cidx, L, M, H, T_total);
  return hipGetLastError();
}

template <int D, int C, Dt IN, Dt OUT>
hipError_t out_t(const void* q, const void* k, const void* v, const float* g, const float* beta,
                 const int32_t* cu, const int32_t* cidx, const float* state_in,
                 const float* fixed, void* o, int max_chunks, int T_total, int H,
                 hipStream_t stream) {
  hipLaunchKernelGGL((chunk_out_kernel<D, C, IN, OUT>), dim3(max_chunks, H), dim3(256), 0, stream,
                     q, k, v, g, beta, cu, cidx, state_in, fixed, o, H, T_total);
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
  if (dk == 128) GDR_LOCAL(128, 16, Dt::F32);
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
  if (dk == 128) GDR_OUT(128, 16, Dt::F32);
  GDR_OUT(64, 16, Dt::F32);
#undef GDR_OUT
}

}  // namespace gdr
