// The unmasked second-order HLA forward, o_t = q_t^T S_t C_t
// ("Higher-order Linear Attention", arXiv 2510.27258, summaries on
// gist.science: method section 1 -- the plain product of the key moment and
// the query-value accumulator, before the cross summaries remove its future
// terms; key contribution 2 -- associative operators for the unmasked
// setting, with and without decay; method section 4 -- segment summaries
// joined by an exclusive scan).
//
// With decay g per head (S, C, m each decay once per token), 0-based
// positions tau, i, j inside a tile of Lt tokens and the tile's starting
// state (S, C, m):
//   p_tau   = g^(tau+1) S q_tau + sum_{i<=tau} g^(tau-i) (q_tau.k_i) k_i   (= S_tau q_tau)
//   num_tau = g^(tau+1) C^T p_tau + sum_{j<=tau} g^(tau-j) (p_tau.q_j) v_j (= C_tau^T p_tau)
//   den_tau = g^(tau+1) p_tau.m   + sum_{j<=tau} g^(tau-j) (p_tau.q_j)
//   S <- g^Lt S + K^T diag(w) K,  C <- g^Lt C + Q^T diag(w) V,  m <- g^Lt m + Q^T w,
//   w_i = g^(Lt-1-i).
// A segment's summary is (S, C, m) reached from zero; the combine has no
// cross term (S = a S_A + S_B, likewise C and m, a = g^(length of B)), so the
// exclusive scan is a decayed running sum over the segments of a unit,
// element by element.
//
// One workgroup owns one segment of one (batch, head) unit.  Its waves split
// into S waves (column blocks of S; they produce the matching columns of P
// and update S) and C waves (column blocks of C; they produce the matching
// columns of the output and update C and m).  The state lives in fp32 MFMA
// accumulators; P goes through LDS (row-major, bf16 for bf16 inputs) for the
// score tiles and the state term C^T p.  Q, K and V are double-buffered by
// tile parity: the next tile is loaded into registers one tile ahead and
// staged while the current one is in use.  Three barriers per tile in the
// output kernel; with bf16 inputs (P double-buffered) the C waves produce a
// tile's outputs and apply its C and m updates one tile late, beside the S
// waves' P and S update of the next tile: [P, S update of t | outputs, C and m
// updates of t - 1] -> [p.m, B scores of t; staging of t + 1] -> [A' of t + 1].
#include <type_traits>

#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int UT = 64;   // tokens per tile

enum { U_SUMMARY = 0, U_OUTPUT = 1 };

template <typename T, int D, int E>
struct ULayout {
  static constexpr int PADT = 16 / (int)sizeof(T);
  static constexpr int DP = D < MM<T>::KS ? MM<T>::KS : D;   // d zero-padded to one MFMA K step
  static constexpr int LDD = DP + PADT;   // Q, K, P: [tok][d]
  static constexpr int LDV = E + PADT;    // V: [tok][e]
  static constexpr int LDT = UT + PADT;   // A', B: [tok][tok]
  static constexpr size_t QB = (size_t)UT * LDD * sizeof(T);
  static constexpr size_t VB = (size_t)UT * LDV * sizeof(T);
  // Q, K, V double-buffered by tile parity: the next tile is staged while the
  // current one is in use, and the C update of a tile runs one tile late
  static constexpr size_t Qs = 0, Ks = 2 * QB, Vs = 4 * QB;
  // bf16: P double-buffered, so that a tile's outputs (C waves) run beside the
  // next tile's P (S waves); fp32 tiles leave no room for a second P buffer
  static constexpr bool DEFER = sizeof(T) == 2;
  static constexpr int NPS = DEFER ? 2 : 1;
  static constexpr size_t Ps = Vs + 2 * VB;
  static constexpr size_t AB = Ps + NPS * QB;
  static constexpr size_t BB = AB + (size_t)UT * LDT * sizeof(T);
  static constexpr size_t TILE_END = BB + (size_t)UT * LDT * sizeof(T);
  static constexpr size_t W = (TILE_END + 15) / 16 * 16;
  // pw, w1, wS[2], pm [UT]; bpart [UT/16][UT]; mst [D]
  static constexpr size_t TOTAL = W + (size_t)(5 * UT + (UT / 16) * UT + D) * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
};

template <typename T>
__device__ __forceinline__ void ustore4(T* p, f32x4 x);
template <>
__device__ __forceinline__ void ustore4<__bf16>(__bf16* p, f32x4 x) {
  bf16x4 y;
  y[0] = (__bf16)x[0]; y[1] = (__bf16)x[1]; y[2] = (__bf16)x[2]; y[3] = (__bf16)x[3];
  *reinterpret_cast<bf16x4*>(p) = y;
}
template <>
__device__ __forceinline__ void ustore4<float>(float* p, f32x4 x) {
  *reinterpret_cast<f32x4*>(p) = x;
}

template <typename T, int D, int E, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void unmasked_kernel(ChunkArgs a) {
  constexpr int NTHR = 64 * NW;
  using L = ULayout<T, D, E>;
  using MMT = MM<T>;
  using FR = Frag<T>;
  constexpr int KS = MMT::KS, CH = MMT::CH, DP = L::DP;
  constexpr int DT = D / 16, ET = E / 16, TR = UT / 16, NKS = UT / KS;
  constexpr int NTRI = TR * (TR + 1) / 2;
  constexpr int QSK = KS == 32 ? (DT + 1) / 2 : DT * 4;   // K steps of a d-contraction
  constexpr int NOWN = NW / 2, HT = NTHR / 2;
  constexpr int SB = (DT + NOWN - 1) / NOWN, CB = (ET + NOWN - 1) / NOWN;
  // every block index is in range when the blocks divide evenly over a role
  constexpr bool SFULL = DT % NOWN == 0, CFULL = ET % NOWN == 0;
  constexpr bool OUT = MODE == U_OUTPUT;

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  auto Qb = [&](int p) { return reinterpret_cast<T*>(smem + L::Qs + p * L::QB); };
  auto Kb = [&](int p) { return reinterpret_cast<T*>(smem + L::Ks + p * L::QB); };
  auto Vb = [&](int p) { return reinterpret_cast<T*>(smem + L::Vs + p * L::VB); };
  auto Psb = [&](int p) { return reinterpret_cast<T*>(smem + L::Ps + (L::NPS == 2 && p ? L::QB : 0)); };
  T* AB = reinterpret_cast<T*>(smem + L::AB);
  T* BB = reinterpret_cast<T*>(smem + L::BB);
  float* pw = reinterpret_cast<float*>(smem + L::W);
  float* w1 = pw + UT;
  auto wSb = [&](int p) { return w1 + UT + p * UT; };
  float* pm = w1 + 3 * UT;
  float* bpart = pm + UT;
  float* mst = bpart + TR * UT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg4 = lane >> 4;
  const bool sRole = wave < NOWN;
  const int rw = sRole ? wave : wave - NOWN;
  const int nspan = a.nspan;
  const int unit = blockIdx.x / nspan, span = blockIdx.x - unit * nspan;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float lgg = log2f(g);
  const int Lspan = a.chunk;
  const size_t tok0 = (size_t)unit * (size_t)a.T + (size_t)span * (size_t)Lspan;
  const T* gq = reinterpret_cast<const T*>(a.q) + tok0 * D;
  const T* gk = reinterpret_cast<const T*>(a.k) + tok0 * D;
  const T* gv = reinterpret_cast<const T*>(a.v) + tok0 * E;
  const size_t sidx = (size_t)unit * nspan + span;
  const int ntiles = (Lspan + UT - 1) / UT;
  auto tile_len = [&](int ti) { return (Lspan - ti * UT) < UT ? (Lspan - ti * UT) : UT; };

  // zero the tile region once: padding columns [D, DP) of Q, K, P and the
  // upper score tiles are read as zeros and never written
  for (size_t i = tid; i < L::TILE_END / 16; i += NTHR)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  if (tid < UT) {
    pw[tid] = gpow(g, lgg, tid);
    w1[tid] = gpow(g, lgg, tid + 1);
  }
  for (int i = tid; i < D; i += NTHR) mst[i] = OUT ? a.m[sidx * D + i] : 0.f;

  // the role's state: S waves hold S[:, 16 cb + lr], C waves C[:, 16 ce + lr]
  // (accumulator tiles t over rows 16 t + 4 lg4 + [0, 4)), from the prefix or zero
  constexpr int NB = SB > CB ? SB : CB;
  f32x4 St[NB][DT];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int cb = rw + NOWN * b;
    const bool own = sRole ? (b < SB && cb < DT) : (b < CB && cb < ET);
    const float* src = sRole ? a.S + sidx * D * D : a.C + sidx * D * E;
    const int ld = sRole ? D : E;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        St[b][t][j] = (OUT && own) ? src[(size_t)(16 * t + 4 * lg4 + j) * ld + 16 * cb + lr] : 0.f;
  }

  // ---- tile staging through registers: 16-byte chunks of Q, K and V, each
  // buffer in a loop of its own (a buffer chosen per lane at run time would
  // put a table of pointers in scratch memory); rows past the segment end
  // read as zeros ----
  constexpr int QCH = UT * D / CH, VCH = UT * E / CH;
  constexpr int NQ = (QCH + NTHR - 1) / NTHR, NV = (VCH + NTHR - 1) / NTHR;
  uint4 xq[NQ], xk[NQ], xv[NV];
  auto load_rows = [&](uint4* x, auto n, const T* src, int W, int nch, int t0, int Lt) {
#pragma unroll
    for (int i = 0; i < decltype(n)::value; ++i) {
      const int c = tid + NTHR * i;
      const int row = c / (W / CH), col = (c % (W / CH)) * CH;
      x[i] = make_uint4(0, 0, 0, 0);
      if (c < nch && row < Lt) x[i] = *reinterpret_cast<const uint4*>(src + (size_t)(t0 + row) * W + col);
    }
  };
  auto store_rows = [&](const uint4* x, auto n, T* dst, int W, int LD, int nch) {
#pragma unroll
    for (int i = 0; i < decltype(n)::value; ++i) {
      const int c = tid + NTHR * i;
      const int row = c / (W / CH), col = (c % (W / CH)) * CH;
      if (c < nch) *reinterpret_cast<uint4*>(dst + row * LD + col) = x[i];
    }
  };
  using NQc = std::integral_constant<int, NQ>;
  using NVc = std::integral_constant<int, NV>;
  auto load_tile = [&](int ti) {
    const int t0 = ti * UT, Lt = tile_len(ti);
    load_rows(xq, NQc{}, gq, D, QCH, t0, Lt);
    load_rows(xk, NQc{}, gk, D, QCH, t0, Lt);
    load_rows(xv, NVc{}, gv, E, VCH, t0, Lt);
  };
  auto store_tile = [&](int p) {
    store_rows(xq, NQc{}, Qb(p), D, L::LDD, QCH);
    store_rows(xk, NQc{}, Kb(p), D, L::LDD, QCH);
    store_rows(xv, NVc{}, Vb(p), E, L::LDV, VCH);
  };
  // update weights w_i = g^(Lt-1-i) of tile ti (0 past its end)
  auto set_weights = [&](int ti) {
    const int Lt = tile_len(ti);
    if (tid < UT) wSb(ti & 1)[tid] = tid < Lt ? gpow(g, lgg, Lt - 1 - tid) : 0.f;
  };

  // A'[tau][i] = g^(tau-i) q_tau.k_i (i <= tau) of the tile in buffers p, score
  // tiles first, first + stride, ... of this wave
  auto a_tiles = [&](int p, int first, int stride) {
    const T* Qx = Qb(p);
    const T* Kx = Kb(p);
    for (int idx = first; idx < NTRI; idx += stride) {
      int r, c;
      tri_block(idx, r, c);
      f32x4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DP; k0 += KS)
        acc = MMT::mma(MMT::ld(Kx, L::LDD, 16 * c, k0, lane), MMT::ld(Qx, L::LDD, 16 * r, k0, lane), acc);
      const int tau = 16 * r + lr;   // lane: position tau, keys i = 16 c + 4 lg4 + j
      f32x4 val;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * c + 4 * lg4 + j;
        val[j] = acc[j] * masked_pow(pw, tau, i);
      }
      ustore4<T>(AB + tau * L::LDT + 16 * c + 4 * lg4, val);
    }
  };
  // S waves: S[:, own] <- g^Lt S + K^T diag(w) K[:, own] for the tile in buffers p
  auto s_update = [&](int p, float gL) {
    const T* Kx = Kb(p);
    const float* wS = wSb(p);
    typename MMT::F bk[SB][NKS];
#pragma unroll
    for (int b = 0; b < SB; ++b)
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk)
        bk[b][kk] = FR::scale(FR::tr(Kx, L::LDD, kk * KS, 16 * ((rw + NOWN * b) % DT), lane), wS, kk * KS, lane);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      f32x4 acc[SB];
#pragma unroll
      for (int b = 0; b < SB; ++b) acc[b] = St[b][t] * gL;
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        const auto ak = FR::tr(Kx, L::LDD, kk * KS, 16 * t, lane);   // shared by the blocks
#pragma unroll
        for (int b = 0; b < SB; ++b) acc[b] = MMT::mma(ak, bk[b][kk], acc[b]);
      }
#pragma unroll
      for (int b = 0; b < SB; ++b)
        if (SFULL || rw + NOWN * b < DT) St[b][t] = acc[b];
    }
  };
  // C waves: C[:, own] <- g^Lt C + Q^T diag(w) V[:, own] and m <- g^Lt m + Q^T w
  // for the tile in buffers p
  auto c_update = [&](int p, float gL) {
    const T* Qx = Qb(p);
    const T* Vx = Vb(p);
    const float* wS = wSb(p);
    typename MMT::F bv[CB][NKS];
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk)
        bv[b][kk] = FR::scale(FR::tr(Vx, L::LDV, kk * KS, 16 * ((rw + NOWN * b) % ET), lane), wS, kk * KS, lane);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      f32x4 acc[CB];
#pragma unroll
      for (int b = 0; b < CB; ++b) acc[b] = St[b][t] * gL;
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        const auto aq = FR::tr(Qx, L::LDD, kk * KS, 16 * t, lane);   // shared by the blocks
#pragma unroll
        for (int b = 0; b < CB; ++b) acc[b] = MMT::mma(aq, bv[b][kk], acc[b]);
      }
#pragma unroll
      for (int b = 0; b < CB; ++b)
        if (CFULL || rw + NOWN * b < ET) St[b][t] = acc[b];
    }
    // m: TPD threads per row d, each over UT / TPD tokens in four
    // independent partial sums, then a fixed-order shuffle reduction
    constexpr int TPD = HT / D < 1 ? 1 : (HT / D > 16 ? 16 : HT / D);
    constexpr int TPT = UT / TPD;
    const int ct = tid - HT;
    if (ct >= 0 && ct < TPD * D) {
      const int d = ct / TPD, part = ct % TPD;
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int tau = part * TPT + i;
        ps[i & 3] += wS[tau] * (float)Qx[tau * L::LDD + d];
      }
      float acc = (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
      for (int off = 1; off < TPD; off *= 2) acc += __shfl_xor(acc, off, 64);
      if (part == 0) mst[d] = gL * mst[d] + acc;
    }
  };

  // ---- pieces of the output kernel ----
  // S waves: P[:, own] = g^(tau+1) Q S[:, own] + A' K[:, own] of the tile in
  // buffers p, to P buffer p
  auto p_tile = [&](int p) {
    T* Px = Psb(p);
    const T* Qx = Qb(p);
    const T* Kx = Kb(p);
    f32x4 pacc[SB][TR];
#pragma unroll
    for (int b = 0; b < SB; ++b)
#pragma unroll
      for (int r = 0; r < TR; ++r) pacc[b][r] = zero4();
#pragma unroll
    for (int kk = 0; kk < QSK; ++kk) {
      typename MMT::F bs[SB];
#pragma unroll
      for (int b = 0; b < SB; ++b) bs[b] = FR::acc_b(St[b], kk);
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const auto aq = FR::perm(Qx, L::LDD, 16 * r, kk, lane);   // shared by the blocks
#pragma unroll
        for (int b = 0; b < SB; ++b) pacc[b][r] = MMT::mma(aq, bs[b], pacc[b][r]);
      }
    }
#pragma unroll
    for (int r = 0; r < TR; ++r) {
#pragma unroll
      for (int b = 0; b < SB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) pacc[b][r][j] *= w1[16 * r + 4 * lg4 + j];
      for (int k0 = 0; k0 < 16 * r + 16; k0 += KS) {
        const auto aa = MMT::ld(AB, L::LDT, 16 * r, k0, lane);
#pragma unroll
        for (int b = 0; b < SB; ++b)
          pacc[b][r] = MMT::mma(aa, FR::tr(Kx, L::LDD, k0, 16 * ((rw + NOWN * b) % DT), lane), pacc[b][r]);
      }
      // lane: P[tau = 16 r + 4 lg4 + j][d = 16 cb + lr]
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int cb = rw + NOWN * b;
        if (SFULL || cb < DT) {
#pragma unroll
          for (int j = 0; j < 4; ++j) Px[(16 * r + 4 * lg4 + j) * L::LDD + 16 * cb + lr] = (T)pacc[b][r][j];
        }
      }
    }
  };
  // all waves: p.m and B[tau][j] = g^(tau-j) p_tau.q_j (j <= tau) of the tile in buffers p
  auto score_tile = [&](int p) {
    const T* Px = Psb(p);
    {
      constexpr int LPR = NTHR / UT;
      const int tau = tid / LPR, part = tid % LPR;
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int c = part * (D / LPR); c < (part + 1) * (D / LPR); ++c)
        ps[c & 1] += (float)Px[tau * L::LDD + c] * mst[c];
      float acc = ps[0] + ps[1];
#pragma unroll
      for (int off = 1; off < LPR; off *= 2) acc += __shfl_xor(acc, off, 64);
      if (part == 0) pm[tau] = acc;
    }
    {
      const T* Qx = Qb(p);
      for (int idx = wave; idx < NTRI; idx += NW) {
        int r, c;
        tri_block(idx, r, c);
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DP; k0 += KS)
          acc = MMT::mma(MMT::ld(Qx, L::LDD, 16 * c, k0, lane), MMT::ld(Px, L::LDD, 16 * r, k0, lane), acc);
        const int tau = 16 * r + lr;   // lane: position tau, values j = 16 c + 4 lg4 + jj
        f32x4 val;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 16 * c + 4 * lg4 + jj;
          val[jj] = acc[jj] * masked_pow(pw, tau, j);
        }
        ustore4<T>(BB + tau * L::LDT + 16 * c + 4 * lg4, val);
        const float rs = sum_rows4(val[0] + val[1] + val[2] + val[3]);
        if (lg4 == 0) bpart[c * UT + tau] = rs;
      }
    }
  };
  // C waves: O = g^(tau+1) P C + B V for tile tp (Ltp tokens, buffers pp), its
  // B scores, p.m and row sums in BB, pm, bpart; written with its den
  auto out_tile = [&](int tp, int Ltp, int pp) {
    const T* Px = Psb(pp);
    const T* Vx = Vb(pp);
    float* go = a.o + (tok0 + (size_t)tp * UT) * E;
    // O^T = C^T P^T + V^T B^T (C^T from the accumulators as the A
    // operand: the A and B layouts are alike), so that a lane holds four
    // adjacent columns of one token and stores them at once
    f32x4 oacc[CB][TR];
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
      for (int r = 0; r < TR; ++r) oacc[b][r] = zero4();
#pragma unroll
    for (int kk = 0; kk < QSK; ++kk) {
      typename MMT::F bc[CB];
#pragma unroll
      for (int b = 0; b < CB; ++b) bc[b] = FR::acc_b(St[b], kk);
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const auto bp = FR::perm(Px, L::LDD, 16 * r, kk, lane);   // shared by the blocks
#pragma unroll
        for (int b = 0; b < CB; ++b) oacc[b][r] = MMT::mma(bc[b], bp, oacc[b][r]);
      }
    }
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      const int tau = 16 * r + lr;
#pragma unroll
      for (int b = 0; b < CB; ++b) oacc[b][r] *= w1[tau];
      for (int k0 = 0; k0 < 16 * r + 16; k0 += KS) {
        const auto bb = MMT::ld(BB, L::LDT, 16 * r, k0, lane);
#pragma unroll
        for (int b = 0; b < CB; ++b)
          oacc[b][r] = MMT::mma(FR::tr(Vx, L::LDV, k0, 16 * ((rw + NOWN * b) % ET), lane), bb, oacc[b][r]);
      }
      float scale = 1.f;
      if (a.normalize) {
        float dn = w1[tau] * pm[tau];
        for (int c = 0; c <= r; ++c) dn += bpart[c * UT + tau];
        scale = 1.f / (dn + a.eps);
      }
      // lane: O[tau][e = 16 ce + 4 lg4 + j]
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const int ce = rw + NOWN * b;
        if ((CFULL || ce < ET) && tau < Ltp)
          *reinterpret_cast<f32x4*>(go + (size_t)tau * E + 16 * ce + 4 * lg4) = oacc[b][r] * scale;
      }
    }
    const int mt = tid - HT;
    if (a.den != nullptr && mt < Ltp) {
      a.den[tok0 + (size_t)tp * UT + mt] = add_lower_blocks(w1[mt] * pm[mt], bpart, UT, mt);
    }
  };

  // prologue: tile 0 to LDS, tile 1 to registers (and A' of tile 0)
  load_tile(0);
  store_tile(0);
  set_weights(0);
  __syncthreads();
  if (ntiles > 1) load_tile(1);
  if constexpr (OUT) {
    a_tiles(0, wave, NW);
    __syncthreads();
  }

  // output kernel: the C waves (outputs, C and m updates) issue first when
  // both roles are ready (measured at B4 H16 T16384 d128: 0.415 -> 0.404 ms)
  if constexpr (OUT) {
    if (!sRole) __builtin_amdgcn_s_setprio(2);
  }
  float gL_prev = 1.f;
  for (int ti = 0; ti < ntiles; ++ti) {
    const int p = ti & 1;
    const int t0 = ti * UT, Lt = tile_len(ti);
    const float gL = gpow(g, lgg, Lt);
    if constexpr (OUT && L::DEFER) {
      // [S waves: P and S update of tile ti | C waves: outputs, C and m
      // updates of tile ti - 1] -> [p.m, B scores of ti; stage ti + 1] -> [A' of ti + 1]
      if (sRole) {
        p_tile(p);
        s_update(p, gL);
      } else if (ti > 0) {
        out_tile(ti - 1, UT, p ^ 1);   // only the last tile can be short
        c_update(p ^ 1, gL_prev);
      }
      __syncthreads();
      score_tile(p);
      if (ti + 1 < ntiles) {
        store_tile(p ^ 1);
        set_weights(ti + 1);
        if (ti + 2 < ntiles) load_tile(ti + 2);
      }
      __syncthreads();
      if (ti + 1 < ntiles) {
        a_tiles(p ^ 1, wave, NW);
        __syncthreads();
      }
    } else if constexpr (OUT) {
      // [S waves: P | C waves: C and m updates of the previous tile] ->
      // [p.m, B scores; stage the next tile] -> [S waves: S update, next A' | C waves: outputs]
      if (sRole) p_tile(p);
      else if (ti > 0) c_update(p ^ 1, gL_prev);
      __syncthreads();
      score_tile(p);
      if (ti + 1 < ntiles) {
        store_tile(p ^ 1);
        set_weights(ti + 1);
        if (ti + 2 < ntiles) load_tile(ti + 2);
      }
      __syncthreads();
      if (sRole) {
        s_update(p, gL);
        if (ti + 1 < ntiles) a_tiles(p ^ 1, rw, NOWN);
      } else {
        out_tile(ti, Lt, p);
      }
      __syncthreads();
    } else {
      if (sRole) s_update(p, gL);
      else c_update(p, gL);
      if (ti + 1 < ntiles) {
        store_tile(p ^ 1);
        set_weights(ti + 1);
      }
      __syncthreads();
      if (ti + 2 < ntiles) load_tile(ti + 2);
    }
    gL_prev = gL;
  }
  if constexpr (OUT && L::DEFER) {
    if (!sRole) out_tile(ntiles - 1, tile_len(ntiles - 1), (ntiles - 1) & 1);
  }

  if constexpr (!OUT) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int cb = rw + NOWN * b;
      const bool own = sRole ? (b < SB && cb < DT) : (b < CB && cb < ET);
      float* dst = sRole ? a.S + sidx * D * D : a.C + sidx * D * E;
      const int ld = sRole ? D : E;
      if (own) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[(size_t)(16 * t + 4 * lg4 + j) * ld + 16 * cb + lr] = St[b][t][j];
      }
    }
    for (int i = tid; i < D; i += NTHR) a.m[sidx * D + i] = mst[i];
  }
}

// Exclusive decayed running sum over the n segments of each unit, in place:
// X[s] <- sum_{r<s} a^(s-1-r) X[r], a = g^chunk (the unmasked combine), for
// the three moments S, C, m ([units, n, F_i] each) in one launch: blockIdx.x
// runs over the blocks of S, then of C, then of m; each thread owns four
// consecutive floats and keeps eight segments' loads in flight.
struct UScanArgs {
  float* X[3];
  int F[3], nb[3];    // floats per segment, blocks of 256 threads
  const float* gamma;
  int H, n, chunk;
};

__global__ __launch_bounds__(256) void unmasked_scan_kernel(UScanArgs a) {
  const int unit = blockIdx.y;
  int b = blockIdx.x, f = 0;
  if (b >= a.nb[0]) {
    b -= a.nb[0];
    f = 1;
    if (b >= a.nb[1]) {
      b -= a.nb[1];
      f = 2;
    }
  }
  const int F = a.F[f];
  const int e4 = b * 256 + threadIdx.x;
  if (4 * e4 >= F) return;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float sa = gpow(g, log2f(g), a.chunk);
  f32x4 run = zero4();
  f32x4* p = reinterpret_cast<f32x4*>(a.X[f] + (size_t)unit * a.n * F) + e4;
  const size_t step = F / 4;
  constexpr int NB = 8;
  for (int s0 = 0; s0 < a.n; s0 += NB) {
    f32x4 x[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) x[i] = s0 + i < a.n ? p[(size_t)(s0 + i) * step] : zero4();
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (s0 + i < a.n) {
        p[(size_t)(s0 + i) * step] = run;
        run = run * sa + x[i];
      }
    }
  }
}

// One decode step of the unmasked variant per unit (one workgroup of UDEC
// threads): S' = g S + k k^T, C' = g C + q v^T, m' = g m + q, a = S' q,
// num = C'^T a, den = a.m'.  Every state element is read once and written
// once (16-byte non-temporal accesses); the reductions go through shuffles
// and LDS.
constexpr int UDEC = 512;

template <typename T, int D, int E>
__global__ __launch_bounds__(UDEC) void unmasked_decode_kernel(DecodeArgs a) {
  constexpr int CPR_S = D / 4, RP_S = UDEC / CPR_S, NP_S = (D + RP_S - 1) / RP_S;
  constexpr int CPR_C = E / 4, RP_C = UDEC / CPR_C, NP_C = (D + RP_C - 1) / RP_C;
  constexpr int NRG = RP_C < D ? RP_C : D;   // row groups that hold C rows
  __shared__ __attribute__((aligned(16))) float sq[D], sk[D], sv[E], sm[D], aval[D];
  __shared__ __attribute__((aligned(16))) float rz[NRG][E];
  __shared__ float sden;

  const int unit = blockIdx.x, tid = threadIdx.x;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  f32x4* S = reinterpret_cast<f32x4*>(a.S + (size_t)unit * D * D);
  f32x4* C = reinterpret_cast<f32x4*>(a.C + (size_t)unit * D * E);
  float* m = a.m + (size_t)unit * D;
  const int ccS = tid % CPR_S, rgS = tid / CPR_S;
  const int ccC = tid % CPR_C, rgC = tid / CPR_C;
  f32x4 rS[NP_S], rC[NP_C];
#pragma unroll
  for (int i = 0; i < NP_S; ++i) {
    const int d = rgS + RP_S * i;
    if (d < D) rS[i] = __builtin_nontemporal_load(S + d * CPR_S + ccS);
  }
#pragma unroll
  for (int i = 0; i < NP_C; ++i) {
    const int d = rgC + RP_C * i;
    if (d < D) rC[i] = __builtin_nontemporal_load(C + d * CPR_C + ccC);
  }
  const T* q = reinterpret_cast<const T*>(a.q) + (size_t)unit * D;
  const T* k = reinterpret_cast<const T*>(a.k) + (size_t)unit * D;
  const T* v = reinterpret_cast<const T*>(a.v) + (size_t)unit * E;
  for (int t = tid; t < D; t += UDEC) {
    sq[t] = (float)q[t];
    sk[t] = (float)k[t];
    sm[t] = m[t];
  }
  for (int t = tid; t < E; t += UDEC) sv[t] = (float)v[t];
  __syncthreads();

  // S' = g S + k k^T; a = S' q (row sums over the CPR_S lanes of a row)
  {
    const f32x4 q4 = *reinterpret_cast<const f32x4*>(sq + 4 * ccS);
    const f32x4 k4 = *reinterpret_cast<const f32x4*>(sk + 4 * ccS);
#pragma unroll
    for (int i = 0; i < NP_S; ++i) {
      const int d = rgS + RP_S * i;
      float ap = 0.f;
      if (d < D) {
        const f32x4 sn = rS[i] * g + k4 * sk[d];
        __builtin_nontemporal_store(sn, S + d * CPR_S + ccS);
        ap = sn[0] * q4[0] + sn[1] * q4[1] + sn[2] * q4[2] + sn[3] * q4[3];
      }
#pragma unroll
      for (int off = 1; off < CPR_S; off *= 2) ap += __shfl_xor(ap, off, 64);
      if (d < D && ccS == 0) aval[d] = ap;
    }
  }
  __syncthreads();

  // C' = g C + q v^T; partial z = C'^T a over this thread's rows; m' and den
  {
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(sv + 4 * ccC);
    f32x4 pz = zero4();
#pragma unroll
    for (int i = 0; i < NP_C; ++i) {
      const int d = rgC + RP_C * i;
      if (d < D) {
        const f32x4 cn = rC[i] * g + v4 * sq[d];
        __builtin_nontemporal_store(cn, C + d * CPR_C + ccC);
        pz += cn * aval[d];
      }
    }
    if (rgC < NRG) *reinterpret_cast<f32x4*>(&rz[rgC][4 * ccC]) = pz;
  }
  for (int t = tid; t < D; t += UDEC) m[t] = g * sm[t] + sq[t];
  if (tid < 64) {
    float dn = 0.f;
    for (int d = tid; d < D; d += 64) dn += aval[d] * (g * sm[d] + sq[d]);
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) dn += __shfl_xor(dn, off, 64);
    if (tid == 0) sden = dn;
  }
  __syncthreads();
  const float den = sden;
  for (int e = tid; e < E; e += UDEC) {
    float z = 0.f;
    for (int r = 0; r < NRG; ++r) z += rz[r][e];
    a.o[(size_t)unit * E + e] = a.normalize ? z / (den + a.eps) : z;
  }
  if (a.den != nullptr && tid == 0) a.den[unit] = den;
}

template <int D, int E>
struct UWaves {
  static constexpr int value = (D == 128 || E == 128) ? 8 : 4;
};

template <int MODE>
hipError_t launch_unmasked_mode(int dtype, int d, int dv, int units, const ChunkArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)units * (unsigned)a.nspan);
#define HLA_CASE(T, D, E)                                                                      \
  if (d == D && dv == E) {                                                                     \
    constexpr int NW = UWaves<D, E>::value;                                                    \
    hipLaunchKernelGGL((unmasked_kernel<T, D, E, MODE, NW>), grid, dim3(64 * NW), 0, s, a);    \
    return hipGetLastError();                                                                  \
  }
  if (dtype == 1) {
    HLA_CASE(__bf16, 16, 16) HLA_CASE(__bf16, 16, 32) HLA_CASE(__bf16, 32, 16)
    HLA_CASE(__bf16, 32, 32) HLA_CASE(__bf16, 32, 64) HLA_CASE(__bf16, 64, 32)
    HLA_CASE(__bf16, 64, 64) HLA_CASE(__bf16, 64, 128) HLA_CASE(__bf16, 128, 64)
    HLA_CASE(__bf16, 128, 128)
  } else {
    HLA_CASE(float, 16, 16) HLA_CASE(float, 16, 32) HLA_CASE(float, 32, 16)
    HLA_CASE(float, 32, 32) HLA_CASE(float, 32, 64) HLA_CASE(float, 64, 32)
    HLA_CASE(float, 64, 64)
  }
#undef HLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_unmasked_summaries(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                     hipStream_t s) {
  return launch_unmasked_mode<U_SUMMARY>(dtype, d, dv, units, a, s);
}

hipError_t launch_unmasked_outputs(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                   hipStream_t s) {
  return launch_unmasked_mode<U_OUTPUT>(dtype, d, dv, units, a, s);
}

hipError_t launch_unmasked_decode(int dtype, int d, int dv, int units, const DecodeArgs& a,
                                  hipStream_t s) {
#define HLA_CASE(T, D, E)                                                                       \
  if (d == D && dv == E) {                                                                      \
    hipLaunchKernelGGL((unmasked_decode_kernel<T, D, E>), dim3(units), dim3(UDEC), 0, s, a);    \
    return hipGetLastError();                                                                   \
  }
  if (dtype == 1) {
    HLA_CASE(__bf16, 16, 16) HLA_CASE(__bf16, 16, 32) HLA_CASE(__bf16, 32, 16)
    HLA_CASE(__bf16, 32, 32) HLA_CASE(__bf16, 32, 64) HLA_CASE(__bf16, 64, 32)
    HLA_CASE(__bf16, 64, 64) HLA_CASE(__bf16, 64, 128) HLA_CASE(__bf16, 128, 64)
    HLA_CASE(__bf16, 128, 128)
  } else {
    HLA_CASE(float, 16, 16) HLA_CASE(float, 16, 32) HLA_CASE(float, 32, 16)
    HLA_CASE(float, 32, 32) HLA_CASE(float, 32, 64) HLA_CASE(float, 64, 32)
    HLA_CASE(float, 64, 64) HLA_CASE(float, 64, 128) HLA_CASE(float, 128, 64)
    HLA_CASE(float, 128, 128)
  }
#undef HLA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_unmasked_scan(const ChunkArgs& a, int units, int d, int dv, hipStream_t s) {
  UScanArgs u;
  u.X[0] = a.S; u.X[1] = a.C; u.X[2] = a.m;
  u.F[0] = d * d; u.F[1] = d * dv; u.F[2] = d;
  for (int i = 0; i < 3; ++i) u.nb[i] = (u.F[i] / 4 + 255) / 256;
  u.gamma = a.gamma; u.H = a.H; u.n = a.nspan; u.chunk = a.chunk;
  const dim3 grid((unsigned)(u.nb[0] + u.nb[1] + u.nb[2]), (unsigned)units);
  hipLaunchKernelGGL(unmasked_scan_kernel, grid, dim3(256), 0, s, u);
  return hipGetLastError();
}

}  // namespace hla
