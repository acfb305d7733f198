// The asymmetric variant AHLA of the second-order forward ("Higher-order
// Linear Attention", arXiv 2510.27258, summaries on gist.science: method
// section 2 -- the operator Q (K^T Q)(K^T V), a single path through an
// intermediate key index, streaming summaries P^KV, m^K, E, n; method
// section 4 -- segment summaries joined by an exclusive scan).
//
// Causal form read here: o_t = sum_{i<=t} sum_{j<=i} (q_t.k_i)(q_i.k_j) v_j,
// with P_t = sum_{j<=t} k_j v_j^T, m_t = sum_{j<=t} k_j, r_i = P_i^T q_i,
// E_t = sum_{i<=t} k_i r_i^T, n_t = sum_{i<=t} k_i (q_i.m_i), o_t = E_t^T q_t,
// den_t = q_t.n_t; decay g multiplies every moment once per token.  Per tile
// (0-based tau, Lt tokens, A'[tau][i] = g^(tau-i) q_tau.k_i for i <= tau):
//   R = g^(tau+1) Q P + A' V,   O = g^(tau+1) Q E + A' R,
//   P <- g^Lt P + K^T diag(w) V,  E <- g^Lt E + K^T diag(w) R,  w_i = g^(Lt-1-i).
// A segment's summary also carries X = sum_i k_i q_i^T (no decay): the
// combine (A then B, a = g^(length of B)) is P = a P_A + P_B,
// E = a E_A + E_B + a X_B P_A (m, n likewise with m in place of P).
//
// One workgroup per (unit, segment) with one wave per 16-column block of the
// values (at least four waves); each wave keeps its blocks of P and E in fp32
// MFMA accumulators and its R tile in registers, so the waves share only the
// staged tile and the A' scores.  m and n (and q.m, den) are vector work for
// all threads, in LDS.  The scan walks a unit's segments in order, one
// workgroup per (unit, column block).  The decode step updates (P, m, E, n)
// in place for one token per unit.
#include <type_traits>

#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int AT = 64;   // tokens per tile

enum { A_SUMMARY = 0, A_OUTPUT = 1 };

template <typename T, int D, int E>
struct ALayout {
  static constexpr int PADT = 16 / (int)sizeof(T);
  static constexpr int DP = D < MM<T>::KS ? MM<T>::KS : D;
  static constexpr int LDD = DP + PADT;    // Q, K: [tok][d]
  static constexpr int LDV = E + PADT;     // V: [tok][e]
  static constexpr int LDT = AT + PADT;    // A': [tok][tok]
  // Q, K, V double-buffered by tile parity: a tile is staged while the
  // previous one's den and m, n updates still read its buffers
  static constexpr size_t QB = (size_t)AT * LDD * sizeof(T);
  static constexpr size_t VB = (size_t)AT * LDV * sizeof(T);
  static constexpr size_t Qs = 0, Ks = 2 * QB, Vs = 4 * QB;
  static constexpr size_t AB = Vs + 2 * VB;
  static constexpr size_t TILE_END = AB + (size_t)AT * LDT * sizeof(T);
  // output tiles of the value blocks, fp32 [block][tok][LDO], held until den is known
  static constexpr int LDO = 20;
  static constexpr size_t OB = (TILE_END + 15) / 16 * 16;
  static constexpr size_t W = OB + (size_t)(E / 16) * AT * LDO * 4;
  // pw, w1, wS[2], qm, qn, rm, den [AT]; bpart [AT / 16][AT]; m, n [D]
  static constexpr size_t TOTAL = W + (size_t)(8 * AT + (AT / 16) * AT + 2 * D) * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
};

// K^T fragment (rows d = n0 + (lane & 15), K = tokens) in the K order of
// Frag<T>::acc_b, from K stored [tok][d]: bf16 step kk holds tokens
// 32 kk + 4 g + [0, 4) and 32 kk + 16 + 4 g + [0, 4) (two transposing reads
// of four rows each); fp32 step kk holds token 16 (kk >> 2) + 4 g + (kk & 3).
template <typename T>
__device__ __forceinline__ typename MM<T>::F kt_acc_order(const T* X, int ldm, int kk, int n0, int lane);
template <>
__device__ __forceinline__ bf16x8 kt_acc_order<__bf16>(const __bf16* X, int ldm, int kk, int n0, int lane) {
  const int l = lane & 15, g = lane >> 4;
  __bf16* p0 = const_cast<__bf16*>(X) + (32 * kk + 4 * g + (l >> 2)) * ldm + n0 + 4 * (l & 3);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 16 * ldm));
  const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}
template <>
__device__ __forceinline__ float kt_acc_order<float>(const float* X, int ldm, int kk, int n0, int lane) {
  return X[(16 * (kk >> 2) + 4 * (lane >> 4) + (kk & 3)) * ldm + n0 + (lane & 15)];
}

template <typename T, int D, int E, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void ahla_kernel(AhlaArgs a) {
  constexpr int NTHR = 64 * NW;
  using L = ALayout<T, D, E>;
  using MMT = MM<T>;
  using FR = Frag<T>;
  using F = typename MMT::F;
  constexpr int KS = MMT::KS, CH = MMT::CH, DP = L::DP;
  constexpr int DT = D / 16, ET = E / 16, TR = AT / 16, NKS = AT / KS;
  constexpr int NTRI = TR * (TR + 1) / 2;
  constexpr int QSK = KS == 32 ? (DT + 1) / 2 : DT * 4;   // K steps over d
  constexpr int TSK = KS == 32 ? TR / 2 : TR * 4;          // K steps over the tile's tokens
  constexpr int XB = (DT + NW - 1) / NW;                   // X column blocks per wave
  constexpr bool OUT = MODE == A_OUTPUT;
  static_assert(NW >= ET && NW >= 4, "one wave per 16-column block of the values, at least four");

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  auto Qb = [&](int p) { return reinterpret_cast<T*>(smem + L::Qs + p * L::QB); };
  auto Kb = [&](int p) { return reinterpret_cast<T*>(smem + L::Ks + p * L::QB); };
  auto Vb = [&](int p) { return reinterpret_cast<T*>(smem + L::Vs + p * L::VB); };
  T* AB = reinterpret_cast<T*>(smem + L::AB);
  float* OBs = reinterpret_cast<float*>(smem + L::OB);
  float* pw = reinterpret_cast<float*>(smem + L::W);
  float* w1 = pw + AT;
  auto wSb = [&](int p) { return w1 + AT + p * AT; };
  float* qm = w1 + 3 * AT;
  float* qn = qm + AT;
  float* rmv = qn + AT;
  float* denv = rmv + AT;
  float* bpart = denv + AT;
  float* mst = bpart + TR * AT;
  float* nst = mst + D;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg4 = lane >> 4;
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
  const int ntiles = (Lspan + AT - 1) / AT;
  const int cb = wave;                 // this wave's value block (none past ET)
  const bool vblk = cb < ET;

  for (size_t i = tid; i < L::TILE_END / 16; i += NTHR)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  if (tid < AT) {
    pw[tid] = gpow(g, lgg, tid);
    w1[tid] = gpow(g, lgg, tid + 1);
  }
  for (int i = tid; i < D; i += NTHR) {
    mst[i] = OUT ? a.m[sidx * D + i] : 0.f;
    nst[i] = OUT ? a.n[sidx * D + i] : 0.f;
  }

  // P and E blocks of this wave (rows 16 t + 4 lg4 + j, column 16 cb + lr),
  // from the prefix or zero
  f32x4 Pt[DT], Et[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * t + 4 * lg4 + j;
      const bool ld = OUT && vblk;
      Pt[t][j] = ld ? a.P[(sidx * D + row) * E + 16 * cb + lr] : 0.f;
      Et[t][j] = ld ? a.E[(sidx * D + row) * E + 16 * cb + lr] : 0.f;
    }
  f32x4 Xt[XB][DT];
#pragma unroll
  for (int b = 0; b < XB; ++b)
#pragma unroll
    for (int t = 0; t < DT; ++t) Xt[b][t] = zero4();
  __syncthreads();   // the cleared tile region before the first staging

  // tile staging through registers, one loop per buffer
  constexpr int QCH = AT * D / CH, VCH = AT * E / CH;
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
  auto tile_len = [&](int ti) { return (Lspan - ti * AT) < AT ? (Lspan - ti * AT) : AT; };

  auto load_tile = [&](int ti) {
    const int t0 = ti * AT, Lt = tile_len(ti);
    load_rows(xq, NQc{}, gq, D, QCH, t0, Lt);
    load_rows(xk, NQc{}, gk, D, QCH, t0, Lt);
    load_rows(xv, NVc{}, gv, E, VCH, t0, Lt);
  };
  // tile ti from registers to the buffers of its parity, with its update weights
  auto stage_tile = [&](int ti) {
    const int p = ti & 1, Lt = tile_len(ti);
    store_rows(xq, NQc{}, Qb(p), D, L::LDD, QCH);
    store_rows(xk, NQc{}, Kb(p), D, L::LDD, QCH);
    store_rows(xv, NVc{}, Vb(p), E, L::LDV, VCH);
    if (tid < AT) wSb(p)[tid] = tid < Lt ? gpow(g, lgg, Lt - 1 - tid) : 0.f;
  };
  // outputs of tile tp (normalised by den when asked): lane l writes columns
  // 4 (l & 3) .. +3 of rows 16 i + (l >> 2) of this wave's block
  auto store_out = [&](int tp, int Ltp) {
    float* go = a.o + (tok0 + (size_t)tp * AT) * E + 16 * cb;
    const float* ob = OBs + (size_t)cb * AT * L::LDO;
#pragma unroll
    for (int i = 0; i < AT / 16; ++i) {
      const int tau = 16 * i + (lane >> 2), c4 = 4 * (lane & 3);
      f32x4 o = *reinterpret_cast<const f32x4*>(ob + tau * L::LDO + c4);
      if (a.normalize) o *= 1.f / (denv[tau] + a.eps);
      if (tau < Ltp) *reinterpret_cast<f32x4*>(go + (size_t)tau * E + c4) = o;
    }
  };

  // Three barriers per tile:
  //   [A' and q.m, q.n of tile t; outputs of t - 1] -> [q.m at every token;
  //   the value blocks of t] -> [den, m, n updates of t; stage t + 1].
  load_tile(0);
  stage_tile(0);
  __syncthreads();
  if (ntiles > 1) load_tile(1);
  for (int ti = 0; ti < ntiles; ++ti) {
    const int p = ti & 1;
    const int t0 = ti * AT, Lt = tile_len(ti);
    const float gL = gpow(g, lgg, Lt);
    const T* Qs = Qb(p);
    const T* Ks = Kb(p);
    const T* Vs = Vb(p);
    const float* wS = wSb(p);

    // ---- A'[tau][i] = g^(tau-i) q_tau.k_i (i <= tau) and its row sums, over
    //      all waves; q.m (and q.n) by all threads ----
    for (int idx = wave; idx < NTRI; idx += NW) {
      int r, c;
      tri_block(idx, r, c);
      f32x4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DP; k0 += KS)
        acc = MMT::mma(MMT::ld(Ks, L::LDD, 16 * c, k0, lane), MMT::ld(Qs, L::LDD, 16 * r, k0, lane), acc);
      const int tau = 16 * r + lr;
      f32x4 val;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * c + 4 * lg4 + j;
        val[j] = acc[j] * masked_pow(pw, tau, i);
      }
      if constexpr (sizeof(T) == 2) {
        bf16x4 y;
        y[0] = (__bf16)val[0]; y[1] = (__bf16)val[1]; y[2] = (__bf16)val[2]; y[3] = (__bf16)val[3];
        *reinterpret_cast<bf16x4*>(AB + tau * L::LDT + 16 * c + 4 * lg4) = y;
      } else {
        *reinterpret_cast<f32x4*>(AB + tau * L::LDT + 16 * c + 4 * lg4) = val;
      }
      const float rs = sum_rows4(val[0] + val[1] + val[2] + val[3]);
      if (lg4 == 0) bpart[c * AT + tau] = rs;
    }
    {
      constexpr int LPR = NTHR / AT;
      const int tau = tid / LPR, part = tid % LPR;
      float sm = 0.f, sn = 0.f;
      for (int c = part; c < D; c += LPR) {
        const float x = (float)Qs[tau * L::LDD + c];
        sm += x * mst[c];
        sn += x * nst[c];
      }
#pragma unroll
      for (int off = 1; off < LPR; off *= 2) {
        sm += __shfl_xor(sm, off, 64);
        sn += __shfl_xor(sn, off, 64);
      }
      if (part == 0) {
        qm[tau] = sm;
        qn[tau] = sn;
      }
    }
    if constexpr (OUT) {
      if (vblk && ti > 0) store_out(ti - 1, AT);   // only the last tile can be short
    }
    __syncthreads();

    // ---- rm = q.m at every token (threads); the waves' value blocks ----
    if (tid < AT) {
      rmv[tid] = add_lower_blocks(w1[tid] * qm[tid], bpart, AT, tid);
    }
    if (vblk) {
      // R = g^(tau+1) Q P + A' V (and O = g^(tau+1) Q E + A' R in the output kernel)
      f32x4 Rt[TR], Ot[TR];
#pragma unroll
      for (int r = 0; r < TR; ++r) { Rt[r] = zero4(); Ot[r] = zero4(); }
#pragma unroll
      for (int kk = 0; kk < QSK; ++kk) {
        const F bp = FR::acc_b(Pt, kk);
        F be;
        if constexpr (OUT) be = FR::acc_b(Et, kk);
#pragma unroll
        for (int r = 0; r < TR; ++r) {
          const F aq = FR::perm(Qs, L::LDD, 16 * r, kk, lane);
          Rt[r] = MMT::mma(aq, bp, Rt[r]);
          if constexpr (OUT) Ot[r] = MMT::mma(aq, be, Ot[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < TR; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Rt[r][j] *= w1[16 * r + 4 * lg4 + j];
          if constexpr (OUT) Ot[r][j] *= w1[16 * r + 4 * lg4 + j];
        }
        for (int k0 = 0; k0 < 16 * r + 16; k0 += KS)
          Rt[r] = MMT::mma(MMT::ld(AB, L::LDT, 16 * r, k0, lane), FR::tr(Vs, L::LDV, k0, 16 * cb, lane), Rt[r]);
      }
      if constexpr (OUT) {
        // A' R: R's tiles stacked along the tokens are the B operand
#pragma unroll
        for (int kk = 0; kk < TSK; ++kk) {
          const F br = FR::acc_b(Rt, kk);
#pragma unroll
          for (int r = 0; r < TR; ++r)
            if (KS * kk < 16 * r + 16) Ot[r] = MMT::mma(FR::perm(AB, L::LDT, 16 * r, kk, lane), br, Ot[r]);
        }
        // park the output tile in LDS until den is known
        float* ob = OBs + (size_t)cb * AT * L::LDO;
#pragma unroll
        for (int r = 0; r < TR; ++r)
#pragma unroll
          for (int j = 0; j < 4; ++j) ob[(16 * r + 4 * lg4 + j) * L::LDO + lr] = Ot[r][j];
      }
      // ---- P <- g^Lt P + K^T diag(w) V, E <- g^Lt E + K^T diag(w) R ----
#pragma unroll
      for (int r = 0; r < TR; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) Rt[r][j] *= wS[16 * r + 4 * lg4 + j];
      F bv[NKS], bw[TSK];
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) bv[kk] = FR::scale(FR::tr(Vs, L::LDV, kk * KS, 16 * cb, lane), wS, kk * KS, lane);
#pragma unroll
      for (int kk = 0; kk < TSK; ++kk) bw[kk] = FR::acc_b(Rt, kk);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 p = Pt[t] * gL, e = Et[t] * gL;
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) p = MMT::mma(FR::tr(Ks, L::LDD, kk * KS, 16 * t, lane), bv[kk], p);
#pragma unroll
        for (int kk = 0; kk < TSK; ++kk) e = MMT::mma(kt_acc_order<T>(Ks, L::LDD, kk, 16 * t, lane), bw[kk], e);
        Pt[t] = p;
        Et[t] = e;
      }
    }
    if constexpr (!OUT) {
      // X[:, blocks] += K^T Q[:, blocks] (rows past the segment end are zero)
#pragma unroll
      for (int b = 0; b < XB; ++b) {
        const int xc = wave + NW * b;
        if (xc < DT) {
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            f32x4 x = Xt[b][t];
#pragma unroll
            for (int kk = 0; kk < NKS; ++kk)
              x = MMT::mma(FR::tr(Ks, L::LDD, kk * KS, 16 * t, lane), FR::tr(Qs, L::LDD, kk * KS, 16 * xc, lane), x);
            Xt[b][t] = x;
          }
        }
      }
    }
    __syncthreads();

    // ---- den = g^(tau+1) q.n + A' rm (output kernel); m and n updates:
    //      TPD threads per row d, each over AT / TPD tokens ----
    if constexpr (OUT) {
      if (tid < AT) {
        float dn = w1[tid] * qn[tid];
        for (int i = 0; i <= tid; ++i) dn += (float)AB[tid * L::LDT + i] * rmv[i];
        denv[tid] = dn;
        if (a.den != nullptr && tid < Lt) a.den[tok0 + (size_t)t0 + tid] = dn;
      }
    }
    {
      constexpr int TPD = NTHR / D > 16 ? 16 : NTHR / D;
      constexpr int TPT = AT / TPD;
      if (tid < TPD * D) {
        const int d = tid / TPD, part = tid % TPD;
        float sm = 0.f, sn = 0.f;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
          const int tau = part * TPT + i;
          const float kw = wS[tau] * (float)Ks[tau * L::LDD + d];
          sm += kw;
          sn += kw * rmv[tau];
        }
#pragma unroll
        for (int off = 1; off < TPD; off *= 2) {
          sm += __shfl_xor(sm, off, 64);
          sn += __shfl_xor(sn, off, 64);
        }
        if (part == 0) {
          mst[d] = gL * mst[d] + sm;
          nst[d] = gL * nst[d] + sn;
        }
      }
    }
    if (ti + 1 < ntiles) {
      stage_tile(ti + 1);
      if (ti + 2 < ntiles) load_tile(ti + 2);
    }
    __syncthreads();
  }
  if constexpr (OUT) {
    if (vblk) store_out(ntiles - 1, tile_len(ntiles - 1));
  }

  if constexpr (!OUT) {
    if (vblk) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * t + 4 * lg4 + j;
          a.P[(sidx * D + row) * E + 16 * cb + lr] = Pt[t][j];
          a.E[(sidx * D + row) * E + 16 * cb + lr] = Et[t][j];
        }
    }
    for (int i = tid; i < D; i += NTHR) {
      a.m[sidx * D + i] = mst[i];
      a.n[sidx * D + i] = nst[i];
    }
#pragma unroll
    for (int b = 0; b < XB; ++b) {
      const int xc = wave + NW * b;
      if (xc < DT) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            a.X[(sidx * D + 16 * t + 4 * lg4 + j) * D + 16 * xc + lr] = Xt[b][t][j];
      }
    }
  }
}

// Exclusive scan of the AHLA summaries of each unit, in order, for one
// 16-column block of (P, E) (block ET: m, n as a single column):
// prefix_s = run; run <- a run + x_s, E picking up a X_s P_run (a = g^chunk).
// In place; X is only read.  The state after the last segment is not wanted,
// so that segment's X is neither loaded nor multiplied.  One workgroup of 4
// waves per (unit, block): X_s
// is staged in LDS and X_s P_run runs on fp32 MFMA, each wave owning row tiles
// of the block; the running E stays in the owning lanes' registers.
template <int D, int E>
__global__ __launch_bounds__(256) void ahla_scan_kernel(AhlaArgs a) {
  constexpr int ET = E / 16, DT = D / 16, LX = D + 4;
  constexpr int RB = (DT + 3) / 4;   // row tiles per wave
  __shared__ __attribute__((aligned(16))) float Xs[D * LX];
  __shared__ __attribute__((aligned(16))) float Pr[D * 16];
  const int unit = blockIdx.x / (ET + 1), cb = blockIdx.x % (ET + 1);
  const bool mblk = cb == ET;
  const int n = a.nspan, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg4 = lane >> 4;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float sa = gpow(g, log2f(g), a.chunk);
  for (int i = tid; i < D * 16; i += 256) Pr[i] = 0.f;
  f32x4 er[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) er[b] = zero4();
  const bool col_ok = !mblk || lr == 0;
  // X_s is loaded into registers one segment ahead, so its loads overlap the
  // previous segment's products
  constexpr int NXR = (D * D / 4 + 255) / 256;
  f32x4 xr[NXR];
  auto load_x = [&](int s) {
    const f32x4* X = reinterpret_cast<const f32x4*>(a.X + ((size_t)unit * n + s) * D * D);
#pragma unroll
    for (int k = 0; k < NXR; ++k) {
      const int i = tid + 256 * k;
      if (i < D * D / 4) xr[k] = X[i];
    }
  };
  if (n > 1) load_x(0);
  for (int s = 0; s < n; ++s) {
    const size_t sidx = (size_t)unit * n + s;
    const bool last = s == n - 1;   // uniform
    // this segment's summary entries of the lanes' own rows, read before the
    // products so that their loads overlap them
    float px[RB][4], ex[RB][4];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int t = wave + 4 * b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * t + 4 * lg4 + j;
        px[b][j] = ex[b][j] = 0.f;
        if (t < DT && col_ok && !last) {
          px[b][j] = mblk ? a.m[sidx * D + row] : a.P[(sidx * D + row) * E + 16 * cb + lr];
          ex[b][j] = mblk ? a.n[sidx * D + row] : a.E[(sidx * D + row) * E + 16 * cb + lr];
        }
      }
    }
    if (!last) {
#pragma unroll
      for (int k = 0; k < NXR; ++k) {
        const int i = tid + 256 * k;
        if (i < D * D / 4) {
          const int r = (4 * i) / D, c = (4 * i) % D;
          *reinterpret_cast<f32x4*>(Xs + r * LX + c) = xr[k];
        }
      }
    }
    if (s + 2 < n) load_x(s + 1);
    __syncthreads();
    f32x4 cross[RB], pold[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int t = wave + 4 * b;
      cross[b] = zero4();
      if (t < DT) {
        if (!last) cross[b] = gemm_f32_tile<D>(Xs, LX, Pr, 16, 16 * t, 0, lane, cross[b]);
#pragma unroll
        for (int j = 0; j < 4; ++j) pold[b][j] = Pr[(16 * t + 4 * lg4 + j) * 16 + lr];
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int t = wave + 4 * b;
      if (t < DT && col_ok) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * t + 4 * lg4 + j;
          float* pp = mblk ? a.m + sidx * D + row : a.P + (sidx * D + row) * E + 16 * cb + lr;
          float* ep = mblk ? a.n + sidx * D + row : a.E + (sidx * D + row) * E + 16 * cb + lr;
          *pp = pold[b][j];
          *ep = er[b][j];
          Pr[row * 16 + lr] = sa * pold[b][j] + px[b][j];
          er[b][j] = sa * er[b][j] + ex[b][j] + sa * cross[b][j];
        }
      }
    }
    __syncthreads();
  }
}

// One AHLA decode step per unit (one workgroup of ADEC threads):
//   P' = g P + k v^T, m' = g m + k, r = P'^T q, E' = g E + k r^T,
//   n' = g n + k (q.m'), o = E'^T q = g (E^T q) + (q.k) r, den = q.n'.
// Each state element is read once and written once (16-byte non-temporal
// accesses); E stays in registers until r is reduced.
constexpr int ADEC = 512;

template <typename T, int D, int E>
__global__ __launch_bounds__(ADEC) void ahla_decode_kernel(AhlaArgs a) {
  constexpr int CPR = E / 4, RP = ADEC / CPR, NP = (D + RP - 1) / RP;
  constexpr int NRG = RP < D ? RP : D;
  __shared__ __attribute__((aligned(16))) float sq[D], sk[D], sv[E], sm[D], sn[D], rr[E], yy[E];
  __shared__ __attribute__((aligned(16))) float pr[NRG][E], py[NRG][E];
  __shared__ float scal[3];
  const int unit = blockIdx.x, tid = threadIdx.x;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  f32x4* P = reinterpret_cast<f32x4*>(a.P + (size_t)unit * D * E);
  f32x4* Em = reinterpret_cast<f32x4*>(a.E + (size_t)unit * D * E);
  float* m = a.m + (size_t)unit * D;
  float* n = a.n + (size_t)unit * D;
  const int cc = tid % CPR, rg = tid / CPR;
  f32x4 rP[NP], rE[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int d = rg + RP * i;
    if (d < D) {
      rP[i] = __builtin_nontemporal_load(P + d * CPR + cc);
      rE[i] = __builtin_nontemporal_load(Em + d * CPR + cc);
    }
  }
  const T* q = reinterpret_cast<const T*>(a.q) + (size_t)unit * D;
  const T* k = reinterpret_cast<const T*>(a.k) + (size_t)unit * D;
  const T* v = reinterpret_cast<const T*>(a.v) + (size_t)unit * E;
  for (int t = tid; t < D; t += ADEC) {
    sq[t] = (float)q[t];
    sk[t] = (float)k[t];
    sm[t] = m[t];
    sn[t] = n[t];
  }
  for (int t = tid; t < E; t += ADEC) sv[t] = (float)v[t];
  __syncthreads();

  // P' = g P + k v^T (stored); partial r = P'^T q and y = E^T q over this thread's rows
  {
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(sv + 4 * cc);
    f32x4 ar = zero4(), ay = zero4();
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int d = rg + RP * i;
      if (d < D) {
        const f32x4 pn = rP[i] * g + v4 * sk[d];
        __builtin_nontemporal_store(pn, P + d * CPR + cc);
        ar += pn * sq[d];
        ay += rE[i] * sq[d];
      }
    }
    if (rg < NRG) {
      *reinterpret_cast<f32x4*>(&pr[rg][4 * cc]) = ar;
      *reinterpret_cast<f32x4*>(&py[rg][4 * cc]) = ay;
    }
  }
  if (tid < 64) {
    float qk = 0.f, qm = 0.f, qn = 0.f;
    for (int d = tid; d < D; d += 64) {
      qk += sq[d] * sk[d];
      qm += sq[d] * sm[d];
      qn += sq[d] * sn[d];
    }
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) {
      qk += __shfl_xor(qk, off, 64);
      qm += __shfl_xor(qm, off, 64);
      qn += __shfl_xor(qn, off, 64);
    }
    if (tid == 0) { scal[0] = qk; scal[1] = g * qm + qk; scal[2] = qn; }   // q.k, q.m', q.n
  }
  __syncthreads();
  for (int e = tid; e < E; e += ADEC) {
    float sr = 0.f, sy = 0.f;
    for (int r = 0; r < NRG; ++r) { sr += pr[r][e]; sy += py[r][e]; }
    rr[e] = sr;
    yy[e] = sy;
  }
  __syncthreads();
  const float qk = scal[0], rm = scal[1];
  const float den = g * scal[2] + qk * rm;
  // E' = g E + k r^T; m', n'; o = g y + (q.k) r
  {
    const f32x4 r4 = *reinterpret_cast<const f32x4*>(rr + 4 * cc);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int d = rg + RP * i;
      if (d < D) __builtin_nontemporal_store(rE[i] * g + r4 * sk[d], Em + d * CPR + cc);
    }
  }
  for (int t = tid; t < D; t += ADEC) {
    m[t] = g * sm[t] + sk[t];
    n[t] = g * sn[t] + sk[t] * rm;
  }
  for (int e = tid; e < E; e += ADEC) {
    const float o = g * yy[e] + qk * rr[e];
    a.o[(size_t)unit * E + e] = a.normalize ? o / (den + a.eps) : o;
  }
  if (a.den != nullptr && tid == 0) a.den[unit] = den;
}

template <int D, int E>
struct AWaves {
  static constexpr int value = E / 16 > 4 ? E / 16 : 4;
};

template <int MODE>
hipError_t launch_ahla_mode(int dtype, int d, int dv, int units, const AhlaArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)units * (unsigned)a.nspan);
#define HLA_CASE(T, D, E)                                                                     \
  if (d == D && dv == E) {                                                                    \
    constexpr int NW = AWaves<D, E>::value;                                                   \
    hipLaunchKernelGGL((ahla_kernel<T, D, E, MODE, NW>), grid, dim3(64 * NW), 0, s, a);       \
    return hipGetLastError();                                                                 \
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

hipError_t launch_ahla_summaries(int dtype, int d, int dv, int units, const AhlaArgs& a, hipStream_t s) {
  return launch_ahla_mode<A_SUMMARY>(dtype, d, dv, units, a, s);
}

hipError_t launch_ahla_outputs(int dtype, int d, int dv, int units, const AhlaArgs& a, hipStream_t s) {
  return launch_ahla_mode<A_OUTPUT>(dtype, d, dv, units, a, s);
}

hipError_t launch_ahla_decode(int dtype, int d, int dv, int units, const AhlaArgs& a, hipStream_t s) {
#define HLA_CASE(T, D, E)                                                                   \
  if (d == D && dv == E) {                                                                  \
    hipLaunchKernelGGL((ahla_decode_kernel<T, D, E>), dim3(units), dim3(ADEC), 0, s, a);    \
    return hipGetLastError();                                                               \
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

hipError_t launch_ahla_scan(int d, int dv, int units, const AhlaArgs& a, hipStream_t s) {
#define HLA_CASE(D, E)                                                                         \
  if (d == D && dv == E) {                                                                     \
    hipLaunchKernelGGL((ahla_scan_kernel<D, E>), dim3((unsigned)units * (E / 16 + 1)), dim3(256), \
                       0, s, a);                                                               \
    return hipGetLastError();                                                                  \
  }
  HLA_CASE(16, 16) HLA_CASE(16, 32) HLA_CASE(32, 16) HLA_CASE(32, 32) HLA_CASE(32, 64)
  HLA_CASE(64, 32) HLA_CASE(64, 64) HLA_CASE(64, 128) HLA_CASE(128, 64) HLA_CASE(128, 128)
#undef HLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace hla
