// Segment summaries and segment outputs of the masked second-order HLA
// forward ("Higher-order Linear Attention", arXiv 2510.27258, summaries on
// gist.science: method section 1 for the state and the output, section 4
// for segment summaries and the chunk-parallel scheme, key contribution 2 for
// decay).
//
// One workgroup (8 waves) owns one segment of `chunk` tokens of one
// (batch, head) unit and walks it in tiles of TT = 64 tokens.  Inside a
// segment it does not carry (S, C, m, G, h) but the equivalent pair (S, M)
// with M_t = S_t C_t - G_t, using the identity
//     S_t C_t - G_t = sum_{j<=t} g^(2(t-j)) S_j q_j v_j^T,
// so that per tile (tau, i, j = 0-based positions inside the tile, Lt tokens):
//     A'[tau,i] = g^(tau-i) q_tau.k_i            (i <= tau)
//     p_tau     = sum_{i<=tau} A'[tau,i] k_i + g^(tau+1) S_prev q_tau  (= S_tau q_tau)
//     B[tau,j]  = g^(2(tau-j)) q_tau.p_j         (j <= tau)
//     num_tau   = sum_{j<=tau} B[tau,j] v_j + g^(2(tau+1)) q_tau^T M_prev
//     den_tau   = sum_{j<=tau} B[tau,j]     + g^(2(tau+1)) q_tau.n_prev
//     S <- g^Lt S + sum_i g^(Lt-1-i) k_i k_i^T
//     M <- g^(2Lt) M + sum_j g^(2(Lt-1-j)) p_j v_j^T,  n likewise with v = 1.
// The summary kernel also accumulates C and m and, at the end of the
// segment, converts back to the method's summary: G = S C - M, h = S m - n.
// The output kernel starts from the segment's exclusive prefix
// (S_P, C_P, m_P, G_P, h_P) with M = S_P C_P - G_P and n = S_P m_P - h_P.
//
// All products of the tile run on MFMA (bf16 operands for bf16 inputs, fp32
// operands for fp32 inputs) with fp32 accumulation; the state (S, M, C) is
// kept in fp32 accumulator registers and copied to LDS as an MFMA operand
// once per tile.  Segment-boundary products (S C, S m) run on fp32 MFMA.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr int TT = 64;      // tokens per tile
constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;

enum { MODE_SUMMARY = 0, MODE_OUTPUT = 1 };

template <typename T, int D, int E, int MODE>
struct ChunkLayout {
  static constexpr int PADT = 16 / (int)sizeof(T);
  static constexpr int LDD = D + PADT;       // [tok][d] buffers
  static constexpr int LDT = TT + PADT;      // [d][tok] buffers
  static constexpr int LDSM = D + PADT;      // S operand [d][d'] / M operand [e][d]
  static constexpr size_t Qs = 0;
  static constexpr size_t Ks = Qs + (size_t)TT * LDD * sizeof(T);
  static constexpr size_t Kt = Ks + (size_t)TT * LDD * sizeof(T);
  static constexpr size_t Vt = Kt + (size_t)D * LDT * sizeof(T);
  static constexpr size_t X1 = Vt + (size_t)E * LDT * sizeof(T);  // Qt (summary) / Ps (output)
  static constexpr size_t X1B = MODE == MODE_SUMMARY ? (size_t)D * LDT * sizeof(T)
                                                     : (size_t)TT * LDD * sizeof(T);
  static constexpr size_t Pt = X1 + X1B;
  static constexpr size_t AB = Pt + (size_t)D * LDT * sizeof(T);
  static constexpr size_t SM = AB + (size_t)TT * LDT * sizeof(T);
  static constexpr int SMROWS = (MODE == MODE_OUTPUT && E > D) ? E : D;
  static constexpr size_t TILE_END = SM + (size_t)SMROWS * LDSM * sizeof(T);
  // fp32 overlay used at segment boundaries: S [D][D+4], C [D][E+4]
  static constexpr int LFS = D + 4, LFC = E + 4;
  static constexpr size_t FS = 0;
  static constexpr size_t FC = FS + (size_t)D * LFS * 4;
  static constexpr size_t F_END = FC + (size_t)D * LFC * 4;
  static constexpr size_t BIG = TILE_END > F_END ? TILE_END : F_END;
  static constexpr size_t W = (BIG + 15) / 16 * 16;
  // w1, w2, wS, wM, pw, pw2, qn [TT]; bpart [TR][TT]; pcol [TR][D]; nst, mst [D]
  static constexpr size_t TOTAL = W + (size_t)(7 * TT + (TT / 16) * TT + (TT / 16) * D + 2 * D) * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
};

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 x);
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, f32x4 x) {
  bf16x4 y;
  y[0] = (__bf16)x[0]; y[1] = (__bf16)x[1]; y[2] = (__bf16)x[2]; y[3] = (__bf16)x[3];
  *reinterpret_cast<bf16x4*>(p) = y;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 x) {
  *reinterpret_cast<f32x4*>(p) = x;
}

template <typename T, int D, int E, int MODE>
__global__ __launch_bounds__(NTHR) void chunk_kernel(ChunkArgs a) {
  using L = ChunkLayout<T, D, E, MODE>;
  using MMT = MM<T>;
  constexpr int KS = MMT::KS;
  constexpr int CH = MMT::CH;
  constexpr int DT = D / 16, ET = E / 16, TR = TT / 16;
  constexpr int PT = (TR * DT + NWAVE - 1) / NWAVE;   // P tiles per wave
  constexpr int OT = (TR * ET + NWAVE - 1) / NWAVE;   // O tiles per wave
  constexpr int ST = (DT * DT + NWAVE - 1) / NWAVE;   // S tiles per wave
  constexpr int MT = (DT * ET + NWAVE - 1) / NWAVE;   // M, C, G tiles per wave
  constexpr int CT = MODE == MODE_SUMMARY ? MT : 1;

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  T* Qs = reinterpret_cast<T*>(smem + L::Qs);
  T* Ks = reinterpret_cast<T*>(smem + L::Ks);
  T* Kt = reinterpret_cast<T*>(smem + L::Kt);
  T* Vt = reinterpret_cast<T*>(smem + L::Vt);
  T* X1 = reinterpret_cast<T*>(smem + L::X1);   // Qt or Ps
  T* Pt = reinterpret_cast<T*>(smem + L::Pt);
  T* AB = reinterpret_cast<T*>(smem + L::AB);
  T* SM = reinterpret_cast<T*>(smem + L::SM);
  float* FS = reinterpret_cast<float*>(smem + L::FS);
  float* FC = reinterpret_cast<float*>(smem + L::FC);
  float* w1 = reinterpret_cast<float*>(smem + L::W);
  float* w2 = w1 + TT;
  float* wS = w2 + TT;
  float* wM = wS + TT;
  float* pw = wM + TT;
  float* pw2 = pw + TT;
  float* qn = pw2 + TT;
  float* bpart = qn + TT;        // [TR][TT]: row sums of B per 16-column block (fixed order)
  float* pcol = bpart + TR * TT; // [TR][D]: weighted column sums of P per 16-row block
  float* nst = pcol + TR * D;
  float* mst = nst + D;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg4 = lane >> 4;
  const int nspan = a.nspan;
  const int unit = blockIdx.x / nspan, span = blockIdx.x - unit * nspan;
  const int head = unit % a.H;
  const float g = a.gamma ? a.gamma[head] : 1.f;
  const float lgg = log2f(g);
  const int Lspan = a.chunk;
  const size_t tok0 = (size_t)unit * (size_t)a.T + (size_t)span * (size_t)Lspan;
  const T* gq = reinterpret_cast<const T*>(a.q) + tok0 * D;
  const T* gk = reinterpret_cast<const T*>(a.k) + tok0 * D;
  const T* gv = reinterpret_cast<const T*>(a.v) + tok0 * E;
  const size_t sidx = (size_t)unit * nspan + span;
  const bool need_n = MODE == MODE_SUMMARY || a.normalize || a.den != nullptr;

  f32x4 Sreg[ST], Mreg[MT], Creg[CT];

  if (tid < TT) {
    pw[tid] = gpow(g, lgg, tid);
    pw2[tid] = gpow(g, lgg, 2 * tid);
    w1[tid] = gpow(g, lgg, tid + 1);
    w2[tid] = gpow(g, lgg, 2 * tid + 2);
  }

  // ---- initial state -------------------------------------------------------
  if (MODE == MODE_SUMMARY) {
#pragma unroll
    for (int s = 0; s < ST; ++s) Sreg[s] = zero4();
#pragma unroll
    for (int s = 0; s < MT; ++s) Mreg[s] = zero4();
#pragma unroll
    for (int s = 0; s < CT; ++s) Creg[s] = zero4();
    for (int i = tid; i < D; i += NTHR) { nst[i] = 0.f; mst[i] = 0.f; }
  } else {
    const float* pS = a.S + sidx * D * D;
    const float* pC = a.C + sidx * D * E;
    const float* pG = a.G + sidx * D * E;
    for (int i = tid; i < D * D / 4; i += NTHR) {
      const int r = (4 * i) / D, c = (4 * i) % D;
      *reinterpret_cast<f32x4*>(FS + r * L::LFS + c) = reinterpret_cast<const f32x4*>(pS)[i];
    }
    for (int i = tid; i < D * E / 4; i += NTHR) {
      const int r = (4 * i) / E, c = (4 * i) % E;
      *reinterpret_cast<f32x4*>(FC + r * L::LFC + c) = reinterpret_cast<const f32x4*>(pC)[i];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      const int id = wave + NWAVE * s;
      if (id < DT * DT) {
        const int r0 = 16 * (id / DT), c0 = 16 * (id % DT);
#pragma unroll
        for (int j = 0; j < 4; ++j) Sreg[s][j] = FS[(r0 + 4 * lg4 + j) * L::LFS + c0 + lr];
      }
    }
#pragma unroll
    for (int s = 0; s < MT; ++s) {
      const int id = wave + NWAVE * s;
      if (id < DT * ET) {
        const int r0 = 16 * (id / ET), c0 = 16 * (id % ET);
        f32x4 acc = gemm_f32_tile<D>(FS, L::LFS, FC, L::LFC, r0, c0, lane, zero4());
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] -= pG[(size_t)(r0 + 4 * lg4 + j) * E + c0 + lr];
        Mreg[s] = acc;
      }
    }
    if (need_n) {
      const float* pm = a.m + sidx * D;
      const float* ph = a.h + sidx * D;
      for (int r = tid; r < D; r += NTHR) {
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc += FS[r * L::LFS + c] * pm[c];
        nst[r] = acc - ph[r];
      }
    }
  }
  __syncthreads();

  // ---- tile staging (global -> registers -> LDS) -----------------------------
  constexpr int QCH = TT * D / CH, VCH = TT * E / CH;
  constexpr int QPT = (QCH + NTHR - 1) / NTHR, VPT = (VCH + NTHR - 1) / NTHR;
  uint4 rq[QPT], rk[QPT], rv[VPT];
  auto load_tile = [&](int t0, int Lt) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int c = tid + NTHR * i;
      rq[i] = make_uint4(0, 0, 0, 0);
      rk[i] = make_uint4(0, 0, 0, 0);
      if (c < QCH) {
        const int row = c / (D / CH), col = (c % (D / CH)) * CH;
        if (row < Lt) {
          rq[i] = *reinterpret_cast<const uint4*>(gq + (size_t)(t0 + row) * D + col);
          rk[i] = *reinterpret_cast<const uint4*>(gk + (size_t)(t0 + row) * D + col);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + NTHR * i;
      rv[i] = make_uint4(0, 0, 0, 0);
      if (c < VCH) {
        const int row = c / (E / CH), col = (c % (E / CH)) * CH;
        if (row < Lt) rv[i] = *reinterpret_cast<const uint4*>(gv + (size_t)(t0 + row) * E + col);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int c = tid + NTHR * i;
      if (c < QCH) {
        const int row = c / (D / CH), col = (c % (D / CH)) * CH;
        *reinterpret_cast<uint4*>(Qs + row * L::LDD + col) = rq[i];
        *reinterpret_cast<uint4*>(Ks + row * L::LDD + col) = rk[i];
        const T* ke = reinterpret_cast<const T*>(&rk[i]);
#pragma unroll
        for (int e = 0; e < CH; ++e) Kt[(col + e) * L::LDT + row] = ke[e];
        if (MODE == MODE_SUMMARY) {
          const T* qe = reinterpret_cast<const T*>(&rq[i]);
#pragma unroll
          for (int e = 0; e < CH; ++e) X1[(col + e) * L::LDT + row] = qe[e];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + NTHR * i;
      if (c < VCH) {
        const int row = c / (E / CH), col = (c % (E / CH)) * CH;
        const T* ve = reinterpret_cast<const T*>(&rv[i]);
#pragma unroll
        for (int e = 0; e < CH; ++e) Vt[(col + e) * L::LDT + row] = ve[e];
      }
    }
  };

  const int ntiles = (Lspan + TT - 1) / TT;
  load_tile(0, Lspan < TT ? Lspan : TT);
  int Lt_prev = -1;

  for (int ti = 0; ti < ntiles; ++ti) {
    const int t0 = ti * TT;
    const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;

    // ---- step 0: stage tile, state operand, per-tile weights ----------------
    store_tile();
    if (ti + 1 < ntiles) {
      const int t1 = t0 + TT;
      load_tile(t1, (Lspan - t1) < TT ? (Lspan - t1) : TT);
    }
    if (Lt != Lt_prev && tid < TT) {
      wS[tid] = tid < Lt ? gpow(g, lgg, Lt - 1 - tid) : 0.f;
      wM[tid] = tid < Lt ? gpow(g, lgg, 2 * (Lt - 1 - tid)) : 0.f;
    }
    Lt_prev = Lt;
    // S operand: SM[n][k] = S[k][n]
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      const int id = wave + NWAVE * s;
      if (id < DT * DT) {
        const int r0 = 16 * (id / DT), c0 = 16 * (id % DT);
        store4<T>(SM + (c0 + lr) * L::LDSM + r0 + 4 * lg4, Sreg[s]);
      }
    }
    __syncthreads();

    if (need_n && MODE == MODE_OUTPUT && tid < TT) {
      // q_tau . n_prev for the denominator (n is updated later in the tile)
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) acc += (float)Qs[tid * L::LDD + c] * nst[c];
      qn[tid] = acc;
    }

    // ---- step 1: A' = (Q K^T) o decay, lower triangle ------------------------
    for (int id = wave; id < TR * TR; id += NWAVE) {
      const int r = id / TR, c = id % TR;
      f32x4 acc = zero4();
      if (c <= r) {
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS)
          acc = MMT::mma(MMT::ld(Qs, L::LDD, 16 * r, k0, lane), MMT::ld(Ks, L::LDD, 16 * c, k0, lane), acc);
      }
      const int i = 16 * c + lr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tau = 16 * r + 4 * lg4 + j;
        const float val = (i <= tau) ? acc[j] * pw[tau - i] : 0.f;
        AB[tau * L::LDT + i] = (T)val;
      }
    }
    __syncthreads();

    // ---- step 2: P = g^(tau+1) Q S_prev + A' K ---------------------------------
    f32x4 Preg[PT];
#pragma unroll
    for (int s = 0; s < PT; ++s) {
      const int id = wave + NWAVE * s;
      Preg[s] = zero4();
      if (id < TR * DT) {
        const int r = id % TR, n0 = 16 * (id / TR);
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS)
          acc = MMT::mma(MMT::ld(Qs, L::LDD, 16 * r, k0, lane), MMT::ld(SM, L::LDSM, n0, k0, lane), acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= w1[16 * r + 4 * lg4 + j];
        const int kend = 16 * r + 16;
        for (int k0 = 0; k0 < kend; k0 += KS)
          acc = MMT::mma(MMT::ld(AB, L::LDT, 16 * r, k0, lane), MMT::ld(Kt, L::LDT, n0, k0, lane), acc);
        Preg[s] = acc;
        // Pt[d][tau] = g^(2(Lt-1-tau)) p_tau[d] (M update operand, weighted once)
        f32x4 pwv;
#pragma unroll
        for (int j = 0; j < 4; ++j) pwv[j] = acc[j] * wM[16 * r + 4 * lg4 + j];
        store4<T>(Pt + (n0 + lr) * L::LDT + 16 * r + 4 * lg4, pwv);
        if (MODE == MODE_OUTPUT) {
#pragma unroll
          for (int j = 0; j < 4; ++j) X1[(16 * r + 4 * lg4 + j) * L::LDD + n0 + lr] = (T)acc[j];
        }
        if (need_n) {
          const float cs = sum_rows4(pwv[0] + pwv[1] + pwv[2] + pwv[3]);
          if (lg4 == 0) pcol[r * D + n0 + lr] = cs;
        }
      }
    }
    __syncthreads();

    // ---- step 3: state updates, B = (Q P^T) o decay, M operand ---------------
    if (MODE == MODE_OUTPUT) {
      // M operand (state before this tile): SM[e][d] = M[d][e]
#pragma unroll
      for (int s = 0; s < MT; ++s) {
        const int id = wave + NWAVE * s;
        if (id < DT * ET) {
          const int r0 = 16 * (id / ET), c0 = 16 * (id % ET);
          store4<T>(SM + (c0 + lr) * L::LDSM + r0 + 4 * lg4, Mreg[s]);
        }
      }
      for (int id = wave; id < TR * TR; id += NWAVE) {
        const int r = id / TR, c = id % TR;
        f32x4 acc = zero4();
        if (c <= r) {
#pragma unroll
          for (int k0 = 0; k0 < D; k0 += KS)
            acc = MMT::mma(MMT::ld(Qs, L::LDD, 16 * r, k0, lane), MMT::ld(X1, L::LDD, 16 * c, k0, lane), acc);
        }
        const int jj = 16 * c + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tau = 16 * r + 4 * lg4 + j;
          const float val = (jj <= tau) ? acc[j] * pw2[tau - jj] : 0.f;
          AB[tau * L::LDT + jj] = (T)val;
          if (need_n) {
            const float rs = sum16(val);
            if (lr == 0) bpart[c * TT + tau] = rs;
          }
        }
      }
    }
    {
      const float gL = gpow(g, lgg, Lt), g2L = gpow(g, lgg, 2 * Lt);
#pragma unroll
      for (int s = 0; s < ST; ++s) {
        const int id = wave + NWAVE * s;
        if (id < DT * DT) {
          const int r0 = 16 * (id / DT), c0 = 16 * (id % DT);
          f32x4 acc = Sreg[s] * gL;
#pragma unroll
          for (int k0 = 0; k0 < TT; k0 += KS)
            acc = MMT::mma(MMT::ldw(Kt, L::LDT, r0, k0, lane, wS), MMT::ld(Kt, L::LDT, c0, k0, lane), acc);
          Sreg[s] = acc;
        }
      }
#pragma unroll
      for (int s = 0; s < MT; ++s) {
        const int id = wave + NWAVE * s;
        if (id < DT * ET) {
          const int r0 = 16 * (id / ET), c0 = 16 * (id % ET);
          f32x4 acc = Mreg[s] * g2L;
#pragma unroll
          for (int k0 = 0; k0 < TT; k0 += KS)
            acc = MMT::mma(MMT::ld(Pt, L::LDT, r0, k0, lane), MMT::ld(Vt, L::LDT, c0, k0, lane), acc);
          Mreg[s] = acc;
          if (MODE == MODE_SUMMARY) {
            f32x4 cacc = Creg[s] * gL;
#pragma unroll
            for (int k0 = 0; k0 < TT; k0 += KS)
              cacc = MMT::mma(MMT::ldw(X1, L::LDT, r0, k0, lane, wS), MMT::ld(Vt, L::LDT, c0, k0, lane), cacc);
            Creg[s] = cacc;
          }
        }
      }
      if (MODE == MODE_SUMMARY) {
        for (int r = tid; r < D; r += NTHR) {
          float acc = 0.f;
          for (int t = 0; t < Lt; ++t) acc += wS[t] * (float)Qs[t * L::LDD + r];
          mst[r] = gL * mst[r] + acc;
        }
      }
      if (need_n) {
        for (int r = tid; r < D; r += NTHR) {
          float acc = 0.f;
#pragma unroll
          for (int rr = 0; rr < TR; ++rr) acc += pcol[rr * D + r];
          nst[r] = g2L * nst[r] + acc;
        }
      }
    }
    __syncthreads();

    // ---- step 4: outputs ------------------------------------------------------
    if (MODE == MODE_OUTPUT) {
      float* go = a.o + (tok0 + t0) * E;
      // denominator of row tau: the B row sums of the column blocks c <= tau/16 in
      // a fixed order, plus the prefix term
      auto den_of = [&](int tau) {
        float acc = 0.f;
        for (int c = 0; c <= tau / 16; ++c) acc += bpart[c * TT + tau];
        return acc + w2[tau] * qn[tau];
      };
#pragma unroll
      for (int s = 0; s < OT; ++s) {
        const int id = wave + NWAVE * s;
        if (id < TR * ET) {
          const int r = id % TR, e0 = 16 * (id / TR);
          f32x4 acc = zero4();
#pragma unroll
          for (int k0 = 0; k0 < D; k0 += KS)
            acc = MMT::mma(MMT::ld(Qs, L::LDD, 16 * r, k0, lane), MMT::ld(SM, L::LDSM, e0, k0, lane), acc);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] *= w2[16 * r + 4 * lg4 + j];
          const int kend = 16 * r + 16;
          for (int k0 = 0; k0 < kend; k0 += KS)
            acc = MMT::mma(MMT::ld(AB, L::LDT, 16 * r, k0, lane), MMT::ld(Vt, L::LDT, e0, k0, lane), acc);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tau = 16 * r + 4 * lg4 + j;
            float val = acc[j];
            if (a.normalize) val = val / (den_of(tau) + a.eps);
            if (tau < Lt) go[(size_t)tau * E + e0 + lr] = val;
          }
        }
      }
      if (a.den != nullptr && tid < Lt) a.den[tok0 + t0 + tid] = den_of(tid);
      __syncthreads();
    }
  }

  // ---- segment summary: S, C, m, G = S C - M, h = S m - n ----------------------
  if (MODE == MODE_SUMMARY) {
    float* oS = a.S + sidx * D * D;
    float* oC = a.C + sidx * D * E;
    float* oG = a.G + sidx * D * E;
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      const int id = wave + NWAVE * s;
      if (id < DT * DT) {
        const int r0 = 16 * (id / DT), c0 = 16 * (id % DT);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = r0 + 4 * lg4 + j;
          FS[r * L::LFS + c0 + lr] = Sreg[s][j];
          oS[(size_t)r * D + c0 + lr] = Sreg[s][j];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < CT; ++s) {
      const int id = wave + NWAVE * s;
      if (id < DT * ET) {
        const int r0 = 16 * (id / ET), c0 = 16 * (id % ET);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = r0 + 4 * lg4 + j;
          FC[r * L::LFC + c0 + lr] = Creg[s][j];
          oC[(size_t)r * E + c0 + lr] = Creg[s][j];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < MT; ++s) {
      const int id = wave + NWAVE * s;
      if (id < DT * ET) {
        const int r0 = 16 * (id / ET), c0 = 16 * (id % ET);
        f32x4 acc = gemm_f32_tile<D>(FS, L::LFS, FC, L::LFC, r0, c0, lane, zero4());
#pragma unroll
        for (int j = 0; j < 4; ++j) oG[(size_t)(r0 + 4 * lg4 + j) * E + c0 + lr] = acc[j] - Mreg[s][j];
      }
    }
    for (int r = tid; r < D; r += NTHR) {
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc += FS[r * L::LFS + c] * mst[c];
      a.m[sidx * D + r] = mst[r];
      a.h[sidx * D + r] = acc - nst[r];
    }
  }
}

// ---- dispatch ------------------------------------------------------------------

template <int MODE>
static hipError_t launch_mode(int dtype, int d, int dv, int units, const ChunkArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)units * (unsigned)a.nspan), block(NTHR);
#define HLA_CASE(T, D, E)                                                            \
  if (d == D && dv == E) {                                                           \
    hipLaunchKernelGGL((chunk_kernel<T, D, E, MODE>), grid, block, 0, s, a);         \
    return hipGetLastError();                                                        \
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

bool chunk_shape_supported(int dtype, int d, int dv) {
  auto ok = [](int x) { return x == 16 || x == 32 || x == 64 || x == 128; };
  if (!ok(d) || !ok(dv)) return false;
  if (d > 2 * dv || dv > 2 * d) return false;
  if (dtype == 0 && (d > 64 || dv > 64)) return false;
  return dtype == 0 || dtype == 1;
}

hipError_t launch_chunk_summaries(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                  hipStream_t s) {
  return launch_mode<MODE_SUMMARY>(dtype, d, dv, units, a, s);
}

hipError_t launch_chunk_outputs(int dtype, int d, int dv, int units, const ChunkArgs& a,
                                hipStream_t s) {
  return launch_mode<MODE_OUTPUT>(dtype, d, dv, units, a, s);
}

}  // namespace hla
