// Segment summaries and segment outputs of the masked second-order HLA
// forward ("Higher-order Linear Attention", arXiv 2510.27258, summaries on
// gist.science: method section 1 for the state and the output, section 4
// for segment summaries and the chunk-parallel scheme, key contribution 2 for
// decay).
//
// One workgroup owns one segment of `chunk` tokens of one (batch, head) unit
// and walks it in tiles of TT = 64 tokens.  Inside a segment it does not carry
// (S, C, m, G, h) but the equivalent pair (S, M) with M_t = S_t C_t - G_t,
// using the identity
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
// Layout on chip.  The tile is staged row-major only (Q, K, V in LDS);
// operands that need the token index contiguous per lane are read with the
// transposing LDS read.  The state lives in fp32 MFMA accumulators: wave w
// owns column block w (16 columns, all rows) of S and of M (and C), and feeds
// those accumulators straight back into the MFMA as the B operand of Q S and
// Q M (Frag::acc_b), so the state never goes through LDS inside the loop.
// The wave that owns S column block w also produces column block w of P and
// writes it transposed (P^T, token-contiguous) to LDS; the wave that owns M
// column block w produces column block w of the output.  Score tiles are
// computed transposed (K Q^T, P Q^T) so that each lane stores four
// consecutive positions and sums its column in registers.
//
// All products run on MFMA (bf16 operands for bf16 inputs, fp32 operands for
// fp32 inputs) with fp32 accumulation; segment-boundary products (S C, S m)
// run on fp32 MFMA.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr int TT = 64;      // tokens per tile

enum { MODE_SUMMARY = 0, MODE_OUTPUT = 1 };

template <typename T, int D, int E, int MODE>
struct ChunkLayout {
  static constexpr int PADT = 16 / (int)sizeof(T);
  // d-contractions run in steps of MM<T>::KS; a smaller d is zero-padded to one step
  static constexpr int DP = D < MM<T>::KS ? MM<T>::KS : D;
  static constexpr int LDD = DP + PADT;      // Qs, Ks: [tok][d]
  static constexpr int LDV = E + PADT;       // Vs: [tok][e]
  static constexpr int LDT = TT + PADT;      // PsT: [d][tok], AB: [tok][tok]
  static constexpr size_t Qs = 0;
  static constexpr size_t Ks = Qs + (size_t)TT * LDD * sizeof(T);
  static constexpr size_t Vs = Ks + (size_t)TT * LDD * sizeof(T);
  static constexpr size_t PsT = Vs + (size_t)TT * LDV * sizeof(T);
  static constexpr size_t AB = PsT + (size_t)DP * LDT * sizeof(T);
  static constexpr size_t TILE_END = AB + (size_t)TT * LDT * sizeof(T);
  // fp32 overlay used at segment boundaries: S [D][D+4]
  static constexpr int LFS = D + 4;
  static constexpr size_t F_END = (size_t)D * LFS * 4;
  static constexpr size_t BIG = TILE_END > F_END ? TILE_END : F_END;
  static constexpr size_t W = (BIG + 15) / 16 * 16;
  // w1, w2, wS, wM, pw, pw2, qn [TT]; bpart [TR][TT]; pcol, nst, mst [D]
  static constexpr size_t TOTAL = W + (size_t)(7 * TT + (TT / 16) * TT + 3 * D) * 4;
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

// Lower-triangular 16x16 tile number idx (row block r of the later position,
// column block c <= r) of the TR*(TR+1)/2 such tiles.
__device__ __forceinline__ void tri_tile(int idx, int& r, int& c) {
  r = 0;
  while (idx > r) { idx -= r + 1; ++r; }
  c = idx;
}

template <typename T, int D, int E, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_kernel(ChunkArgs a) {
  constexpr int NTHR = 64 * NW;
  using L = ChunkLayout<T, D, E, MODE>;
  using MMT = MM<T>;
  using FR = Frag<T>;
  using F = typename MMT::F;
  constexpr int KS = MMT::KS;
  constexpr int CH = MMT::CH;
  constexpr int DP = L::DP;
  constexpr int DT = D / 16, ET = E / 16, TR = TT / 16, NKS = TT / KS;
  constexpr int NTRI = TR * (TR + 1) / 2;
  constexpr int QSK = KS == 32 ? (DT + 1) / 2 : DT * 4;   // K steps of Q S and Q M
  static_assert(DT <= NW && ET <= NW, "one state column block per wave");

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  T* Qs = reinterpret_cast<T*>(smem + L::Qs);
  T* Ks = reinterpret_cast<T*>(smem + L::Ks);
  T* Vs = reinterpret_cast<T*>(smem + L::Vs);
  T* PsT = reinterpret_cast<T*>(smem + L::PsT);
  T* AB = reinterpret_cast<T*>(smem + L::AB);
  float* FS = reinterpret_cast<float*>(smem);
  float* w1 = reinterpret_cast<float*>(smem + L::W);
  float* w2 = w1 + TT;
  float* wS = w2 + TT;
  float* wM = wS + TT;
  float* pw = wM + TT;
  float* pw2 = pw + TT;
  float* qn = pw2 + TT;
  float* bpart = qn + TT;        // [TR][TT]: B column sums per 16-row block of j
  float* pcol = bpart + TR * TT; // [D]: weighted column sums of P (one writer per column)
  float* nst = pcol + D;
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
  const bool ownS = wave < DT, ownM = wave < ET;   // column block `wave` of S / of M, C, G
  const int cs0 = 16 * wave;                        // first column of the owned block

  f32x4 Sreg[DT], Mreg[DT], Creg[MODE == MODE_SUMMARY ? DT : 1];

  if (tid < TT) {
    pw[tid] = gpow(g, lgg, tid);
    pw2[tid] = gpow(g, lgg, 2 * tid);
    w1[tid] = gpow(g, lgg, tid + 1);
    w2[tid] = gpow(g, lgg, 2 * tid + 2);
  }

  // ---- initial state -------------------------------------------------------
#pragma unroll
  for (int t = 0; t < DT; ++t) { Sreg[t] = zero4(); Mreg[t] = zero4(); }
  if (MODE == MODE_SUMMARY) {
#pragma unroll
    for (int t = 0; t < DT; ++t) Creg[t] = zero4();
    for (int i = tid; i < D; i += NTHR) { nst[i] = 0.f; mst[i] = 0.f; }
  } else {
    // S from the prefix; M = S_P C_P - G_P with S_P staged in LDS (fp32) as the
    // A operand and the wave's column block of C_P as the B operand
    const float* pS = a.S + sidx * D * D;
    const float* pC = a.C + sidx * D * E;
    const float* pG = a.G + sidx * D * E;
    for (int i = tid; i < D * D / 4; i += NTHR) {
      const int r = (4 * i) / D, c = (4 * i) % D;
      *reinterpret_cast<f32x4*>(FS + r * L::LFS + c) = reinterpret_cast<const f32x4*>(pS)[i];
    }
    __syncthreads();
    if (ownS) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) Sreg[t][j] = FS[(16 * t + 4 * lg4 + j) * L::LFS + cs0 + lr];
    }
    if (ownM) {
      f32x4 cp[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) cp[t][j] = pC[(size_t)(16 * t + 4 * lg4 + j) * E + cs0 + lr];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < D / 4; ++kk)
          acc = MM<float>::mma(FS[(16 * t + lr) * L::LFS + 16 * (kk >> 2) + 4 * lg4 + (kk & 3)],
                               Frag<float>::acc_b(cp, kk), acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] -= pG[(size_t)(16 * t + 4 * lg4 + j) * E + cs0 + lr];
        Mreg[t] = acc;
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
    __syncthreads();
  }
  // zero the tile region once: the upper score tiles and any padding columns
  // [D, DP) / rows of P^T are read as zeros and never written
  for (size_t i = tid; i < L::TILE_END / 16; i += NTHR)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // ---- tile staging: global -> registers -> LDS, row-major, 16-byte chunks ---
  // The summary kernel issues the loads of tile t+1 in the middle of tile t
  // (step 2) and writes them to LDS at the start of tile t+1.  The output
  // kernel holds more state and would spill, so it loads and stores each
  // tile at its start (all loads issued before the first store).
  constexpr int QCH = TT * D / CH, VCH = TT * E / CH;
  constexpr int NCH = 2 * QCH + VCH;
  constexpr int SPT = (NCH + NTHR - 1) / NTHR;
  uint4 xs[SPT];   // prefetched tile (summary kernel only)
  auto load_tile = [&](uint4 (&xs)[SPT], int t0, int Lt) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int c = tid + NTHR * i;
      xs[i] = make_uint4(0, 0, 0, 0);
      if (c < NCH) {
        const T* src;
        int cl, W;
        if (c < QCH) { src = gq; cl = c; W = D; }
        else if (c < 2 * QCH) { src = gk; cl = c - QCH; W = D; }
        else { src = gv; cl = c - 2 * QCH; W = E; }
        const int row = cl / (W / CH), col = (cl % (W / CH)) * CH;
        if (row < Lt) xs[i] = *reinterpret_cast<const uint4*>(src + (size_t)(t0 + row) * W + col);
      }
    }
  };
  auto store_tile = [&](const uint4 (&xs)[SPT]) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int c = tid + NTHR * i;
      if (c < NCH) {
        T* dst;
        int cl, W, LD;
        if (c < QCH) { dst = Qs; cl = c; W = D; LD = L::LDD; }
        else if (c < 2 * QCH) { dst = Ks; cl = c - QCH; W = D; LD = L::LDD; }
        else { dst = Vs; cl = c - 2 * QCH; W = E; LD = L::LDV; }
        const int row = cl / (W / CH), col = (cl % (W / CH)) * CH;
        *reinterpret_cast<uint4*>(dst + row * LD + col) = xs[i];
      }
    }
  };
  auto prefetch_next = [&](int ti) {
    const int t1 = (ti + 1) * TT;
    if (t1 < Lspan) load_tile(xs, t1, (Lspan - t1) < TT ? (Lspan - t1) : TT);
  };

  const int ntiles = (Lspan + TT - 1) / TT;
  int Lt_prev = -1;
  if constexpr (MODE == MODE_SUMMARY) load_tile(xs, 0, Lspan < TT ? Lspan : TT);

  for (int ti = 0; ti < ntiles; ++ti) {
    const int t0 = ti * TT;
    const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;

    // ---- step 0: stage the tile and the per-tile weights --------------------
    if constexpr (MODE == MODE_SUMMARY) {
      store_tile(xs);
    } else {
      uint4 xt[SPT];
      load_tile(xt, t0, Lt);
      store_tile(xt);
    }
    if (Lt != Lt_prev && tid < TT) {
      wS[tid] = tid < Lt ? gpow(g, lgg, Lt - 1 - tid) : 0.f;
      wM[tid] = tid < Lt ? gpow(g, lgg, 2 * (Lt - 1 - tid)) : 0.f;
    }
    Lt_prev = Lt;
    __syncthreads();

    // ---- step 1: A'^T = (K Q^T) o decay, q.n for the denominator ---------------
    if (need_n && MODE == MODE_OUTPUT) {
      constexpr int LPR = NTHR / TT;
      const int tau = tid / LPR, part = tid % LPR;
      float acc = 0.f;
#pragma unroll
      for (int c = part * (D / LPR); c < (part + 1) * (D / LPR); ++c)
        acc += (float)Qs[tau * L::LDD + c] * nst[c];
#pragma unroll
      for (int off = 1; off < LPR; off *= 2) acc += __shfl_xor(acc, off, 64);
      if (part == 0) qn[tau] = acc;
    }
    for (int idx = wave; idx < NTRI; idx += NW) {
      int r, c;
      tri_tile(idx, r, c);
      f32x4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DP; k0 += KS)
        acc = MMT::mma(MMT::ld(Ks, L::LDD, 16 * c, k0, lane), MMT::ld(Qs, L::LDD, 16 * r, k0, lane), acc);
      // lane: position tau = 16 r + lr, keys i = 16 c + 4 lg4 + j
      const int tau = 16 * r + lr;
      f32x4 val;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * c + 4 * lg4 + j;
        val[j] = (i <= tau) ? acc[j] * pw[tau - i] : 0.f;
      }
      store4<T>(AB + tau * L::LDT + 16 * c + 4 * lg4, val);
    }
    __syncthreads();

    // ---- step 2: P = g^(tau+1) Q S_prev + A' K; S update -----------------------
    if constexpr (MODE == MODE_SUMMARY) prefetch_next(ti);
    if (ownS) {
      f32x4 pacc[TR];
#pragma unroll
      for (int r = 0; r < TR; ++r) pacc[r] = zero4();
#pragma unroll
      for (int kk = 0; kk < QSK; ++kk) {
        const F b = FR::acc_b(Sreg, kk);
#pragma unroll
        for (int r = 0; r < TR; ++r) pacc[r] = MMT::mma(FR::perm(Qs, L::LDD, 16 * r, kk, lane), b, pacc[r]);
      }
      float ncol = 0.f;
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        pacc[r] *= *reinterpret_cast<const f32x4*>(w1 + 16 * r + 4 * lg4);
        for (int k0 = 0; k0 < 16 * r + 16; k0 += KS)
          pacc[r] = MMT::mma(MMT::ld(AB, L::LDT, 16 * r, k0, lane), FR::tr(Ks, L::LDD, k0, cs0, lane), pacc[r]);
        // P^T[d][tau], d = cs0 + lr, tau = 16 r + 4 lg4 + j
        store4<T>(PsT + (cs0 + lr) * L::LDT + 16 * r + 4 * lg4, pacc[r]);
        const f32x4 wm = *reinterpret_cast<const f32x4*>(wM + 16 * r + 4 * lg4);
        ncol += pacc[r][0] * wm[0] + pacc[r][1] * wm[1] + pacc[r][2] * wm[2] + pacc[r][3] * wm[3];
      }
      if (need_n) {
        ncol = sum_rows4(ncol);
        if (lg4 == 0) pcol[cs0 + lr] = ncol;
      }
      // S[:, block] <- g^Lt S + K^T diag(wS) K[:, block]
      const float gL = gpow(g, lgg, Lt);
      F bk[NKS];
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) bk[kk] = FR::scale(FR::tr(Ks, L::LDD, kk * KS, cs0, lane), wS, kk * KS, lane);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 acc = Sreg[t] * gL;
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) acc = MMT::mma(FR::tr(Ks, L::LDD, kk * KS, 16 * t, lane), bk[kk], acc);
        Sreg[t] = acc;
      }
    }
    __syncthreads();

    // ---- step 3: B^T = (P Q^T) o decay; M (and C, m) update; O = Q M_prev ------
    const float gL = gpow(g, lgg, Lt), g2L = gpow(g, lgg, 2 * Lt);
    f32x4 oacc[MODE == MODE_OUTPUT ? TR : 1];
    if (MODE == MODE_OUTPUT) {
      for (int idx = wave; idx < NTRI; idx += NW) {
        int r, c;
        tri_tile(idx, r, c);
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DP; k0 += KS)
          acc = MMT::mma(FR::tr(PsT, L::LDT, k0, 16 * c, lane), MMT::ld(Qs, L::LDD, 16 * r, k0, lane), acc);
        const int tau = 16 * r + lr;
        f32x4 val;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int jj = 16 * c + 4 * lg4 + j;
          val[j] = (jj <= tau) ? acc[j] * pw2[tau - jj] : 0.f;
        }
        store4<T>(AB + tau * L::LDT + 16 * c + 4 * lg4, val);
        if (need_n) {
          const float rs = sum_rows4(val[0] + val[1] + val[2] + val[3]);
          if (lg4 == 0) bpart[c * TT + tau] = rs;
        }
      }
      if (ownM) {
#pragma unroll
        for (int r = 0; r < TR; ++r) oacc[r] = zero4();
#pragma unroll
        for (int kk = 0; kk < QSK; ++kk) {
          const F b = FR::acc_b(Mreg, kk);
#pragma unroll
          for (int r = 0; r < TR; ++r) oacc[r] = MMT::mma(FR::perm(Qs, L::LDD, 16 * r, kk, lane), b, oacc[r]);
        }
#pragma unroll
        for (int r = 0; r < TR; ++r) oacc[r] *= *reinterpret_cast<const f32x4*>(w2 + 16 * r + 4 * lg4);
      }
    }
    if (ownM) {
      // M[:, block] <- g^2Lt M + P^T diag(wM) V[:, block]; C likewise with Q and wS
      F bv[NKS];
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) bv[kk] = FR::scale(FR::tr(Vs, L::LDV, kk * KS, cs0, lane), wM, kk * KS, lane);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 acc = Mreg[t] * g2L;
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) acc = MMT::mma(MMT::ld(PsT, L::LDT, 16 * t, kk * KS, lane), bv[kk], acc);
        Mreg[t] = acc;
      }
      if (MODE == MODE_SUMMARY) {
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) bv[kk] = FR::scale(FR::tr(Vs, L::LDV, kk * KS, cs0, lane), wS, kk * KS, lane);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          f32x4 acc = Creg[t] * gL;
#pragma unroll
          for (int kk = 0; kk < NKS; ++kk) acc = MMT::mma(FR::tr(Qs, L::LDD, kk * KS, 16 * t, lane), bv[kk], acc);
          Creg[t] = acc;
        }
      }
    }
    if (MODE == MODE_SUMMARY) {
      // m <- g^Lt m + sum_tau wS[tau] q_tau: NTHR / D lanes per column
      constexpr int LPC = NTHR / D;
      const int col = tid / LPC, part = tid % LPC;
      float acc = 0.f;
      for (int t = part; t < Lt; t += LPC) acc += wS[t] * (float)Qs[t * L::LDD + col];
#pragma unroll
      for (int off = 1; off < LPC; off *= 2) acc += __shfl_xor(acc, off, 64);
      if (part == 0) mst[col] = gL * mst[col] + acc;
    }
    if (need_n) {
      for (int r = tid; r < D; r += NTHR) nst[r] = g2L * nst[r] + pcol[r];
    }
    __syncthreads();

    // ---- step 4: O += B V; write the outputs ------------------------------------
    if (MODE == MODE_OUTPUT) {
      if (ownM) {
        float* go = a.o + (tok0 + t0) * E;
#pragma unroll
        for (int r = 0; r < TR; ++r) {
          for (int k0 = 0; k0 < 16 * r + 16; k0 += KS)
            oacc[r] = MMT::mma(MMT::ld(AB, L::LDT, 16 * r, k0, lane), FR::tr(Vs, L::LDV, k0, cs0, lane), oacc[r]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tau = 16 * r + 4 * lg4 + j;
            float val = oacc[r][j];
            if (a.normalize) {
              float dn = 0.f;
              for (int c = 0; c <= r; ++c) dn += bpart[c * TT + tau];
              val = val / (dn + w2[tau] * qn[tau] + a.eps);
            }
            if (tau < Lt) go[(size_t)tau * E + cs0 + lr] = val;
          }
        }
      }
      if (a.den != nullptr && tid < Lt) {
        float dn = 0.f;
        for (int c = 0; c <= tid / 16; ++c) dn += bpart[c * TT + tid];
        a.den[tok0 + t0 + tid] = dn + w2[tid] * qn[tid];
      }
      __syncthreads();
    }
  }

  // ---- segment summary: S, C, m, G = S C - M, h = S m - n ----------------------
  if (MODE == MODE_SUMMARY) {
    float* oS = a.S + sidx * D * D;
    float* oC = a.C + sidx * D * E;
    float* oG = a.G + sidx * D * E;
    // the tile region is free now: S goes to LDS (fp32) as the A operand of S C
    if (ownS) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * t + 4 * lg4 + j;
          FS[r * L::LFS + cs0 + lr] = Sreg[t][j];
          oS[(size_t)r * D + cs0 + lr] = Sreg[t][j];
        }
    }
    __syncthreads();
    if (ownM) {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < D / 4; ++kk)
          acc = MM<float>::mma(FS[(16 * t + lr) * L::LFS + 16 * (kk >> 2) + 4 * lg4 + (kk & 3)],
                               Frag<float>::acc_b(Creg, kk), acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const size_t e = (size_t)(16 * t + 4 * lg4 + j) * E + cs0 + lr;
          oC[e] = Creg[t][j];
          oG[e] = acc[j] - Mreg[t][j];
        }
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

template <int D, int E>
struct Waves {
  // one wave per 16-column block of the wider state, at least 4
  static constexpr int M = D > E ? D / 16 : E / 16;
  static constexpr int value = M > 4 ? M : 4;
};

template <int MODE>
static hipError_t launch_mode(int dtype, int d, int dv, int units, const ChunkArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)units * (unsigned)a.nspan);
#define HLA_CASE(T, D, E)                                                                    \
  if (d == D && dv == E) {                                                                   \
    constexpr int NW = Waves<D, E>::value;                                                   \
    hipLaunchKernelGGL((chunk_kernel<T, D, E, MODE, NW>), grid, dim3(64 * NW), 0, s, a);     \
    return hipGetLastError();                                                                \
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
