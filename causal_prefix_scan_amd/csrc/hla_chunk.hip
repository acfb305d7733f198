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

enum { MODE_SUMMARY = 0, MODE_OUTPUT = 1 };

template <typename T, int D, int E, int MODE>
struct ChunkLayout {
  static constexpr int PADT = 16 / (int)sizeof(T);
  // d-contractions run in steps of MM<T>::KS; a smaller d is zero-padded to one step
  static constexpr int DP = D < MM<T>::KS ? MM<T>::KS : D;
  static constexpr int LDD = DP + PADT;      // [tok][d] buffers
  static constexpr int LDT = TT + PADT;      // [d][tok] buffers
  static constexpr int LDSM = DP + PADT;     // S operand [d][d'] / M operand [e][d]
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

// Four consecutive elements of one LDS row (8 bytes for bf16, 16 for fp32).
template <typename T>
__device__ __forceinline__ void store4_raw(T* p, T a, T b, T c, T d);
template <>
__device__ __forceinline__ void store4_raw<__bf16>(__bf16* p, __bf16 a, __bf16 b, __bf16 c, __bf16 d) {
  bf16x4 y;
  y[0] = a; y[1] = b; y[2] = c; y[3] = d;
  *reinterpret_cast<bf16x4*>(p) = y;
}
template <>
__device__ __forceinline__ void store4_raw<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Ownership of the 16x16 tiles of an R x CB grid (R row blocks, CB column
// blocks) by the NW waves of a workgroup.  Slot s of wave w holds tile (rb, cb):
//   CB >= NW: cb = w + NW * (s / R), rb = s % R
//   CB <  NW: cb = w % CB,          rb = w / CB + (NW / CB) * s
// so consecutive slots of a wave share a column block, and therefore the B
// fragments of a product whose B operand depends only on the column.
template <int R, int CB, int NW>
struct Owner {
  static constexpr int SLOTS = (R * CB + NW - 1) / NW;
  __device__ static __forceinline__ bool tile(int w, int s, int& rb, int& cb) {
    if (CB >= NW) {
      cb = w + NW * (s / R);
      rb = s % R;
      return cb < CB;
    }
    cb = w % CB;
    rb = w / CB + (NW / CB) * s;
    return rb < R;
  }
  __device__ static __forceinline__ bool new_col(int s) { return CB >= NW ? (s % R) == 0 : s == 0; }
};

template <typename T, int D, int E, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_kernel(ChunkArgs a) {
  constexpr int NTHR = 64 * NW;
  using L = ChunkLayout<T, D, E, MODE>;
  using MMT = MM<T>;
  using F = typename MMT::F;
  constexpr int KS = MMT::KS;
  constexpr int CH = MMT::CH;
  constexpr int DP = L::DP;
  constexpr int DT = D / 16, ET = E / 16, TR = TT / 16, NKS = TT / KS;
  static_assert(NW % TR == 0, "row-block ownership of P and O tiles needs TR | NW");
  using OS = Owner<DT, DT, NW>;                   // S tiles
  using OM = Owner<DT, ET, NW>;                   // M, C and G tiles
  constexpr int PSL = (TR * DT + NW - 1) / NW;    // P slots per wave (row block wave % TR)
  constexpr int OSL = (TR * ET + NW - 1) / NW;    // O slots per wave
  constexpr int CT = MODE == MODE_SUMMARY ? OM::SLOTS : 1;

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  T* Qs = reinterpret_cast<T*>(smem + L::Qs);
  T* Ks = reinterpret_cast<T*>(smem + L::Ks);
  T* Kt = reinterpret_cast<T*>(smem + L::Kt);
  T* Vt = reinterpret_cast<T*>(smem + L::Vt);
  T* X1 = reinterpret_cast<T*>(smem + L::X1);   // Qt (summary) or Ps (output)
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
  float* bpart = qn + TT;        // [TR][TT]: row sums of B per 16-column block
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

  f32x4 Sreg[OS::SLOTS], Mreg[OM::SLOTS], Creg[CT];

  if (tid < TT) {
    pw[tid] = gpow(g, lgg, tid);
    pw2[tid] = gpow(g, lgg, 2 * tid);
    w1[tid] = gpow(g, lgg, tid + 1);
    w2[tid] = gpow(g, lgg, 2 * tid + 2);
  }

  // ---- initial state -------------------------------------------------------
  if (MODE == MODE_SUMMARY) {
#pragma unroll
    for (int s = 0; s < OS::SLOTS; ++s) Sreg[s] = zero4();
#pragma unroll
    for (int s = 0; s < OM::SLOTS; ++s) Mreg[s] = zero4();
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
    for (int s = 0; s < OS::SLOTS; ++s) {
      int rb, cb;
      if (OS::tile(wave, s, rb, cb)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) Sreg[s][j] = FS[(16 * rb + 4 * lg4 + j) * L::LFS + 16 * cb + lr];
      }
    }
#pragma unroll
    for (int s = 0; s < OM::SLOTS; ++s) {
      int rb, cb;
      if (OM::tile(wave, s, rb, cb)) {
        f32x4 acc = gemm_f32_tile<D>(FS, L::LFS, FC, L::LFC, 16 * rb, 16 * cb, lane, zero4());
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] -= pG[(size_t)(16 * rb + 4 * lg4 + j) * E + 16 * cb + lr];
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
  // The next tile is not prefetched into registers: with the state held in
  // accumulators the extra live registers spill, which costs more than the
  // exposed load latency.
  // Row-major copies (Qs, Ks): thread <-> consecutive 16-byte chunks of a row,
  // so both the global loads and the LDS writes are contiguous.
  // Transposed copies (Kt, Vt and, for summaries, Qt = X1): one item is 4 rows x
  // one 16-byte column chunk; the 16 lanes of a quarter-wave take 16 row
  // quads of the same column chunk, so each packed 4-row write of a column is
  // one 8-byte (bf16) / 16-byte (fp32) store into consecutive LDS words.
  constexpr int RCH = TT * D / CH;                       // row chunks per tensor
  constexpr int RPT = (2 * RCH + NTHR - 1) / NTHR;
  constexpr int IK = (TT / 4) * (D / CH), IV = (TT / 4) * (E / CH);
  constexpr int NIT = IK + IV + (MODE == MODE_SUMMARY ? IK : 0);
  constexpr int TPT = (NIT + NTHR - 1) / NTHR;
  uint4 rrow[RPT];
  uint4 rtr[TPT][4];
  auto load_tile = [&](int t0, int Lt) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = tid + NTHR * i;
      rrow[i] = make_uint4(0, 0, 0, 0);
      if (c < 2 * RCH) {
        const int cl = c < RCH ? c : c - RCH;
        const T* src = c < RCH ? gq : gk;
        const int row = cl / (D / CH), col = (cl % (D / CH)) * CH;
        if (row < Lt) rrow[i] = *reinterpret_cast<const uint4*>(src + (size_t)(t0 + row) * D + col);
      }
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int it = tid + NTHR * i;
#pragma unroll
      for (int r = 0; r < 4; ++r) rtr[i][r] = make_uint4(0, 0, 0, 0);
      if (it < NIT) {
        const T* src;
        int loc, W;
        if (it < IK) { src = gk; loc = it; W = D; }
        else if (it < IK + IV) { src = gv; loc = it - IK; W = E; }
        else { src = gq; loc = it - IK - IV; W = D; }
        const int rq4 = 4 * (loc % (TT / 4)), col = (loc / (TT / 4)) * CH;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (rq4 + r < Lt)
            rtr[i][r] = *reinterpret_cast<const uint4*>(src + (size_t)(t0 + rq4 + r) * W + col);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = tid + NTHR * i;
      if (c < 2 * RCH) {
        const int cl = c < RCH ? c : c - RCH;
        T* dst = c < RCH ? Qs : Ks;
        const int row = cl / (D / CH), col = (cl % (D / CH)) * CH;
        *reinterpret_cast<uint4*>(dst + row * L::LDD + col) = rrow[i];
      }
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int it = tid + NTHR * i;
      if (it < NIT) {
        T* dst;
        int loc;
        if (it < IK) { dst = Kt; loc = it; }
        else if (it < IK + IV) { dst = Vt; loc = it - IK; }
        else { dst = X1; loc = it - IK - IV; }
        const int rq4 = 4 * (loc % (TT / 4)), col = (loc / (TT / 4)) * CH;
        const T* e0 = reinterpret_cast<const T*>(&rtr[i][0]);
        const T* e1 = reinterpret_cast<const T*>(&rtr[i][1]);
        const T* e2 = reinterpret_cast<const T*>(&rtr[i][2]);
        const T* e3 = reinterpret_cast<const T*>(&rtr[i][3]);
#pragma unroll
        for (int e = 0; e < CH; ++e) store4_raw<T>(dst + (col + e) * L::LDT + rq4, e0[e], e1[e], e2[e], e3[e]);
      }
    }
  };

  if (DP > D) {
    // padding columns [D, DP) of the d-contraction buffers must read as zero
    for (size_t i = tid; i < L::TILE_END / 16; i += NTHR)
      reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }
  const int ntiles = (Lspan + TT - 1) / TT;
  int Lt_prev = -1;
  const int rw = wave % TR;   // row block of the wave's P and O tiles

  for (int ti = 0; ti < ntiles; ++ti) {
    const int t0 = ti * TT;
    const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;

    // ---- step 0: stage tile, state operand, per-tile weights ----------------
    load_tile(t0, Lt);
    store_tile();
    if (Lt != Lt_prev && tid < TT) {
      wS[tid] = tid < Lt ? gpow(g, lgg, Lt - 1 - tid) : 0.f;
      wM[tid] = tid < Lt ? gpow(g, lgg, 2 * (Lt - 1 - tid)) : 0.f;
    }
    Lt_prev = Lt;
    // S operand: SM[n][k] = S[k][n]
#pragma unroll
    for (int s = 0; s < OS::SLOTS; ++s) {
      int rb, cb;
      if (OS::tile(wave, s, rb, cb)) store4<T>(SM + (16 * cb + lr) * L::LDSM + 16 * rb + 4 * lg4, Sreg[s]);
    }
    __syncthreads();

    if (need_n && MODE == MODE_OUTPUT) {
      // q_tau . n_prev for the denominator (n is updated later in the tile)
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

    // ---- step 1: A' = (Q K^T) o decay, lower triangle ------------------------
    for (int id = wave; id < TR * TR; id += NW) {
      const int r = id / TR, c = id % TR;
      f32x4 acc = zero4();
      if (c <= r) {
#pragma unroll
        for (int k0 = 0; k0 < DP; k0 += KS)
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
    {
      F qf[DP / KS];
#pragma unroll
      for (int kk = 0; kk < DP / KS; ++kk) qf[kk] = MMT::ld(Qs, L::LDD, 16 * rw, kk * KS, lane);
      const f32x4 w1v = *reinterpret_cast<const f32x4*>(w1 + 16 * rw + 4 * lg4);
      const f32x4 wMv = *reinterpret_cast<const f32x4*>(wM + 16 * rw + 4 * lg4);
#pragma unroll
      for (int s = 0; s < PSL; ++s) {
        const int cb = wave / TR + (NW / TR) * s;
        if (cb < DT) {
          const int n0 = 16 * cb;
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < DP / KS; ++kk)
            acc = MMT::mma(qf[kk], MMT::ld(SM, L::LDSM, n0, kk * KS, lane), acc);
          acc *= w1v;
          const int kend = 16 * rw + 16;
          for (int k0 = 0; k0 < kend; k0 += KS)
            acc = MMT::mma(MMT::ld(AB, L::LDT, 16 * rw, k0, lane), MMT::ld(Kt, L::LDT, n0, k0, lane), acc);
          // Pt[d][tau] = g^(2(Lt-1-tau)) p_tau[d] (M update operand, weighted once)
          const f32x4 pwv = acc * wMv;
          store4<T>(Pt + (n0 + lr) * L::LDT + 16 * rw + 4 * lg4, pwv);
          if (MODE == MODE_OUTPUT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) X1[(16 * rw + 4 * lg4 + j) * L::LDD + n0 + lr] = (T)acc[j];
          }
          if (need_n) {
            const float cs = sum_rows4(pwv[0] + pwv[1] + pwv[2] + pwv[3]);
            if (lg4 == 0) pcol[rw * D + n0 + lr] = cs;
          }
        }
      }
    }
    __syncthreads();

    // ---- step 3: state updates, B = (Q P^T) o decay, M operand ---------------
    if (MODE == MODE_OUTPUT) {
      // M operand (state before this tile): SM[e][d] = M[d][e]
#pragma unroll
      for (int s = 0; s < OM::SLOTS; ++s) {
        int rb, cb;
        if (OM::tile(wave, s, rb, cb)) store4<T>(SM + (16 * cb + lr) * L::LDSM + 16 * rb + 4 * lg4, Mreg[s]);
      }
      for (int id = wave; id < TR * TR; id += NW) {
        const int r = id / TR, c = id % TR;
        f32x4 acc = zero4();
        if (c <= r) {
#pragma unroll
          for (int k0 = 0; k0 < DP; k0 += KS)
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
      // S <- g^Lt S + K^T diag(wS) K; the weights ride on the B fragments,
      // which a wave shares across the tiles of one column block
      {
        F bk[NKS];
#pragma unroll
        for (int s = 0; s < OS::SLOTS; ++s) {
          int rb, cb;
          if (OS::tile(wave, s, rb, cb)) {
            if (OS::new_col(s)) {
#pragma unroll
              for (int kk = 0; kk < NKS; ++kk) bk[kk] = MMT::ldw(Kt, L::LDT, 16 * cb, kk * KS, lane, wS);
            }
            f32x4 acc = Sreg[s] * gL;
#pragma unroll
            for (int kk = 0; kk < NKS; ++kk)
              acc = MMT::mma(MMT::ld(Kt, L::LDT, 16 * rb, kk * KS, lane), bk[kk], acc);
            Sreg[s] = acc;
          }
        }
      }
      // M <- g^2Lt M + Pt V (Pt carries the weights); C <- g^Lt C + Q^T diag(wS) V
      {
        F bv[NKS], bvw[MODE == MODE_SUMMARY ? NKS : 1];
#pragma unroll
        for (int s = 0; s < OM::SLOTS; ++s) {
          int rb, cb;
          if (OM::tile(wave, s, rb, cb)) {
            if (OM::new_col(s)) {
#pragma unroll
              for (int kk = 0; kk < NKS; ++kk) {
                bv[kk] = MMT::ld(Vt, L::LDT, 16 * cb, kk * KS, lane);
                if (MODE == MODE_SUMMARY) bvw[kk] = MMT::ldw(Vt, L::LDT, 16 * cb, kk * KS, lane, wS);
              }
            }
            f32x4 acc = Mreg[s] * g2L;
#pragma unroll
            for (int kk = 0; kk < NKS; ++kk)
              acc = MMT::mma(MMT::ld(Pt, L::LDT, 16 * rb, kk * KS, lane), bv[kk], acc);
            Mreg[s] = acc;
            if (MODE == MODE_SUMMARY) {
              f32x4 cacc = Creg[s] * gL;
#pragma unroll
              for (int kk = 0; kk < NKS; ++kk)
                cacc = MMT::mma(MMT::ld(X1, L::LDT, 16 * rb, kk * KS, lane), bvw[kk], cacc);
              Creg[s] = cacc;
            }
          }
        }
      }
      if (MODE == MODE_SUMMARY) {
        // m <- g^Lt m + sum_tau wS[tau] q_tau: NTHR / D lanes per column,
        // interleaved rows, then a shuffle reduction
        constexpr int LPC = NTHR / D;
        const int col = tid / LPC, part = tid % LPC;
        float acc = 0.f;
        for (int t = part; t < Lt; t += LPC) acc += wS[t] * (float)Qs[t * L::LDD + col];
#pragma unroll
        for (int off = 1; off < LPC; off *= 2) acc += __shfl_xor(acc, off, 64);
        if (part == 0) mst[col] = gL * mst[col] + acc;
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
      F qf[DP / KS];
#pragma unroll
      for (int kk = 0; kk < DP / KS; ++kk) qf[kk] = MMT::ld(Qs, L::LDD, 16 * rw, kk * KS, lane);
      const f32x4 w2v = *reinterpret_cast<const f32x4*>(w2 + 16 * rw + 4 * lg4);
#pragma unroll
      for (int s = 0; s < OSL; ++s) {
        const int cb = wave / TR + (NW / TR) * s;
        if (cb < ET) {
          const int e0 = 16 * cb;
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < DP / KS; ++kk)
            acc = MMT::mma(qf[kk], MMT::ld(SM, L::LDSM, e0, kk * KS, lane), acc);
          acc *= w2v;
          const int kend = 16 * rw + 16;
          for (int k0 = 0; k0 < kend; k0 += KS)
            acc = MMT::mma(MMT::ld(AB, L::LDT, 16 * rw, k0, lane), MMT::ld(Vt, L::LDT, e0, k0, lane), acc);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tau = 16 * rw + 4 * lg4 + j;
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
    for (int s = 0; s < OS::SLOTS; ++s) {
      int rb, cb;
      if (OS::tile(wave, s, rb, cb)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * rb + 4 * lg4 + j;
          FS[r * L::LFS + 16 * cb + lr] = Sreg[s][j];
          oS[(size_t)r * D + 16 * cb + lr] = Sreg[s][j];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < CT; ++s) {
      int rb, cb;
      if (OM::tile(wave, s, rb, cb)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * rb + 4 * lg4 + j;
          FC[r * L::LFC + 16 * cb + lr] = Creg[s][j];
          oC[(size_t)r * E + 16 * cb + lr] = Creg[s][j];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < OM::SLOTS; ++s) {
      int rb, cb;
      if (OM::tile(wave, s, rb, cb)) {
        f32x4 acc = gemm_f32_tile<D>(FS, L::LFS, FC, L::LFC, 16 * rb, 16 * cb, lane, zero4());
#pragma unroll
        for (int j = 0; j < 4; ++j)
          oG[(size_t)(16 * rb + 4 * lg4 + j) * E + 16 * cb + lr] = acc[j] - Mreg[s][j];
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
  const dim3 grid((unsigned)units * (unsigned)a.nspan);
#define HLA_CASE(T, D, E)                                                                    \
  if (d == D && dv == E) {                                                                   \
    constexpr int NW = 8;                                                                    \
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
