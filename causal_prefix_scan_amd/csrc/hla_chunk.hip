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
// As it needs C, m, M and n only there, it weights each token by its decay
// to the segment end (g^(L-1-j) for C and m, g^(2(L-1-j)) for M and n) and
// never rescales those running sums; S is rescaled per tile as above.
// The output kernel starts from the segment's exclusive prefix
// (S_P, C_P, m_P, G_P, h_P) with M = S_P C_P - G_P and n = S_P m_P - h_P.
//
// Layout on chip.  The tile is staged row-major only (Q, K, V in LDS);
// operands that need the token index contiguous per lane are read with the
// transposing LDS read.  The state lives in fp32 MFMA accumulators and never
// goes through LDS inside the loop.  The waves split into two roles with a
// tile loop each (same barriers): the S waves own column blocks of S, produce
// the matching column blocks of P = Q S (S fed back as the MFMA B operand,
// Frag::acc_b), write them transposed (P^T, token-contiguous) to LDS, and
// compute the B score tiles; the M waves own column blocks of M (and of C in
// the summary kernel), produce the matching column blocks of the output and
// update M from P^T.  Each wave owns two column blocks when a head dimension
// is 128, so every A fragment read from LDS feeds two MFMAs.  Score tiles are
// computed transposed (K Q^T, P Q^T) so that each lane stores four
// consecutive positions and sums its column in registers.
//
// All products run on MFMA (bf16 operands for bf16 inputs, fp32 operands for
// fp32 inputs) with fp32 accumulation; segment-boundary products (S C, S m)
// run on fp32 MFMA.
#include <type_traits>

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
  // Q S and Q M take the state in the natural K order (lane swaps, bf16 with
  // 8 waves) or read Q in the state's K order (otherwise; fewer registers)
  static constexpr bool NAT = sizeof(T) == 2 && (D == 128 || E == 128);
  // 8-wave kernels (a head dimension of 128, one workgroup per CU) pipeline
  // the score tiles: the next tile's Q (and K in the summary kernel) is staged
  // while the current one is in use, so Q (and K) are double-buffered
  static constexpr bool PIPE = D == 128 || E == 128;
  static constexpr int NQB = PIPE ? 2 : 1, NKB = (PIPE && MODE == 0) ? 2 : 1;
  // Qs, Ks: [tok][d].  With NAT, rows are padded by 32 bytes, which makes the
  // row-major fragment reads free of LDS bank conflicts; the permuted reads
  // prefer 16 (measured)
  static constexpr int LDD = DP + (NAT ? 2 * PADT : PADT);
  static constexpr int LDV = E + PADT;       // Vs: [tok][e]
  static constexpr int LDT = TT + PADT;      // PsT: [d][tok], AB: [tok][tok]
  static constexpr size_t QB = (size_t)TT * LDD * sizeof(T);   // one Q or K buffer
  static constexpr size_t Qs = 0;
  static constexpr size_t Ks = Qs + NQB * QB;
  // V and P^T are double-buffered by tile parity: the M update of a tile runs
  // while the next tile is staged and its P produced
  static constexpr size_t Vs0 = Ks + NKB * QB;
  static constexpr size_t Vs1 = Vs0 + (size_t)TT * LDV * sizeof(T);
  static constexpr size_t PsT0 = Vs1 + (size_t)TT * LDV * sizeof(T);
  static constexpr size_t PsT1 = PsT0 + (size_t)DP * LDT * sizeof(T);
  static constexpr size_t AB = PsT1 + (size_t)DP * LDT * sizeof(T);
  // output kernel: B scores of a tile, read while the next tile's A' is in AB
  static constexpr size_t BB = AB + (size_t)TT * LDT * sizeof(T);
  static constexpr size_t TILE_END = BB + (MODE == 1 ? (size_t)TT * LDT * sizeof(T) : 0);
  // fp32 overlay used at segment boundaries: S [D][D+4]
  static constexpr int LFS = D + 4;
  static constexpr size_t F_END = (size_t)D * LFS * 4;
  static constexpr size_t BIG = TILE_END > F_END ? TILE_END : F_END;
  static constexpr size_t W = (BIG + 15) / 16 * 16;
  // w1, w2, wS, wM0, wM1, pw, pw2, qn0, qn1 [TT]; bpart [TR][TT]; nst, mst [D]
  static constexpr size_t TOTAL = W + (size_t)(9 * TT + (TT / 16) * TT + 2 * D) * 4;
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

template <typename T, int D, int E, int MODE, int NW>
// (4-wave kernels are held to two workgroups per CU: 256 registers per lane)
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void chunk_kernel(ChunkArgs a) {
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
  // Two roles of NOWN waves each: S waves own column blocks of S, M waves own
  // column blocks of M (and of C in the summary kernel).  Block b of the wave
  // with role index rw is column block rw + NOWN * b.
  constexpr int NOWN = NW / 2;
  constexpr int SB = (DT + NOWN - 1) / NOWN, MB = (ET + NOWN - 1) / NOWN;
  constexpr bool SUM = MODE == MODE_SUMMARY;
  // output kernel: add B V and write a tile's outputs during the next tile's
  // main phase (8 waves), or in a phase of its own (4 waves: fewer registers)
  constexpr bool DEFER = !SUM && NW == 8;
  // every block index is in range when the blocks divide evenly over a role
  constexpr bool SFULL = DT % NOWN == 0, MFULL = ET % NOWN == 0;
  // the summary kernel at bf16, d = dv = 128 can also write the segment-local p
  constexpr bool WPK = SUM && sizeof(T) == 2 && D == 128 && E == 128;

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  T* Qs = reinterpret_cast<T*>(smem + L::Qs);
  T* Ks = reinterpret_cast<T*>(smem + L::Ks);
  // Q and K buffers of tile parity p (one buffer each unless pipelined)
  auto Qb = [&](int p) { return reinterpret_cast<T*>(smem + L::Qs + (L::NQB == 2 && p ? L::QB : 0)); };
  auto Kb = [&](int p) { return reinterpret_cast<T*>(smem + L::Ks + (L::NKB == 2 && p ? L::QB : 0)); };
  // buffers of tile parity p
  auto Vsb = [&](int p) { return reinterpret_cast<T*>(smem + (p ? L::Vs1 : L::Vs0)); };
  auto PsTb = [&](int p) { return reinterpret_cast<T*>(smem + (p ? L::PsT1 : L::PsT0)); };
  T* AB = reinterpret_cast<T*>(smem + L::AB);
  T* BB = reinterpret_cast<T*>(smem + L::BB);
  float* FS = reinterpret_cast<float*>(smem);
  float* w1 = reinterpret_cast<float*>(smem + L::W);
  float* w2 = w1 + TT;
  float* wS = w2 + TT;
  auto wMb = [&](int p) { return wS + (p ? 2 * TT : TT); };
  float* pw = wS + 3 * TT;
  float* pw2 = pw + TT;
  float* qn = pw2 + TT;          // [2][TT]: q.n by tile parity
  auto qnb = [&](int p) { return qn + p * TT; };
  float* wC = qn;                // summary kernel (no q.n there): C and m weights
  float* bpart = qn + 2 * TT;    // [TR][TT]: B column sums per 16-row block of j
  float* nst = bpart + TR * TT;
  float* mst = nst + D;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg4 = lane >> 4;
  // Q times a register-resident state (Q S, and Q M as (Q M)^T = M^T Q^T), the
  // state tiles being the B operand (the A operand for M^T: the two operand
  // layouts are alike): in the natural K order (lane swaps) with Q a plain
  // row-major read, or in the accumulator's K order with Q read to match
  auto state_b = [&](const auto& tiles, int kk) {
    if constexpr (L::NAT) return FR::acc_b_nat(tiles, kk);
    else return FR::acc_b(tiles, kk);
  };
  auto state_a = [&](const T* X, int row0, int kk) {
    if constexpr (L::NAT) return MMT::ld(X, L::LDD, row0, 32 * kk, lane);
    else return FR::perm(X, L::LDD, row0, kk, lane);
  };
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
  // the segment's rows as raw buffers: rows at or past the segment end read as zeros
  const auto rq = buf_rsrc(gq, Lspan * D * (int)sizeof(T));
  const auto rk = buf_rsrc(gk, Lspan * D * (int)sizeof(T));
  const auto rv = buf_rsrc(gv, Lspan * E * (int)sizeof(T));
  const size_t sidx = (size_t)unit * nspan + span;
  const bool need_n = SUM || a.normalize || a.den != nullptr;
  const bool sRole = wave < NOWN;
  const int rw = sRole ? wave : wave - NOWN;
  const int ntiles = (Lspan + TT - 1) / TT;

  // output kernel with 4 waves (short segments are common there): the prefix
  // S_P (every thread, to LDS) and the M waves' column blocks of C_P are
  // loaded together before anything waits on them
  constexpr bool EARLY = !SUM && NW == 4;
  constexpr int FSN = (D * D / 4 + NTHR - 1) / NTHR;
  f32x4 fsx[EARLY ? FSN : 1];
  f32x4 cpx[EARLY ? MB : 1][EARLY ? DT : 1];
  if constexpr (EARLY) {
    const f32x4* pS = reinterpret_cast<const f32x4*>(a.S + sidx * D * D);
#pragma unroll
    for (int i = 0; i < FSN; ++i) {
      const int e = tid + NTHR * i;
      fsx[i] = e < D * D / 4 ? pS[e] : zero4();
    }
    if (!sRole) {
      const float* pC = a.C + sidx * D * E;
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int cb = (rw + NOWN * b) % ET;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) cpx[b][t][j] = pC[(size_t)(16 * t + 4 * lg4 + j) * E + 16 * cb + lr];
      }
    }
  }
  if (tid < TT) {
    pw[tid] = gpow(g, lgg, tid);
    pw2[tid] = gpow(g, lgg, 2 * tid);
    w1[tid] = gpow(g, lgg, tid + 1);
    w2[tid] = gpow(g, lgg, 2 * tid + 2);
  }
  if constexpr (SUM) {
    for (int i = tid; i < D; i += NTHR) { nst[i] = 0.f; mst[i] = 0.f; }
  } else {
    // S_P to LDS (fp32): the S waves take their columns of it, the M waves use
    // it as the A operand of S_P C_P, and n = S_P m_P - h_P reads it
    if constexpr (EARLY) {
#pragma unroll
      for (int i = 0; i < FSN; ++i) {
        const int e = tid + NTHR * i;
        if (e < D * D / 4) {
          const int r = (4 * e) / D, c = (4 * e) % D;
          *reinterpret_cast<f32x4*>(FS + r * L::LFS + c) = fsx[i];
        }
      }
    } else {
      const float* pS = a.S + sidx * D * D;
      for (int i = tid; i < D * D / 4; i += NTHR) {
        const int r = (4 * i) / D, c = (4 * i) % D;
        *reinterpret_cast<f32x4*>(FS + r * L::LFS + c) = reinterpret_cast<const f32x4*>(pS)[i];
      }
    }
  }
  __syncthreads();

  // ---- pieces shared by both roles (every thread runs them) -----------------
  // after the role's initial state: n from the prefix, then zero the tile
  // region once (the upper score tiles and any padding columns [D, DP) / rows
  // of P^T are read as zeros and never written)
  auto finish_init = [&]() {
    if (!SUM && need_n) {
      const float* pm = a.m + sidx * D;
      const float* ph = a.h + sidx * D;
      for (int r = tid; r < D; r += NTHR) {
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc += FS[r * L::LFS + c] * pm[c];
        nst[r] = acc - ph[r];
      }
    }
    __syncthreads();
    // the score buffers' upper tiles are read as zeros and never written; with
    // d < DP so are the padding columns of Q, K and rows of P^T
    constexpr size_t Z0 = DP > D ? 0 : L::AB;
    for (size_t i = Z0 / 16 + tid; i < L::TILE_END / 16; i += NTHR)
      reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  };

  // Tile staging: global -> registers -> LDS, row-major, 16-byte chunks (Q
  // chunks [0, QCH), K chunks [QCH, 2 QCH), V chunks [2 QCH, NCH)).  The
  // loads of tile t+1 are issued in the middle of tile t and written to LDS at
  // the start of tile t+1, the S waves carrying Q and K and the M waves V
  // (tile 0 is loaded and stored by all threads).  The 4-wave output kernels
  // keep two workgroups per CU with these registers (measured: B1 H32 T65536
  // d64, outputs 0.39 -> 0.36 ms against staging each tile at its start).
  constexpr int QCH = TT * D / CH, VCH = TT * E / CH;
  constexpr int NCH = 2 * QCH + VCH;
  constexpr int HT = NTHR / 2;
  constexpr int NXS = (2 * QCH + HT - 1) / HT, NXM = (VCH + HT - 1) / HT, NXA = (NCH + NTHR - 1) / NTHR;
  using QK = std::integral_constant<int, 0>;
  using VB = std::integral_constant<int, 2 * QCH>;
  using END = std::integral_constant<int, NCH>;
  using HALF = std::integral_constant<int, HT>;
  using ALL = std::integral_constant<int, NTHR>;
  // chunks [C0, C1) of tile ti by P threads, lt = this thread's index among them
  // slots [I0, I1) of the n = ceil((C1 - C0) / P) slots (default: all)
  auto load_slots = [&](auto& x, int ti, int lt, auto C0, auto C1, auto P, auto I0, auto I1) {
    constexpr int c0 = decltype(C0)::value, c1 = decltype(C1)::value, np = decltype(P)::value;
    constexpr int i0 = decltype(I0)::value, i1 = decltype(I1)::value;
    const int t0 = ti * TT;
    // when every slot i (chunks c0 + np i + [0, np)) lies inside one of Q, K, V,
    // the buffer is known per slot at compile time; otherwise plain loads with
    // a row test (a per-lane choice of buffer would need a waterfall loop)
    constexpr bool SLOT = c0 % np == 0 && QCH % np == 0 && (c1 - c0) % np == 0;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int cb = c0 + np * i, c = cb + lt;
      x[i] = make_uint4(0, 0, 0, 0);
      if constexpr (SLOT) {
        if (cb < QCH) x[i] = buf_load16(rq, (t0 * D + c * CH) * (int)sizeof(T));
        else if (cb < 2 * QCH) x[i] = buf_load16(rk, (t0 * D + (c - QCH) * CH) * (int)sizeof(T));
        else x[i] = buf_load16(rv, (t0 * E + (c - 2 * QCH) * CH) * (int)sizeof(T));
      } else if (c < c1) {
        const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;
        const T* src;
        int cl, W;
        if (c < QCH) { src = gq; cl = c; W = D; }
        else if (c < 2 * QCH) { src = gk; cl = c - QCH; W = D; }
        else { src = gv; cl = c - 2 * QCH; W = E; }
        if (cl / (W / CH) < Lt) x[i] = *reinterpret_cast<const uint4*>(src + (size_t)t0 * W + cl * CH);
      }
    }
  };
  auto load_part = [&](auto& x, int ti, int lt, auto C0, auto C1, auto P) {
    constexpr int n = (decltype(C1)::value - decltype(C0)::value + decltype(P)::value - 1) / decltype(P)::value;
    load_slots(x, ti, lt, C0, C1, P, std::integral_constant<int, 0>{}, std::integral_constant<int, n>{});
  };
  auto store_part = [&](const auto& x, int lt, T* Qd, T* Kd, T* Vs, auto C0, auto C1, auto P) {
    constexpr int c0 = decltype(C0)::value, c1 = decltype(C1)::value, np = decltype(P)::value;
    constexpr int n = (c1 - c0 + np - 1) / np;
    constexpr bool SLOT = c0 % np == 0 && QCH % np == 0 && (c1 - c0) % np == 0;
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int cb = c0 + np * i, c = cb + lt;
      if (SLOT || c < c1) {
        T* dst;
        int cl, W, LD;
        const int cs = SLOT ? cb : c;   // decides the buffer
        if (cs < QCH) { dst = Qd; cl = c; W = D; LD = L::LDD; }
        else if (cs < 2 * QCH) { dst = Kd; cl = c - QCH; W = D; LD = L::LDD; }
        else { dst = Vs; cl = c - 2 * QCH; W = E; LD = L::LDV; }
        const int row = cl / (W / CH), col = (cl % (W / CH)) * CH;
        *reinterpret_cast<uint4*>(dst + row * LD + col) = x[i];
      }
    }
  };
  // the summary kernel's share of the staging for the calling role
  auto load_role = [&](auto& x, int ti, auto s_wave) {
    if constexpr (decltype(s_wave)::value) load_part(x, ti, tid, QK{}, VB{}, HALF{});
    else load_part(x, ti, tid - HT, VB{}, END{}, HALF{});
  };
  auto store_role = [&](const auto& x, T* Vs, auto s_wave) {
    if constexpr (decltype(s_wave)::value) store_part(x, tid, Qs, Ks, Vs, QK{}, VB{}, HALF{});
    else store_part(x, tid - HT, Qs, Ks, Vs, VB{}, END{}, HALF{});
  };

  // Summary kernel: C, m, M and n are needed only at the end of the segment, so
  // their updates weight each token by its decay to the segment end (the
  // tile's rows of sum_j g^(L-1-j) q_j v_j^T and sum_j g^(2(L-1-j)) p_j v_j^T)
  // and the running sums are never rescaled.  Tile t, thread tid < TT.
  auto end_weights = [&](int t, int Lt) {
    const int after = Lspan - t * TT - 1 - tid;   // tokens after this one
    wC[tid] = tid < Lt ? gpow(g, lgg, after) : 0.f;
    wMb(t & 1)[tid] = tid < Lt ? gpow(g, lgg, 2 * after) : 0.f;
  };

  // steps 0 and 1 of tile ti: stage the tile and its weights, then
  // A'^T = (K Q^T) o decay over all waves and q.n for the denominator
  int Lt_prev = -1;
  // x: this role's prefetched part of the tile
  auto tile_head = [&](int ti, int Lt, auto& x, auto s_wave) {
    store_role(x, Vsb(ti & 1), s_wave);
    // wS for this tile; wM[ti & 1] was last written for tile ti - 2
    if ((ti < 2 || Lt != Lt_prev) && tid < TT) {
      wS[tid] = tid < Lt ? gpow(g, lgg, Lt - 1 - tid) : 0.f;
      if constexpr (!SUM) wMb(ti & 1)[tid] = tid < Lt ? gpow(g, lgg, 2 * (Lt - 1 - tid)) : 0.f;
    }
    if constexpr (SUM) {
      if (tid < TT) end_weights(ti, Lt);
    }
    Lt_prev = Lt;
    __syncthreads();

    if (need_n && !SUM) {
      constexpr int LPR = NTHR / TT;
      const int tau = tid / LPR, part = tid % LPR;
      float acc = 0.f;
#pragma unroll
      for (int c = part * (D / LPR); c < (part + 1) * (D / LPR); ++c)
        acc += (float)Qs[tau * L::LDD + c] * nst[c];
#pragma unroll
      for (int off = 1; off < LPR; off *= 2) acc += __shfl_xor(acc, off, 64);
      if (part == 0) qnb(ti & 1)[tau] = acc;
    }
    for (int idx = wave; idx < NTRI; idx += NW) {
      int r, c;
      tri_block(idx, r, c);
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
        val[j] = acc[j] * masked_pow(pw, tau, i);
      }
      store4<T>(AB + tau * L::LDT + 16 * c + 4 * lg4, val);
    }
    __syncthreads();
    if (ti + 1 < ntiles) load_role(x, ti + 1, s_wave);
  };

  // B^T = (P Q^T) o decay for tile ti (output kernel), the tiles shared by all
  // waves with DEFER, else by the S waves (the M waves then hold Q M_prev)
  constexpr int NBW = DEFER ? NW : NOWN;
  auto b_scores = [&](int ti) {
    const T* PsT = PsTb(ti & 1);
    for (int idx = DEFER ? wave : rw; idx < NTRI; idx += NBW) {
      int r, c;
      tri_block(idx, r, c);
      f32x4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DP; k0 += KS)
        acc = MMT::mma(FR::tr(PsT, L::LDT, k0, 16 * c, lane), MMT::ld(Qs, L::LDD, 16 * r, k0, lane), acc);
      const int tau = 16 * r + lr;
      f32x4 val;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int jj = 16 * c + 4 * lg4 + j;
        val[j] = acc[j] * masked_pow(pw2, tau, jj);
      }
      store4<T>(BB + tau * L::LDT + 16 * c + 4 * lg4, val);
      if (need_n) {
        const float rs = sum_rows4(val[0] + val[1] + val[2] + val[3]);
        if (lg4 == 0) bpart[c * TT + tau] = rs;
      }
    }
  };


  // end of the segment, for every thread: m and h = S m - n (S in FS)
  auto write_mh = [&]() {
    for (int r = tid; r < D; r += NTHR) {
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc += FS[r * L::LFS + c] * mst[c];
      a.m[sidx * D + r] = mst[r];
      a.h[sidx * D + r] = acc - nst[r];
    }
  };

  // ---- pieces of the pipelined (8-wave) kernels ----
  // decay weights of tile t (wS, and wM by parity), by the threads tid < TT;
  // only the last tile can be short, so tiles 2 .. ntiles-2 reuse earlier values
  // (the summary kernel's weights to the segment end change every tile)
  auto weights = [&](int t) {
    const int Lt = (Lspan - t * TT) < TT ? (Lspan - t * TT) : TT;
    if ((t < 2 || t == ntiles - 1) && tid < TT) {
      wS[tid] = tid < Lt ? gpow(g, lgg, Lt - 1 - tid) : 0.f;
      if constexpr (!SUM) wMb(t & 1)[tid] = tid < Lt ? gpow(g, lgg, 2 * (Lt - 1 - tid)) : 0.f;
    }
    if constexpr (SUM) {
      if (tid < TT) end_weights(t, Lt);
    }
  };
  // A' score tile idx (rows 16 r + lr of the later position, masked and
  // decayed) of the tile in buffers p, left in registers
  auto a_tile = [&](int idx, int p) {
    int r, c;
    tri_block(idx, r, c);
    const T* Qx = Qb(p);
    const T* Kx = Kb(p);
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < DP; k0 += KS)
      acc = MMT::mma(MMT::ld(Kx, L::LDD, 16 * c, k0, lane), MMT::ld(Qx, L::LDD, 16 * r, k0, lane), acc);
    const int tau = 16 * r + lr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 16 * c + 4 * lg4 + j;
      acc[j] = acc[j] * masked_pow(pw, tau, i);
    }
    return acc;
  };
  auto a_store = [&](int idx, f32x4 val) {
    int r, c;
    tri_block(idx, r, c);
    store4<T>(AB + (16 * r + lr) * L::LDT + 16 * c + 4 * lg4, val);
  };
  // B^T score tile idx of the tile whose P^T and Q sit in buffers p, to BB
  // (and its column sums to bpart)
  auto b_tile = [&](int idx, int p) {
    int r, c;
    tri_block(idx, r, c);
    const T* PsT = PsTb(p);
    const T* Qx = Qb(p);
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < DP; k0 += KS)
      acc = MMT::mma(FR::tr(PsT, L::LDT, k0, 16 * c, lane), MMT::ld(Qx, L::LDD, 16 * r, k0, lane), acc);
    const int tau = 16 * r + lr;
    f32x4 val;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int jj = 16 * c + 4 * lg4 + j;
      val[j] = acc[j] * masked_pow(pw2, tau, jj);
    }
    store4<T>(BB + tau * L::LDT + 16 * c + 4 * lg4, val);
    if (need_n) {
      const float rs = sum_rows4(val[0] + val[1] + val[2] + val[3]);
      if (lg4 == 0) bpart[c * TT + tau] = rs;
    }
  };
  // q.n of the tile in buffers p (n as it stands), for its denominator
  auto q_dot_n = [&](int p) {
    constexpr int LPR = NTHR / TT;
    const T* Qx = Qb(p);
    const int tau = tid / LPR, part = tid % LPR;
    float acc = 0.f;
#pragma unroll
    for (int c = part * (D / LPR); c < (part + 1) * (D / LPR); ++c) acc += (float)Qx[tau * L::LDD + c] * nst[c];
#pragma unroll
    for (int off = 1; off < LPR; off *= 2) acc += __shfl_xor(acc, off, 64);
    if (part == 0) qnb(p)[tau] = acc;
  };
  // tile 0 (and the summary kernel's tile 1 Q, K) to LDS, then A' of tile 0
  auto prologue = [&]() {
    {
      uint4 xt[NXA];
      load_part(xt, 0, tid, QK{}, END{}, ALL{});
      store_part(xt, tid, Qb(0), Kb(0), Vsb(0), QK{}, END{}, ALL{});
    }
    if (SUM && ntiles > 1) {
      constexpr int NXQ = (2 * QCH + NTHR - 1) / NTHR;
      uint4 xt[NXQ];
      load_part(xt, 1, tid, QK{}, VB{}, ALL{});
      store_part(xt, tid, Qb(1), Kb(1), nullptr, QK{}, VB{}, ALL{});
    }
    weights(0);
    __syncthreads();
    for (int idx = wave; idx < NTRI; idx += NW) a_store(idx, a_tile(idx, 0));
    if (!SUM && need_n) q_dot_n(0);
    __syncthreads();
  };
  // output kernel, after tile ti's P^T is complete and tile ti + 1 is staged:
  // B scores of ti and A' of ti + 1 (2 NTRI tiles over the waves), q.n of ti + 1
  auto score_phase = [&](int ti) {
    const bool nxt = ti + 1 < ntiles;
    // 2 NTRI jobs (B tiles of ti, then A' tiles of ti + 1): the M waves take
    // one each, as their main phase is the longer one (measured), the S waves
    // the rest
    constexpr int NJ = 2 * NTRI, SJ = NJ - NOWN;
    auto job = [&](int idx) {
      if (idx < NTRI) b_tile(idx, ti & 1);
      else if (nxt && idx < NJ) a_store(idx - NTRI, a_tile(idx - NTRI, (ti + 1) & 1));
    };
    if (sRole) {
#pragma unroll
      for (int sl = 0; sl < (SJ + NOWN - 1) / NOWN; ++sl) {
        const int idx = rw + NOWN * sl;
        if (idx < SJ) job(idx);
      }
    } else {
      job(SJ + rw);
    }
    if (need_n && nxt) q_dot_n((ti + 1) & 1);
  };

  if (sRole) {
    // ======== S waves: P = g^(tau+1) Q S_prev + A' K, P^T to LDS, S update;
    //          B^T = (P Q^T) o decay in the output kernel ========
    f32x4 St[SB][DT];
#pragma unroll
    for (int b = 0; b < SB; ++b) {
      const int cb = rw + NOWN * b;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          St[b][t][j] = (!SUM && (SFULL || cb < DT)) ? FS[(16 * t + 4 * lg4 + j) * L::LFS + 16 * cb + lr] : 0.f;
    }
    // step 2 of tile ti (tile in Qx, Kx; A' in AB): P, P^T to LDS, n and S
    // updates; mid() runs between Q S and the rest
    auto s_step2 = [&](int ti, float gL, float g2L, const T* Qx, const T* Kx, auto&& mid) {
      T* PsT = PsTb(ti & 1);
      f32x4 pacc[SB][TR];
#pragma unroll
      for (int b = 0; b < SB; ++b)
#pragma unroll
        for (int r = 0; r < TR; ++r) pacc[b][r] = zero4();
#pragma unroll
      for (int kk = 0; kk < QSK; ++kk) {
        F bs[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) bs[b] = state_b(St[b], kk);
#pragma unroll
        for (int r = 0; r < TR; ++r) {
          const F aq = state_a(Qx, 16 * r, kk);
#pragma unroll
          for (int b = 0; b < SB; ++b) pacc[b][r] = MMT::mma(aq, bs[b], pacc[b][r]);
        }
      }
      mid();
      // the segment-local p of this tile to global memory, when asked: per
      // tile, (column block, row block) 16x16 fragments of 512 contiguous
      // bytes in the accumulator's lane order (lane l: tokens 16 r + 4 (l >> 4)
      // + [0, 4) of column 16 cb + (l & 15)), so each store is one coalesced run
      T* plt = nullptr;
      if constexpr (WPK) {
        if (a.pl) plt = reinterpret_cast<T*>(a.pl) + (sidx * (size_t)ntiles + (size_t)ti) * (size_t)(D * TT);
      }
      float ncol[SB];
#pragma unroll
      for (int b = 0; b < SB; ++b) ncol[b] = 0.f;
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const f32x4 w1v = *reinterpret_cast<const f32x4*>(w1 + 16 * r + 4 * lg4);
#pragma unroll
        for (int b = 0; b < SB; ++b) pacc[b][r] *= w1v;
        for (int k0 = 0; k0 < 16 * r + 16; k0 += KS) {
          const F aa = MMT::ld(AB, L::LDT, 16 * r, k0, lane);
#pragma unroll
          for (int b = 0; b < SB; ++b)
            if (SFULL || rw + NOWN * b < DT)
              pacc[b][r] = MMT::mma(aa, FR::tr(Kx, L::LDD, k0, 16 * (rw + NOWN * b), lane), pacc[b][r]);
        }
        const f32x4 wm = *reinterpret_cast<const f32x4*>(wMb(ti & 1) + 16 * r + 4 * lg4);
#pragma unroll
        for (int b = 0; b < SB; ++b) {
          const int cb = rw + NOWN * b;
          if (SFULL || cb < DT) {
            // P^T[d][tau], d = 16 cb + lr, tau = 16 r + 4 lg4 + j
            store4<T>(PsT + (16 * cb + lr) * L::LDT + 16 * r + 4 * lg4, pacc[b][r]);
            if constexpr (WPK) {
              if (plt) store4<T>(plt + ((cb * TR + r) * 64 + lane) * 4, pacc[b][r]);
            }
            ncol[b] += pacc[b][r][0] * wm[0] + pacc[b][r][1] * wm[1] + pacc[b][r][2] * wm[2] +
                       pacc[b][r][3] * wm[3];
          }
        }
      }
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int cb = rw + NOWN * b;
        if (need_n && (SFULL || cb < DT)) {
          // n <- g^2Lt n + P^T wM (summary: n + P^T wM, weights to the segment
          // end): one writer per column; q.n of this tile is already taken
          const float cs = sum_rows4(ncol[b]);
          if (lg4 == 0) nst[16 * cb + lr] = (SUM ? nst[16 * cb + lr] : g2L * nst[16 * cb + lr]) + cs;
        }
      }
      // S[:, blocks] <- g^Lt S + K^T diag(wS) K[:, blocks]; the K^T fragments are shared
      {
        F bk[SB][NKS];
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
            const F ak = FR::tr(Kx, L::LDD, kk * KS, 16 * t, lane);
#pragma unroll
            for (int b = 0; b < SB; ++b) acc[b] = MMT::mma(ak, bk[b][kk], acc[b]);
          }
#pragma unroll
          for (int b = 0; b < SB; ++b)
            if (SFULL || rw + NOWN * b < DT) St[b][t] = acc[b];
        }
      }
    };
    uint4 xq[NXS];
    // output kernel: the S waves (P, the B scores both roles wait for) issue
    // first when both roles are ready (measured at B1 H32 T65536 d64: outputs
    // 0.298 -> 0.293 ms; the summary kernel gains nothing either way)
    if constexpr (!SUM) __builtin_amdgcn_s_setprio(2);
    if constexpr (L::PIPE) {
      finish_init();
      prologue();
      // the S waves carry Q and K two tiles ahead (summary) or one (output);
      // in the summary kernel the loads of a tile are issued in two halves,
      // the second one inside the next main phase, so that the vector memory
      // queue drains meanwhile (the output kernel is slower that way: measured)
      constexpr int AHEAD = SUM ? 2 : 1;
      using H0 = std::integral_constant<int, 0>;
      using H1 = std::integral_constant<int, SUM ? NXS / 2 : NXS>;
      using H2 = std::integral_constant<int, NXS>;
      if (AHEAD < ntiles) load_slots(xq, AHEAD, tid, QK{}, VB{}, HALF{}, H0{}, H1{});
      // summary: A' tiles of the next tile, shared with the M waves
      constexpr int NAS = SUM ? (NTRI + NW - 1) / NW : 1;
      for (int ti = 0; ti < ntiles; ++ti) {
        const int t0 = ti * TT;
        const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;
        s_step2(ti, gpow(g, lgg, Lt), gpow(g, lgg, 2 * Lt), Qb(ti & 1), Kb(ti & 1), [&]() {
          if (ti + AHEAD < ntiles) load_slots(xq, ti + AHEAD, tid, QK{}, VB{}, HALF{}, H1{}, H2{});
        });
        // summary: A' of the next tile (staged a tile ago), kept in registers
        // until every S wave of this tile has read AB
        f32x4 an[NAS];
        if constexpr (SUM) {
          if (ti + 1 < ntiles) {
#pragma unroll
            for (int sl = 0; sl < NAS; ++sl)
              if (wave + NW * sl < NTRI) an[sl] = a_tile(wave + NW * sl, (ti + 1) & 1);
          }
        }
        __syncthreads();
        // stage Q, K of tile ti + AHEAD (their buffers were last read in this step 2
        // or, in the output kernel, by the B scores of tile ti - 1)
        if (ti + AHEAD < ntiles)
          store_part(xq, tid, Qb((ti + AHEAD) & 1), Kb((ti + AHEAD) & 1), nullptr, QK{}, VB{}, HALF{});
        if constexpr (SUM) {
          if (ti + 1 < ntiles) {
#pragma unroll
            for (int sl = 0; sl < NAS; ++sl)
              if (wave + NW * sl < NTRI) a_store(wave + NW * sl, an[sl]);
          }
        }
        if (ti + 1 < ntiles) weights(ti + 1);
        __syncthreads();
        if constexpr (!SUM) score_phase(ti);
        if (ti + AHEAD + 1 < ntiles) load_slots(xq, ti + AHEAD + 1, tid, QK{}, VB{}, HALF{}, H0{}, H1{});
        if constexpr (!SUM) __syncthreads();
      }
    } else {
      load_role(xq, 0, std::true_type{});
      finish_init();

      for (int ti = 0; ti < ntiles; ++ti) {
        const int t0 = ti * TT;
        const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;
        const float gL = gpow(g, lgg, Lt), g2L = gpow(g, lgg, 2 * Lt);
        tile_head(ti, Lt, xq, std::true_type{});
        s_step2(ti, gL, g2L, Qs, Ks, []() {});
        __syncthreads();

        // ---- step 3 (output kernel): B^T scores, shared with the M waves ----
        if (!SUM) {
          b_scores(ti);
          __syncthreads();
          if constexpr (!DEFER) __syncthreads();   // step 4: the M waves write the outputs
        }
      }
    }
    if (SUM) {
      __syncthreads();   // the M waves' last M update has read P^T and V
      // S to LDS (fp32, the tile region is free now) as the A operand of S C
      float* oS = a.S + sidx * D * D;
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int cb = rw + NOWN * b;
        if (SFULL || cb < DT) {
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 16 * t + 4 * lg4 + j;
              FS[r * L::LFS + 16 * cb + lr] = St[b][t][j];
              oS[(size_t)r * D + 16 * cb + lr] = St[b][t][j];
            }
        }
      }
      __syncthreads();
      write_mh();
    }
  } else {
    // ======== M waves: O = g^(2(tau+1)) Q M_prev + B V and the M update
    //          (output kernel); C and M updates, G = S C - M (summary) ========
    f32x4 St[MB][DT];
    f32x4 Ct[SUM ? MB : 1][SUM ? DT : 1];
    if (SUM) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int t = 0; t < DT; ++t) { St[b][t] = zero4(); Ct[b][t] = zero4(); }
    } else {
      // M = S_P C_P - G_P: S_P from LDS is the A operand, the block of C_P the B operand
      const float* pG = a.G + sidx * D * E;
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int cb = rw + NOWN * b;
#pragma unroll
        for (int t = 0; t < DT; ++t) St[b][t] = zero4();
        if (MFULL || cb < ET) {
          f32x4 cp[DT];
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            if constexpr (EARLY) {
              cp[t] = cpx[b][t];
            } else {
              const float* pC = a.C + sidx * D * E;
#pragma unroll
              for (int j = 0; j < 4; ++j) cp[t][j] = pC[(size_t)(16 * t + 4 * lg4 + j) * E + 16 * cb + lr];
            }
          }
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < D / 4; ++kk)
              acc = MM<float>::mma(FS[(16 * t + lr) * L::LFS + 16 * (kk >> 2) + 4 * lg4 + (kk & 3)],
                                   Frag<float>::acc_b(cp, kk), acc);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] -= pG[(size_t)(16 * t + 4 * lg4 + j) * E + 16 * cb + lr];
            St[b][t] = acc;
          }
        }
      }
    }
    uint4 xv[NXM];

    // M[:, blocks] <- g^2L M + P^T diag(wM) V[:, blocks] for tile tp (its P^T, V
    // and wM are in the buffers of tp's parity); the P^T fragments are shared.
    // Summary kernel: M + P^T diag(wM) V, wM the weights to the segment end
    auto m_update = [&](int tp, float g2Lp) {
      const T* PsT = PsTb(tp & 1);
      const T* Vs = Vsb(tp & 1);
      const float* wM = wMb(tp & 1);
      F bv[MB][NKS];
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk)
          bv[b][kk] = FR::scale(FR::tr(Vs, L::LDV, kk * KS, 16 * ((rw + NOWN * b) % ET), lane), wM, kk * KS, lane);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 acc[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[b] = SUM ? St[b][t] : St[b][t] * g2Lp;
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const F ap = MMT::ld(PsT, L::LDT, 16 * t, kk * KS, lane);
#pragma unroll
          for (int b = 0; b < MB; ++b) acc[b] = MMT::mma(ap, bv[b][kk], acc[b]);
        }
#pragma unroll
        for (int b = 0; b < MB; ++b)
          if (MFULL || rw + NOWN * b < ET) St[b][t] = acc[b];
      }
    };

    // output kernel: oacc holds g^(2(tau+1)) (Q M_prev)^T of a tile until its B V
    // is added one tile later (B scores in BB, V and q.n in the tile's parity
    // buffers); then the tile is normalised and written with its denominator.
    // The outputs are accumulated transposed (O^T: the state or V^T is the A
    // operand), so that a lane holds four adjacent output columns of one token
    // and writes them with one 16-byte store.
    f32x4 oacc[SUM ? 1 : MB][TR];
    auto finish_out = [&](int tp, int Ltp) {
      const T* Vs = Vsb(tp & 1);
      const float* qnp = qnb(tp & 1);
      // the tile's Ltp output rows as a raw buffer: rows past them are dropped
      const auto ro = buf_rsrc(a.o + (tok0 + (size_t)tp * TT) * E, Ltp * E * (int)sizeof(float));
      F vf[MB][NKS];
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) vf[b][kk] = FR::tr(Vs, L::LDV, kk * KS, 16 * ((rw + NOWN * b) % ET), lane);
#pragma unroll
      for (int r = 0; r < TR; ++r)
#pragma unroll
        for (int k0 = 0; k0 < 16 * r + 16; k0 += KS) {
          const F bb = MMT::ld(BB, L::LDT, 16 * r, k0, lane);
#pragma unroll
          for (int b = 0; b < MB; ++b)
            if (MFULL || rw + NOWN * b < ET) oacc[b][r] = MMT::mma(vf[b][k0 / KS], bb, oacc[b][r]);
        }
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const int tau = 16 * r + lr;
        if (a.normalize) {
          float dn = 0.f;
          for (int c = 0; c <= r; ++c) dn += bpart[c * TT + tau];
          const float scale = 1.f / (dn + w2[tau] * qnp[tau] + a.eps);
#pragma unroll
          for (int b = 0; b < MB; ++b) oacc[b][r] *= scale;
        }
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const int cb = rw + NOWN * b;
          if (MFULL || cb < ET)
            buf_store16(ro, (tau * E + 16 * cb + 4 * lg4) * (int)sizeof(float), oacc[b][r]);
        }
      }
      const int mt = tid - HT;
      if (a.den != nullptr && mt < Ltp) {
        float dn = 0.f;
        for (int c = 0; c <= mt / 16; ++c) dn += bpart[c * TT + mt];
        a.den[tok0 + (size_t)tp * TT + mt] = dn + w2[mt] * qnp[mt];
      }
    };

    // (Q M_prev)^T of the tile in Qx, scaled by g^(2(tau+1)), into oacc (output kernel)
    auto qm = [&](const T* Qx) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int r = 0; r < TR; ++r) oacc[b][r] = zero4();
#pragma unroll
      for (int kk = 0; kk < QSK; ++kk) {
        F bm[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) bm[b] = state_b(St[b], kk);
#pragma unroll
        for (int r = 0; r < TR; ++r) {
          const F aq = state_a(Qx, 16 * r, kk);
#pragma unroll
          for (int b = 0; b < MB; ++b) oacc[b][r] = MMT::mma(bm[b], aq, oacc[b][r]);
        }
      }
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const float w2t = w2[16 * r + lr];
#pragma unroll
        for (int b = 0; b < MB; ++b) oacc[b][r] *= w2t;
      }
    };
    // C[:, blocks] <- C + Q^T diag(wC) V[:, blocks] (summary; wC: the weights to
    // the segment end); the Q^T fragments are shared
    auto c_update = [&](const T* Qx, const T* Vs) {
      F bv[MB][NKS];
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk)
          bv[b][kk] = FR::scale(FR::tr(Vs, L::LDV, kk * KS, 16 * ((rw + NOWN * b) % ET), lane), wC, kk * KS, lane);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 acc[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[b] = Ct[b][t];
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const F aq = FR::tr(Qx, L::LDD, kk * KS, 16 * t, lane);
#pragma unroll
          for (int b = 0; b < MB; ++b) acc[b] = MMT::mma(aq, bv[b][kk], acc[b]);
        }
#pragma unroll
        for (int b = 0; b < MB; ++b)
          if (MFULL || rw + NOWN * b < ET) Ct[b][t] = acc[b];
      }
    };
    // m <- m + Q^T wC (summary) on MFMA: the B operand is wC in column 0
    // and zeros elsewhere, so column 0 of the product (lanes lr == 0) is m for
    // the rows 16 t + [0, 16) of this wave's blocks t = rw + NOWN s
    constexpr int MS = (DT + NOWN - 1) / NOWN;
    f32x4 macc[SUM ? MS : 1];
#pragma unroll
    for (int sm = 0; sm < (SUM ? MS : 1); ++sm) macc[sm] = zero4();
    auto m_mma = [&](const T* Qx) {
      // every lane reads its weights (32-byte aligned runs of wC) and keeps them
      // only in column 0, so that no read waits behind a branch of its own
      F wc[NKS];
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        if constexpr (sizeof(T) == 2) {
          const f32x4* w8 = reinterpret_cast<const f32x4*>(wC + kk * KS + 8 * lg4);
          const f32x4 lo = w8[0], hi = w8[1];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            wc[kk][i] = (T)(lr == 0 ? lo[i] : 0.f);
            wc[kk][4 + i] = (T)(lr == 0 ? hi[i] : 0.f);
          }
        } else {
          const float w = wC[kk * KS + lg4];
          wc[kk] = lr == 0 ? w : 0.f;
        }
      }
#pragma unroll
      for (int sm = 0; sm < MS; ++sm) {
        const int t = rw + NOWN * sm;
        if (t < DT) {
          f32x4 acc = macc[sm];
#pragma unroll
          for (int kk = 0; kk < NKS; ++kk) acc = MMT::mma(FR::tr(Qx, L::LDD, kk * KS, 16 * t, lane), wc[kk], acc);
          macc[sm] = acc;
        }
      }
    };

    float g2L_prev = 1.f;
    if constexpr (L::PIPE) {
      finish_init();
      prologue();
      // V one tile ahead, its loads issued in two halves like Q and K (summary)
      using H0 = std::integral_constant<int, 0>;
      using H1 = std::integral_constant<int, SUM ? NXM / 2 : NXM>;
      using H2 = std::integral_constant<int, NXM>;
      if (1 < ntiles) load_slots(xv, 1, tid - HT, VB{}, END{}, HALF{}, H0{}, H1{});
      constexpr int NAS = SUM ? (NTRI + NW - 1) / NW : 1;
      for (int ti = 0; ti < ntiles; ++ti) {
        const int t0 = ti * TT;
        const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;
        const float g2L = gpow(g, lgg, 2 * Lt);
        // summary: the previous tile's M update, the C and m updates of this
        // tile and A' tiles of the next one; output: the previous tile's
        // outputs, the M update, then (Q M)^T of this tile
        f32x4 an[NAS];
        if constexpr (SUM) {
          if (ti > 0) m_update(ti - 1, g2L_prev);
          if (ti + 1 < ntiles) load_slots(xv, ti + 1, tid - HT, VB{}, END{}, HALF{}, H1{}, H2{});
          __builtin_amdgcn_sched_barrier(0);
          c_update(Qb(ti & 1), Vsb(ti & 1));
          m_mma(Qb(ti & 1));
          if (ti + 1 < ntiles) {
#pragma unroll
            for (int sl = 0; sl < NAS; ++sl)
              if (wave + NW * sl < NTRI) an[sl] = a_tile(wave + NW * sl, (ti + 1) & 1);
          }
        } else {
          if (ti > 0) finish_out(ti - 1, TT);   // only the last tile can be short
          if (ti + 1 < ntiles) load_slots(xv, ti + 1, tid - HT, VB{}, END{}, HALF{}, H1{}, H2{});
          __builtin_amdgcn_sched_barrier(0);
          if (ti > 0) m_update(ti - 1, g2L_prev);
          __builtin_amdgcn_sched_barrier(0);
          qm(Qb(ti & 1));
        }
        g2L_prev = g2L;
        __syncthreads();
        // V of tile ti + 1 to the buffer last read by this step's updates of tile ti - 1
        if (ti + 1 < ntiles) {
          store_part(xv, tid - HT, nullptr, nullptr, Vsb((ti + 1) & 1), VB{}, END{}, HALF{});
          if constexpr (SUM) {
#pragma unroll
            for (int sl = 0; sl < NAS; ++sl)
              if (wave + NW * sl < NTRI) a_store(wave + NW * sl, an[sl]);
          }
        }
        __syncthreads();
        if constexpr (!SUM) score_phase(ti);
        if (ti + 2 < ntiles) load_slots(xv, ti + 2, tid - HT, VB{}, END{}, HALF{}, H0{}, H1{});
        if constexpr (!SUM) __syncthreads();
      }
      if constexpr (!SUM) finish_out(ntiles - 1, (Lspan - (ntiles - 1) * TT));
    } else {
      load_role(xv, 0, std::false_type{});
      finish_init();
      for (int ti = 0; ti < ntiles; ++ti) {
        const int t0 = ti * TT;
        const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;
        const float g2L = gpow(g, lgg, 2 * Lt);
        tile_head(ti, Lt, xv, std::false_type{});

        // ---- step 2: the previous tile's outputs (output kernel) and M update,
        //      then Q M (output) or the C update (summary) ----
        if constexpr (DEFER) {
          if (ti > 0) finish_out(ti - 1, TT);   // only the last tile can be short
          __builtin_amdgcn_sched_barrier(0);
        }
        if (ti > 0) m_update(ti - 1, g2L_prev);
        __builtin_amdgcn_sched_barrier(0);   // keep the two updates' operand loads apart
        if constexpr (!SUM) qm(Qs);
        else c_update(Qs, Vsb(ti & 1));
        if constexpr (SUM) m_mma(Qs);
        g2L_prev = g2L;
        __syncthreads();

        // ---- step 3: B scores (with the S waves); step 4 without DEFER ----
        if constexpr (!SUM) {
          if constexpr (DEFER) b_scores(ti);
          __syncthreads();
        }
        if constexpr (!SUM && !DEFER) {
          finish_out(ti, Lt);
          __syncthreads();
        }
      }
      if constexpr (DEFER) finish_out(ntiles - 1, (Lspan - (ntiles - 1) * TT));
    }
    if (SUM) {
      m_update(ntiles - 1, g2L_prev);
      if (lr == 0) {
#pragma unroll
        for (int sm = 0; sm < MS; ++sm) {
          const int t = rw + NOWN * sm;
          if (t < DT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) mst[16 * t + 4 * lg4 + j] = macc[sm][j];
          }
        }
      }
      __syncthreads();
    }
    if (SUM) {
      // G = S C - M with S from LDS (written by the S waves) as the A operand
      float* oC = a.C + sidx * D * E;
      float* oG = a.G + sidx * D * E;
      __syncthreads();
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int cb = rw + NOWN * b;
        if (MFULL || cb < ET) {
          // G = S C - M accumulated onto -M, the row blocks interleaved
#pragma unroll
          for (int t = 0; t < DT; ++t) St[b][t] = -St[b][t];
#pragma unroll
          for (int kk = 0; kk < D / 4; ++kk) {
            const float bk = Frag<float>::acc_b(Ct[b], kk);
#pragma unroll
            for (int t = 0; t < DT; ++t)
              St[b][t] = MM<float>::mma(FS[(16 * t + lr) * L::LFS + 16 * (kk >> 2) + 4 * lg4 + (kk & 3)],
                                        bk, St[b][t]);
          }
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const size_t e = (size_t)(16 * t + 4 * lg4 + j) * E + 16 * cb + lr;
              oC[e] = Ct[b][t][j];
              oG[e] = St[b][t][j];
            }
          // one column block at a time: keeps the S loads of the next block from
          // being hoisted (and spilled) while C and M are both live
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      write_mh();
    }
  }
}

// ---- dispatch ------------------------------------------------------------------

template <int D, int E>
struct Waves {
  // two roles (S waves, M waves) of 4 waves when a head dimension is 128, else of 2
  static constexpr int value = (D == 128 || E == 128) ? 8 : 4;
};

// bf16 kernels with a head dimension of 64 (and none of 128) also come with 8
// waves: a grid of at most one workgroup per CU (256) leaves the second
// 4-wave workgroup of a CU unused, and 8 waves hide more latency (measured:
// 16 spans of 256 tokens per head, B2 H8 d64: summaries 23 -> 20 us, outputs
// 36 -> 27 us; with two workgroups per CU the 4-wave kernels stay faster)
template <int D, int E>
struct Wide8 {
  static constexpr bool value = (D == 64 || E == 64) && D <= 64 && E <= 64 && D >= 32 && E >= 32;
};

template <int MODE>
static hipError_t launch_mode(int dtype, int d, int dv, int units, const ChunkArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)units * (unsigned)a.nspan);
  const bool one_per_cu = (long long)units * a.nspan <= 256;
#define HLA_CASE(T, D, E)                                                                    \
  if (d == D && dv == E) {                                                                   \
    constexpr int NW = Waves<D, E>::value;                                                   \
    if constexpr (sizeof(T) == 2 && Wide8<D, E>::value) {                                    \
      if (one_per_cu) {                                                                      \
        hipLaunchKernelGGL((chunk_kernel<T, D, E, MODE, 8>), grid, dim3(512), 0, s, a);      \
        return hipGetLastError();                                                            \
      }                                                                                      \
    }                                                                                        \
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
