// Segment outputs of the masked second-order HLA forward from the
// segment-local p ("Higher-order Linear Attention", arXiv 2510.27258,
// summaries on gist.science: method section 1 for the output, section 4 for
// the chunk-parallel scheme, key contribution 2 for decay).
//
// Inside a segment that starts from the exclusive prefix (S_P, M_P, n_P), the
// state at position j (0-based in the segment) is
//     S_j = g^(j+1) S_P + S^loc_j,
// S^loc being the same recurrence from zero at the segment start, so
//     p_j = S_j q_j = g^(j+1) S_P q_j + p^loc_j.
// The summary kernel already forms p^loc for every token (it walks the
// segment's S recurrence) and writes it out (bf16, per 64-token tile its 16x16
// fragments in the MFMA accumulator's lane order, which is the order the P
// waves here hold P in).  This kernel therefore carries no S recurrence:
// per tile (tau, j = positions inside the tile, t0 = the tile's first position)
//     P        = g^(t0+tau+1) Q S_P + P^loc
//     B[tau,j] = g^(2(tau-j)) q_tau.p_j          (j <= tau)
//     num_tau  = sum_{j<=tau} B[tau,j] v_j + g^(2(tau+1)) q_tau^T M_prev
//     den_tau  = sum_{j<=tau} B[tau,j]     + g^(2(tau+1)) q_tau.n_prev
//     M <- g^(2Lt) M + P^T diag(wM) V,  n likewise with v = 1.
// With S no longer updated, S_P is a constant operand (bf16 fragments held
// in registers).  Sixteen waves (four per SIMD, at most 128 registers each):
// P waves 0..7 own column block w of P (16 columns of S_P), M waves 8..15
// column block w - 8 of M and the outputs.  Two barriers per tile:
//   [q.n; P waves: P (P^loc prefetched into registers a tile ahead), P^T to
//    LDS and its column sums for n | M waves: (Q M)^T]  ->  barrier  ->
//   [P waves: B^T score tiles, n update; the next tile staged from
//    registers and the one after it loaded]  ->  barrier  ->
//   [M waves: B V, normalisation, output stores; M update].
// bf16 inputs with d = dv = 128; every product on MFMA with fp32
// accumulation; segment-boundary products (S_P C_P, S_P m_P) on fp32 MFMA.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

namespace {

constexpr int PT_TT = 64;   // tokens per tile

struct OutPLayout {
  static constexpr int D = 128, E = 128, TT = PT_TT;
  static constexpr int LDD = D + 16;   // Q rows (row-major fragment reads conflict-free)
  static constexpr int LDV = E + 8;    // V rows
  static constexpr int LDT = TT + 8;   // P^T rows, B score rows
  static constexpr size_t QB = (size_t)TT * LDD * 2, VB = (size_t)TT * LDV * 2, PB = (size_t)D * LDT * 2;
  static constexpr size_t Q0 = 0, V0 = 2 * QB, P0 = V0 + 2 * VB, BBo = P0 + 2 * PB;
  static constexpr size_t TILE_END = BBo + (size_t)TT * LDT * 2;
  static constexpr int LFS = D + 4;    // fp32 S_P overlay at the segment start
  static_assert((size_t)D * LFS * 4 <= TILE_END, "S_P overlay");
  static constexpr size_t W = (TILE_END + 15) / 16 * 16;
  // w1, w2, wM[2], pw, pw2, qn[2] [TT]; bpart [TR][TT]; nst [D]
  static constexpr size_t TOTAL = W + (size_t)(8 * TT + (TT / 16) * TT + D) * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
};

__device__ __forceinline__ void st_bf16x4(__bf16* p, f32x4 x) {
  bf16x4 y;
  y[0] = (__bf16)x[0]; y[1] = (__bf16)x[1]; y[2] = (__bf16)x[2]; y[3] = (__bf16)x[3];
  *reinterpret_cast<bf16x4*>(p) = y;
}

__global__ __launch_bounds__(1024, 1) void outp_kernel(ChunkArgs a) {
  using L = OutPLayout;
  using T = __bf16;
  using MMT = MM<T>;
  using FR = Frag<T>;
  using F = MMT::F;
  constexpr int D = L::D, E = L::E, TT = L::TT, NT = 1024, KS = 32, CH = 8;
  constexpr int DT = D / 16, TR = TT / 16, NKS = TT / KS, QK = D / KS;
  constexpr int NTRI = TR * (TR + 1) / 2;
  constexpr int QCH = TT * D / CH, VCH = TT * E / CH;   // 16-byte chunks per tile
  constexpr int NXQ = QCH / NT, NXV = VCH / NT;
  static_assert(QCH % NT == 0 && VCH % NT == 0, "chunks per thread");

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  auto Qb = [&](int p) { return reinterpret_cast<T*>(smem + L::Q0 + (p ? L::QB : 0)); };
  auto Vb = [&](int p) { return reinterpret_cast<T*>(smem + L::V0 + (p ? L::VB : 0)); };
  auto Pb = [&](int p) { return reinterpret_cast<T*>(smem + L::P0 + (p ? L::PB : 0)); };
  T* BB = reinterpret_cast<T*>(smem + L::BBo);
  float* FS = reinterpret_cast<float*>(smem);
  float* w1 = reinterpret_cast<float*>(smem + L::W);
  float* w2 = w1 + TT;
  auto wMb = [&](int p) { return w2 + TT + p * TT; };
  float* pw = w2 + 3 * TT;
  float* pw2 = pw + TT;
  auto qnb = [&](int p) { return pw2 + TT + p * TT; };
  float* bpart = pw2 + 3 * TT;   // [TR][TT]
  float* nst = bpart + TR * TT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg4 = lane >> 4;
  const int nspan = a.nspan;
  const int unit = blockIdx.x / nspan, span = blockIdx.x - unit * nspan;
  const int head = unit % a.H;
  const float g = a.gamma ? a.gamma[head] : 1.f;
  const float lgg = log2f(g);
  const int Lspan = a.chunk;
  const int ntiles = (Lspan + TT - 1) / TT;
  const size_t tok0 = (size_t)unit * (size_t)a.T + (size_t)span * (size_t)Lspan;
  const size_t sidx = (size_t)unit * nspan + span;
  const bool need_n = a.normalize || a.den != nullptr;
  const T* gq = reinterpret_cast<const T*>(a.q) + tok0 * D;
  const T* gv = reinterpret_cast<const T*>(a.v) + tok0 * E;
  const T* gp = reinterpret_cast<const T*>(a.pl) + sidx * (size_t)ntiles * (size_t)(D * TT);
  // the segment's rows as raw buffers: rows past the end read as zeros
  const auto rq = buf_rsrc(gq, Lspan * D * 2);
  const auto rv = buf_rsrc(gv, Lspan * E * 2);
  const bool pRole = wave < 8;
  const int cb = pRole ? wave : wave - 8;   // this wave's column block of P or of M

  // ---- segment start: S_P to LDS (fp32), tables ----
  {
    const f32x4* pS = reinterpret_cast<const f32x4*>(a.S + sidx * D * D);
    for (int i = tid; i < D * D / 4; i += NT) {
      const int r = (4 * i) / D, c = (4 * i) % D;
      *reinterpret_cast<f32x4*>(FS + r * L::LFS + c) = pS[i];
    }
  }
  const int Llast = Lspan - (ntiles - 1) * TT;
  if (tid < TT) {
    pw[tid] = gpow(g, lgg, tid);
    pw2[tid] = gpow(g, lgg, 2 * tid);
    w1[tid] = gpow(g, lgg, tid + 1);
    w2[tid] = gpow(g, lgg, 2 * tid + 2);
    // M weights g^(2(Lt-1-j)) of a full tile in both parities; a short last
    // tile's are written before its first use
    const float wf = gpow(g, lgg, 2 * (TT - 1 - tid));
    wMb(0)[tid] = wf;
    wMb(1)[tid] = wf;
    if (ntiles == 1) wMb(0)[tid] = tid < Llast ? gpow(g, lgg, 2 * (Llast - 1 - tid)) : 0.f;
  }
  __syncthreads();

  // ---- tile staging through registers: Q and V rows of a tile ----
  uint4 xq[NXQ], xv[NXV];
  auto load_tile = [&](int ti) {
    const int t0 = ti * TT;
#pragma unroll
    for (int i = 0; i < NXQ; ++i) xq[i] = buf_load16(rq, (t0 * D + (tid + NT * i) * CH) * 2);
#pragma unroll
    for (int i = 0; i < NXV; ++i) xv[i] = buf_load16(rv, (t0 * E + (tid + NT * i) * CH) * 2);
  };
  auto store_tile = [&](int p) {
#pragma unroll
    for (int i = 0; i < NXQ; ++i) {
      const int c = tid + NT * i, row = c / (D / CH), col = (c % (D / CH)) * CH;
      *reinterpret_cast<uint4*>(Qb(p) + row * L::LDD + col) = xq[i];
    }
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int c = tid + NT * i, row = c / (E / CH), col = (c % (E / CH)) * CH;
      *reinterpret_cast<uint4*>(Vb(p) + row * L::LDV + col) = xv[i];
    }
  };
  // q.n of the tile in buffers p (n as it stands), for its denominator
  auto q_dot_n = [&](int p) {
    constexpr int LPR = NT / TT;
    const T* Qx = Qb(p);
    const int tau = tid / LPR, part = tid % LPR;
    float acc = 0.f;
#pragma unroll
    for (int c = part * (D / LPR); c < (part + 1) * (D / LPR); ++c) acc += (float)Qx[tau * L::LDD + c] * nst[c];
#pragma unroll
    for (int off = 1; off < LPR; off *= 2) acc += __shfl_xor(acc, off, 64);
    if (part == 0) qnb(p)[tau] = acc;
  };
  // B^T score tile idx of the tile in buffers p, to BB (and its column sums to bpart)
  auto b_tile = [&](int idx, int p) {
    int r, c;
    tri_block(idx, r, c);
    const T* PsT = Pb(p);
    const T* Qx = Qb(p);
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += KS)
      acc = MMT::mma(FR::tr(PsT, L::LDT, k0, 16 * c, lane), MMT::ld(Qx, L::LDD, 16 * r, k0, lane), acc);
    const int tau = 16 * r + lr;
    f32x4 val;
#pragma unroll
    for (int j = 0; j < 4; ++j) val[j] = acc[j] * masked_pow(pw2, tau, 16 * c + 4 * lg4 + j);
    st_bf16x4(BB + tau * L::LDT + 16 * c + 4 * lg4, val);
    if (need_n) {
      const float rs = sum_rows4(val[0] + val[1] + val[2] + val[3]);
      if (lg4 == 0) bpart[c * TT + tau] = rs;
    }
  };

  // n = S_P m_P - h_P; then the B score buffer's upper blocks (read as zeros,
  // never written) and tile 0 (over the S_P overlay, once every wave has read
  // its part of S_P)
  auto prologue_tail = [&]() {
    if (need_n) {
      const float* pm = a.m + sidx * D;
      const float* ph = a.h + sidx * D;
      for (int r = tid; r < D; r += NT) {
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc += FS[r * L::LFS + c] * pm[c];
        nst[r] = acc - ph[r];
      }
    }
    __syncthreads();
    for (size_t i = L::BBo / 16 + tid; i < L::TILE_END / 16; i += NT)
      reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
    load_tile(0);
    store_tile(0);
    if (ntiles > 1) load_tile(1);
    __syncthreads();
  };
  // every thread, between the two barriers of tile ti: the next tile staged
  // from registers and the one after it loaded; a short last tile's M weights
  auto stage_next = [&](int ti, int p) {
    if (ti + 1 < ntiles) {
      store_tile(p ^ 1);
      if (ti + 2 < ntiles) load_tile(ti + 2);
      if (ti + 2 == ntiles && Llast < TT && tid < TT)
        wMb(p ^ 1)[tid] = tid < Llast ? gpow(g, lgg, 2 * (Llast - 1 - tid)) : 0.f;
    }
  };

  // The two roles run tile loops of their own with the same barriers, so
  // that each role's registers are allocated apart.
  if (pRole) {
    // ======== P waves: P = g^(t0+tau+1) Q S_P + P^loc, its column sums for
    //          n; the B^T score tiles ========
    // S_P's column block as bf16 B fragments (natural K order: lane group g
    // holds K rows 32 kk + 8 g + [0, 8))
    F spf[QK];
#pragma unroll
    for (int kk = 0; kk < QK; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) spf[kk][i] = (T)FS[(32 * kk + 8 * lg4 + i) * L::LFS + 16 * cb + lr];
    // this wave's fragments of P^loc (row blocks r of column block cb, 512
    // contiguous bytes each, lane order), a tile ahead
    bf16x4 xpl[TR];
    auto load_pl = [&](int ti) {
      const T* src = gp + (size_t)ti * (D * TT) + (size_t)cb * (TR * 256) + lane * 4;
#pragma unroll
      for (int r = 0; r < TR; ++r) xpl[r] = *reinterpret_cast<const bf16x4*>(src + r * 256);
    };
    load_pl(0);
    prologue_tail();
    for (int ti = 0; ti < ntiles; ++ti) {
      const int p = ti & 1;
      const int t0 = ti * TT;
      const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;
      const float g2L = gpow(g, lgg, 2 * Lt);
      const float gt0 = gpow(g, lgg, t0);
      T* PsT = Pb(p);
      const T* Qx = Qb(p);
      if (need_n) q_dot_n(p);
      f32x4 pacc[TR];
#pragma unroll
      for (int r = 0; r < TR; ++r) pacc[r] = zero4();
#pragma unroll
      for (int kk = 0; kk < QK; ++kk)
#pragma unroll
        for (int r = 0; r < TR; ++r) pacc[r] = MMT::mma(MMT::ld(Qx, L::LDD, 16 * r, 32 * kk, lane), spf[kk], pacc[r]);
      float ncol = 0.f;
      const float* wm = wMb(p);
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        // P^T[d][tau], d = 16 cb + lr, tau = 16 r + 4 lg4 + j
        T* pp = PsT + (16 * cb + lr) * L::LDT + 16 * r + 4 * lg4;
        const f32x4 w1v = *reinterpret_cast<const f32x4*>(w1 + 16 * r + 4 * lg4);
        const f32x4 wmv = *reinterpret_cast<const f32x4*>(wm + 16 * r + 4 * lg4);
        f32x4 pv;
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[j] = pacc[r][j] * (gt0 * w1v[j]) + (float)xpl[r][j];
        st_bf16x4(pp, pv);
        ncol += pv[0] * wmv[0] + pv[1] * wmv[1] + pv[2] * wmv[2] + pv[3] * wmv[3];
      }
      const float ncs = need_n ? sum_rows4(ncol) : 0.f;
      if (ti + 1 < ntiles) load_pl(ti + 1);
      __syncthreads();
      for (int idx = cb; idx < NTRI; idx += 8) b_tile(idx, p);
      stage_next(ti, p);
      // n <- g^2Lt n + P^T wM: one writer per column; q.n of this tile is taken
      if (need_n && lg4 == 0) nst[16 * cb + lr] = g2L * nst[16 * cb + lr] + ncs;
      __syncthreads();
    }
  } else {
    // ======== M waves: (Q M)^T, B V and the outputs; the M update ========
    // M's column block: M = S_P C_P - G_P (fp32 MFMA, S_P from LDS as the A operand)
    f32x4 St[DT];
    {
      const float* pC = a.C + sidx * D * E;
      const float* pG = a.G + sidx * D * E;
      f32x4 cp[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) cp[t][j] = pC[(size_t)(16 * t + 4 * lg4 + j) * E + 16 * cb + lr];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < D / 4; ++kk)
          acc = MM<float>::mma(FS[(16 * t + lr) * L::LFS + 16 * (kk >> 2) + 4 * lg4 + (kk & 3)],
                               Frag<float>::acc_b(cp, kk), acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] -= pG[(size_t)(16 * t + 4 * lg4 + j) * E + 16 * cb + lr];
        St[t] = acc;
      }
    }
    prologue_tail();
    // the M waves' chain (B V, the outputs, the M update, Q M) bounds the
    // tile while the P waves wait at the barriers for it: they issue first
    // when both are ready (measured: outputs 0.281 -> 0.270 ms)
    __builtin_amdgcn_s_setprio(2);
    for (int ti = 0; ti < ntiles; ++ti) {
      const int p = ti & 1;
      const int t0 = ti * TT;
      const int Lt = (Lspan - t0) < TT ? (Lspan - t0) : TT;
      const float g2L = gpow(g, lgg, 2 * Lt);
      const T* PsT = Pb(p);
      const T* Qx = Qb(p);
      if (need_n) q_dot_n(p);
      // (Q M)^T of the tile, scaled by g^(2(tau+1))
      f32x4 oacc[TR];
#pragma unroll
      for (int r = 0; r < TR; ++r) oacc[r] = zero4();
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) {
        const F bm = FR::acc_b_nat(St, kk);
#pragma unroll
        for (int r = 0; r < TR; ++r) oacc[r] = MMT::mma(bm, MMT::ld(Qx, L::LDD, 16 * r, 32 * kk, lane), oacc[r]);
      }
#pragma unroll
      for (int r = 0; r < TR; ++r) oacc[r] *= w2[16 * r + lr];
      __syncthreads();
      stage_next(ti, p);
      __syncthreads();
      // B V and the outputs of tile ti
      const T* Vs = Vb(p);
      const float* qnp = qnb(p);
      F vf[NKS];
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) vf[kk] = FR::tr(Vs, L::LDV, kk * KS, 16 * cb, lane);
#pragma unroll
      for (int r = 0; r < TR; ++r)
#pragma unroll
        for (int k0 = 0; k0 < 16 * r + 16; k0 += KS)
          oacc[r] = MMT::mma(vf[k0 / KS], MMT::ld(BB, L::LDT, 16 * r, k0, lane), oacc[r]);
      // the tile's Lt output rows as a raw buffer: rows past them are dropped
      const auto ro = buf_rsrc(a.o + (tok0 + (size_t)t0) * E, Lt * E * (int)sizeof(float));
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const int tau = 16 * r + lr;
        if (a.normalize) {
          float dn = 0.f;
          for (int c = 0; c <= r; ++c) dn += bpart[c * TT + tau];
          oacc[r] *= 1.f / (dn + w2[tau] * qnp[tau] + a.eps);
        }
        buf_store16(ro, (tau * E + 16 * cb + 4 * lg4) * (int)sizeof(float), oacc[r]);
      }
      const int mt = tid - NT / 2;
      if (a.den != nullptr && mt < Lt) {
        float dn = 0.f;
        for (int c = 0; c <= mt / 16; ++c) dn += bpart[c * TT + mt];
        a.den[tok0 + (size_t)t0 + mt] = dn + w2[mt] * qnp[mt];
      }
      // M <- g^2Lt M + P^T diag(wM) V[:, block]
      const float* wM = wMb(p);
      F bv[NKS];
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) bv[kk] = FR::scale(FR::tr(Vs, L::LDV, kk * KS, 16 * cb, lane), wM, kk * KS, lane);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 acc = St[t] * g2L;
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) acc = MMT::mma(MMT::ld(PsT, L::LDT, 16 * t, kk * KS, lane), bv[kk], acc);
        St[t] = acc;
      }
    }
  }
}

}  // namespace

bool outp_supported(int dtype, int d, int dv) { return dtype == 1 && d == 128 && dv == 128; }

size_t outp_plocal_bytes(int64_t units, int64_t T, int chunk, int d) {
  const int64_t nspan = T / chunk, ntiles = (chunk + PT_TT - 1) / PT_TT;
  return (size_t)units * (size_t)nspan * (size_t)ntiles * (size_t)d * PT_TT * 2;
}

hipError_t launch_outputs_from_p(int units, const ChunkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(outp_kernel, dim3((unsigned)units * (unsigned)a.nspan), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace hla
