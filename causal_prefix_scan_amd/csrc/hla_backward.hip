// Backward pass of the masked second-order HLA forward on gfx950.
//
// The pages motivate the chunk-parallel form by training ("Higher-order
// Linear Attention", method section on parallel training by associative
// scans) but give no backward.  Writing the forward's closed form as two
// stacked first-order sums, p_t = S_t q_t = sum_{i<=t} g^(t-i) (q_t.k_i) k_i
// and o_t = sum_{j<=t} g^(2(t-j)) (q_t.p_j) v_j, the chain rule turns the
// gradient into seven first-order decayed sums (four of them over the future
// tokens):
//   p   = sum_{i<=t} g^(t-i)      (q_t.k_i)   k_i
//   dp  = sum_{t>=j} g^(2(t-j))   (v_j.dO_t)  q_t
//   dv  = sum_{t>=j} g^(2(t-j))   (p_j.q_t)   dO_t
//   dq  = sum_{j<=t} g^(2(t-j))   (dO_t.v_j)  p_j  +  sum_{i<=t} g^(t-i) (dp_t.k_i) k_i
//   dk  = sum_{t>=i} g^(t-i)      (k_i.q_t)   dp_t +  sum_{t>=i} g^(t-i) (k_i.dp_t) q_t
// Each is y_t = sum_{s<=t} lam^(t-s) (a_t.b_s) c_s in a walk order (forward,
// or reverse for the sums over the future), computed chunk-parallel like the
// forward: segment states H = sum_s lam^(L-1-s) b_s c_s^T, an exclusive
// decayed running sum over the segments, then per tile (64 tokens; 32 for fp32)
// Y = lam^(tau+1) A H_prev + ((A B^T) o decay) C and H <- lam^L H + B^T diag(w) C.
// Sums with the same states share them: S dp starts from the prefixes of p,
// dv from those of dp read transposed, and the two dk sums are one sum over
// the symmetric states lam^(..) (q dp^T + dp q^T).
// Precision follows the forward: with bf16 inputs every operand (q, k, v, the
// intermediates p and dp, which are stored as bf16, and the upstream
// gradient) is staged to LDS as bf16 and contracted with
// v_mfma_f32_16x16x32_bf16 into fp32 accumulators; with fp32 inputs
// everything stays fp32 (v_mfma_f32_16x16x4_f32).  States and the outputs
// dq, dk, dv are fp32 either way.

#include <type_traits>

#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

enum { L_SUMMARY = 0, L_OUTPUT = 1 };

// waves per workgroup: one per 16 columns of c, at least four
template <int Dc>
struct LWaves {
  static constexpr int value = Dc / 16 > 4 ? Dc / 16 : 4;
};

template <typename T, int Da, int Dc, bool SYM>
struct LLayout {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int LT = BF ? 64 : 32;           // tokens per tile
  static constexpr int DP = Da < MM<T>::KS ? MM<T>::KS : Da;   // zero-padded to one MFMA step
  static constexpr int LDA = DP + (BF ? 8 : 4);     // a, b rows: [tok][DP]
  static constexpr int LDC = Dc + (BF ? 8 : 16);    // c rows: [tok][Dc]
  static constexpr int LDS_ = LT + (BF ? 8 : 4);    // scores: [tau][s]
  static constexpr size_t As = 0;
  static constexpr size_t Bs = As + (size_t)LT * LDA * sizeof(T);
  static constexpr size_t Cs = Bs + (size_t)LT * LDA * sizeof(T);
  static constexpr size_t Ss = Cs + (size_t)LT * LDC * sizeof(T);
  static constexpr size_t Ss2 = Ss + (size_t)LT * LDS_ * sizeof(T);   // scores against c (SYM)
  static constexpr size_t W = (Ss2 + (SYM ? (size_t)LT * LDS_ * sizeof(T) : 0) + 15) / 16 * 16;
  // pw (lam^n), w1 (lam^(tau+1)), wS (lam^(L-1-tau)) [LT]
  static constexpr size_t TOTAL = W + 3 * LT * 4;
  static_assert(TOTAL <= 80 * 1024, "LDS budget of the first-order sum kernel (two per CU)");
  static_assert(!SYM || (Da == Dc && DP == Da), "mirrored pair: b and c rows share one layout");
};

template <typename T> struct Vec4;
template <> struct Vec4<float> { using V = f32x4; };
template <> struct Vec4<__bf16> { using V = bf16x4; };

// One operand's rows [t0, t0 + LT) of the walk, columns [0, W), held in
// registers as raw 4-element groups (8 bytes from a bf16 source, 16 from an
// fp32 one; the source type is fixed at compile time so that bf16 groups
// take two registers) between the global loads and the LDS stores, so that
// a whole tile's loads are in flight together and the next tile's overlap
// the current one's products.  Rows past `end` read as zero.
template <int W, int NTHR, int LT, bool F32>
struct TileRows {
  static constexpr int G = W / 4;                      // groups per row
  static constexpr int N = (LT * G + NTHR - 1) / NTHR; // groups per thread
  using R = typename std::conditional<F32, uint4, uint2>::type;
  R r[N];

  // A null operand is the unit channel: rows (1, 0, ..., 0), formed here
  // rather than read.
  __device__ __forceinline__ void load(const LaOperand& op, size_t urow, int nT, bool rev, int t0,
                                       int end, int tid) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    const E* base = reinterpret_cast<const E*>(op.p);
    if (!base) {
      R one{};
      one.x = F32 ? 0x3F800000u : 0x3F80u;   // 1.0 in the first element
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int idx = tid + NTHR * i, row = idx / G, l = t0 + row;
        r[i] = (idx < LT * G && l < end && idx % G == 0) ? one : R{};
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + NTHR * i, row = idx / G, col = (idx % G) * 4, l = t0 + row;
      r[i] = R{};
      if (idx < LT * G && l < end) {
        const size_t phys = (size_t)(rev ? nT - 1 - l : l);
        r[i] = *reinterpret_cast<const R*>(base + (urow + phys) * W + col);
      }
    }
  }

  // the held rows, rounded to bf16, to a dense [rows][W] copy (fp32 sources)
  __device__ __forceinline__ void write_bf16_copy(void* dst, size_t urow, int nT, bool rev, int t0,
                                                  int end, int tid) const {
    static_assert(F32, "only fp32 sources are copied");
    __bf16* base = reinterpret_cast<__bf16*>(dst);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + NTHR * i, row = idx / G, col = (idx % G) * 4, l = t0 + row;
      if (idx < LT * G && l < end) {
        const f32x4 f = __builtin_bit_cast(f32x4, r[i]);
        const size_t phys = (size_t)(rev ? nT - 1 - l : l);
        *reinterpret_cast<bf16x4*>(base + (urow + phys) * W + col) =
            bf16x4{(__bf16)f[0], (__bf16)f[1], (__bf16)f[2], (__bf16)f[3]};
      }
    }
  }

  template <typename T>
  __device__ __forceinline__ void store(T* dst, int ldd, int tid) const {
    using V = typename Vec4<T>::V;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + NTHR * i, row = idx / G, col = (idx % G) * 4;
      if (idx < LT * G) {
        V v;
        if constexpr (F32) {
          const f32x4 f = __builtin_bit_cast(f32x4, r[i]);
          v = V{(T)f[0], (T)f[1], (T)f[2], (T)f[3]};
        } else {
          const bf16x4 b = __builtin_bit_cast(bf16x4, r[i]);
          v = V{(T)b[0], (T)b[1], (T)b[2], (T)b[3]};
        }
        *reinterpret_cast<V*>(dst + row * ldd + col) = v;
      }
    }
  }
};

// One workgroup per (unit, segment); wave w owns columns 16 w .. +15 of c and
// of the state.  MODE L_SUMMARY writes the segment's state; L_OUTPUT starts
// from the exclusive prefix (or zero when there is none) and writes (or
// adds) y.  SYM adds the mirrored pair (b and c swapped) from the same staged
// tiles: a second score block against c weighting b, and C^T diag(w) B in
// the state update.
// SRCF marks the fp32 sources (bit 0: a, 1: b, 2: c; the others are bf16)
// and, with bit 3, that c is the same tensor as b.
// The bf16 kernels fit 128 VGPRs without spills, which lets two 8-wave
// workgroups share a CU.
template <typename T, int Da, int Dc, int MODE, int NW, bool SYM, int SRCF, bool ACC, bool CH>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 4 : 1))) void la_kernel(LaArgs a) {
  using L = LLayout<T, Da, Dc, SYM>;
  using MMT = MM<T>;
  using FR = Frag<T>;
  constexpr int NTHR = 64 * NW;
  constexpr int LT = L::LT;
  constexpr int KS = MMT::KS;
  constexpr int DT = Da / 16, TR = LT / 16;
  constexpr int QK = KS == 32 ? (DT + 1) / 2 : DT * 4;   // K steps over Da against the state
  constexpr bool OUT = MODE == L_OUTPUT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  T* As = reinterpret_cast<T*>(smem + L::As);
  T* Bs = reinterpret_cast<T*>(smem + L::Bs);
  // SRCF bit 3: c is the same tensor as b (Da == Dc), so its tile is b's
  constexpr bool CB = (SRCF & 8) != 0;
  static_assert(!CB || (Da == Dc && !SYM), "c = b needs equal widths");
  constexpr int LDC = CB ? L::LDA : L::LDC;
  T* Cs = CB ? Bs : reinterpret_cast<T*>(smem + L::Cs);
  T* Ss = reinterpret_cast<T*>(smem + L::Ss);
  T* Ss2 = reinterpret_cast<T*>(smem + L::Ss2);
  float* pw = reinterpret_cast<float*>(smem + L::W);
  float* w1 = pw + LT;
  float* wS = w1 + LT;
  // (CH) the scalar channel: its values in the tile, its state by tile parity
  __shared__ float c2s[CH ? LT : 1];
  __shared__ float h2s[2][CH ? Da : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int us = blockIdx.x;
  const int unit = us / a.nseg, seg = us - unit * a.nseg;
  float lam = a.gamma ? a.gamma[unit % a.H] : 1.f;
  lam = a.gexp == 3 ? lam * lam * lam : a.gexp == 2 ? lam * lam : lam;
  const float lgl = log2f(lam);
  const int nT = a.T;
  const bool rev = a.reverse != 0;
  const int s0 = seg * a.seg, s1 = s0 + a.seg < nT ? s0 + a.seg : nT;
  const size_t urow = (size_t)unit * (size_t)nT;
  const bool cols = wave * 16 < Dc;       // this wave owns columns 16 wave .. +15
  const int col = 16 * wave + lr;
  const size_t hbase = (size_t)us * Da * Dc;

  // padding columns past Da and the score block above the diagonal are read
  // as zeros by whole MFMA steps and never written
  for (size_t i = tid; i < L::W / 16; i += NTHR)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  if (tid < LT) pw[tid] = gpow(lam, lgl, tid);
  if (tid < LT) w1[tid] = gpow(lam, lgl, tid + 1);
  // (CH, summary passes) a second sum with the same a, b and lam whose value
  // is the scalar in column 0 of c2's 16-wide rows: its state rides along
  constexpr bool ch = CH;
  static_assert(!CH || MODE == L_SUMMARY, "the scalar channel is for summary passes");
  if constexpr (ch) {
    for (int k = tid; k < Da; k += NTHR) h2s[0][k] = 0.f;
  }
  __syncthreads();

  // this wave's columns of the state: H[16 t + 4 lg + j][col]
  f32x4 Ht[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      Ht[t][j] = (OUT && a.Hp && cols)
                     ? a.Hp[hbase + (a.hp_transposed ? (size_t)col * Da + (16 * t + 4 * lg + j)
                                                     : (size_t)(16 * t + 4 * lg + j) * Dc + col)]
                     : 0.f;

  TileRows<Da, NTHR, LT, (SRCF & 1) != 0> ra;
  TileRows<Da, NTHR, LT, (SRCF & 2) != 0> rb;
  TileRows<Dc, NTHR, LT, (SRCF & 4) != 0> rc;
  float c2v = 0.f;   // (ch) this thread's token's channel value, a tile ahead
  auto load_tile = [&](int t0) {
    if (OUT) ra.load(a.a, urow, nT, rev, t0, s1, tid);
    rb.load(a.b, urow, nT, rev, t0, s1, tid);
    if constexpr (!CB) rc.load(a.c, urow, nT, rev, t0, s1, tid);
    if constexpr (ch) {
      if (tid < LT) {
      const int l = t0 + tid;
      const size_t o = (urow + (size_t)(rev ? nT - 1 - l : l)) * 16;
      c2v = l >= s1 ? 0.f
            : !a.c2.p ? 1.f
            : a.c2.bf16 ? (float)reinterpret_cast<const __bf16*>(a.c2.p)[o]
                        : reinterpret_cast<const float*>(a.c2.p)[o];
      }
    }
  };
  int par = 0;   // tile parity: the channel's state is h2s[par]
  load_tile(s0);
  for (int t0 = s0; t0 < s1; t0 += LT) {
    const int Lt = s1 - t0 < LT ? s1 - t0 : LT;
    if (OUT) ra.store(As, L::LDA, tid);
    rb.store(Bs, L::LDA, tid);
    if constexpr ((SRCF & 2) != 0 && sizeof(T) == 2) {
      if (a.b_copy) rb.write_bf16_copy(a.b_copy, urow, nT, rev, t0, s1, tid);
    }
    if constexpr (!CB) rc.store(Cs, LDC, tid);
    if (tid < LT) wS[tid] = tid < Lt ? gpow(lam, lgl, Lt - 1 - tid) : 0.f;
    if constexpr (ch) {
      if (tid < LT) c2s[tid] = c2v;
    }
    __syncthreads();
    // the next tile's loads, which stay in flight during the products
    if (t0 + LT < s1) load_tile(t0 + LT);

    if constexpr (OUT) {
      // scores Ss[tau][s] = lam^(tau-s) a_tau.b_s for s <= tau (the lower 16x16
      // blocks; the block above the diagonal stays zero); with SYM also
      // Ss2[tau][s] = lam^(tau-s) a_tau.c_s
      constexpr int NB = TR * (TR + 1) / 2;
      for (int idx = wave; idx < (SYM ? 2 * NB : NB); idx += NW) {
        const bool mirror = SYM && idx >= NB;
        const T* Xs = mirror ? Cs : Bs;
        const int ldx = mirror ? LDC : L::LDA;
        T* So = mirror ? Ss2 : Ss;
        int r, c;
        tri_block(mirror ? idx - NB : idx, r, c);
        f32x4 acc = zero4();
#pragma unroll 8
        for (int k0 = 0; k0 < L::DP; k0 += KS)
          acc = MMT::mma(MMT::ld(As, L::LDA, 16 * r, k0, lane), MMT::ld(Xs, ldx, 16 * c, k0, lane), acc);
        const int s = 16 * c + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tau = 16 * r + 4 * lg + j;
          So[tau * L::LDS_ + s] = (T)(acc[j] * masked_pow(pw, tau, s));
        }
      }
      __syncthreads();
      if (cols) {
        // Y = lam^(tau+1) A H_prev + S C for this wave's 16 columns, as Y^T
        // (the state and C blocks are the A operands): a lane holds columns
        // 16 wave + 4 lg .. + 3 of token 16 r + lr and stores them at once
#pragma unroll
        for (int r = 0; r < TR; ++r) {
          const int l = t0 + 16 * r + lr;
          const size_t o = (urow + (size_t)(rev ? nT - 1 - l : l)) * Dc + 16 * wave + 4 * lg;
          // (accumulating calls) the previous outputs, in flight during the products
          f32x4 yold = zero4();
          if constexpr (ACC) {
            if (l < s1) yold = *reinterpret_cast<const f32x4*>(a.y + o);
          }
          f32x4 y = zero4();
#pragma unroll
          for (int kk = 0; kk < QK; ++kk) y = MMT::mma(FR::acc_b(Ht, kk), FR::perm(As, L::LDA, 16 * r, kk, lane), y);
          y *= w1[16 * r + lr];
#pragma unroll
          for (int k0 = 0; k0 < 16 * r + 16; k0 += KS)
            y = MMT::mma(FR::tr(Cs, LDC, k0, 16 * wave, lane), MMT::ld(Ss, L::LDS_, 16 * r, k0, lane), y);
          if constexpr (SYM) {
#pragma unroll
            for (int k0 = 0; k0 < 16 * r + 16; k0 += KS)
              y = MMT::mma(FR::tr(Bs, L::LDA, k0, 16 * wave, lane), MMT::ld(Ss2, L::LDS_, 16 * r, k0, lane), y);
          }
          if (l < s1) {
            if constexpr (ACC) {
              *reinterpret_cast<f32x4*>(a.y + o) = yold + y;
            } else if (a.y_bf16) {
              *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.y) + o) =
                  bf16x4{(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
            } else {
              *reinterpret_cast<f32x4*>(a.y + o) = y;
            }
          }
        }
      }
    }
    if (cols) {
      // H <- lam^Lt H + B^T diag(w) C (+ C^T diag(w) B with SYM)
      const float gL = gpow(lam, lgl, Lt);
      typename MMT::F bw[LT / KS], bw2[SYM ? LT / KS : 1];
#pragma unroll
      for (int kk = 0; kk < LT / KS; ++kk) bw[kk] = FR::scale(FR::tr(Cs, LDC, KS * kk, 16 * wave, lane), wS, KS * kk, lane);
      if constexpr (SYM) {
#pragma unroll
        for (int kk = 0; kk < LT / KS; ++kk) bw2[kk] = FR::scale(FR::tr(Bs, L::LDA, KS * kk, 16 * wave, lane), wS, KS * kk, lane);
      }
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 h = Ht[t] * gL;
#pragma unroll
        for (int kk = 0; kk < LT / KS; ++kk) h = MMT::mma(FR::tr(Bs, L::LDA, KS * kk, 16 * t, lane), bw[kk], h);
        if constexpr (SYM) {
#pragma unroll
          for (int kk = 0; kk < LT / KS; ++kk) h = MMT::mma(FR::tr(Cs, LDC, KS * kk, 16 * t, lane), bw2[kk], h);
        }
        Ht[t] = h;
      }
    }
    if constexpr (ch) {
      // the channel's state: h2 <- lam^Lt h2 + B^T diag(w) c2, P consecutive
      // threads per row of h2
      constexpr int P = NTHR / Da, SQ = LT / P;
      static_assert(NTHR % Da == 0 && LT % P == 0, "channel state threads");
      const int k = tid / P, part = tid % P;
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < SQ; ++i) {
        const int sx = part * SQ + i;
        v += (float)Bs[sx * L::LDA + k] * (wS[sx] * c2s[sx]);
      }
#pragma unroll
      for (int off = 1; off < P; off *= 2) v += __shfl_xor(v, off, 64);
      if (part == 0) h2s[par ^ 1][k] = gpow(lam, lgl, Lt) * h2s[par][k] + v;
    }
    if constexpr (ch) par ^= 1;
    __syncthreads();
  }

  float* Ho = OUT ? a.Hout : a.Hp;
  if (Ho && cols) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) Ho[hbase + (size_t)(16 * t + 4 * lg + j) * Dc + col] = Ht[t][j];
  }
  if (ch && a.Hp2) {
    for (int i = tid; i < Da * 16; i += NTHR)
      a.Hp2[(size_t)us * Da * 16 + i] = (i & 15) == 0 ? h2s[par][i >> 4] : 0.f;
  }
}

// Exclusive decayed running sum over the segments of each unit, in place:
// H_s <- sum_{r<s} lam^(L (s-1-r)) H_r.  One thread per state element.
__global__ __launch_bounds__(256) void la_scan_kernel(LaArgs a, int elems) {
  const int per = (elems + 255) / 256;
  const int unit = blockIdx.x / per;
  const int e = (blockIdx.x - unit * per) * 256 + threadIdx.x;
  if (e >= elems) return;
  float lam = a.gamma ? a.gamma[unit % a.H] : 1.f;
  lam = a.gexp == 3 ? lam * lam * lam : a.gexp == 2 ? lam * lam : lam;
  const float aL = gpow(lam, log2f(lam), a.seg);
  float run = 0.f;
  float* p = a.Hp + (size_t)unit * a.nseg * elems + e;
  // eight segments' loads in flight at a time rather than one dependent
  // load per segment
  constexpr int NB = 8;
  for (int s0 = 0; s0 < a.nseg; s0 += NB) {
    float x[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) x[i] = s0 + i < a.nseg ? p[(size_t)(s0 + i) * elems] : 0.f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (s0 + i < a.nseg) {
        p[(size_t)(s0 + i) * elems] = run;
        run = aL * run + x[i];
      }
    }
  }
}

template <typename T, int DA, int DC, int MODE, bool SYM, int SRCF, bool ACC = false, bool CH = false>
hipError_t launch_k(int units, const LaArgs& a, hipStream_t s) {
  constexpr int NW = LWaves<DC>::value;
  hipLaunchKernelGGL((la_kernel<T, DA, DC, MODE, NW, SYM, SRCF, ACC, CH>), dim3((unsigned)units * a.nseg),
                     dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// Picks the instantiation for the operands' source types.  fp32 MFMA takes
// fp32 sources only; bf16 MFMA takes bf16 sources with at most one fp32
// operand (the upstream gradient), and bf16 sources only for the symmetric
// and the accumulating sums.
template <typename T, int DA, int DC, int MODE>
hipError_t launch_dims(int units, const LaArgs& a, hipStream_t s) {
  int srcf = (a.a.bf16 ? 0 : 1) | (a.b.bf16 ? 0 : 2) | (a.c.bf16 ? 0 : 4);
  if (MODE == L_SUMMARY) srcf &= 6;   // a is not read
  if (a.ch) {   // the scalar channel (summary passes): sources of the MFMA type, plain sums
    if constexpr (MODE == L_SUMMARY) {
      constexpr int F = sizeof(T) == 4 ? 6 : 0;
      if (a.sym || a.reverse || a.b_copy || srcf != F || a.c2.bf16 != (sizeof(T) == 2 ? 1 : 0))
        return hipErrorInvalidValue;
      return launch_k<T, DA, DC, MODE, false, F, false, true>(units, a, s);
    }
    return hipErrorInvalidValue;
  }
  // c the same tensor as b (k in p = S q and S dp): its tile is staged once
  const bool cb = sizeof(T) == 2 && DA == DC && !a.sym && srcf == 0 && a.c.p == a.b.p &&
                  a.c.bf16 == a.b.bf16;
  if (MODE == L_OUTPUT && a.accumulate) {
    if (a.sym) return hipErrorInvalidValue;
    if constexpr (MODE == L_OUTPUT) {
      constexpr int F = sizeof(T) == 4 ? 7 : 0;
      if constexpr (sizeof(T) == 2 && DA == DC) {
        if (cb) return launch_k<T, DA, DC, MODE, false, 8, true>(units, a, s);
      }
      if (srcf == F) return launch_k<T, DA, DC, MODE, false, F, true>(units, a, s);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (sizeof(T) == 2 && DA == DC) {
    if (cb) return launch_k<T, DA, DC, MODE, false, 8>(units, a, s);
  }
  if constexpr (sizeof(T) == 4) {
    constexpr int F = MODE == L_SUMMARY ? 6 : 7;
    if (srcf != F) return hipErrorInvalidValue;
    if (a.sym) {
      if constexpr (DA == DC) return launch_k<T, DA, DC, MODE, true, F>(units, a, s);
      return hipErrorInvalidValue;
    }
    return launch_k<T, DA, DC, MODE, false, F>(units, a, s);
  } else {
    if (a.sym) {
      if constexpr (DA == DC && DA >= MM<T>::KS) {
        if (srcf == 0) return launch_k<T, DA, DC, MODE, true, 0>(units, a, s);
      }
      return hipErrorInvalidValue;
    }
    switch (srcf) {
      case 0: return launch_k<T, DA, DC, MODE, false, 0>(units, a, s);
      case 2: return launch_k<T, DA, DC, MODE, false, 2>(units, a, s);
      case 4: return launch_k<T, DA, DC, MODE, false, 4>(units, a, s);
      case 1:
        if constexpr (MODE == L_OUTPUT) return launch_k<T, DA, DC, MODE, false, 1>(units, a, s);
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
}

template <typename T, int MODE>
hipError_t launch_la_mode(int Da, int Dc, int units, const LaArgs& a, hipStream_t s) {
#define HLA_CASE(DA, DC) \
  if (Da == DA && Dc == DC) return launch_dims<T, DA, DC, MODE>(units, a, s);
  HLA_CASE(16, 16) HLA_CASE(16, 32) HLA_CASE(16, 64) HLA_CASE(16, 128)
  HLA_CASE(32, 16) HLA_CASE(32, 32) HLA_CASE(32, 64) HLA_CASE(32, 128)
  HLA_CASE(64, 16) HLA_CASE(64, 32) HLA_CASE(64, 64) HLA_CASE(64, 128)
  HLA_CASE(128, 16) HLA_CASE(128, 32) HLA_CASE(128, 64) HLA_CASE(128, 128)
#undef HLA_CASE
  return hipErrorInvalidValue;
}

// y_i += lam^(t - s0 + 1) a_t^T Hp_i for the three outputs of PrefixTermArgs:
// the part of a first-order sum that the exclusive segment prefix adds to
// the segment-local sum (the state at position t is lam^(t-s0+1) Hp plus the
// local state), so a pass that already has the local outputs needs no scores
// and no state recurrence for it.  One workgroup per (unit, segment); the 16-
// column blocks of the three outputs are dealt to the waves two at a time,
// each wave holding its blocks of Hp in registers for the whole segment.
// The outputs' rows go through LDS (loaded a tile ahead, whole rows per
// group of lanes, and stored back the same way): read and written straight
// from the product layout, every lane touched 8 bytes of a 32-byte piece of
// a row (measured at B4 H16 T16384 d128, 2048-token segments: 385 -> 333 µs).
constexpr int pt_waves(int da, int e) { return (da / 16 + e / 16 + 2) / 2; }

// [LT][W] rows of a T matrix in groups of four elements, consecutive threads
// on consecutive groups of a row: loads to registers, stores to LDS, and the
// LDS copy's rows back to global memory.  Rows at or past `end` are zero on
// load and not stored.
template <typename T, int W, int NTHR, int LT>
struct RowTile {
  static constexpr int G = W / 4, N = (LT * G + NTHR - 1) / NTHR;
  using V = typename Vec4<T>::V;
  V r[N];
  __device__ __forceinline__ void load(const T* base, size_t urow, int t0, int end, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + NTHR * i, row = idx / G, col = (idx % G) * 4;
      r[i] = V{};
      if (idx < LT * G && t0 + row < end) r[i] = *reinterpret_cast<const V*>(base + (urow + t0 + row) * W + col);
    }
  }
  __device__ __forceinline__ void to_lds(T* dst, int ld, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + NTHR * i, row = idx / G, col = (idx % G) * 4;
      if (idx < LT * G) *reinterpret_cast<V*>(dst + row * ld + col) = r[i];
    }
  }
  static __device__ __forceinline__ void from_lds(const T* src, int ld, T* base, size_t urow, int t0, int end,
                                                  int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + NTHR * i, row = idx / G, col = (idx % G) * 4;
      if (idx < LT * G && t0 + row < end)
        *reinterpret_cast<V*>(base + (urow + t0 + row) * W + col) = *reinterpret_cast<const V*>(src + row * ld + col);
    }
  }
};

template <int Da, int E>
struct PtShape {
  static constexpr int NB0 = Da / 16, NB1 = E / 16, NB = NB0 + NB1 + 1;
  static constexpr int NW = pt_waves(Da, E);
};

template <typename T, int Da, int E>
__global__ __launch_bounds__(64 * pt_waves(Da, E)) void prefix_term_kernel(PrefixTermArgs a) {
  using L = LLayout<T, Da, 16, false>;
  using MMT = MM<T>;
  using FR = Frag<T>;
  using Sh = PtShape<Da, E>;
  constexpr int NW = Sh::NW, NTHR = 64 * NW, LT = L::LT, TR = LT / 16, DT = Da / 16;
  constexpr int KS = MMT::KS;
  constexpr int QK = KS == 32 ? (DT + 1) / 2 : DT * 4;   // K steps over Da (as in la_kernel)
  __shared__ __attribute__((aligned(16))) T As[LT * L::LDA];
  // the tile's rows of the three outputs, rows padded by 16 bytes
  constexpr int PY = 16 / (int)sizeof(T), L0 = Da + PY, L1 = E + PY, L2 = 16 + PY;
  __shared__ __attribute__((aligned(16))) T Ys[LT * (L0 + L1 + L2)];
  __shared__ float w1[LT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int us = blockIdx.x;
  const int unit = us / a.nseg, seg = us - unit * a.nseg;
  float lam = a.gamma ? a.gamma[unit % a.H] : 1.f;
  lam = a.gexp == 3 ? lam * lam * lam : a.gexp == 2 ? lam * lam : lam;
  const float lgl = log2f(lam);
  const int nT = a.T;
  const int s0 = seg * a.seg, s1 = s0 + a.seg < nT ? s0 + a.seg : nT;
  const size_t urow = (size_t)unit * (size_t)nT;

  // columns past Da (a zero-padded MFMA step) read as zeros
  for (int i = tid; i < LT * L::LDA; i += NTHR) As[i] = (T)0.f;
  if (tid < LT) w1[tid] = gpow(lam, lgl, tid + 1);

  // this wave's two column blocks: output oi[b], block cbk[b] of it, width wd[b]
  int oi[2], cbk[2], wd[2];
  bool own[2];
  f32x4 Ht[2][DT];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int gb = 2 * wave + b;
    own[b] = gb < Sh::NB;
    oi[b] = gb < Sh::NB0 ? 0 : gb < Sh::NB0 + Sh::NB1 ? 1 : 2;
    cbk[b] = oi[b] == 0 ? gb : oi[b] == 1 ? gb - Sh::NB0 : 0;
    wd[b] = oi[b] == 0 ? Da : oi[b] == 1 ? E : 16;
    const float* hp = a.Hp[oi[b]] + (size_t)us * Da * wd[b];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        Ht[b][t][j] = own[b] ? hp[(size_t)(16 * t + 4 * lg + j) * wd[b] + 16 * cbk[b] + lr] : 0.f;
  }
  // bf16: the blocks as MFMA operands in the natural K order, formed once, so
  // that a's rows are read with plain 16-byte row reads
  constexpr bool NATK = sizeof(T) == 2;
  typename MMT::F hb[2][NATK ? QK : 1];
  if constexpr (NATK) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) hb[b][kk] = FR::acc_b_nat(Ht[b], kk);
  }
  __syncthreads();

  T* const y0 = reinterpret_cast<T*>(a.y[0]);
  T* const y1 = reinterpret_cast<T*>(a.y[1]);
  T* const y2 = reinterpret_cast<T*>(a.y[2]);
  T* const Y0 = Ys;
  T* const Y1 = Ys + LT * L0;
  T* const Y2 = Y1 + LT * L1;
  TileRows<Da, NTHR, LT, sizeof(T) == 4> ra;
  RowTile<T, Da, NTHR, LT> r0t;
  RowTile<T, E, NTHR, LT> r1t;
  RowTile<T, 16, NTHR, LT> r2t;
  ra.load(a.a, urow, nT, false, s0, s1, tid);
  r0t.load(y0, urow, s0, s1, tid);
  r1t.load(y1, urow, s0, s1, tid);
  r2t.load(y2, urow, s0, s1, tid);
  for (int t0 = s0; t0 < s1; t0 += LT) {
    ra.store(As, L::LDA, tid);
    r0t.to_lds(Y0, L0, tid);
    r1t.to_lds(Y1, L1, tid);
    r2t.to_lds(Y2, L2, tid);
    __syncthreads();
    if (t0 + LT < s1) {
      ra.load(a.a, urow, nT, false, t0 + LT, s1, tid);
      r0t.load(y0, urow, t0 + LT, s1, tid);
      r1t.load(y1, urow, t0 + LT, s1, tid);
      r2t.load(y2, urow, t0 + LT, s1, tid);
    }
    const float gt0 = gpow(lam, lgl, t0 - s0);
    // y^T per row block (Hp's block is the A operand), so that a lane holds
    // four adjacent columns of one token, added to the local output in LDS
    // in place
    using V = typename Vec4<T>::V;
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      const float wt = gt0 * w1[16 * r + lr];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (!own[b]) continue;
        f32x4 y = zero4();
#pragma unroll
        for (int kk = 0; kk < QK; ++kk) {
          if constexpr (NATK)
            y = MMT::mma(hb[b][kk], MMT::ld(As, L::LDA, 16 * r, 32 * kk, lane), y);
          else
            y = MMT::mma(FR::acc_b(Ht[b], kk), FR::perm(As, L::LDA, 16 * r, kk, lane), y);
        }
        T* const yb = oi[b] == 0 ? Y0 : oi[b] == 1 ? Y1 : Y2;
        const int ly = oi[b] == 0 ? L0 : oi[b] == 1 ? L1 : L2;
        V* const slot = reinterpret_cast<V*>(yb + (16 * r + lr) * ly + 16 * cbk[b] + 4 * lg);
        const V yl = *slot;
        V o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (T)((float)yl[j] + y[j] * wt);
        *slot = o;
      }
    }
    __syncthreads();
    RowTile<T, Da, NTHR, LT>::from_lds(Y0, L0, y0, urow, t0, s1, tid);
    RowTile<T, E, NTHR, LT>::from_lds(Y1, L1, y1, urow, t0, s1, tid);
    RowTile<T, 16, NTHR, LT>::from_lds(Y2, L2, y2, urow, t0, s1, tid);
    __syncthreads();
  }
}

template <typename T, int DA, int E>
hipError_t launch_pt(int units, const PrefixTermArgs& a, hipStream_t s) {
  // bf16 operands come from bf16 tensors, fp32 ones from fp32 tensors
  if (a.a.bf16 != (sizeof(T) == 2 ? 1 : 0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefix_term_kernel<T, DA, E>), dim3((unsigned)units * a.nseg),
                     dim3(64 * pt_waves(DA, E)), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_pt_dims(int Da, int E, int units, const PrefixTermArgs& a, hipStream_t s) {
#define HLA_CASE(DA, DE) \
  if (Da == DA && E == DE) return launch_pt<T, DA, DE>(units, a, s);
  HLA_CASE(16, 16) HLA_CASE(16, 32) HLA_CASE(32, 16) HLA_CASE(32, 32) HLA_CASE(32, 64)
  HLA_CASE(64, 32) HLA_CASE(64, 64) HLA_CASE(64, 128) HLA_CASE(128, 64) HLA_CASE(128, 128)
#undef HLA_CASE
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch_la(int Da, int Dc, int units, const LaArgs& a, hipStream_t s) {
  return a.mfma_bf16 ? launch_la_mode<__bf16, MODE>(Da, Dc, units, a, s)
                     : launch_la_mode<float, MODE>(Da, Dc, units, a, s);
}

// Upstream gradients of the ratio-normalised output o = num / (den + eps),
// one thread per token: dL/dnum = dO / (den + eps) (row of dv values) and
// dL/dden = -(dO . num) / (den + eps)^2, written as column 0 of a row of
// NC values whose other columns are 0, beside a row holding 1 in column 0 (the
// value channel v = 1 that turns num into den).  Out is bf16 or fp32 (the
// MFMA operand type of the sums that read it).
template <typename T>
__global__ __launch_bounds__(256) void norm_grad_kernel(const float* num, const float* den,
                                                        const float* dout, float eps, size_t tokens,
                                                        int dv, T* g_num, T* g_den, T* one) {
  constexpr int NC = 16;
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= tokens) return;
  const float r = 1.f / (den[t] + eps);
  const float* x = dout + t * dv;
  const float* y = num + t * dv;
  float dot = 0.f;
  for (int e = 0; e < dv; ++e) {
    dot += x[e] * y[e];
    g_num[t * dv + e] = (T)(x[e] * r);
  }
  g_den[t * NC] = (T)(-dot * r * r);
  one[t * NC] = (T)1.f;
  for (int e = 1; e < NC; ++e) {
    g_den[t * NC + e] = (T)0.f;
    one[t * NC + e] = (T)0.f;
  }
}

// dp (fp32, accumulated) to the operand type of the later sums
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* x, __bf16* y, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = (__bf16)x[i];
}

}  // namespace

hipError_t launch_norm_grad(int bf16, const float* num, const float* den, const float* dout,
                            float eps, size_t tokens, int dv, void* g_num, void* g_den, void* one,
                            hipStream_t s) {
  const dim3 grid((unsigned)((tokens + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(norm_grad_kernel<__bf16>, grid, dim3(256), 0, s, num, den, dout, eps, tokens,
                       dv, (__bf16*)g_num, (__bf16*)g_den, (__bf16*)one);
  else
    hipLaunchKernelGGL(norm_grad_kernel<float>, grid, dim3(256), 0, s, num, den, dout, eps, tokens, dv,
                       (float*)g_num, (float*)g_den, (float*)one);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* x, void* y, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x,
                     (__bf16*)y, n);
  return hipGetLastError();
}

hipError_t launch_prefix_terms(int Da, int E, int units, const PrefixTermArgs& a, hipStream_t s) {
  return a.mfma_bf16 ? launch_pt_dims<__bf16>(Da, E, units, a, s) : launch_pt_dims<float>(Da, E, units, a, s);
}

hipError_t launch_first_order_states(int Da, int Dc, int units, const LaArgs& a, hipStream_t s) {
  if (a.y_bf16 || a.accumulate || a.sym || a.b_copy) return hipErrorInvalidValue;
  return launch_la<L_SUMMARY>(Da, Dc, units, a, s);
}

hipError_t launch_first_order_sum(int Da, int Dc, int units, const LaArgs& a, hipStream_t s,
                                  bool prefixes_ready) {
  if (a.y_bf16 && a.accumulate) return hipErrorInvalidValue;
  if (a.b_copy && (!a.mfma_bf16 || a.b.bf16)) return hipErrorInvalidValue;
  LaArgs b = a;
  if (a.nseg > 1 && !prefixes_ready) {
    if (hipError_t e = launch_la<L_SUMMARY>(Da, Dc, units, a, s)) return e;
    const int elems = Da * Dc;
    hipLaunchKernelGGL(la_scan_kernel, dim3((unsigned)units * ((elems + 255) / 256)), dim3(256), 0, s,
                       a, elems);
    if (hipError_t e = hipGetLastError()) return e;
    if (a.b_copy) {   // the summary pass wrote the copy: read it
      b.b = LaOperand{a.b_copy, 1};
      b.b_copy = nullptr;
    }
  }
  if (a.nseg == 1) b.Hp = nullptr;
  return launch_la<L_OUTPUT>(Da, Dc, units, b, s);
}

}  // namespace hla
