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
// decayed running sum over the segments, then per 32-token tile
// Y = lam^(tau+1) A H_prev + ((A B^T) o decay) C and H <- lam^L H + B^T diag(w) C.
// Operands are staged to LDS as fp32 (bf16 inputs widened exactly) and
// contracted with v_mfma_f32_16x16x4_f32, so the intermediates p, dp and the
// upstream gradient keep full fp32 precision.

#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int LT = 32;     // tokens per tile
constexpr int LNW = 4;     // waves per workgroup
constexpr int LCB = 64;    // columns of c (and of the state) per workgroup: 16 per wave

enum { L_SUMMARY = 0, L_OUTPUT = 1 };

template <int Da, int Dc>
struct LLayout {
  static constexpr int CB = Dc < LCB ? Dc : LCB;
  static constexpr int LDA = Da + 4;       // a, b rows: [tok][Da]
  static constexpr int LDC = CB + 16;      // c rows: [tok][CB]
  static constexpr int LDS_ = LT + 4;      // scores: [tau][s]
  static constexpr size_t As = 0;
  static constexpr size_t Bs = As + (size_t)LT * LDA * 4;
  static constexpr size_t Cs = Bs + (size_t)LT * LDA * 4;
  static constexpr size_t Ss = Cs + (size_t)LT * LDC * 4;
  static constexpr size_t W = Ss + (size_t)LT * LDS_ * 4;
  // pw (lam^n), w1 (lam^(tau+1)), wS (lam^(L-1-tau)) [LT]
  static constexpr size_t TOTAL = W + 3 * LT * 4;
  static_assert(TOTAL <= 64 * 1024, "LDS budget of the first-order sum kernel");
};

// Rows [t0, t0 + LT) of the walk, columns [c0, c0 + width) of an operand with
// `ld` elements per token, widened to fp32 into LDS (rows past `end` are zero).
__device__ __forceinline__ void stage_rows(const LaOperand& x, size_t unit_row0, int T, bool rev,
                                           int t0, int end, int ld, int c0, int width, float* dst,
                                           int ldd, int tid) {
  const int n4 = LT * width / 4;
  for (int i = tid; i < n4; i += 64 * LNW) {
    const int row = i / (width / 4), col = (i % (width / 4)) * 4;
    const int l = t0 + row;
    f32x4 val = zero4();
    if (l < end) {
      const int phys = rev ? T - 1 - l : l;
      const size_t off = (unit_row0 + (size_t)phys) * (size_t)ld + (size_t)(c0 + col);
      if (x.bf16) {
        const bf16x4 b = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(x.p) + off);
        val = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
      } else {
        val = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x.p) + off);
      }
    }
    *reinterpret_cast<f32x4*>(dst + row * ldd + col) = val;
  }
}

// One workgroup per (unit, segment, block of 64 columns of c).  MODE
// L_SUMMARY writes the segment's state; L_OUTPUT starts from the exclusive
// prefix (or zero when there is none) and writes (or adds) y.
template <int Da, int Dc, int MODE>
__global__ __launch_bounds__(64 * LNW) void la_kernel(LaArgs a) {
  using L = LLayout<Da, Dc>;
  using MMT = MM<float>;
  using FR = Frag<float>;
  constexpr int CB = L::CB, NCB = Dc / CB, DT = Da / 16, TR = LT / 16;
  constexpr bool OUT = MODE == L_OUTPUT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  float* As = reinterpret_cast<float*>(smem + L::As);
  float* Bs = reinterpret_cast<float*>(smem + L::Bs);
  float* Cs = reinterpret_cast<float*>(smem + L::Cs);
  float* Ss = reinterpret_cast<float*>(smem + L::Ss);
  float* pw = reinterpret_cast<float*>(smem + L::W);
  float* w1 = pw + LT;
  float* wS = w1 + LT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int cb = blockIdx.x % NCB;
  const int us = blockIdx.x / NCB;
  const int unit = us / a.nseg, seg = us - unit * a.nseg;
  float lam = a.gamma ? a.gamma[unit % a.H] : 1.f;
  if (a.gexp == 2) lam *= lam;
  const float lgl = log2f(lam);
  const int T = a.T;
  const bool rev = a.reverse != 0;
  const int s0 = seg * a.seg, s1 = s0 + a.seg < T ? s0 + a.seg : T;
  const size_t urow = (size_t)unit * (size_t)T;
  const bool cols = wave * 16 < CB;       // this wave owns columns 16 wave .. +15 of the block
  const int col = cb * CB + 16 * wave + lr;
  const size_t hbase = (size_t)us * Da * Dc;

  if (tid < LT) pw[tid] = gpow(lam, lgl, tid);
  if (tid < LT) w1[tid] = gpow(lam, lgl, tid + 1);

  // this wave's columns of the state: H[16 t + 4 lg + j][col]
  f32x4 Ht[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      Ht[t][j] = (OUT && a.Hp && cols) ? a.Hp[hbase + (size_t)(16 * t + 4 * lg + j) * Dc + col] : 0.f;

  for (int t0 = s0; t0 < s1; t0 += LT) {
    const int Lt = s1 - t0 < LT ? s1 - t0 : LT;
    if (OUT) stage_rows(a.a, urow, T, rev, t0, s1, Da, 0, Da, As, L::LDA, tid);
    stage_rows(a.b, urow, T, rev, t0, s1, Da, 0, Da, Bs, L::LDA, tid);
    stage_rows(a.c, urow, T, rev, t0, s1, Dc, cb * CB, CB, Cs, L::LDC, tid);
    if (tid < LT) wS[tid] = tid < Lt ? gpow(lam, lgl, Lt - 1 - tid) : 0.f;
    __syncthreads();

    if constexpr (OUT) {
      // scores Ss[tau][s] = lam^(tau-s) a_tau.b_s for s <= tau (the lower 16x16
      // blocks; the block above the diagonal is never read)
      for (int idx = wave; idx < TR * (TR + 1) / 2; idx += LNW) {
        int r = 0, c = idx;
        while (c > r) { c -= r + 1; ++r; }
        f32x4 acc = zero4();
#pragma unroll 8
        for (int k0 = 0; k0 < Da; k0 += 4)
          acc = MMT::mma(MMT::ld(As, L::LDA, 16 * r, k0, lane), MMT::ld(Bs, L::LDA, 16 * c, k0, lane), acc);
        const int s = 16 * c + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tau = 16 * r + 4 * lg + j;
          Ss[tau * L::LDS_ + s] = s <= tau ? acc[j] * pw[tau - s] : 0.f;
        }
      }
      __syncthreads();
      if (cols) {
        // Y = lam^(tau+1) A H_prev + S C for this wave's 16 columns
#pragma unroll
        for (int r = 0; r < TR; ++r) {
          f32x4 y = zero4();
#pragma unroll
          for (int kk = 0; kk < Da / 4; ++kk) y = MMT::mma(FR::perm(As, L::LDA, 16 * r, kk, lane), FR::acc_b(Ht, kk), y);
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] *= w1[16 * r + 4 * lg + j];
#pragma unroll
          for (int k0 = 0; k0 < 16 * r + 16; k0 += 4)
            y = MMT::mma(MMT::ld(Ss, L::LDS_, 16 * r, k0, lane), FR::tr(Cs, L::LDC, k0, 16 * wave, lane), y);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int l = t0 + 16 * r + 4 * lg + j;
            if (l < s1) {
              const int phys = rev ? T - 1 - l : l;
              float* dst = a.y + (urow + (size_t)phys) * Dc + col;
              *dst = a.accumulate ? *dst + y[j] : y[j];
            }
          }
        }
      }
    }
    if (cols) {
      // H <- lam^Lt H + B^T diag(w) C
      const float gL = gpow(lam, lgl, Lt);
      float bw[LT / 4];
#pragma unroll
      for (int kk = 0; kk < LT / 4; ++kk) bw[kk] = FR::scale(FR::tr(Cs, L::LDC, 4 * kk, 16 * wave, lane), wS, 4 * kk, lane);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        f32x4 h = Ht[t] * gL;
#pragma unroll
        for (int kk = 0; kk < LT / 4; ++kk) h = MMT::mma(FR::tr(Bs, L::LDA, 4 * kk, 16 * t, lane), bw[kk], h);
        Ht[t] = h;
      }
    }
    __syncthreads();
  }

  if constexpr (!OUT) {
    if (cols) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) a.Hp[hbase + (size_t)(16 * t + 4 * lg + j) * Dc + col] = Ht[t][j];
    }
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
  if (a.gexp == 2) lam *= lam;
  const float aL = gpow(lam, log2f(lam), a.seg);
  float run = 0.f;
  float* p = a.Hp + (size_t)unit * a.nseg * elems + e;
  for (int s = 0; s < a.nseg; ++s) {
    const float x = p[(size_t)s * elems];
    p[(size_t)s * elems] = run;
    run = aL * run + x;
  }
}

template <int MODE>
hipError_t launch_la_mode(int Da, int Dc, int units, const LaArgs& a, hipStream_t s) {
#define HLA_CASE(DA, DC)                                                                     \
  if (Da == DA && Dc == DC) {                                                                \
    constexpr int NCB = DC / LLayout<DA, DC>::CB;                                            \
    hipLaunchKernelGGL((la_kernel<DA, DC, MODE>), dim3((unsigned)units * a.nseg * NCB),      \
                       dim3(64 * LNW), 0, s, a);                                             \
    return hipGetLastError();                                                                \
  }
  HLA_CASE(16, 16) HLA_CASE(16, 32) HLA_CASE(16, 64) HLA_CASE(16, 128)
  HLA_CASE(32, 16) HLA_CASE(32, 32) HLA_CASE(32, 64) HLA_CASE(32, 128)
  HLA_CASE(64, 16) HLA_CASE(64, 32) HLA_CASE(64, 64) HLA_CASE(64, 128)
  HLA_CASE(128, 16) HLA_CASE(128, 32) HLA_CASE(128, 64) HLA_CASE(128, 128)
#undef HLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_first_order_sum(int Da, int Dc, int units, const LaArgs& a, hipStream_t s) {
  if (a.nseg > 1) {
    if (hipError_t e = launch_la_mode<L_SUMMARY>(Da, Dc, units, a, s)) return e;
    const int elems = Da * Dc;
    hipLaunchKernelGGL(la_scan_kernel, dim3((unsigned)units * ((elems + 255) / 256)), dim3(256), 0, s,
                       a, elems);
    if (hipError_t e = hipGetLastError()) return e;
  }
  LaArgs b = a;
  if (a.nseg == 1) b.Hp = nullptr;
  return launch_la_mode<L_OUTPUT>(Da, Dc, units, b, s);
}

}  // namespace hla
