// Exclusive Blelloch scan of segment summaries under the semidirect-product
// combine ("Higher-order Linear Attention", arXiv 2510.27258, summaries on
// gist.science: method section 4 -- associative operator with cross term
// S_B C_A, exclusive Blelloch scan equal to the serial activations; key
// contribution 2 -- decayed operators).
//
// Combine of A followed by B with a = gamma^(tokens in B):
//   S = a S_A + S_B, C = a C_A + C_B, m = a m_A + m_B,
//   G = a^2 G_A + G_B + a S_B C_A, h = a^2 h_A + h_B + a S_B m_A.
// The identity is all zeros with length 0 (a = 1).
//
// The n summaries of each (b, h) unit are scanned as an array of N = 2^ceil(log2 n)
// slots; slots >= n are identities kept in a caller-provided workspace.  Each
// tree level is one launch (grid: pairs x units, one workgroup per combine),
// so the whole array level finishes before the next starts.  A workgroup
// reads everything it needs (the cross-term operands into LDS) before it
// writes, so the in-place down-sweep (left <- parent, right <- parent (+) left)
// has no read/write race.  The D x D by D x dv cross term runs on fp32 MFMA.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr int SCAN_THR = 512;
constexpr int SCAN_WAVES = SCAN_THR / 64;

struct Slot {
  float *S, *C, *m, *G, *h;
};

__device__ __forceinline__ Slot slot_ptr(const ScanArgs& a, int unit, int idx) {
  const int d = a.d, dv = a.dv;
  Slot s;
  if (idx < a.n) {
    const size_t k = (size_t)unit * a.n + idx;
    s.S = a.S + k * d * d; s.C = a.C + k * d * dv; s.m = a.m + k * d;
    s.G = a.G + k * d * dv; s.h = a.h + k * d;
  } else {
    const size_t k = (size_t)unit * (a.N - a.n) + (idx - a.n);
    s.S = a.wS + k * d * d; s.C = a.wC + k * d * dv; s.m = a.wm + k * d;
    s.G = a.wG + k * d * dv; s.h = a.wh + k * d;
  }
  return s;
}

// Number of real segments in the slot range [lo, hi].
__device__ __forceinline__ int real_len(int lo, int hi, int n) {
  const int h = hi < n - 1 ? hi : n - 1;
  return h >= lo ? h - lo + 1 : 0;
}

template <int D, int E>
__global__ __launch_bounds__(SCAN_THR) void scan_level_kernel(ScanArgs a, int down) {
  constexpr int LDS_ = D + 4, LDC = E + 4;
  constexpr int DT = D / 16, ET = E / 16;
  __shared__ __attribute__((aligned(16))) float sS[D * LDS_];
  __shared__ __attribute__((aligned(16))) float sC[D * LDC];
  __shared__ float sm[D];

  const int unit = blockIdx.y;
  const int step = a.step;
  const int j = (blockIdx.x + 1) * 2 * step - 1;
  const int i = j - step;
  if (i - step + 1 >= a.n) return;   // both subtrees are padding: identity (+) identity

  // up-sweep:   x[j] <- x[i] (+) x[j]                    (A = x[i], B = x[j])
  // down-sweep: x[i] <- x[j];  x[j] <- x[j] (+) old x[i]  (A = x[j], B = x[i])
  const Slot xi = slot_ptr(a, unit, i), xj = slot_ptr(a, unit, j);
  const Slot A = down ? xj : xi;
  const Slot B = down ? xi : xj;
  const int lenB = down ? real_len(i - step + 1, i, a.n) : real_len(j - step + 1, j, a.n);
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float al = gpow(g, log2f(g), lenB * a.chunk);
  const float al2 = al * al;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int t = tid; t < D * D / 4; t += SCAN_THR) {
    const int r = (4 * t) / D, c = (4 * t) % D;
    *reinterpret_cast<f32x4*>(sS + r * LDS_ + c) = reinterpret_cast<const f32x4*>(B.S)[t];
  }
  for (int t = tid; t < D * E / 4; t += SCAN_THR) {
    const int r = (4 * t) / E, c = (4 * t) % E;
    *reinterpret_cast<f32x4*>(sC + r * LDC + c) = reinterpret_cast<const f32x4*>(A.C)[t];
  }
  for (int t = tid; t < D; t += SCAN_THR) sm[t] = A.m[t];
  __syncthreads();

  // G = a^2 G_A + G_B + a S_B C_A
  for (int id = wave; id < DT * ET; id += SCAN_WAVES) {
    const int r0 = 16 * (id / ET), c0 = 16 * (id % ET);
    const f32x4 acc = gemm_f32_tile<D>(sS, LDS_, sC, LDC, r0, c0, lane, zero4());
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const size_t e = (size_t)(r0 + 4 * (lane >> 4) + q) * E + c0 + (lane & 15);
      const float gA = A.G[e], gB = B.G[e];
      xj.G[e] = al2 * gA + gB + al * acc[q];
      if (down) xi.G[e] = gA;
    }
  }
  // h = a^2 h_A + h_B + a S_B m_A
  for (int r = tid; r < D; r += SCAN_THR) {
    float acc = 0.f;
    for (int c = 0; c < D; ++c) acc += sS[r * LDS_ + c] * sm[c];
    const float hA = A.h[r], hB = B.h[r];
    xj.h[r] = al2 * hA + hB + al * acc;
    if (down) xi.h[r] = hA;
  }
  // S, C, m: a X_A + X_B
  for (int t = tid; t < D * D / 4; t += SCAN_THR) {
    const f32x4 sa = reinterpret_cast<const f32x4*>(A.S)[t];
    const f32x4 sb = reinterpret_cast<const f32x4*>(B.S)[t];
    reinterpret_cast<f32x4*>(xj.S)[t] = sa * al + sb;
    if (down) reinterpret_cast<f32x4*>(xi.S)[t] = sa;
  }
  for (int t = tid; t < D * E / 4; t += SCAN_THR) {
    const f32x4 ca = reinterpret_cast<const f32x4*>(A.C)[t];
    const f32x4 cb = reinterpret_cast<const f32x4*>(B.C)[t];
    reinterpret_cast<f32x4*>(xj.C)[t] = ca * al + cb;
    if (down) reinterpret_cast<f32x4*>(xi.C)[t] = ca;
  }
  for (int t = tid; t < D; t += SCAN_THR) {
    const float ma = A.m[t], mb = B.m[t];
    xj.m[t] = al * ma + mb;
    if (down) xi.m[t] = ma;
  }
}

// Root handling between the sweeps: optionally copy the inclusive total
// (slot N-1) out, then reset the root to the identity.
__global__ __launch_bounds__(256) void scan_root_kernel(ScanArgs a, float* tS, float* tC, float* tm,
                                                        float* tG, float* th) {
  const int unit = blockIdx.x;
  const Slot r = slot_ptr(a, unit, a.N - 1);
  const int d = a.d, dv = a.dv;
  for (int t = threadIdx.x; t < d * d; t += blockDim.x) {
    if (tS) tS[(size_t)unit * d * d + t] = r.S[t];
    r.S[t] = 0.f;
  }
  for (int t = threadIdx.x; t < d * dv; t += blockDim.x) {
    if (tC) tC[(size_t)unit * d * dv + t] = r.C[t];
    if (tG) tG[(size_t)unit * d * dv + t] = r.G[t];
    r.C[t] = 0.f;
    r.G[t] = 0.f;
  }
  for (int t = threadIdx.x; t < d; t += blockDim.x) {
    if (tm) tm[(size_t)unit * d + t] = r.m[t];
    if (th) th[(size_t)unit * d + t] = r.h[t];
    r.m[t] = 0.f;
    r.h[t] = 0.f;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, size_t count) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < count; t += stride) p[t] = 0.f;
}

template <int D, int E>
static hipError_t run_scan(int units, ScanArgs a, float* tS, float* tC, float* tm, float* tG,
                           float* th, hipStream_t s) {
  if (a.N > a.n) {
    // padding slots start as identities (one contiguous workspace region)
    const size_t per = (size_t)D * D + 2 * (size_t)D * E + 2 * (size_t)D;
    const size_t count = per * (size_t)units * (size_t)(a.N - a.n);
    size_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.wS, count);
    if (hipError_t e = hipGetLastError()) return e;
  }
  for (int step = 1; step < a.N; step *= 2) {
    a.step = step;
    hipLaunchKernelGGL((scan_level_kernel<D, E>), dim3(a.N / (2 * step), units), dim3(SCAN_THR), 0, s,
                       a, 0);
    if (hipError_t e = hipGetLastError()) return e;
  }
  hipLaunchKernelGGL(scan_root_kernel, dim3(units), dim3(256), 0, s, a, tS, tC, tm, tG, th);
  if (hipError_t e = hipGetLastError()) return e;
  for (int step = a.N / 2; step >= 1; step /= 2) {
    a.step = step;
    hipLaunchKernelGGL((scan_level_kernel<D, E>), dim3(a.N / (2 * step), units), dim3(SCAN_THR), 0, s,
                       a, 1);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

hipError_t launch_scan(int units, int d, int dv, const ScanArgs& a, float* tS, float* tC, float* tm,
                       float* tG, float* th, hipStream_t s) {
#define HLA_CASE(D, E) \
  if (d == D && dv == E) return run_scan<D, E>(units, a, tS, tC, tm, tG, th, s);
  HLA_CASE(16, 16) HLA_CASE(16, 32) HLA_CASE(32, 16) HLA_CASE(32, 32) HLA_CASE(32, 64)
  HLA_CASE(64, 32) HLA_CASE(64, 64) HLA_CASE(64, 128) HLA_CASE(128, 64) HLA_CASE(128, 128)
#undef HLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace hla
