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
// tree level is one or two launches, so a level finishes before the next one
// starts:
//   up-sweep level:   x[j] <- x[i] (+) x[j]
//   down-sweep level: swap x[i] and x[j] (left <- parent prefix, right <- left
//                     sum), then x[j] <- x[i] (+) x[j] (= parent (+) left sum)
// with i = j - step for every pair of the level.  The combine is split over
// workgroups by 16-row blocks of the D-row state: a workgroup reads and writes
// only rows of x[j] it owns, and x[i] is read-only, so there is no race.  The
// cross terms S_B C_A and S_B m_A run on fp32 MFMA with C_A staged in LDS.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr int SCAN_THR = 256;
constexpr int SCAN_WAVES = SCAN_THR / 64;
constexpr int SCAN_RB = 16;      // state rows per combine workgroup

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

// x[j] <- x[i] (+) x[j] for every pair of one level; blockIdx.x = pair * (D/RB) + row block.
// a = gamma^(tokens in x[j]'s subtree): the right subtree (up-sweep) or, after
// the swap, the left subtree (down-sweep).
template <int D, int E>
__global__ __launch_bounds__(SCAN_THR) void scan_combine_kernel(ScanArgs a, int down) {
  constexpr int LDC = E + 4, LDS_ = D + 4, ET = E / 16, NRB = D / SCAN_RB;
  __shared__ __attribute__((aligned(16))) float sC[D * LDC];
  __shared__ __attribute__((aligned(16))) float sS[SCAN_RB * LDS_];
  __shared__ float sm[D];

  const int unit = blockIdx.y;
  const int step = a.step;
  const int pair = blockIdx.x / NRB, rb = blockIdx.x % NRB;
  const int j = (pair + 1) * 2 * step - 1;
  const int i = j - step;
  if (i - step + 1 >= a.n) return;   // both subtrees are padding: identity (+) identity
  const Slot A = slot_ptr(a, unit, i), B = slot_ptr(a, unit, j);
  const int lenB = down ? real_len(i - step + 1, i, a.n) : real_len(j - step + 1, j, a.n);
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float al = gpow(g, log2f(g), lenB * a.chunk);
  const float al2 = al * al;
  const int r0 = rb * SCAN_RB;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int t = tid; t < D * E / 4; t += SCAN_THR) {
    const int r = (4 * t) / E, c = (4 * t) % E;
    *reinterpret_cast<f32x4*>(sC + r * LDC + c) = reinterpret_cast<const f32x4*>(A.C)[t];
  }
  for (int t = tid; t < SCAN_RB * D / 4; t += SCAN_THR) {
    const int r = (4 * t) / D, c = (4 * t) % D;
    *reinterpret_cast<f32x4*>(sS + r * LDS_ + c) =
        reinterpret_cast<const f32x4*>(B.S + (size_t)r0 * D)[t];
  }
  for (int t = tid; t < D; t += SCAN_THR) sm[t] = A.m[t];
  __syncthreads();

  // G rows [r0, r0 + 16): a^2 G_A + G_B + a S_B C_A
  for (int et = wave; et < ET; et += SCAN_WAVES) {
    const f32x4 acc = gemm_f32_tile<D>(sS, LDS_, sC, LDC, 0, 16 * et, lane, zero4());
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const size_t e = (size_t)(r0 + 4 * (lane >> 4) + q) * E + 16 * et + (lane & 15);
      B.G[e] = al2 * A.G[e] + B.G[e] + al * acc[q];
    }
  }
  // h rows: a^2 h_A + h_B + a S_B m_A
  for (int r = tid; r < SCAN_RB; r += SCAN_THR) {
    float acc = 0.f;
    for (int c = 0; c < D; ++c) acc += sS[r * LDS_ + c] * sm[c];
    B.h[r0 + r] = al2 * A.h[r0 + r] + B.h[r0 + r] + al * acc;
  }
  // S, C, m rows: a X_A + X_B
  for (int t = tid; t < SCAN_RB * D / 4; t += SCAN_THR) {
    const size_t e = (size_t)r0 * D / 4 + t;
    reinterpret_cast<f32x4*>(B.S)[e] = reinterpret_cast<const f32x4*>(A.S)[e] * al +
                                       reinterpret_cast<const f32x4*>(B.S)[e];
  }
  for (int t = tid; t < SCAN_RB * E / 4; t += SCAN_THR) {
    const size_t e = (size_t)r0 * E / 4 + t;
    reinterpret_cast<f32x4*>(B.C)[e] = reinterpret_cast<const f32x4*>(A.C)[e] * al +
                                       reinterpret_cast<const f32x4*>(B.C)[e];
  }
  for (int t = tid; t < SCAN_RB; t += SCAN_THR) B.m[r0 + t] = al * A.m[r0 + t] + B.m[r0 + t];
}

// Down-sweep first half: x[i] <-> x[j] for every pair of one level.
// blockIdx.x = pair * parts + part; every element is swapped by one thread.
__global__ __launch_bounds__(256) void scan_swap_kernel(ScanArgs a, int parts) {
  const int unit = blockIdx.y;
  const int pair = blockIdx.x / parts, part = blockIdx.x % parts;
  const int j = (pair + 1) * 2 * a.step - 1;
  const int i = j - a.step;
  if (i - a.step + 1 >= a.n) return;
  const Slot x = slot_ptr(a, unit, i), y = slot_ptr(a, unit, j);
  const int d = a.d, dv = a.dv;
  const int nS = d * d / 4, nC = d * dv / 4;
  const int stride = parts * 256;
  for (int t = part * 256 + threadIdx.x; t < nS + 2 * nC + d / 2; t += stride) {
    f32x4* p;
    f32x4* q;
    int o;
    if (t < nS) { p = reinterpret_cast<f32x4*>(x.S); q = reinterpret_cast<f32x4*>(y.S); o = t; }
    else if (t < nS + nC) { p = reinterpret_cast<f32x4*>(x.C); q = reinterpret_cast<f32x4*>(y.C); o = t - nS; }
    else if (t < nS + 2 * nC) { p = reinterpret_cast<f32x4*>(x.G); q = reinterpret_cast<f32x4*>(y.G); o = t - nS - nC; }
    else if (t < nS + 2 * nC + d / 4) { p = reinterpret_cast<f32x4*>(x.m); q = reinterpret_cast<f32x4*>(y.m); o = t - nS - 2 * nC; }
    else { p = reinterpret_cast<f32x4*>(x.h); q = reinterpret_cast<f32x4*>(y.h); o = t - nS - 2 * nC - d / 4; }
    const f32x4 u = p[o], w = q[o];
    p[o] = w;
    q[o] = u;
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
  constexpr int NRB = D / SCAN_RB;
  constexpr int VEC = (D * D + 2 * D * E + 2 * D) / 4;       // f32x4 per summary
  constexpr int PARTS = VEC / 1024 > 0 ? VEC / 1024 : 1;    // swap workgroups per pair
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
    hipLaunchKernelGGL((scan_combine_kernel<D, E>), dim3(a.N / (2 * step) * NRB, units),
                       dim3(SCAN_THR), 0, s, a, 0);
    if (hipError_t e = hipGetLastError()) return e;
  }
  hipLaunchKernelGGL(scan_root_kernel, dim3(units), dim3(256), 0, s, a, tS, tC, tm, tG, th);
  if (hipError_t e = hipGetLastError()) return e;
  for (int step = a.N / 2; step >= 1; step /= 2) {
    a.step = step;
    hipLaunchKernelGGL(scan_swap_kernel, dim3(a.N / (2 * step) * PARTS, units), dim3(256), 0, s, a,
                       PARTS);
    if (hipError_t e = hipGetLastError()) return e;
    hipLaunchKernelGGL((scan_combine_kernel<D, E>), dim3(a.N / (2 * step) * NRB, units),
                       dim3(SCAN_THR), 0, s, a, 1);
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
