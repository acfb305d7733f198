// Third-order HLA on gfx950: the segment scan with its segment map, the
// glue of the chunk-parallel forward, and the decode step.
//
// Source: the summaries of "Higher-order Linear Attention" (arXiv
// 2510.27258) on gist.science -- method section 3 (the masked third-order
// interaction A A^T A with A = Q K^T, prefix moments S^K, S^Q, P^KV and
// cross summaries), method section 4 (the third-order scan, whose operator
// carries segment-level linear maps M^KQP, M^KQm) and key contribution 3
// (online update, streaming kernel, exact chunk-parallel algorithm).
//
// With p_j = S_j q_j and u_j = P_j^T q_j (S the decayed key moment, P the
// decayed key-value moment), the masked output is
//     num_t = q_t^T R_t,  R_t = sum_{j<=t} g^(3(t-j)) p_j u_j^T,
// and den_t = q_t . r_t with u_j replaced by q_j . m_j.  A segment's summary
// (from the zero state, a = g^L) is S, Q = sum q q^T, P, m and the cross
// summaries V = sum g^(2(L-j)) p_j q_j^T, Z = sum g^(2(L-j)) q_j u_j^T,
// z = sum g^(2(L-j)) (q_j.m_j) q_j, R, r.  The combine (A then B, a of B):
//     moments: X = a X_A + X_B,
//     R = a^3 R_A + R_B + a S_A Z_B + M P_A,  r = a^3 r_A + r_B + a S_A z_B + M m_A,
//     M = a^2 S_A Q_B + a V_B   (the segment map, applied to P_A and m_A).
// The exclusive scan walks each unit's segments in order: the moments by an
// elementwise decayed running sum, then R and r by the combine above with
// the moments' prefixes in place of the running S_A, P_A, m_A.
//
// The m, z, r and unit-channel arrays are kept as [.., d][16] with the value
// in column 0 (the layout of a first-order sum whose value operand is 16
// wide); `ldm` is their row stride (16, or 1 for plain [.., d] arrays).
#include <type_traits>

#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

// Exclusive decayed running sum over each unit's nseg segments, in place
// (x_s <- sum_{r<s} a^(s-1-r) x_r, a = g^seg), one thread per element; the
// inclusive total of every element goes to `total` when it is not null.
__global__ __launch_bounds__(256) void moments_scan_kernel(float* x, float* total, const float* gamma,
                                                           int H, int seg, int nseg, int elems) {
  const int per = (elems + 255) / 256;
  const int unit = blockIdx.x / per;
  const int e = (blockIdx.x - unit * per) * 256 + threadIdx.x;
  if (e >= elems) return;
  const float g = gamma ? gamma[unit % H] : 1.f;
  const float a = gpow(g, log2f(g), seg);
  float* p = x + (size_t)unit * nseg * elems + e;
  float run = 0.f;
  constexpr int NB = 8;   // loads of eight segments in flight
  for (int s0 = 0; s0 < nseg; s0 += NB) {
    float v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) v[i] = s0 + i < nseg ? p[(size_t)(s0 + i) * elems] : 0.f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (s0 + i < nseg) {
        p[(size_t)(s0 + i) * elems] = run;
        run = a * run + v[i];
      }
    }
  }
  if (total) total[(size_t)unit * elems + e] = run;
}

// R and r through the segments of one unit, one workgroup per (unit, block
// of 16 rows), four waves.  On entry R, r hold the segment summaries; on exit
// their exclusive prefixes (each step reads its segment's rows before writing
// the prefix over them).  Sp, Pp, mp: the moments' exclusive prefixes; Q, V,
// Z, z: the segments' summaries.  All products on fp32 MFMA, operands read
// from global memory (L2-resident) with the helper tile product.
template <int D, int E>
__global__ __launch_bounds__(256) void r_scan_kernel(R3ScanArgs a) {
  constexpr int LS = D + 4;
  __shared__ float Mk[16 * LS];      // the segment map's 16 rows
  __shared__ float rrun[16];
  const int nrb = D / 16;
  const int unit = blockIdx.x / nrb, rb = blockIdx.x - unit * nrb, r0 = 16 * rb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float a1 = gpow(g, log2f(g), a.seg), a2 = a1 * a1, a3 = a2 * a1;
  constexpr int NCE = (E / 16 + 3) / 4;   // column blocks of R per wave
  f32x4 Rrun[NCE];
#pragma unroll
  for (int i = 0; i < NCE; ++i) Rrun[i] = zero4();
  if (tid < 16) rrun[tid] = 0.f;
  const int row = tid >> 4, part = tid & 15;   // the r update: 16 lanes per row
  for (int s = 0; s < a.nseg; ++s) {
    const size_t us = (size_t)unit * a.nseg + s;
    const float* SA = a.Sp + us * D * D + (size_t)r0 * D;     // 16 rows of S_A
    const float* QB = a.Q + us * D * D;
    const float* VB = a.V + us * D * D + (size_t)r0 * D;
    const float* ZB = a.Z + us * D * E;
    const float* PA = a.Pp + us * D * E;
    const float* mA = a.mp + us * D * a.ldm;
    const float* zB = a.z + us * D * a.ldm;
    float* RB = a.R + us * D * E + (size_t)r0 * E;
    float* rB = a.r + us * D * a.ldm + (size_t)r0 * a.ldm;
    // the map's rows: M = a^2 S_A Q_B + a V_B
    for (int cb = wave; cb < D / 16; cb += 4) {
      f32x4 acc = gemm_f32_tile<D>(SA, D, QB, D, 0, 16 * cb, lane, zero4());
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 4 * lg + j, cc = 16 * cb + lr;
        Mk[rr * LS + cc] = a2 * acc[j] + a1 * VB[(size_t)rr * D + cc];
      }
    }
    __syncthreads();
    // R rows: a^3 R_A + R_B + a S_A Z_B + M P_A; the prefix is R_A
#pragma unroll
    for (int i = 0; i < NCE; ++i) {
      const int ce = wave + 4 * i;
      if (ce < E / 16) {
        f32x4 rb4;
#pragma unroll
        for (int j = 0; j < 4; ++j) rb4[j] = RB[(size_t)(4 * lg + j) * E + 16 * ce + lr];
        f32x4 t1 = gemm_f32_tile<D>(SA, D, ZB, E, 0, 16 * ce, lane, zero4());
        f32x4 t2 = gemm_f32_tile<D>(Mk, LS, PA, E, 0, 16 * ce, lane, zero4());
#pragma unroll
        for (int j = 0; j < 4; ++j) RB[(size_t)(4 * lg + j) * E + 16 * ce + lr] = Rrun[i][j];
        Rrun[i] = Rrun[i] * a3 + rb4 + t1 * a1 + t2;
      }
    }
    // r rows: a^3 r_A + r_B + a S_A z_B + M m_A
    float sz = 0.f, mm = 0.f;
    for (int c = part; c < D; c += 16) {
      sz += SA[(size_t)row * D + c] * zB[(size_t)c * a.ldm];
      mm += Mk[row * LS + c] * mA[(size_t)c * a.ldm];
    }
#pragma unroll
    for (int off = 1; off < 16; off *= 2) {
      sz += __shfl_xor(sz, off, 64);
      mm += __shfl_xor(mm, off, 64);
    }
    if (part == 0) {
      const float rbv = rB[(size_t)row * a.ldm];
      rB[(size_t)row * a.ldm] = rrun[row];
      rrun[row] = a3 * rrun[row] + rbv + a1 * sz + mm;
    }
    __syncthreads();
  }
  if (a.tR) {
#pragma unroll
    for (int i = 0; i < NCE; ++i) {
      const int ce = wave + 4 * i;
      if (ce < E / 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a.tR[(size_t)unit * D * E + (size_t)(r0 + 4 * lg + j) * E + 16 * ce + lr] = Rrun[i][j];
      }
    }
  }
  if (a.tr && tid < 16) a.tr[(size_t)unit * D + r0 + tid] = rrun[tid];
}

// The unit channel: one[t][0] = 1, one[t][1..15] = 0 (bf16 or fp32).
template <typename T>
__global__ __launch_bounds__(256) void unit_channel_kernel(T* one, size_t tokens) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < tokens * 16) one[i] = (T)((i & 15) == 0 ? 1.f : 0.f);
}

// den[t] = den16[t][0]; with normalize, o[t][:] /= den[t] + eps.
__global__ __launch_bounds__(256) void finish_kernel(float* o, const float* den16, float* den,
                                                     size_t tokens, int E, int normalize, float eps) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= tokens) return;
  const float dn = den16[t * 16];
  if (den) den[t] = dn;
  if (normalize) {
    const float sc = 1.f / (dn + eps);
    f32x4* row = reinterpret_cast<f32x4*>(o + t * E);
    for (int e = 0; e < E / 4; ++e) row[e] = row[e] * sc;
  }
}

// Column 0 of [n][16] rows to a plain [n] array.
__global__ __launch_bounds__(256) void gather_col0_kernel(const float* x, float* y, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = x[i * 16];
}

// One decode step per unit (one workgroup of 256 threads):
//   S' = g S + k k^T, P' = g P + k v^T, m' = g m + k,
//   p = S' q = g S q + (k.q) k,  u = P'^T q = g P^T q + (k.q) v,  qm = q.m',
//   R' = g^3 R + p u^T,  r' = g^3 r + qm p,
//   num = R'^T q = g^3 R^T q + (q.p) u,  den = q.r' = g^3 q.r + qm (q.p).
// S, P and R are each read and written once (16-byte accesses).
template <typename T, int D, int E>
__global__ __launch_bounds__(256) void decode3_kernel(Decode3Args a) {
  constexpr int NT = 256;
  __shared__ float qs[D], ks[D], vs[E], ps[D], us[E], part[NT];
  __shared__ float red[8];
  const int unit = blockIdx.x, tid = threadIdx.x;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float g3 = g * g * g;
  const T* q = reinterpret_cast<const T*>(a.q) + (size_t)unit * D;
  const T* k = reinterpret_cast<const T*>(a.k) + (size_t)unit * D;
  const T* v = reinterpret_cast<const T*>(a.v) + (size_t)unit * E;
  for (int i = tid; i < D; i += NT) { qs[i] = (float)q[i]; ks[i] = (float)k[i]; }
  for (int i = tid; i < E; i += NT) vs[i] = (float)v[i];
  __syncthreads();
  // block sum of one value per thread (all threads call it)
  auto bsum = [&](float x) {
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    const float r = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return r;
  };
  const float kq = bsum(tid < D ? qs[tid] * ks[tid] : 0.f);
  // m' and q.m'
  float* m = a.m + (size_t)unit * D;
  float mn = 0.f;
  if (tid < D) {
    mn = g * m[tid] + ks[tid];
    m[tid] = mn;
  }
  const float qm = bsum(tid < D ? qs[tid] * mn : 0.f);
  // S: p_i = g (S q)_i + (k.q) k_i; S' written in place.  Threads cover rows
  // in groups of TPR = NT / D lanes, each lane D / TPR columns as float4s.
  {
    constexpr int TPR = NT / D > 0 ? NT / D : 1;
    constexpr int RPI = D / (NT / TPR);          // rows per thread pass
    float* S = a.S + (size_t)unit * D * D;
    const int lane_r = tid % TPR, r_base = tid / TPR;
#pragma unroll
    for (int pass = 0; pass < (RPI > 0 ? RPI : 1); ++pass) {
      const int i = r_base + pass * (NT / TPR);
      if (i < D) {
        float acc = 0.f;
        f32x4* rowp = reinterpret_cast<f32x4*>(S + (size_t)i * D);
        for (int c4 = lane_r; c4 < D / 4; c4 += TPR) {
          const f32x4 x = __builtin_nontemporal_load(rowp + c4);
          acc += x[0] * qs[4 * c4] + x[1] * qs[4 * c4 + 1] + x[2] * qs[4 * c4 + 2] + x[3] * qs[4 * c4 + 3];
          f32x4 y;
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = g * x[j] + ks[i] * ks[4 * c4 + j];
          __builtin_nontemporal_store(y, rowp + c4);
        }
        for (int off = 1; off < TPR; off *= 2) acc += __shfl_xor(acc, off, 64);
        if (lane_r == 0) ps[i] = g * acc + kq * ks[i];
      }
    }
  }
  // P: u_e = g (P^T q)_e + (k.q) v_e; P' in place.  Thread (column group cg of
  // four columns, row group rg) sums its rows; the row groups meet in LDS.
  // X' = gain X + rowv colv^T in place; out_cols = q^T X over the old X
  auto col_pass = [&](float* X, const float* rowv, const float* colv, float gain, float* out_cols) {
    constexpr int CG = E / 4, RG = NT / CG;
    const int cg = tid % CG, rg = tid / CG;
    f32x4 acc = zero4();
    for (int i = rg; i < D; i += RG) {
      f32x4* p4 = reinterpret_cast<f32x4*>(X + (size_t)i * E) + cg;
      const f32x4 x = __builtin_nontemporal_load(p4);
      f32x4 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = gain * x[j] + rowv[i] * colv[4 * cg + j];
      __builtin_nontemporal_store(y, p4);
      acc += x * qs[i];
    }
    // reduce the RG row groups
    for (int j = 0; j < 4; ++j) {
      part[tid] = acc[j];
      __syncthreads();
      if (rg == 0) {
        float s = 0.f;
        for (int r = 0; r < RG; ++r) s += part[r * CG + cg];
        out_cols[4 * cg + j] = s;
      }
      __syncthreads();
    }
  };
  // u: sum_i q_i P_ie over the old P, then P' = g P + k v^T
  col_pass(a.P + (size_t)unit * D * E, ks, vs, g, us);
  for (int e = tid; e < E; e += NT) us[e] = g * us[e] + kq * vs[e];
  __syncthreads();
  const float qp = bsum(tid < D ? qs[tid] * ps[tid] : 0.f);
  // R' = g^3 R + p u^T; num = g^3 R^T q + (q.p) u (R^T q over the old R)
  __shared__ float rq[E];
  col_pass(a.R + (size_t)unit * D * E, ps, us, g3, rq);
  // r' = g^3 r + qm p; den = g^3 q.r + qm (q.p)
  float* r = a.r + (size_t)unit * D;
  float qr_old = 0.f;
  if (tid < D) {
    const float ro = r[tid];
    qr_old = qs[tid] * ro;
    r[tid] = g3 * ro + qm * ps[tid];
  }
  const float qr = bsum(qr_old);
  const float den = g3 * qr + qm * qp;
  const float sc = a.normalize ? 1.f / (den + a.eps) : 1.f;
  for (int e = tid; e < E; e += NT) a.o[(size_t)unit * E + e] = (g3 * rq[e] + qp * us[e]) * sc;
  if (a.den && tid == 0) a.den[unit] = den;
}

}  // namespace

hipError_t launch_moments_scan(float* x, float* total, const float* gamma, int H, int seg, int nseg,
                               int elems, int units, hipStream_t s) {
  const int per = (elems + 255) / 256;
  hipLaunchKernelGGL(moments_scan_kernel, dim3((unsigned)(units * per)), dim3(256), 0, s, x, total,
                     gamma, H, seg, nseg, elems);
  return hipGetLastError();
}

hipError_t launch_r_scan(int d, int dv, int units, const R3ScanArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(units * (d / 16)));
#define HLA_CASE(D, E) \
  if (d == D && dv == E) { hipLaunchKernelGGL((r_scan_kernel<D, E>), grid, dim3(256), 0, s, a); return hipGetLastError(); }
  HLA_CASE(16, 16) HLA_CASE(16, 32) HLA_CASE(32, 16) HLA_CASE(32, 32) HLA_CASE(32, 64)
  HLA_CASE(64, 32) HLA_CASE(64, 64) HLA_CASE(64, 128) HLA_CASE(128, 64) HLA_CASE(128, 128)
#undef HLA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_unit_channel(int bf16, void* one, size_t tokens, hipStream_t s) {
  const dim3 grid((unsigned)((tokens * 16 + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(unit_channel_kernel<__bf16>, grid, dim3(256), 0, s, (__bf16*)one, tokens);
  else
    hipLaunchKernelGGL(unit_channel_kernel<float>, grid, dim3(256), 0, s, (float*)one, tokens);
  return hipGetLastError();
}

hipError_t launch_finish3(float* o, const float* den16, float* den, size_t tokens, int dv,
                          int normalize, float eps, hipStream_t s) {
  hipLaunchKernelGGL(finish_kernel, dim3((unsigned)((tokens + 255) / 256)), dim3(256), 0, s, o, den16,
                     den, tokens, dv, normalize, eps);
  return hipGetLastError();
}

hipError_t launch_gather_col0(const float* x, float* y, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(gather_col0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

hipError_t launch_decode3(int dtype, int d, int dv, int units, const Decode3Args& a, hipStream_t s) {
#define HLA_CASE(T, D, E)                                                                         \
  if (d == D && dv == E) {                                                                        \
    hipLaunchKernelGGL((decode3_kernel<T, D, E>), dim3((unsigned)units), dim3(256), 0, s, a);     \
    return hipGetLastError();                                                                     \
  }
  if (dtype == 1) {
    HLA_CASE(__bf16, 16, 16) HLA_CASE(__bf16, 16, 32) HLA_CASE(__bf16, 32, 16) HLA_CASE(__bf16, 32, 32)
    HLA_CASE(__bf16, 32, 64) HLA_CASE(__bf16, 64, 32) HLA_CASE(__bf16, 64, 64) HLA_CASE(__bf16, 64, 128)
    HLA_CASE(__bf16, 128, 64) HLA_CASE(__bf16, 128, 128)
  } else {
    HLA_CASE(float, 16, 16) HLA_CASE(float, 16, 32) HLA_CASE(float, 32, 16) HLA_CASE(float, 32, 32)
    HLA_CASE(float, 32, 64) HLA_CASE(float, 64, 32) HLA_CASE(float, 64, 64) HLA_CASE(float, 64, 128)
    HLA_CASE(float, 128, 64) HLA_CASE(float, 128, 128)
  }
#undef HLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace hla
