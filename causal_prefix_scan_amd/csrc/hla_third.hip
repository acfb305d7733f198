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
// The exclusive scan: the moments by an elementwise decayed running sum over
// each unit's segments; then every segment's own term of R's and r's combine
// at once (the moments' prefixes in place of S_A, P_A, m_A), and an
// elementwise decayed running sum of those terms.
//
// The m, z, r arrays (and the unit channel) are kept as [.., d][16] with the value
// in column 0 (the layout of a first-order sum whose value operand is 16
// wide); `ldm` is their row stride (16, or 1 for plain [.., d] arrays).
#include <type_traits>

#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

// Exclusive decayed running sum over each unit's nseg segments, in place
// (x_s <- sum_{r<s} a^(s-1-r) x_r, a = g^seg), one thread per element, for
// up to three arrays in one launch (per unit, blockIdx.x runs over the
// blocks of x[0], then x[1], then x[2]); the inclusive total of every
// element goes to total[i] when it is not null.
struct MomentsScanArgs {
  float* x[3];
  float* total[3];
  int elems[3], nb[3];
  const float* gamma;
  int H, seg, nseg;
};

__global__ __launch_bounds__(256) void moments_scan_kernel(MomentsScanArgs m) {
  const int per = m.nb[0] + m.nb[1] + m.nb[2];
  const int unit = blockIdx.x / per;
  int b = blockIdx.x - unit * per, f = 0;
  if (b >= m.nb[0]) {
    b -= m.nb[0];
    f = 1;
    if (b >= m.nb[1]) {
      b -= m.nb[1];
      f = 2;
    }
  }
  const int elems = m.elems[f];
  const int e = b * 256 + threadIdx.x;
  if (e >= elems) return;
  const int nseg = m.nseg;
  const float g = m.gamma ? m.gamma[unit % m.H] : 1.f;
  const float a = gpow(g, log2f(g), m.seg);
  float* total = m.total[f];
  float* p = m.x[f] + (size_t)unit * nseg * elems + e;
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

// The R and r terms of every segment at once.  Over a unit's segments the
// exclusive prefixes obey
//     R_P(k+1) = a^3 R_P(k) + X_k,   X_k = R_k + a S_P(k) Z_k + M_k P_P(k),
//     M_k = a^2 S_P(k) Q_k + a V_k   (r likewise with z_k and m_P(k)),
// so once the moments' prefixes are known no X_k waits for another: one
// workgroup per (unit, segment) forms X_k and x_k in place of R_k and r_k,
// and r_prefix_kernel then turns them into the prefixes by an elementwise
// decayed running sum.  Segment 0 has zero prefixes, so X_0 = R_0 (nothing to
// do).  Wave w owns rows 16 w .. 16 w + 15.  Z_k, then Q_k, share one LDS
// buffer and P_P(k) has its own, so every operand matrix is read from HBM
// once per segment and shared by all waves; the staged rows are padded by 16
// floats, which makes the fp32 MFMA reads of four rows of 16 columns hit
// distinct banks.  Every product is formed transposed (the staged matrix as
// the A operand, the wave's S_P rows as the B operand): a lane then holds
// four adjacent columns of one row, so M's transposed block is already the
// operand of M P_P(k) (its K order 16 c + 4 (lane / 16) + jj is the one P_P(k)
// is read in), and X's rows are read and written 16 bytes at a time.  All
// products on fp32 MFMA.
template <int D, int E>
__global__ __launch_bounds__(4 * D) void r_x_kernel(R3ScanArgs a) {
  constexpr int NT = 4 * D, LQ = D + 16, LZ = E + 16;
  constexpr int BA = (D * LQ > D * LZ) ? D * LQ : D * LZ;
  __shared__ __attribute__((aligned(16))) float bA[BA];      // Z_k, then Q_k
  __shared__ __attribute__((aligned(16))) float bP[D * LZ];  // P_P(k)
  const int unit = blockIdx.x / a.nseg, s = blockIdx.x - unit * a.nseg;
  if (s == 0) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int r0 = 16 * wave;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float a1 = gpow(g, log2f(g), a.seg), a2 = a1 * a1;
  constexpr int KD = D / 4;               // K steps of a product over D
  constexpr int CD = D / 16, CE = E / 16;  // column blocks of the map and of R
  const size_t us = (size_t)unit * a.nseg + s;
  const float* SA = a.Sp + us * D * D + (size_t)r0 * D;     // 16 rows of S_P(k)
  const float* QB = a.Q + us * D * D;
  const float* VB = a.V + us * D * D + (size_t)r0 * D;
  const float* ZB = a.Z + us * D * E;
  const float* PA = a.Pp + us * D * E;
  const float* mA = a.mp + us * D * a.ldm;
  const float* zB = a.z + us * D * a.ldm;
  float* RB = a.R + us * D * E + (size_t)r0 * E;
  float* rB = a.r + us * D * a.ldm + (size_t)r0 * a.ldm;

  // a row-major [D][W] fp32 matrix: loads to registers (16 bytes per thread
  // and load), then stores to LDS with row stride LW
  auto load_mat = [&](const float* src, f32x4* x, auto Wc) {
    constexpr int W = decltype(Wc)::value, PER = D * W / 4 / NT;
#pragma unroll
    for (int u = 0; u < PER; ++u) x[u] = reinterpret_cast<const f32x4*>(src)[tid + NT * u];
  };
  auto store_mat = [&](const f32x4* x, float* dst, auto Wc, auto LWc) {
    constexpr int W = decltype(Wc)::value, LW = decltype(LWc)::value, PER = D * W / 4 / NT;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + NT * u, rr = i / (W / 4), c4 = i - rr * (W / 4);
      *reinterpret_cast<f32x4*>(dst + rr * LW + 4 * c4) = x[u];
    }
  };
  using DC = std::integral_constant<int, D>;
  using EC = std::integral_constant<int, E>;
  using LQC = std::integral_constant<int, LQ>;
  using LZC = std::integral_constant<int, LZ>;
  constexpr int PQ = D * D / 4 / NT, PZ = D * E / 4 / NT;

  // S_P rows as the B operand (lane: row lr, K slots 4 j + lg); Z_k and
  // P_P(k) staged in LDS; S_P z_k's part of x
  float sa[KD];
#pragma unroll
  for (int j = 0; j < KD; ++j) sa[j] = SA[(size_t)lr * D + 4 * j + lg];
  {
    f32x4 xz[PZ], xp[PZ];
    load_mat(ZB, xz, EC{});
    load_mat(PA, xp, EC{});
    store_mat(xz, bA, EC{}, LZC{});
    store_mat(xp, bP, EC{}, LZC{});
  }
  float sz = 0.f;
#pragma unroll
  for (int j = 0; j < KD; ++j) sz += sa[j] * zB[(size_t)(4 * j + lg) * a.ldm];
  const float rbv = lg == 0 ? rB[(size_t)lr * a.ldm] : 0.f;
  f32x4 xq[PQ];
  load_mat(QB, xq, DC{});   // in flight during S_P Z_k
  __syncthreads();

  // (S_P(k) Z_k)^T: lane holds row lr, columns 16 c + 4 lg + jj
  f32x4 t1[CE];
#pragma unroll
  for (int c = 0; c < CE; ++c) {
    f32x4 acc = zero4();
#pragma unroll
    for (int j = 0; j < KD; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bA[(4 * j + lg) * LZ + 16 * c + lr], sa[j], acc, 0, 0, 0);
    t1[c] = acc;
  }
  __syncthreads();
  store_mat(xq, bA, DC{}, LQC{});
  __syncthreads();
  // the map's rows transposed, M^T = a^2 (S_P(k) Q_k)^T + a V_k^T: lane holds
  // M[16 w + lr][16 c + 4 lg + jj]
  f32x4 mt[CD];
#pragma unroll
  for (int c = 0; c < CD; ++c) {
    const f32x4 vb = *reinterpret_cast<const f32x4*>(VB + (size_t)lr * D + 16 * c + 4 * lg);
    f32x4 acc = zero4();
#pragma unroll
    for (int j = 0; j < KD; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bA[(4 * j + lg) * LQ + 16 * c + lr], sa[j], acc, 0, 0, 0);
    mt[c] = acc * a2 + vb * a1;
  }
  // X rows = R_k + a t1 + M P_P(k), in place: (M P_P(k))^T with P_P(k)'s rows
  // taken in M^T's K order (K step 4 c + jj: row 16 c + 4 lg + jj)
#pragma unroll
  for (int ce = 0; ce < CE; ++ce) {
    f32x4 acc = zero4();
#pragma unroll
    for (int c = 0; c < CD; ++c)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bP[(16 * c + 4 * lg + jj) * LZ + 16 * ce + lr], mt[c][jj],
                                                   acc, 0, 0, 0);
    f32x4* px = reinterpret_cast<f32x4*>(RB + (size_t)lr * E + 16 * ce + 4 * lg);
    *px = *px + t1[ce] * a1 + acc;
  }
  // x rows = r_k + a S_P(k) z_k + M m_P(k)
  float mm = 0.f;
#pragma unroll
  for (int c = 0; c < CD; ++c)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) mm += mt[c][jj] * mA[(size_t)(16 * c + 4 * lg + jj) * a.ldm];
  float xr = a1 * sz + mm;
  xr += __shfl_xor(xr, 16, 64);
  xr += __shfl_xor(xr, 32, 64);
  if (lg == 0) rB[(size_t)lr * a.ldm] = rbv + xr;
}

// R_k, r_k (holding X_k, x_k) become their exclusive prefixes:
// R_P(k) = sum_{j<k} a^(3(k-1-j)) X_j, elementwise, one thread per element of
// R and of r (row stride ldm); the inclusive totals to tR, tr when set.
template <int D, int E>
__global__ __launch_bounds__(256) void r_prefix_kernel(R3ScanArgs a) {
  constexpr int ER = D * E, ALL = ER + D, PER = (ALL + 255) / 256;
  const int unit = blockIdx.x / PER;
  const int e = (blockIdx.x - unit * PER) * 256 + threadIdx.x;
  if (e >= ALL) return;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float a1 = gpow(g, log2f(g), a.seg), a3 = a1 * a1 * a1;
  const bool isR = e < ER;
  const size_t stride = isR ? (size_t)ER : (size_t)D * a.ldm;
  float* p = isR ? a.R + (size_t)unit * a.nseg * ER + e
                 : a.r + (size_t)unit * a.nseg * D * a.ldm + (size_t)(e - ER) * a.ldm;
  float run = 0.f;
  constexpr int NB = 8;   // loads of eight segments in flight
  for (int s0 = 0; s0 < a.nseg; s0 += NB) {
    float v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) v[i] = s0 + i < a.nseg ? p[(size_t)(s0 + i) * stride] : 0.f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (s0 + i < a.nseg) {
        p[(size_t)(s0 + i) * stride] = run;
        run = a3 * run + v[i];
      }
    }
  }
  float* t = isR ? a.tR : a.tr;
  if (t) t[isR ? (size_t)unit * ER + e : (size_t)unit * D + (e - ER)] = run;
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

// One decode step per unit (one workgroup of 512 threads):
//   S' = g S + k k^T, P' = g P + k v^T, m' = g m + k,
//   p = S' q = g S q + (k.q) k,  u = P'^T q = g P^T q + (k.q) v,  qm = q.m',
//   R' = g^3 R + p u^T,  r' = g^3 r + qm p,
//   num = R'^T q = g^3 R^T q + (q.p) u,  den = q.r' = g^3 q.r + qm (q.p).
// Every load of S, P and R is issued up front (16-byte, non-temporal); S' and
// P' are stored at once, R is held in registers until p and u are reduced.
template <typename T, int D, int E>
__global__ __launch_bounds__(512) void decode3_kernel(Decode3Args a) {
  constexpr int NT = 512;
  constexpr int DV4 = D / 4, EV4 = E / 4;
  constexpr int NS = (D * DV4 + NT - 1) / NT;     // float4s of S per thread
  constexpr int NP = (D * EV4 + NT - 1) / NT;     // float4s of P (and R) per thread
  constexpr int RG = NT / EV4;                    // threads sharing a column group of P, R
  __shared__ float qs[D], ks[D], vs[E], ps[D], us[E], rq[E];
  __shared__ f32x4 part[2][NT];
  __shared__ float red[8][4];
  const int unit = blockIdx.x, tid = threadIdx.x, wv = tid >> 6;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float g3 = g * g * g;
  float* S = a.S + (size_t)unit * D * D;
  float* P = a.P + (size_t)unit * D * E;
  float* R = a.R + (size_t)unit * D * E;
  // every state load in flight before any arithmetic waits on one
  f32x4 xs[NS], xp[NP], xr[NP];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int idx = tid + NT * j;
    xs[j] = idx < D * DV4 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S) + idx) : zero4();
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int idx = tid + NT * j;
    xp[j] = idx < D * EV4 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(P) + idx) : zero4();
    xr[j] = idx < D * EV4 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(R) + idx) : zero4();
  }
  const T* q = reinterpret_cast<const T*>(a.q) + (size_t)unit * D;
  const T* k = reinterpret_cast<const T*>(a.k) + (size_t)unit * D;
  const T* v = reinterpret_cast<const T*>(a.v) + (size_t)unit * E;
  float* m = a.m + (size_t)unit * D;
  float* r = a.r + (size_t)unit * D;
  float mo = 0.f, ro = 0.f;
  if (tid < D) {
    qs[tid] = (float)q[tid];
    ks[tid] = (float)k[tid];
    mo = m[tid];
    ro = r[tid];
  }
  if (tid < E) vs[tid] = (float)v[tid];
  __syncthreads();
  // up to four block sums at once (every thread calls it)
  auto bsum4 = [&](f32x4 x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] += __shfl_xor(x[i], off, 64);
    if ((tid & 63) == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wv][i] = x[i];
    __syncthreads();
    f32x4 y = zero4();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] += red[w][i];
    __syncthreads();
    return y;
  };
  const float qd = tid < D ? qs[tid] : 0.f, kd = tid < D ? ks[tid] : 0.f;
  const float mn = g * mo + kd;
  if (tid < D) m[tid] = mn;
  const f32x4 s1 = bsum4(f32x4{qd * kd, qd * mn, qd * ro, 0.f});
  const float kq = s1[0], qm = s1[1], qr_old = s1[2];
  // S: row sums against q (rows of DV4 lanes), S' stored at once
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int idx = tid + NT * j;
    const int i = idx / DV4, c = 4 * (idx % DV4);
    float acc = 0.f;
    if (idx < D * DV4) {
      const f32x4 x = xs[j];
      acc = x[0] * qs[c] + x[1] * qs[c + 1] + x[2] * qs[c + 2] + x[3] * qs[c + 3];
      f32x4 y;
#pragma unroll
      for (int t = 0; t < 4; ++t) y[t] = g * x[t] + ks[i] * ks[c + t];
      __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(S) + idx);
    }
#pragma unroll
    for (int off = 1; off < DV4; off *= 2) acc += __shfl_xor(acc, off, 64);
    if (idx < D * DV4 && (idx % DV4) == 0) ps[i] = g * acc + kq * ks[i];
  }
  // P and R: column partial sums against q over this thread's rows (the old
  // values); P' stored at once
  f32x4 up = zero4(), rp = zero4();
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int idx = tid + NT * j;
    if (idx < D * EV4) {
      const int i = idx / EV4, c = 4 * (idx % EV4);
      up += xp[j] * qs[i];
      rp += xr[j] * qs[i];
      f32x4 y;
#pragma unroll
      for (int t = 0; t < 4; ++t) y[t] = g * xp[j][t] + ks[i] * vs[c + t];
      __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(P) + idx);
    }
  }
  part[0][tid] = up;
  part[1][tid] = rp;
  __syncthreads();
  if (tid < 2 * EV4) {
    const int which = tid / EV4, cg = tid % EV4;
    f32x4 sum = zero4();
    for (int t = cg; t < NT; t += EV4) sum += part[which][t];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (which == 0) us[4 * cg + t] = g * sum[t] + kq * vs[4 * cg + t];
      else rq[4 * cg + t] = sum[t];
    }
  }
  __syncthreads();
  // R' = g^3 R + p u^T
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int idx = tid + NT * j;
    if (idx < D * EV4) {
      const int i = idx / EV4, c = 4 * (idx % EV4);
      f32x4 y;
#pragma unroll
      for (int t = 0; t < 4; ++t) y[t] = g3 * xr[j][t] + ps[i] * us[c + t];
      __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(R) + idx);
    }
  }
  const float pd = tid < D ? ps[tid] : 0.f;
  if (tid < D) r[tid] = g3 * ro + qm * pd;
  const f32x4 s2 = bsum4(f32x4{qd * pd, 0.f, 0.f, 0.f});
  const float qp = s2[0];
  const float den = g3 * qr_old + qm * qp;
  const float sc = a.normalize ? 1.f / (den + a.eps) : 1.f;
  if (tid < E) a.o[(size_t)unit * E + tid] = (g3 * rq[tid] + qp * us[tid]) * sc;
  if (a.den && tid == 0) a.den[unit] = den;
  (void)RG;
}

}  // namespace

hipError_t launch_moments_scan(float* const x[3], float* const total[3], const int elems[3],
                               const float* gamma, int H, int seg, int nseg, int units, hipStream_t s) {
  MomentsScanArgs m;
  int per = 0;
  for (int i = 0; i < 3; ++i) {
    m.x[i] = x[i];
    m.total[i] = total[i];
    m.elems[i] = x[i] ? elems[i] : 0;
    m.nb[i] = (m.elems[i] + 255) / 256;
    per += m.nb[i];
  }
  m.gamma = gamma; m.H = H; m.seg = seg; m.nseg = nseg;
  if (per == 0) return hipSuccess;
  hipLaunchKernelGGL(moments_scan_kernel, dim3((unsigned)(units * per)), dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_r_scan(int d, int dv, int units, const R3ScanArgs& a, hipStream_t s) {
  // every segment's X at once, then the elementwise prefixes
  const dim3 gx((unsigned)units * (unsigned)a.nseg);
#define HLA_CASE(D, E)                                                                              \
  if (d == D && dv == E) {                                                                          \
    hipLaunchKernelGGL((r_x_kernel<D, E>), gx, dim3(4 * D), 0, s, a);                               \
    if (hipError_t e = hipGetLastError()) return e;                                                 \
    const unsigned per = (unsigned)((D * E + D + 255) / 256);                                        \
    hipLaunchKernelGGL((r_prefix_kernel<D, E>), dim3((unsigned)units * per), dim3(256), 0, s, a);   \
    return hipGetLastError();                                                                       \
  }
  HLA_CASE(16, 16) HLA_CASE(16, 32) HLA_CASE(32, 16) HLA_CASE(32, 32) HLA_CASE(32, 64)
  HLA_CASE(64, 32) HLA_CASE(64, 64) HLA_CASE(64, 128) HLA_CASE(128, 64) HLA_CASE(128, 128)
#undef HLA_CASE
  return hipErrorInvalidValue;
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
    hipLaunchKernelGGL((decode3_kernel<T, D, E>), dim3((unsigned)units), dim3(512), 0, s, a);     \
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
