// One streaming decode step of the masked second-order HLA
// ("Higher-order Linear Attention", arXiv 2510.27258, summaries on
// gist.science: method section 1 -- online update of the prefix state and
// the output q^T (S C - G) with its ratio-normalised variant; results and
// claims -- constant work and memory per token).
//
// Per unit (one workgroup of 512 threads), with g the unit's decay and the
// old state (S, C, m, G, h):
//   u = C^T k,  G' = g^2 G + g k u^T,  h' = g^2 h + g k (k.m)
//   S' = g S + k k^T,  C' = g C + q v^T,  m' = g m + q
//   a = S' q,  num = C'^T a - G'^T q,  den = a.m' - q.h'
// expanded so that each state element is read once and written once:
//   num_e = g (C^T a)_e + (a.q) v_e - g^2 (G^T q)_e - g (q.k) u_e
//   den   = g (a.m) + (a.q) - g^2 (q.h) - g (q.k)(k.m).
// The kernel is HBM-bound: the state is streamed with 16-byte coalesced
// non-temporal loads and stores; all reductions go through registers,
// cross-lane shuffles and LDS.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr int DEC_THR = 512;

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

template <typename T, int D, int E>
__global__ __launch_bounds__(DEC_THR) void decode_kernel(DecodeArgs a) {
  constexpr int CPR_S = D / 4, RP_S = DEC_THR / CPR_S, NP_S = (D + RP_S - 1) / RP_S;
  constexpr int CPR_C = E / 4, RP_C = DEC_THR / CPR_C, NP_C = (D + RP_C - 1) / RP_C;
  constexpr int NRG = RP_C < D ? RP_C : D;   // row groups that hold C rows

  __shared__ __attribute__((aligned(16))) float sq[D], sk[D], sv[E], smo[D], sho[D], aval[D];
  __shared__ __attribute__((aligned(16))) float ru[NRG][E], ry[NRG][E], rz[NRG][E];
  __shared__ __attribute__((aligned(16))) float uu[E], yy[E], zz[E];
  __shared__ float scal[5];

  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const float g = a.gamma ? a.gamma[unit % a.H] : 1.f;
  const float g2 = g * g;

  f32x4* S = reinterpret_cast<f32x4*>(a.S + (size_t)unit * D * D);
  f32x4* C = reinterpret_cast<f32x4*>(a.C + (size_t)unit * D * E);
  f32x4* G = reinterpret_cast<f32x4*>(a.G + (size_t)unit * D * E);
  float* m = a.m + (size_t)unit * D;
  float* h = a.h + (size_t)unit * D;

  // stream the state in (all loads issued before any use)
  const int ccS = tid % CPR_S, rgS = tid / CPR_S;
  const int ccC = tid % CPR_C, rgC = tid / CPR_C;
  f32x4 rS[NP_S], rC[NP_C], rG[NP_C];
#pragma unroll
  for (int i = 0; i < NP_S; ++i) {
    const int d = rgS + RP_S * i;
    if (d < D) rS[i] = __builtin_nontemporal_load(S + d * CPR_S + ccS);
  }
#pragma unroll
  for (int i = 0; i < NP_C; ++i) {
    const int d = rgC + RP_C * i;
    if (d < D) {
      rC[i] = __builtin_nontemporal_load(C + d * CPR_C + ccC);
      rG[i] = __builtin_nontemporal_load(G + d * CPR_C + ccC);
    }
  }
  const T* q = reinterpret_cast<const T*>(a.q) + (size_t)unit * D;
  const T* k = reinterpret_cast<const T*>(a.k) + (size_t)unit * D;
  const T* v = reinterpret_cast<const T*>(a.v) + (size_t)unit * E;
  for (int t = tid; t < D; t += DEC_THR) {
    sq[t] = to_f32(q[t]);
    sk[t] = to_f32(k[t]);
    smo[t] = m[t];
    sho[t] = h[t];
  }
  for (int t = tid; t < E; t += DEC_THR) sv[t] = to_f32(v[t]);
  __syncthreads();

  // S' = g S + k k^T; a = S' q (row sums over the CPR_S lanes of a row)
  {
    const f32x4 q4 = *reinterpret_cast<const f32x4*>(sq + 4 * ccS);
    const f32x4 k4 = *reinterpret_cast<const f32x4*>(sk + 4 * ccS);
#pragma unroll
    for (int i = 0; i < NP_S; ++i) {
      const int d = rgS + RP_S * i;
      float ap = 0.f;
      if (d < D) {
        const f32x4 sn = rS[i] * g + k4 * sk[d];
        __builtin_nontemporal_store(sn, S + d * CPR_S + ccS);
        ap = sn[0] * q4[0] + sn[1] * q4[1] + sn[2] * q4[2] + sn[3] * q4[3];
      }
#pragma unroll
      for (int off = 1; off < CPR_S; off *= 2) ap += __shfl_xor(ap, off, 64);
      if (d < D && ccS == 0) aval[d] = ap;
    }
  }
  __syncthreads();

  // C' = g C + q v^T; partial u = C^T k, z = C^T a, y = G^T q over this thread's rows
  {
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(sv + 4 * ccC);
    f32x4 pu = zero4(), pz = zero4(), py = zero4();
#pragma unroll
    for (int i = 0; i < NP_C; ++i) {
      const int d = rgC + RP_C * i;
      if (d < D) {
        const f32x4 c4 = rC[i];
        pu += c4 * sk[d];
        pz += c4 * aval[d];
        py += rG[i] * sq[d];
        __builtin_nontemporal_store(c4 * g + v4 * sq[d], C + d * CPR_C + ccC);
      }
    }
    if (rgC < NRG) {
      *reinterpret_cast<f32x4*>(&ru[rgC][4 * ccC]) = pu;
      *reinterpret_cast<f32x4*>(&rz[rgC][4 * ccC]) = pz;
      *reinterpret_cast<f32x4*>(&ry[rgC][4 * ccC]) = py;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += DEC_THR) {
    float su = 0.f, sy = 0.f, sz = 0.f;
    for (int r = 0; r < NRG; ++r) { su += ru[r][e]; sy += ry[r][e]; sz += rz[r][e]; }
    uu[e] = su; yy[e] = sy; zz[e] = sz;
  }
  if (tid < 64) {
    float aq = 0.f, am = 0.f, qh = 0.f, qk = 0.f, km = 0.f;
    for (int d = tid; d < D; d += 64) {
      aq += aval[d] * sq[d];
      am += aval[d] * smo[d];
      qh += sq[d] * sho[d];
      qk += sq[d] * sk[d];
      km += sk[d] * smo[d];
    }
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) {
      aq += __shfl_xor(aq, off, 64);
      am += __shfl_xor(am, off, 64);
      qh += __shfl_xor(qh, off, 64);
      qk += __shfl_xor(qk, off, 64);
      km += __shfl_xor(km, off, 64);
    }
    if (tid == 0) { scal[0] = aq; scal[1] = am; scal[2] = qh; scal[3] = qk; scal[4] = km; }
  }
  __syncthreads();

  // G' = g^2 G + g k u^T
  {
    const f32x4 u4 = *reinterpret_cast<const f32x4*>(uu + 4 * ccC);
#pragma unroll
    for (int i = 0; i < NP_C; ++i) {
      const int d = rgC + RP_C * i;
      if (d < D) __builtin_nontemporal_store(rG[i] * g2 + u4 * (g * sk[d]), G + d * CPR_C + ccC);
    }
  }
  const float aq = scal[0], am = scal[1], qh = scal[2], qk = scal[3], km = scal[4];
  for (int t = tid; t < D; t += DEC_THR) {
    m[t] = g * smo[t] + sq[t];
    h[t] = g2 * sho[t] + g * sk[t] * km;
  }
  const float den = g * am + aq - g2 * qh - g * qk * km;
  for (int e = tid; e < E; e += DEC_THR) {
    const float num = g * zz[e] + aq * sv[e] - g2 * yy[e] - g * qk * uu[e];
    a.o[(size_t)unit * E + e] = a.normalize ? num / (den + a.eps) : num;
  }
  if (a.den != nullptr && tid == 0) a.den[unit] = den;
}

hipError_t launch_decode(int dtype, int d, int dv, int units, const DecodeArgs& a, hipStream_t s) {
#define HLA_CASE(T, D, E)                                                                      \
  if (d == D && dv == E) {                                                                     \
    hipLaunchKernelGGL((decode_kernel<T, D, E>), dim3(units), dim3(DEC_THR), 0, s, a);         \
    return hipGetLastError();                                                                  \
  }
  if (dtype == 1) {
    HLA_CASE(__bf16, 16, 16) HLA_CASE(__bf16, 16, 32) HLA_CASE(__bf16, 32, 16)
    HLA_CASE(__bf16, 32, 32) HLA_CASE(__bf16, 32, 64) HLA_CASE(__bf16, 64, 32)
    HLA_CASE(__bf16, 64, 64) HLA_CASE(__bf16, 64, 128) HLA_CASE(__bf16, 128, 64)
    HLA_CASE(__bf16, 128, 128)
  } else {
    HLA_CASE(float, 16, 16) HLA_CASE(float, 16, 32) HLA_CASE(float, 32, 16)
    HLA_CASE(float, 32, 32) HLA_CASE(float, 32, 64) HLA_CASE(float, 64, 32)
    HLA_CASE(float, 64, 64) HLA_CASE(float, 64, 128) HLA_CASE(float, 128, 64)
    HLA_CASE(float, 128, 128)
  }
#undef HLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace hla
