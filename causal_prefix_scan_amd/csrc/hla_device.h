// Device-side building blocks shared by the HLA kernels (gfx950 / CDNA4).
//
// MFMA fragments used here (wave64):
//   v_mfma_f32_16x16x32_bf16 : A 16x32, B 32x16, C/D 16x16, fp32 accumulate
//   v_mfma_f32_16x16x4_f32   : A 16x4,  B 4x16,  C/D 16x16
// Lane l holds, for A, row (l & 15) and the K values KS/4*(l >> 4) + [0, KS/4);
// for B, column (l & 15) and the same K values; for C/D, column (l & 15) and
// rows 4*(l >> 4) + [0, 4).  Every operand buffer in LDS is stored with the
// contraction index contiguous ("[row][k]"), so one fragment is one
// 16-byte (bf16) or 4-byte (fp32) LDS read per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <typename T> struct MM;

template <> struct MM<__bf16> {
  static constexpr int KS = 32;   // K per instruction
  static constexpr int CH = 8;    // elements per 16-byte chunk
  using F = bf16x8;
  __device__ static __forceinline__ F ld(const __bf16* base, int ldm, int row0, int k0, int lane) {
    return *reinterpret_cast<const F*>(base + (row0 + (lane & 15)) * ldm + k0 + 8 * (lane >> 4));
  }
  // Fragment scaled by a per-k weight (fp32), rounded once to bf16.
  __device__ static __forceinline__ F ldw(const __bf16* base, int ldm, int row0, int k0, int lane,
                                          const float* w) {
    F x = ld(base, ldm, row0, k0, lane);
    const float* ww = w + k0 + 8 * (lane >> 4);
    F y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (__bf16)((float)x[i] * ww[i]);
    return y;
  }
  __device__ static __forceinline__ f32x4 mma(F a, F b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct MM<float> {
  static constexpr int KS = 4;
  static constexpr int CH = 4;
  using F = float;
  __device__ static __forceinline__ F ld(const float* base, int ldm, int row0, int k0, int lane) {
    return base[(row0 + (lane & 15)) * ldm + k0 + (lane >> 4)];
  }
  __device__ static __forceinline__ F ldw(const float* base, int ldm, int row0, int k0, int lane,
                                          const float* w) {
    return ld(base, ldm, row0, k0, lane) * w[k0 + (lane >> 4)];
  }
  __device__ static __forceinline__ f32x4 mma(F a, F b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// gamma^n for an integer n >= 0, with gamma^0 = 1 and 0^n = 0 for n > 0.
// lg = log2(gamma) (may be -inf for gamma = 0).
__device__ __forceinline__ float gpow(float gamma, float lg, int n) {
  if (n == 0) return 1.f;
  if (gamma == 0.f) return 0.f;
  return exp2f((float)n * lg);
}

// fp32 GEMM tile from LDS with fp32 MFMA: acc += X[r0:r0+16, 0:K] * Y[0:K, c0:c0+16]
// with X stored [row][k] (leading dim ldx) and Y stored [k][col] (leading dim ldy).
template <int K>
__device__ __forceinline__ f32x4 gemm_f32_tile(const float* X, int ldx, const float* Y, int ldy,
                                               int r0, int c0, int lane, f32x4 acc) {
  const float* xp = X + (r0 + (lane & 15)) * ldx + (lane >> 4);
  const float* yp = Y + (lane >> 4) * ldy + c0 + (lane & 15);
#pragma unroll 8
  for (int k = 0; k < K; k += 4) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xp[k], yp[k * ldy], acc, 0, 0, 0);
  }
  return acc;
}

// Sum of v over the 16 lanes that share (lane >> 4) (i.e. across columns of
// a C/D fragment).  Result valid in every lane.
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

// Sum over the 4 lane groups (lane >> 4) with equal (lane & 15) (i.e. across
// rows of a C/D fragment).  Result valid in every lane.
__device__ __forceinline__ float sum_rows4(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

}  // namespace hla
