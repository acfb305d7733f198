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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Raw buffer over nbytes bytes at p (word 3 = 0x00020000, the CDNA data
// format): a load whose byte offset is nbytes or more returns zeros, so a
// ragged last tile needs no row test.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, nbytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// 16-byte store at byte_off; a store at or past the buffer's end is dropped.
// The whole offset goes in the per-lane operand: the scalar offset of a buffer
// access is left out of its range check.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 x) {
  const u32x4 v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 0);
}

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

// ---- operand fragments with other access patterns ------------------------------
//
// ld_tr: operand fragment of a matrix X stored row-major in LDS as X[k][n] (n
// contiguous): lane (n = lane & 15, g = lane >> 4) gets X[k0 + KS/4*g + i][n0 + n].
// For bf16 this is two 64-bit transposing LDS reads (ds_read_b64_tr_b16): inside
// each 16-lane group, lane l receives element (l & 3) of the 4-element vectors
// read by lanes 4j + (l >> 2), j = 0..3, so lane s of the group points at row
// k + (s >> 2), columns n0 + 4 (s & 3) .. +3.
//
// ld_perm: operand fragment whose K order matches an fp32 accumulator used as
// the other operand (see acc_b): for bf16 step kk the K slots of lane group g
// are columns 32 kk + 4 g + [0, 4) and 32 kk + 16 + 4 g + [0, 4); for fp32 step
// kk they are column 16 (kk >> 2) + 4 g + (kk & 3).
//
// acc_b: the same K order read out of 16x16 fp32 accumulator tiles stacked
// along K (tile t covers K rows 16 t .. 16 t + 15): bf16 step kk takes the lane's
// four rows of tiles 2 kk and 2 kk + 1; fp32 step kk takes row (kk & 3) of
// tile kk >> 2.
template <typename T> struct Frag;

template <> struct Frag<__bf16> {
  using F = bf16x8;
  __device__ static __forceinline__ F tr(const __bf16* X, int ldm, int k0, int n0, int lane) {
    const int l = lane & 15, g = lane >> 4;
    __bf16* p0 = const_cast<__bf16*>(X) + (k0 + 8 * g + (l >> 2)) * ldm + n0 + 4 * (l & 3);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * ldm));
    const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(F, c);
  }
  __device__ static __forceinline__ F perm(const __bf16* X, int ldm, int row0, int kk, int lane) {
    const __bf16* p = X + (row0 + (lane & 15)) * ldm + 32 * kk + 4 * (lane >> 4);
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // tiles: accumulator tiles along K; ntiles: how many exist (missing ones read as 0)
  template <int N>
  __device__ static __forceinline__ F acc_b(const f32x4 (&tiles)[N], int kk) {
    F r;
    const f32x4 a = tiles[2 * kk];
    const f32x4 b = (2 * kk + 1 < N) ? tiles[2 * kk + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = (__bf16)a[i]; r[4 + i] = (__bf16)b[i]; }
    return r;
  }
  __device__ static __forceinline__ F scale(F x, const float* w, int k0, int lane) {
    const float* ww = w + k0 + 8 * (lane >> 4);
    F y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (__bf16)((float)x[i] * ww[i]);
    return y;
  }
  // B operand of step kk in the natural K order (lane group g: K rows 32 kk +
  // 8 g + [0, 8)) from fp32 accumulator tiles 2 kk and 2 kk + 1 stacked along
  // K.  Each lane packs its four rows of both tiles to bf16 (rows 4 g' + [0, 4)
  // of group g'); one 32-lane and one 16-lane swap per dword pair then route
  // group g' of tile 2 kk to group g' / 2 (half g' % 2) and of tile 2 kk + 1 to
  // group 2 + g' / 2.
  template <int N>
  __device__ static __forceinline__ F acc_b_nat(const f32x4 (&tiles)[N], int kk) {
    const f32x4 a = tiles[2 * kk];
    const f32x4 b = (2 * kk + 1 < N) ? tiles[2 * kk + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
    auto pk = [](float x, float y) {
      const bf16x2 v = {(__bf16)x, (__bf16)y};
      return __builtin_bit_cast(unsigned, v);
    };
    const auto s0 = __builtin_amdgcn_permlane32_swap(pk(a[0], a[1]), pk(b[0], b[1]), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pk(a[2], a[3]), pk(b[2], b[3]), false, false);
    const auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
    const auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
    const uint4 r = make_uint4(t0[0], t1[0], t0[1], t1[1]);
    return __builtin_bit_cast(F, r);
  }
};

template <> struct Frag<float> {
  using F = float;
  __device__ static __forceinline__ F tr(const float* X, int ldm, int k0, int n0, int lane) {
    return X[(k0 + (lane >> 4)) * ldm + n0 + (lane & 15)];
  }
  __device__ static __forceinline__ F perm(const float* X, int ldm, int row0, int kk, int lane) {
    return X[(row0 + (lane & 15)) * ldm + 16 * (kk >> 2) + 4 * (lane >> 4) + (kk & 3)];
  }
  template <int N>
  __device__ static __forceinline__ F acc_b(const f32x4 (&tiles)[N], int kk) {
    return tiles[kk >> 2][kk & 3];
  }
  __device__ static __forceinline__ F scale(F x, const float* w, int k0, int lane) {
    return x * w[k0 + (lane >> 4)];
  }
};

// gamma^n for an integer n >= 0, with gamma^0 = 1 and 0^n = 0 for n > 0.
// lg = log2(gamma) (may be -inf for gamma = 0).
__device__ __forceinline__ float gpow(float gamma, float lg, int n) {
  if (n == 0) return 1.f;
  if (gamma == 0.f) return 0.f;
  return exp2f((float)n * lg);
}

// Lower-triangular 16x16 block number idx (row block r of the later position,
// column block c <= r, numbered row by row: (0,0), (1,0), (1,1), (2,0), ...) of
// a tile of at most 4 row blocks, without a loop: r is read from a packed table.
__device__ __forceinline__ void tri_block(int idx, int& r, int& c) {
  r = (int)((0x3333222110ull >> (4 * idx)) & 15ull);
  c = idx - (r * (r + 1)) / 2;
}

// pw[tau - i] (pw[n] = gamma^n) for i <= tau, else 0.  The table is read at a
// clamped index whatever the mask, so the read needs no branch around it.
__device__ __forceinline__ float masked_pow(const float* pw, int tau, int i) {
  const int e = tau - i;
  const float w = pw[e > 0 ? e : 0];
  return e >= 0 ? w : 0.f;
}

// init + sum of part[c * ld + tau] over the column blocks c <= tau / 16 of a
// 64-position tile, in the order c = 0, 1, ...; every block is read and the
// ones past the diagonal are dropped by a select, so no read waits on a branch.
__device__ __forceinline__ float add_lower_blocks(float init, const float* part, int ld, int tau) {
  float s = init;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float x = part[c * ld + tau];
    s += c <= tau / 16 ? x : 0.f;
  }
  return s;
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
