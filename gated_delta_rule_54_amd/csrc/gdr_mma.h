// Matrix-core (MFMA) tile products on LDS-resident operands for gfx950.
//
// A product C[m0:m0+16, n0:n0+16] += sum_k A(m, k) * B(k, n) is computed by
// one wave.  Both operands are addressed as (row, k) views of an LDS array:
//   KMIN = false: element (row, k) at p[row * ld + k]   (k contiguous)
//   KMIN = true:  element (row, k) at p[k * ld + row]   (row contiguous)
// For A the row is m; for B the row is n (i.e. B is viewed through B^T).
// k-contiguous views load a whole fragment with one 16-byte LDS read.
//
// Instruction layouts (wave64, 16x16 output tiles):
//   F16Op: v_mfma_f32_16x16x32_f16 - lane l supplies A(m0 + l%16, k0 + 8*(l/16) + i)
//          and B(k0 + 8*(l/16) + i, n0 + l%16) for i = 0..7.
//   F32Op: v_mfma_f32_16x16x4_f32  - lane l supplies A(m0 + l%16, k0 + l/16) and
//          B(k0 + l/16, n0 + l%16).
//   Accumulator: lane l holds C(m0 + 4*(l/16) + i, n0 + l%16), i = 0..3.
#pragma once

#include <hip/hip_runtime.h>

namespace gdr {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct F16Op {
  using E = _Float16;
  static constexpr int KS = 32;  // k per instruction
  template <bool KMIN>
  static __device__ __forceinline__ f16x8 frag(const E* p, int ld, int row, int k) {
    if constexpr (!KMIN) {
      return *reinterpret_cast<const f16x8*>(p + row * ld + k);
    } else {
      f16x8 r;
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = p[(k + i) * ld + row];
      return r;
    }
  }
  static __device__ __forceinline__ f32x4 mma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

struct F32Op {
  using E = float;
  static constexpr int KS = 4;
  template <bool KMIN>
  static __device__ __forceinline__ float frag(const E* p, int ld, int row, int k) {
    return KMIN ? p[k * ld + row] : p[row * ld + k];
  }
  static __device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// acc + A[m0:m0+16, 0:K] * B[0:K, n0:n0+16]; K a multiple of OP::KS.
template <typename OP, bool AKMIN, bool BKMIN>
__device__ __forceinline__ f32x4 mma_tile(f32x4 acc, const typename OP::E* A, int lda, int m0,
                                          const typename OP::E* Bt, int ldb, int n0, int K) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int kl = (lane >> 4) * (OP::KS / 4);
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += OP::KS) {
    const auto a = OP::template frag<AKMIN>(A, lda, m0 + r, k0 + kl);
    const auto b = OP::template frag<BKMIN>(Bt, ldb, n0 + r, k0 + kl);
    acc = OP::mma(a, b, acc);
  }
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row / column of accumulator element i of the calling lane for tile (m0, n0).
__device__ __forceinline__ int acc_row(int m0, int i) { return m0 + ((threadIdx.x & 63) >> 4) * 4 + i; }
__device__ __forceinline__ int acc_col(int n0) { return n0 + (threadIdx.x & 15); }

}  // namespace gdr
