// Device-side helpers shared by the libgdr kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

constexpr float kL2Eps = 1e-6f;  // q/k L2-norm eps (Megatron-LM page, "Why")

typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// ---- typed scalar / 4-vector loads and stores (T = float or bf16_t) ------
template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ void ld4(const T* p, float (&x)[4]);
template <> __device__ __forceinline__ void ld4<float>(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void ld4<bf16_t>(const bf16_t* p, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xffff0000u);
  x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xffff0000u);
}

template <typename T> __device__ __forceinline__ void st1(T* p, float x);
template <> __device__ __forceinline__ void st1<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void st1<bf16_t>(bf16_t* p, float x) { *p = f32_to_bf16(x); }

template <typename T> __device__ __forceinline__ void st4(T* p, const float (&x)[4]);
template <> __device__ __forceinline__ void st4<float>(float* p, const float (&x)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
template <> __device__ __forceinline__ void st4<bf16_t>(bf16_t* p, const float (&x)[4]) {
  uint2 v;
  v.x = static_cast<uint32_t>(f32_to_bf16(x[0])) | (static_cast<uint32_t>(f32_to_bf16(x[1])) << 16);
  v.y = static_cast<uint32_t>(f32_to_bf16(x[2])) | (static_cast<uint32_t>(f32_to_bf16(x[3])) << 16);
  *reinterpret_cast<uint2*>(p) = v;
}

// Fused gate activation: g = -softplus(a) = -(max(a, 0) + log1p(e^-|a|)),
// alpha = exp(g) = 1 / (1 + e^a), beta = sigmoid(b); and the factors that
// take dL/dg and dL/dbeta to dL/da = -sigmoid(a) dL/dg and
// dL/db = beta (1 - beta) dL/dbeta.
__device__ __forceinline__ float fg_log_alpha(float a) { return -(fmaxf(a, 0.f) + log1pf(expf(-fabsf(a)))); }
__device__ __forceinline__ float fg_alpha(float a) { return 1.f / (1.f + expf(a)); }
__device__ __forceinline__ float fg_beta(float b) { return 1.f / (1.f + expf(-b)); }
__device__ __forceinline__ float fg_dlog_alpha(float a) { return -1.f / (1.f + expf(-a)); }
__device__ __forceinline__ float fg_dbeta(float b) {
  const float s = fg_beta(b);
  return s * (1.f - s);
}

// Sum over the lanes whose ids differ only in the bits of [LO, HI) masks,
// i.e. xor-butterfly with masks LO, 2*LO, ..., HI/2.  Every lane ends with
// the same total; the order of additions is fixed (deterministic).
template <int LO, int HI>
__device__ __forceinline__ float xsum(float x) {
#pragma unroll
  for (int m = LO; m < HI; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k+15): four row
// rotations; every lane of the row ends with the same total.  A rotation
// never reads outside the row, so bound_ctrl changes nothing but lets the
// compiler fold each move into its add (v_add_f32_dpp).
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x122, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x121, 0xf, 0xf, true));
  return x;
}

// N (16 or 8) sums over the 16 lanes of a DPP row at once: lane j of the
// row ends with the sum of every lane's v[j N / 16].  Recursive halving: at
// each step a lane pairs with its mirror in the row, its mirror in the
// half-row, its mirror in the quad, then its neighbour; the lane whose bit
// (3, 2, 1, 0 of its row position) is set keeps the upper half of its
// values, the other the lower, and each adds the half its partner gave up
// (with N = 8 the neighbours, holding the same value, just add).  15 adds
// and 30 selects for N = 16, against 64 adds for sixteen full row sums; the
// order of additions is fixed.
template <int H, int CTRL>
__device__ __forceinline__ void row16_halve(const float* in, float* out, bool hi) {
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float keep = hi ? in[k + H] : in[k];
    const float give = hi ? in[k] : in[k + H];
    out[k] = keep + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, give), CTRL, 0xf, 0xf,
                                                                       true));
  }
}
template <int N>
__device__ __forceinline__ float row16_scatter(const float (&v)[N]) {
  static_assert(N == 16 || N == 8, "16 or 8 values per lane");
  const int j = threadIdx.x & 15;
  float a[8], b[4], c[2];
  if constexpr (N == 16) {
    row16_halve<8, 0x140>(v, a, (j & 8) != 0);  // row_mirror: lane 15 - j
    row16_halve<4, 0x141>(a, b, (j & 4) != 0);  // row_half_mirror: lane 7 - j in its half
  } else {
    row16_halve<4, 0x140>(v, b, (j & 8) != 0);
  }
  row16_halve<2, (N == 16 ? 0x1b : 0x141)>(b, c, (j & (N == 16 ? 2 : 4)) != 0);
  float d[1];
  row16_halve<1, (N == 16 ? 0xb1 : 0x1b)>(c, d, (j & (N == 16 ? 1 : 2)) != 0);
  if constexpr (N == 16) {
    return d[0];
  } else {  // quad_perm [1, 0, 3, 2]: the neighbour holds the same value
    return d[0] + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, d[0]), 0xb1, 0xf, 0xf, true));
  }
}

// Sum over the four 16-lane rows (lanes j, j ^ 16, j ^ 32, j ^ 48): every
// lane ends with its row position's total.  gfx950's row swaps exchange
// odd and even rows, then the two halves of the wave, on the VALU (no LDS
// crossbar); the two lanes of a pair add the same two values.  The swaps'
// results are copied out element by element before use (a bit cast taken
// directly of the second element reads the first).
__device__ __forceinline__ float rows4_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned a0 = a[0], a1 = a[1];
  const float y = __uint_as_float(a0) + __uint_as_float(a1);
  const unsigned v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return __uint_as_float(b0) + __uint_as_float(b1);
}

}  // namespace gdr
