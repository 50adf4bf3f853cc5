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

// Sum over aligned groups of N (8 or 16) lanes by DPP adds on the VALU: the
// neighbour, the other pair of the quad, then the mirror in the half-row
// (and for N = 16 in the row); once a group's quads (halves) hold equal
// values, the mirror reaches the other quad (half).  The additions and
// their order are those of the xor butterfly xsum<1, N>.
template <int N>
__device__ __forceinline__ float group_sum_dpp(float x) {
  static_assert(N == 8 || N == 16, "8 or 16 lanes");
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xb1, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4e, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, true));
  if constexpr (N == 16)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xf, 0xf, true));
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
// (with N = 8 the neighbours, holding the same value, just add).  27 adds
// and 6 selects for N = 16, against 64 adds for sixteen full row sums; the
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
// The first two halving steps split the row by bit 3, then bit 2 of the
// lane's row position: whole DPP banks of four lanes, so the bank mask picks
// the lanes an add writes.  The lower banks add their own and their
// partner's v[k], the upper banks v[k + H], into one register: two adds per
// pair and no selects (the builtins take a bank mask only on a move, whose
// add then needs the selects again).  The leading s_nop gives the wait
// states a DPP read needs after a VALU write of its source, which the
// compiler's hazard pass does not check inside inline asm.  Each add is
// partner + own, the same sum as the selecting form.
__device__ __forceinline__ void row16_halve8_mirror(const float* in, float* out) {
  asm("s_nop 4\n"
      "v_add_f32_dpp %0, %8, %8 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %0, %16, %16 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %1, %9, %9 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %1, %17, %17 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %2, %10, %10 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %2, %18, %18 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %3, %11, %11 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %3, %19, %19 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %4, %12, %12 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %4, %20, %20 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %5, %13, %13 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %5, %21, %21 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %6, %14, %14 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %6, %22, %22 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %7, %15, %15 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %7, %23, %23 row_mirror row_mask:0xf bank_mask:0xc\n"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7])
      : "v"(in[0]), "v"(in[1]), "v"(in[2]), "v"(in[3]), "v"(in[4]), "v"(in[5]), "v"(in[6]), "v"(in[7]), "v"(in[8]), "v"(in[9]), "v"(in[10]), "v"(in[11]), "v"(in[12]), "v"(in[13]), "v"(in[14]), "v"(in[15]));
}
__device__ __forceinline__ void row16_halve4_mirror(const float* in, float* out) {
  asm("s_nop 4\n"
      "v_add_f32_dpp %0, %4, %4 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %0, %8, %8 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %1, %5, %5 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %1, %9, %9 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %2, %6, %6 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %2, %10, %10 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %3, %7, %7 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %3, %11, %11 row_mirror row_mask:0xf bank_mask:0xc\n"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
      : "v"(in[0]), "v"(in[1]), "v"(in[2]), "v"(in[3]), "v"(in[4]), "v"(in[5]), "v"(in[6]), "v"(in[7]));
}
__device__ __forceinline__ void row16_halve4_half_mirror(const float* in, float* out) {
  asm("s_nop 4\n"
      "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %0, %8, %8 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %1, %9, %9 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      "v_add_f32_dpp %2, %6, %6 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %2, %10, %10 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      "v_add_f32_dpp %3, %7, %7 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %3, %11, %11 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
      : "v"(in[0]), "v"(in[1]), "v"(in[2]), "v"(in[3]), "v"(in[4]), "v"(in[5]), "v"(in[6]), "v"(in[7]));
}
__device__ __forceinline__ void row16_halve2_half_mirror(const float* in, float* out) {
  asm("s_nop 4\n"
      "v_add_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      "v_add_f32_dpp %1, %3, %3 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      : "=&v"(out[0]), "=&v"(out[1])
      : "v"(in[0]), "v"(in[1]), "v"(in[2]), "v"(in[3]));
}
template <int N>
__device__ __forceinline__ float row16_scatter(const float (&v)[N]) {
  static_assert(N == 16 || N == 8, "16 or 8 values per lane");
  const int j = threadIdx.x & 15;
  float a[8], b[4], c[2];
  if constexpr (N == 16) {
    row16_halve8_mirror(v, a);       // row_mirror: lane 15 - j
    row16_halve4_half_mirror(a, b);  // row_half_mirror: lane 7 - j in its half
    row16_halve<2, 0x1b>(b, c, (j & 2) != 0);
  } else {
    row16_halve4_mirror(v, b);
    row16_halve2_half_mirror(b, c);
  }
  float d[1];
  row16_halve<1, (N == 16 ? 0xb1 : 0x1b)>(c, d, (j & (N == 16 ? 1 : 2)) != 0);
  if constexpr (N == 16) {
    return d[0];
  } else {  // quad_perm [1, 0, 3, 2]: the neighbour holds the same value
    return d[0] + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, d[0]), 0xb1, 0xf, 0xf, true));
  }
}

// Inclusive prefix sum over the wave's 64 lanes in lane order: shifts by 1,
// 2, 4 and 8 lanes inside each 16-lane row (a lane whose source lies before
// the row's start adds 0), then the totals of the rows below carried up by
// the broadcasts of lanes 15 (to rows 1 and 3) and 31 (to rows 2 and 3).
// Every step is a DPP add on the VALU; no LDS crossbar.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
  return x;
}

// The same prefix sum over integers.
__device__ __forceinline__ int wave_prefix_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
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
