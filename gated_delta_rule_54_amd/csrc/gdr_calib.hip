// Device ceilings (include/gdr_calib.h): a streaming copy and a loop of
// fp16 matrix-core products.  They measure the HBM rate and matrix-core rate
// this GPU sustains, the two roofs the gated delta rule kernels are set
// against.

#include <gdr_calib.h>

#include "gdr_internal.h"
#include "gdr_mma.h"

namespace gdr {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte units per thread

// Each thread moves kCopyUnroll 16-byte units, kCopyThreads * 16 bytes
// apart, so every load and store instruction of a wave covers 1 KB of
// consecutive bytes; all loads are issued before the first store.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCopyThreads) void calib_copy_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst, int64_t n16) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * kCopyThreads;
    if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * kCopyThreads;
    if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
  }
}

constexpr int kMfmaChains = 8;  // independent accumulators per wave

// Every wave runs `iters` rounds of kMfmaChains independent products; the
// operands come from the lane id so the compiler cannot fold them.
__global__ __launch_bounds__(256) void calib_mfma_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<_Float16>(0.001f * static_cast<float>((lane + i) & 7));
    b[i] = static_cast<_Float16>(0.002f * static_cast<float>((lane * 3 + i) & 7));
  }
  f32x4 c0 = zero4(), c1 = zero4(), c2 = zero4(), c3 = zero4(), c4 = zero4(), c5 = zero4(), c6 = zero4(),
        c7 = zero4();
  // Each product accumulates in place ("+v": the accumulator is both source
  // C and destination, in VGPRs), so the loop body is eight back-to-back
  // matrix-core instructions and the loop counter.
#define GDR_CALIB_MFMA(c) asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b))
  for (int it = 0; it < iters; ++it) {
    GDR_CALIB_MFMA(c0);
    GDR_CALIB_MFMA(c1);
    GDR_CALIB_MFMA(c2);
    GDR_CALIB_MFMA(c3);
    GDR_CALIB_MFMA(c4);
    GDR_CALIB_MFMA(c5);
    GDR_CALIB_MFMA(c6);
    GDR_CALIB_MFMA(c7);
  }
#undef GDR_CALIB_MFMA
  asm volatile("s_nop 15" ::: "memory");  // the last products' results settle before they are read
  const f32x4 s = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = (s[0] + s[1]) + (s[2] + s[3]);
}

}  // namespace
}  // namespace gdr

extern "C" {

gdr_status gdr_calib_copy(const void* src, void* dst, size_t bytes, void* hip_stream) {
  if (!src || !dst) return GDR_ERR_NULL_ARG;
  if (bytes == 0 || bytes % 16 != 0) return GDR_ERR_BAD_SHAPE;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return GDR_ERR_BAD_ALIGNMENT;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const int64_t per_wg = gdr::kCopyThreads * gdr::kCopyUnroll;
  const int64_t grid = (n16 + per_wg - 1) / per_wg;
  if (grid > 0x7fffffffLL) return GDR_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  {
    gdr::ProfScope ps("calib_copy", st);
    hipLaunchKernelGGL(gdr::calib_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(gdr::kCopyThreads), 0, st,
                       static_cast<const gdr::u32x4*>(src), static_cast<gdr::u32x4*>(dst), n16);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GDR_OK : gdr::record_hip_error(e);
}

gdr_status gdr_calib_mfma(float* out, int64_t workgroups, int64_t iters, double* flops, void* hip_stream) {
  if (!out || !flops) return GDR_ERR_NULL_ARG;
  if (workgroups <= 0 || iters <= 0) return GDR_ERR_BAD_SHAPE;
  if (workgroups > 0x7fffffffLL || iters > 0x7fffffffLL) return GDR_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return GDR_ERR_BAD_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  {
    gdr::ProfScope ps("calib_mfma", st);
    hipLaunchKernelGGL(gdr::calib_mfma_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(256), 0, st, out,
                       static_cast<int>(iters));
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return gdr::record_hip_error(e);
  *flops = static_cast<double>(workgroups) * 4.0 * static_cast<double>(iters) * gdr::kMfmaChains * 16384.0;
  return GDR_OK;
}

}  // extern "C"
