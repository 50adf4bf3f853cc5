// Chunked gated delta rule on the gfx950 matrix cores.
//
// Tokens are grouped in chunks of C.  Inside a chunk, with G_r the running
// sum of g over the chunk, gam_r = exp(G_r), lam_r = exp(G_C - G_r) (G_C the
// chunk's last G) and H0 the state entering the chunk, the recurrence unrolls
// to (the chunk-parallel form behind the "chunked" VJP kernel of the page
// "Adding VJP for gated delta net", ml-explore/mlx pull request 4565):
//
//   (I + A) U = RHS,  A_rs = beta_r exp(G_r - G_s) k_r.k_s  (s < r),
//                     RHS = diag(beta) (V - diag(gam) K H0)
//   O   = diag(gam) Q H0 + P U,  P_rs = exp(G_r - G_s) q_r.k_s (s <= r)
//   H_C = gam_C H0 + K^T diag(lam) U
//
// Only exponents of differences G_r - G_s with r >= s are formed, so no term
// can overflow for g <= 0.  With T = (I + A)^-1 the deltas are U = T RHS.
//
// Kernels:
//   chunk_prep_kernel  - per (b, chunk, v-head): A from K K^T (MFMA), T by
//                        forward substitution in fp32 (one lane per column).
//   chunk_fwd_kernel   - per (b, v-head, value slice): the sequential pass over
//                        chunks carrying H in MFMA accumulators; writes O and
//                        the final state, optionally every chunk's H0.
//   chunk_dh_kernel    - reverse pass carrying dH; writes dv and every
//                        chunk's incoming dH (VJP).
//   chunk_grad_kernel  - per (b, v-head, chunk): all remaining gradients of a
//                        chunk from its H0 and dH (VJP).
//
// Matrix-core operands: fp16 (F16Op, v_mfma_f32_16x16x32_f16) for bf16 io at
// Dk = 128, fp32 (F32Op, v_mfma_f32_16x16x4_f32) otherwise.  Accumulation is
// always fp32; the carried state and all scalar gate math are fp32.

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_mma.h"

namespace gdr {
namespace {

struct CArgs {
  const void *q, *k, *v, *dout;
  const float *g, *beta, *h0, *dht;
  void* o;
  float* ht;
  void* tmat;    // [B][Hv][NC][C][C] E   T = (I + A)^-1
  void* pmat;    // [B][Hv][NC][C][C] E   P (masked, gate-scaled q.k)
  void* hst;     // [B][Hv][NC][Dv][Dk] E   chunk-entry states H0 (transposed)
  void* dhst;    // [B][Hv][NC][Dv][Dk] E   gradient at each chunk's end
  void* dv;
  float* dh0;
  float *pdq, *pdk;   // [B][T][Hv][Dk] per-v-head dq_hat / dk_hat
  float *dg, *dbeta;  // [B][T][Hv]
  int64_t B, T;
  int Hk, Hv, NC, l2;
};

template <typename OP_, int C_, int DK_, int BV_, int BVG_>
struct Cfg {
  using OP = OP_;
  using E = typename OP::E;
  static constexpr int C = C_, DK = DK_, BV = BV_;
  static constexpr int BVG = BVG_;      // value-slice width of chunk_grad_kernel
  static constexpr int PAD = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD;  // pitch of [*][DK] arrays
  static constexpr int LDC = C + PAD;   // pitch of [*][C] arrays
  static constexpr int NW = 4;          // waves per workgroup
};

template <typename E> __device__ __forceinline__ E to_e(float x) { return static_cast<E>(x); }

// Load C rows (t0 .. t0+L-1) of q or k for head kh, normalise each row over
// Dk when l2 is set, and store them as E in dst[r * LDK + i]; rows >= L are 0.
template <typename CF, typename TI>
__device__ __forceinline__ void stage_rows(typename CF::E* dst, const TI* src, int64_t b, int64_t t0,
                                           int L, int kh, const CArgs& a) {
  constexpr int TPR = 256 / CF::C;        // threads per row
  constexpr int EPT = CF::DK / TPR;       // elements per thread
  const int tid = threadIdx.x;
  const int r = tid / TPR, part = tid % TPR;
  float x[EPT];
  float ss = 0.f;
  if (r < L) {
    const TI* p = src + ((b * a.T + t0 + r) * a.Hk + kh) * CF::DK + part * EPT;
    if constexpr (EPT % 4 == 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        float t4[4];
        ld4<TI>(p + e, t4);
        x[e] = t4[0]; x[e + 1] = t4[1]; x[e + 2] = t4[2]; x[e + 3] = t4[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) x[e] = ld1<TI>(p + e);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) x[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) ss += x[e] * x[e];
  if constexpr (TPR > 1) ss = xsum<1, TPR>(ss);
  const float rn = a.l2 ? rsqrtf(ss + kL2Eps) : 1.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) dst[r * CF::LDK + part * EPT + e] = to_e<typename CF::E>(x[e] * rn);
}

// Gate scalars of one chunk (wave 0 writes them; caller barriers):
// G_r, gam_r = exp(G_r), lam_r = exp(G_C - G_r), beta_r (0 beyond L), and
// sc[0] = gam_C.  Rows >= L have g = 0, so G_r = G_C there.
template <int C>
__device__ __forceinline__ void stage_gates(float* G, float* gam, float* lam, float* bet, float* sc,
                                            int64_t b, int64_t t0, int L, int hv, const CArgs& a) {
  const int lane = threadIdx.x;
  if (lane >= 64) return;
  const int64_t row = (b * a.T + t0 + lane) * a.Hv + hv;
  float x = lane < L ? a.g[row] : 0.f;
  const float bt = lane < L ? a.beta[row] : 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  const float gc = __shfl(x, L - 1, 64);
  if (lane < C) {
    G[lane] = x;
    gam[lane] = expf(x);
    lam[lane] = expf(gc - x);
    bet[lane] = bt;
  }
  if (lane == 0) sc[0] = expf(gc);
}

// Copy the chunk's T (C x C, E) from global into LDS with pitch LDC.
template <typename CF>
__device__ __forceinline__ void stage_t(typename CF::E* Ts, const typename CF::E* src) {
  constexpr int N = CF::C * CF::C;
  for (int e = threadIdx.x; e < N; e += 256) Ts[(e / CF::C) * CF::LDC + e % CF::C] = src[e];
}

// ---------------------------------------------------------------------------
// T = (I + A)^-1 and P for one (b, chunk, v-head); one wave.  Lane c computes
// column c of T by forward substitution: x_r = [r == c] - sum_{s<r} A_rs x_s.
// P_rs = exp(G_r - G_s) q_r.k_s for s <= r (0 above the diagonal).
template <typename CF, typename TI>
__global__ __launch_bounds__(64) void chunk_prep_kernel(CArgs a) {
  using E = typename CF::E;
  using OP = typename CF::OP;
  constexpr int C = CF::C, DK = CF::DK, LDK = CF::LDK;
  constexpr int LDA = C + 4;
  __shared__ __align__(16) E Ks[C * LDK];
  __shared__ __align__(16) E Qs[C * LDK];
  __shared__ __align__(16) float A[C * LDA];
  __shared__ float G[C], gam[C], lam[C], bet[C], sc[1];
  const int lane = threadIdx.x;
  const int c = blockIdx.x, hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (a.Hv / a.Hk);
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const int L = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
  const int64_t cbase = (b * a.Hv + hv) * a.NC + c;

  // q and k rows, one lane per row, normalised over Dk
  if (lane < C) {
    const int rc = lane < L ? lane : L - 1;
    for (int which = 0; which < 2; ++which) {
      const TI* p = static_cast<const TI*>(which ? a.q : a.k) + ((b * a.T + t0 + rc) * a.Hk + kh) * DK;
      E* dst = (which ? Qs : Ks) + lane * LDK;
      float x[DK];
#pragma unroll
      for (int i = 0; i < DK; i += 4) {
        float t4[4];
        ld4<TI>(p + i, t4);
        x[i] = t4[0]; x[i + 1] = t4[1]; x[i + 2] = t4[2]; x[i + 3] = t4[3];
      }
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < DK; ++i) ss += x[i] * x[i];
      const float rn = lane < L ? (a.l2 ? rsqrtf(ss + kL2Eps) : 1.f) : 0.f;
#pragma unroll
      for (int i = 0; i < DK; ++i) dst[i] = to_e<E>(x[i] * rn);
    }
  }
  stage_gates<C>(G, gam, lam, bet, sc, b, t0, L, hv, a);
  __syncthreads();
  E* pdst = static_cast<E*>(a.pmat) + cbase * static_cast<int64_t>(C * C);
  for (int tr = 0; tr < C / 16; ++tr)
    for (int tc = 0; tc < C / 16; ++tc) {
      if (tc <= tr) {
        const f32x4 s = mma_tile<OP, false, false>(zero4(), Ks, LDK, 16 * tr, Ks, LDK, 16 * tc, DK);
        const f32x4 qk = mma_tile<OP, false, false>(zero4(), Qs, LDK, 16 * tr, Ks, LDK, 16 * tc, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = acc_row(16 * tr, i), q = acc_col(16 * tc);
          const float e = q <= r ? expf(G[r] - G[q]) : 0.f;
          A[r * LDA + q] = q < r ? bet[r] * e * s[i] : 0.f;
          pdst[r * C + q] = to_e<E>(e * qk[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) pdst[acc_row(16 * tr, i) * C + acc_col(16 * tc)] = to_e<E>(0.f);
      }
    }
  __syncthreads();
  if (lane < C) {
    // four interleaved partial sums per row keep the FMA pipeline busy; the
    // order of additions is fixed (deterministic)
    float x[C];
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float acc[4] = {r == lane ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2) acc[s2 & 3] -= A[r * LDA + s2] * x[s2];
      x[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    E* dst = static_cast<E*>(a.tmat) + cbase * static_cast<int64_t>(C * C);
#pragma unroll
    for (int r = 0; r < C; ++r) dst[r * C + lane] = to_e<E>(x[r]);
  }
}

// ---------------------------------------------------------------------------
// Forward pass over chunks for one (b, v-head, value slice of BV columns).
template <typename CF, typename TI, typename TO, bool WRITE_O, bool STORE_H>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(CArgs a) {
  using E = typename CF::E;
  using OP = typename CF::OP;
  constexpr int C = CF::C, DK = CF::DK, BV = CF::BV, LDK = CF::LDK, LDC = CF::LDC;
  constexpr int NCB = (C / 16) * (BV / 16), QCB = (NCB + 3) / 4;   // C x BV tiles
  constexpr int NCC = (C / 16) * (C / 16), QCC = (NCC + 3) / 4;    // C x C tiles
  constexpr int NKB = (DK / 16) * (BV / 16), QKB = (NKB + 3) / 4;  // DK x BV tiles
  __shared__ __align__(16) E Ks[C * LDK];
  __shared__ __align__(16) E Qs[C * LDK];
  __shared__ __align__(16) E Hs[BV * LDK];   // Hs[j][i] = H[i][j]
  __shared__ __align__(16) E Ts[C * LDC];
  __shared__ __align__(16) E Ps[C * LDC];
  __shared__ __align__(16) E Rs[BV * LDC];   // Rs[j][r] = RHS[r][j]
  __shared__ __align__(16) E Us[BV * LDC];   // Us[j][r] = U[r][j]
  __shared__ __align__(16) E LUs[BV * LDC];  // LUs[j][r] = lam_r U[r][j]
  __shared__ float G[C], gam[C], lam[C], bet[C], sc[1];

  const int tid = threadIdx.x, w = tid >> 6;
  const int slice = blockIdx.x, hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (a.Hv / a.Hk);
  const int j0 = slice * BV;

  // state tiles owned by this wave: tile t = w + 4q -> rows 16*(t / (BV/16)), cols 16*(t % (BV/16))
  f32x4 h[QKB];
#pragma unroll
  for (int q = 0; q < QKB; ++q) {
    const int t = w + 4 * q;
    h[q] = zero4();
    if (t < NKB && a.h0) {
      const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        h[q][i] = a.h0[((b * a.Hv + hv) * DK + acc_row(m0, i)) * DK + j0 + acc_col(n0)];
    }
  }
  auto write_hs = [&]() {
#pragma unroll
    for (int q = 0; q < QKB; ++q) {
      const int t = w + 4 * q;
      if (t < NKB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) Hs[acc_col(n0) * LDK + acc_row(m0, i)] = to_e<E>(h[q][i]);
      }
    }
  };
  write_hs();
  __syncthreads();

  for (int c = 0; c < a.NC; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * C;
    const int L = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
    if constexpr (STORE_H) {
      E* dst = static_cast<E*>(a.hst) + (((b * a.Hv + hv) * a.NC + c) * DK + j0) * static_cast<int64_t>(DK);
      for (int e = tid; e < BV * DK; e += 256) dst[e] = Hs[(e / DK) * LDK + e % DK];
    }
    stage_rows<CF, TI>(Ks, static_cast<const TI*>(a.k), b, t0, L, kh, a);
    if constexpr (WRITE_O) stage_rows<CF, TI>(Qs, static_cast<const TI*>(a.q), b, t0, L, kh, a);
    stage_gates<C>(G, gam, lam, bet, sc, b, t0, L, hv, a);
    stage_t<CF>(Ts, static_cast<const E*>(a.tmat) + ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(C * C));
    __syncthreads();

    // Y = K H0 -> RHS; Z = Q H0 -> O accumulators; P
    f32x4 o[QCB];
#pragma unroll
    for (int q = 0; q < QCB; ++q) {
      const int t = w + 4 * q;
      if (t < NCB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        const f32x4 y = mma_tile<OP, false, false>(zero4(), Ks, LDK, m0, Hs, LDK, n0, DK);
        const int j = acc_col(n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = acc_row(m0, i);
          const float vv = r < L ? ld1<TI>(static_cast<const TI*>(a.v) + ((b * a.T + t0 + r) * a.Hv + hv) * DK + j0 + j) : 0.f;
          Rs[j * LDC + r] = to_e<E>(bet[r] * (vv - gam[r] * y[i]));
        }
        if constexpr (WRITE_O) {
          const f32x4 z = mma_tile<OP, false, false>(zero4(), Qs, LDK, m0, Hs, LDK, n0, DK);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[q][i] = gam[acc_row(m0, i)] * z[i];
        }
      }
    }
    if constexpr (WRITE_O) {
#pragma unroll
      for (int q = 0; q < QCC; ++q) {
        const int t = w + 4 * q;
        if (t < NCC) {
          const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
          const f32x4 p = mma_tile<OP, false, false>(zero4(), Qs, LDK, m0, Ks, LDK, n0, DK);
          const int s = acc_col(n0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = acc_row(m0, i);
            Ps[r * LDC + s] = to_e<E>(s <= r ? expf(G[r] - G[s]) * p[i] : 0.f);
          }
        }
      }
    }
    __syncthreads();

    // U = T RHS
#pragma unroll
    for (int q = 0; q < QCB; ++q) {
      const int t = w + 4 * q;
      if (t < NCB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        const f32x4 u = mma_tile<OP, false, false>(zero4(), Ts, LDC, m0, Rs, LDC, n0, C);
        const int j = acc_col(n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = acc_row(m0, i);
          Us[j * LDC + r] = to_e<E>(u[i]);
          LUs[j * LDC + r] = to_e<E>(lam[r] * u[i]);
        }
      }
    }
    __syncthreads();

    // O += P U; H = gam_C H + K^T (lam U)
    if constexpr (WRITE_O) {
#pragma unroll
      for (int q = 0; q < QCB; ++q) {
        const int t = w + 4 * q;
        if (t < NCB) {
          const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
          o[q] = mma_tile<OP, false, false>(o[q], Ps, LDC, m0, Us, LDC, n0, C);
          const int j = acc_col(n0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = acc_row(m0, i);
            if (r < L) st1<TO>(static_cast<TO*>(a.o) + ((b * a.T + t0 + r) * a.Hv + hv) * DK + j0 + j, o[q][i]);
          }
        }
      }
    }
    const float gc = sc[0];
#pragma unroll
    for (int q = 0; q < QKB; ++q) {
      const int t = w + 4 * q;
      if (t < NKB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        h[q] = h[q] * gc;
        h[q] = mma_tile<OP, true, false>(h[q], Ks, LDK, m0, LUs, LDC, n0, C);
      }
    }
    __syncthreads();  // everyone is done reading Hs / Ks of this chunk
    write_hs();
    __syncthreads();
  }
  if (a.ht) {
#pragma unroll
    for (int q = 0; q < QKB; ++q) {
      const int t = w + 4 * q;
      if (t < NKB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.ht[((b * a.Hv + hv) * DK + acc_row(m0, i)) * DK + j0 + acc_col(n0)] = h[q][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Reverse pass over chunks for one (b, v-head, value slice), carrying the
// gradient dH of the state in MFMA accumulators.  Per chunk (dH = gradient
// at the chunk's end):
//   dU   = P^T dO + diag(lam) K dH
//   dRHS = T^T dU,  dv = diag(beta) dRHS
//   dH  <- gam_C dH + Q^T diag(gam) dO - K^T diag(beta gam) dRHS
// Every chunk's incoming dH is stored (transposed, E) for chunk_grad_kernel.
template <typename CF, typename TI, typename TO>
__global__ __launch_bounds__(256) void chunk_dh_kernel(CArgs a) {
  using E = typename CF::E;
  using OP = typename CF::OP;
  constexpr int C = CF::C, DK = CF::DK, BV = CF::BV, LDK = CF::LDK, LDC = CF::LDC;
  constexpr int NCB = (C / 16) * (BV / 16), QCB = (NCB + 3) / 4;
  constexpr int NCC = (C / 16) * (C / 16), QCC = (NCC + 3) / 4;
  constexpr int NKB = (DK / 16) * (BV / 16), QKB = (NKB + 3) / 4;
  __shared__ __align__(16) E Ks[C * LDK];
  __shared__ __align__(16) E Qs[C * LDK];
  __shared__ __align__(16) E dHs[BV * LDK];   // dHs[j][i] = dH[i][j]
  __shared__ __align__(16) E Ts[C * LDC];
  __shared__ __align__(16) E Ps[C * LDC];
  __shared__ __align__(16) E dOT[BV * LDC];   // dO^T
  __shared__ __align__(16) E gdOT[BV * LDC];  // (diag(gam) dO)^T
  __shared__ __align__(16) E dUT[BV * LDC];   // dU^T
  __shared__ __align__(16) E bRT[BV * LDC];   // (-diag(beta gam) dRHS)^T
  __shared__ float G[C], gam[C], lam[C], bet[C], sc[1];

  const int tid = threadIdx.x, w = tid >> 6;
  const int slice = blockIdx.x, hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (a.Hv / a.Hk);
  const int j0 = slice * BV;

  f32x4 dh[QKB];
#pragma unroll
  for (int q = 0; q < QKB; ++q) {
    const int t = w + 4 * q;
    dh[q] = zero4();
    if (t < NKB && a.dht) {
      const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dh[q][i] = a.dht[((b * a.Hv + hv) * DK + acc_row(m0, i)) * DK + j0 + acc_col(n0)];
    }
  }
  auto write_dhs = [&]() {
#pragma unroll
    for (int q = 0; q < QKB; ++q) {
      const int t = w + 4 * q;
      if (t < NKB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) dHs[acc_col(n0) * LDK + acc_row(m0, i)] = to_e<E>(dh[q][i]);
      }
    }
  };
  write_dhs();
  __syncthreads();

  for (int c = a.NC - 1; c >= 0; --c) {
    const int64_t t0 = static_cast<int64_t>(c) * C;
    const int L = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
    {
      E* dst = static_cast<E*>(a.dhst) + (((b * a.Hv + hv) * a.NC + c) * DK + j0) * static_cast<int64_t>(DK);
      for (int e = tid; e < BV * DK; e += 256) dst[e] = dHs[(e / DK) * LDK + e % DK];
    }
    stage_rows<CF, TI>(Ks, static_cast<const TI*>(a.k), b, t0, L, kh, a);
    stage_rows<CF, TI>(Qs, static_cast<const TI*>(a.q), b, t0, L, kh, a);
    stage_gates<C>(G, gam, lam, bet, sc, b, t0, L, hv, a);
    stage_t<CF>(Ts, static_cast<const E*>(a.tmat) + ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(C * C));
    for (int e = tid; e < C * BV; e += 256) {
      const int r = e / BV, j = e % BV;
      const float x = r < L ? ld1<TI>(static_cast<const TI*>(a.dout) + ((b * a.T + t0 + r) * a.Hv + hv) * DK + j0 + j) : 0.f;
      dOT[j * LDC + r] = to_e<E>(x);
    }
    __syncthreads();

    for (int e = tid; e < C * BV; e += 256) {
      const int r = e % C, j = e / C;
      gdOT[j * LDC + r] = to_e<E>(gam[r] * static_cast<float>(dOT[j * LDC + r]));
    }
    f32x4 du[QCB];
#pragma unroll
    for (int q = 0; q < QCB; ++q) {
      const int t = w + 4 * q;
      if (t < NCB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        du[q] = mma_tile<OP, false, false>(zero4(), Ks, LDK, m0, dHs, LDK, n0, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) du[q][i] *= lam[acc_row(m0, i)];
      }
    }
#pragma unroll
    for (int q = 0; q < QCC; ++q) {
      const int t = w + 4 * q;
      if (t < NCC) {
        const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
        const f32x4 p = mma_tile<OP, false, false>(zero4(), Qs, LDK, m0, Ks, LDK, n0, DK);
        const int s = acc_col(n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = acc_row(m0, i);
          Ps[r * LDC + s] = to_e<E>(s <= r ? expf(G[r] - G[s]) * p[i] : 0.f);
        }
      }
    }
    __syncthreads();

    // dU += P^T dO
#pragma unroll
    for (int q = 0; q < QCB; ++q) {
      const int t = w + 4 * q;
      if (t < NCB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        du[q] = mma_tile<OP, true, false>(du[q], Ps, LDC, m0, dOT, LDC, n0, C);
        const int j = acc_col(n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) dUT[j * LDC + acc_row(m0, i)] = to_e<E>(du[q][i]);
      }
    }
    __syncthreads();

    // dRHS = T^T dU -> dv, bRT
#pragma unroll
    for (int q = 0; q < QCB; ++q) {
      const int t = w + 4 * q;
      if (t < NCB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        const f32x4 dr = mma_tile<OP, true, false>(zero4(), Ts, LDC, m0, dUT, LDC, n0, C);
        const int j = acc_col(n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = acc_row(m0, i);
          if (r < L) st1<TO>(static_cast<TO*>(a.dv) + ((b * a.T + t0 + r) * a.Hv + hv) * DK + j0 + j, bet[r] * dr[i]);
          bRT[j * LDC + r] = to_e<E>(-bet[r] * gam[r] * dr[i]);
        }
      }
    }
    __syncthreads();

    const float gc = sc[0];
#pragma unroll
    for (int q = 0; q < QKB; ++q) {
      const int t = w + 4 * q;
      if (t < NKB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        dh[q] = dh[q] * gc;
        dh[q] = mma_tile<OP, true, false>(dh[q], Qs, LDK, m0, gdOT, LDC, n0, C);
        dh[q] = mma_tile<OP, true, false>(dh[q], Ks, LDK, m0, bRT, LDC, n0, C);
      }
    }
    __syncthreads();
    write_dhs();
    __syncthreads();
  }
  if (a.dh0) {
#pragma unroll
    for (int q = 0; q < QKB; ++q) {
      const int t = w + 4 * q;
      if (t < NKB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.dh0[((b * a.Hv + hv) * DK + acc_row(m0, i)) * DK + j0 + acc_col(n0)] = dh[q][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// All gradients of one chunk except dv and dH, given its entry state H0 and
// the gradient dH at its end (both stored transposed, E).  The value dim is
// walked in slices of BVG columns; the value-dim reductions
//   X1 = dRHS H0^T,  X2 = dO H0^T,  X3 = U dH^T,  dP = dO U^T,  dT = dU RHS^T
// accumulate in registers.  Then
//   dA  = -T^T dT T^T on s < r;  dAm_rs = dA_rs beta_r exp(G_r - G_s)
//   dq  = diag(gam) X2 + dPm K,  dPm_rs = dP_rs exp(G_r - G_s) (s <= r)
//   dk  = -diag(beta gam) X1 + diag(lam) X3 + dPm^T Q + (dAm + dAm^T) K
//   dbeta_r = sum_j dRHS_rj (V - gam Y)_rj + sum_s dA_rs exp(G_r - G_s) k_r.k_s
//   dG_r collects every exp(G) factor: gam in RHS and in O, P, A, lam, gam_C
//   dg   = running sum of dG from the chunk's end backwards.
// dq / dk are written per v-head; the epilogue sums the GQA group and
// applies the L2-norm VJP.
template <typename CF, typename TI>
__global__ __launch_bounds__(256) void chunk_grad_kernel(CArgs a) {
  using E = typename CF::E;
  using OP = typename CF::OP;
  constexpr int C = CF::C, DK = CF::DK, BV = CF::BVG, LDK = CF::LDK, LDC = CF::LDC;
  constexpr int NCB = (C / 16) * (BV / 16), QCB = (NCB + 3) / 4;
  constexpr int NCC = (C / 16) * (C / 16), QCC = (NCC + 3) / 4;
  constexpr int NCK = (C / 16) * (DK / 16), QCK = (NCK + 3) / 4;
  // pool: value-slice phase {Hsub, dHsub, Rs, UT, dOT, dUT, dRT};
  //       C x C phase {X = dT -> M1 -> dA, Y = dPm}
  constexpr int SUB = 2 * BV * LDK + 5 * BV * LDC;
  constexpr int CC = 2 * C * LDC;
  constexpr int POOL = SUB > CC ? SUB : CC;
  __shared__ __align__(16) E Ks[C * LDK];
  __shared__ __align__(16) E Qs[C * LDK];
  __shared__ __align__(16) E Ts[C * LDC];
  __shared__ __align__(16) E Ps[C * LDC];
  __shared__ __align__(16) E pool[POOL];
  __shared__ float G[C], gam[C], lam[C], bet[C], sc[1];
  __shared__ float sG[4][C], sGc[4][C], sB[4][C], red[2][4];
  E* Hsub = pool;                   // Hsub[j][i]  = H0[i][j0 + j]
  E* dHsub = Hsub + BV * LDK;       // dHsub[j][i] = dH[i][j0 + j]
  E* Rs = dHsub + BV * LDK;         // RHS^T
  E* UT = Rs + BV * LDC;            // U^T
  E* dOT = UT + BV * LDC;           // dO^T
  E* dUT = dOT + BV * LDC;          // dU^T
  E* dRT = dUT + BV * LDC;          // dRHS^T
  E* Xs = pool;                     // C x C, pitch LDC
  E* Ys = pool + C * LDC;           // C x C, pitch LDC

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c = blockIdx.x, hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (a.Hv / a.Hk);
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const int L = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
  const int64_t cbase = (b * a.Hv + hv) * a.NC + c;

  for (int e = tid; e < 4 * C; e += 256) {
    sG[e / C][e % C] = 0.f;
    sGc[e / C][e % C] = 0.f;
    sB[e / C][e % C] = 0.f;
  }
  stage_rows<CF, TI>(Ks, static_cast<const TI*>(a.k), b, t0, L, kh, a);
  stage_rows<CF, TI>(Qs, static_cast<const TI*>(a.q), b, t0, L, kh, a);
  stage_gates<C>(G, gam, lam, bet, sc, b, t0, L, hv, a);
  stage_t<CF>(Ts, static_cast<const E*>(a.tmat) + cbase * static_cast<int64_t>(C * C));
  __syncthreads();
#pragma unroll
  for (int q = 0; q < QCC; ++q) {
    const int t = w + 4 * q;
    if (t < NCC) {
      const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
      const f32x4 p = mma_tile<OP, false, false>(zero4(), Qs, LDK, m0, Ks, LDK, n0, DK);
      const int s2 = acc_col(n0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = acc_row(m0, i);
        Ps[r * LDC + s2] = to_e<E>(s2 <= r ? expf(G[r] - G[s2]) * p[i] : 0.f);
      }
    }
  }

  f32x4 x1[QCK], x2[QCK], x3[QCK], dP[QCC], dT[QCC];
#pragma unroll
  for (int q = 0; q < QCK; ++q) x1[q] = x2[q] = x3[q] = zero4();
#pragma unroll
  for (int q = 0; q < QCC; ++q) dP[q] = dT[q] = zero4();
  float hh = 0.f;  // this thread's part of <dH, H0>

  for (int j0 = 0; j0 < DK; j0 += BV) {
    const E* hsrc = static_cast<const E*>(a.hst) + (cbase * DK + j0) * static_cast<int64_t>(DK);
    const E* dhsrc = static_cast<const E*>(a.dhst) + (cbase * DK + j0) * static_cast<int64_t>(DK);
    for (int e = tid; e < BV * DK; e += 256) {
      const E h0e = hsrc[e], dh0e = dhsrc[e];
      Hsub[(e / DK) * LDK + e % DK] = h0e;
      dHsub[(e / DK) * LDK + e % DK] = dh0e;
      hh += static_cast<float>(h0e) * static_cast<float>(dh0e);
    }
    for (int e = tid; e < C * BV; e += 256) {
      const int r = e / BV, j = e % BV;
      const float x = r < L ? ld1<TI>(static_cast<const TI*>(a.dout) + ((b * a.T + t0 + r) * a.Hv + hv) * DK + j0 + j) : 0.f;
      dOT[j * LDC + r] = to_e<E>(x);
    }
    __syncthreads();

    // Y = K H0 -> RHS = diag(beta)(V - diag(gam) Y);  dU starts as lam K dH
    f32x4 vmy[QCB], yy[QCB], du[QCB];
#pragma unroll
    for (int q = 0; q < QCB; ++q) {
      const int t = w + 4 * q;
      if (t < NCB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        yy[q] = mma_tile<OP, false, false>(zero4(), Ks, LDK, m0, Hsub, LDK, n0, DK);
        du[q] = mma_tile<OP, false, false>(zero4(), Ks, LDK, m0, dHsub, LDK, n0, DK);
        const int j = acc_col(n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = acc_row(m0, i);
          const float vv = r < L ? ld1<TI>(static_cast<const TI*>(a.v) + ((b * a.T + t0 + r) * a.Hv + hv) * DK + j0 + j) : 0.f;
          vmy[q][i] = vv - gam[r] * yy[q][i];
          Rs[j * LDC + r] = to_e<E>(bet[r] * vmy[q][i]);
          du[q][i] *= lam[r];
        }
      }
    }
    __syncthreads();
    // U = T RHS;  dU += P^T dO
#pragma unroll
    for (int q = 0; q < QCB; ++q) {
      const int t = w + 4 * q;
      if (t < NCB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        const f32x4 u = mma_tile<OP, false, false>(zero4(), Ts, LDC, m0, Rs, LDC, n0, C);
        du[q] = mma_tile<OP, true, false>(du[q], Ps, LDC, m0, dOT, LDC, n0, C);
        const int j = acc_col(n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          UT[j * LDC + acc_row(m0, i)] = to_e<E>(u[i]);
          dUT[j * LDC + acc_row(m0, i)] = to_e<E>(du[q][i]);
        }
      }
    }
    __syncthreads();
    // dRHS = T^T dU; row sums for dbeta and dG
#pragma unroll
    for (int q = 0; q < QCB; ++q) {
      const int t = w + 4 * q;
      if (t < NCB) {
        const int m0 = 16 * (t / (BV / 16)), n0 = 16 * (t % (BV / 16));
        const f32x4 dr = mma_tile<OP, true, false>(zero4(), Ts, LDC, m0, dUT, LDC, n0, C);
        const int j = acc_col(n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = acc_row(m0, i);
          dRT[j * LDC + r] = to_e<E>(dr[i]);
          const float sb = xsum<1, 16>(dr[i] * vmy[q][i]);
          const float sy = xsum<1, 16>(dr[i] * yy[q][i]);
          if ((lane & 15) == 0) {
            sB[w][r] += sb;
            sG[w][r] -= bet[r] * gam[r] * sy;
          }
        }
      }
    }
    __syncthreads();
    // value-dim reductions
#pragma unroll
    for (int q = 0; q < QCK; ++q) {
      const int t = w + 4 * q;
      if (t < NCK) {
        const int m0 = 16 * (t / (DK / 16)), n0 = 16 * (t % (DK / 16));
        x1[q] = mma_tile<OP, true, true>(x1[q], dRT, LDC, m0, Hsub, LDK, n0, BV);
        x2[q] = mma_tile<OP, true, true>(x2[q], dOT, LDC, m0, Hsub, LDK, n0, BV);
        x3[q] = mma_tile<OP, true, true>(x3[q], UT, LDC, m0, dHsub, LDK, n0, BV);
      }
    }
#pragma unroll
    for (int q = 0; q < QCC; ++q) {
      const int t = w + 4 * q;
      if (t < NCC) {
        const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
        dP[q] = mma_tile<OP, true, true>(dP[q], dOT, LDC, m0, UT, LDC, n0, BV);
        dT[q] = mma_tile<OP, true, true>(dT[q], dUT, LDC, m0, Rs, LDC, n0, BV);
      }
    }
    __syncthreads();
  }

  // ---- C x C stage.  Xs <- dT, Ys <- dPm; P terms of dG.
#pragma unroll
  for (int q = 0; q < QCC; ++q) {
    const int t = w + 4 * q;
    if (t < NCC) {
      const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
      const f32x4 qk = mma_tile<OP, false, false>(zero4(), Qs, LDK, m0, Ks, LDK, n0, DK);
      const int s2 = acc_col(n0);
      float col = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = acc_row(m0, i);
        const float m = s2 <= r ? expf(G[r] - G[s2]) : 0.f;
        Xs[r * LDC + s2] = to_e<E>(dT[q][i]);
        Ys[r * LDC + s2] = to_e<E>(dP[q][i] * m);
        const float dpp = dP[q][i] * m * qk[i];     // dP_rs P_rs
        const float rs = xsum<1, 16>(dpp);
        if ((lane & 15) == 0) sG[w][r] += rs;
        col += dpp;
      }
      col = xsum<16, 64>(col);
      if (lane < 16) sGc[w][s2] += col;
    }
  }
  __syncthreads();
  // M1 = T^T dT (kept in registers across the barrier, then written over Xs)
  f32x4 m1[QCC];
#pragma unroll
  for (int q = 0; q < QCC; ++q) {
    const int t = w + 4 * q;
    if (t < NCC) {
      const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
      m1[q] = mma_tile<OP, true, true>(zero4(), Ts, LDC, m0, Xs, LDC, n0, C);
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < QCC; ++q) {
    const int t = w + 4 * q;
    if (t < NCC) {
      const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
#pragma unroll
      for (int i = 0; i < 4; ++i) Xs[acc_row(m0, i) * LDC + acc_col(n0)] = to_e<E>(m1[q][i]);
    }
  }
  __syncthreads();
  // dA = -M1 T^T on s < r; A terms of dbeta and dG; dAm (symmetrised) over Xs
  f32x4 dam[QCC];
#pragma unroll
  for (int q = 0; q < QCC; ++q) {
    const int t = w + 4 * q;
    if (t < NCC) {
      const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
      const f32x4 da = mma_tile<OP, false, false>(zero4(), Xs, LDC, m0, Ts, LDC, n0, C);
      const f32x4 kk = mma_tile<OP, false, false>(zero4(), Ks, LDK, m0, Ks, LDK, n0, DK);
      const int s2 = acc_col(n0);
      float col = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = acc_row(m0, i);
        const float e = s2 < r ? expf(G[r] - G[s2]) : 0.f;
        const float dav = -da[i] * e;                  // dA_rs exp(G_r - G_s)
        dam[q][i] = dav * bet[r];
        const float rb = xsum<1, 16>(dav * kk[i]);     // dbeta_r
        const float ag = dam[q][i] * kk[i];            // dA_rs A_rs
        const float rg = xsum<1, 16>(ag);
        if ((lane & 15) == 0) {
          sB[w][r] += rb;
          sG[w][r] += rg;
        }
        col += ag;
      }
      col = xsum<16, 64>(col);
      if (lane < 16) sGc[w][s2] += col;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < QCC; ++q) {
    const int t = w + 4 * q;
    if (t < NCC) {
      const int m0 = 16 * (t / (C / 16)), n0 = 16 * (t % (C / 16));
      const int s2 = acc_col(n0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = acc_row(m0, i);
        if (s2 < r) {
          Xs[r * LDC + s2] = to_e<E>(dam[q][i]);
          Xs[s2 * LDC + r] = to_e<E>(dam[q][i]);
        } else if (s2 == r) {
          Xs[r * LDC + r] = to_e<E>(0.f);
        }
      }
    }
  }
  __syncthreads();

  // ---- dq, dk (per v-head) and the X2 / X3 terms of dG
  float gcx = 0.f;  // this lane's part of sum_r lam_r k_r . X3_r (goes to dG_C)
  float* pq = a.pdq;
  float* pk = a.pdk;
#pragma unroll
  for (int q = 0; q < QCK; ++q) {
    const int t = w + 4 * q;
    if (t < NCK) {
      const int m0 = 16 * (t / (DK / 16)), n0 = 16 * (t % (DK / 16));
      f32x4 dqv = mma_tile<OP, false, true>(zero4(), Ys, LDC, m0, Ks, LDK, n0, C);
      f32x4 dkv = mma_tile<OP, true, true>(zero4(), Ys, LDC, m0, Qs, LDK, n0, C);
      dkv = mma_tile<OP, false, true>(dkv, Xs, LDC, m0, Ks, LDK, n0, C);
      const int i2 = acc_col(n0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = acc_row(m0, i);
        const float qn = static_cast<float>(Qs[r * LDK + i2]);
        const float kn = static_cast<float>(Ks[r * LDK + i2]);
        const float rg = xsum<1, 16>(gam[r] * qn * x2[q][i] - lam[r] * kn * x3[q][i]);
        gcx += lam[r] * kn * x3[q][i];
        if ((lane & 15) == 0) sG[w][r] += rg;
        dqv[i] += gam[r] * x2[q][i];
        dkv[i] += lam[r] * x3[q][i] - bet[r] * gam[r] * x1[q][i];
        if (r < L) {
          const int64_t o = ((b * a.T + t0 + r) * a.Hv + hv) * DK + i2;
          pq[o] = dqv[i];
          pk[o] = dkv[i];
        }
      }
    }
  }
  hh = xsum<1, 64>(hh);
  gcx = xsum<1, 64>(gcx);
  if (lane == 0) {
    red[0][w] = hh;
    red[1][w] = gcx;
  }
  __syncthreads();

  // ---- dG -> dg (reverse running sum over valid rows), dbeta
  if (w == 0) {
    const int r = lane;
    float dG = 0.f, dB = 0.f;
    if (r < C) {
      dG = sG[0][r] + sG[1][r] + sG[2][r] + sG[3][r] - (sGc[0][r] + sGc[1][r] + sGc[2][r] + sGc[3][r]);
      dB = sB[0][r] + sB[1][r] + sB[2][r] + sB[3][r];
    }
    if (r == L - 1) {
      const float hsum = red[0][0] + red[0][1] + red[0][2] + red[0][3];
      const float xsum3 = red[1][0] + red[1][1] + red[1][2] + red[1][3];
      dG += sc[0] * hsum + xsum3;
    }
    if (r >= L) dG = 0.f;
    // suffix sum: dg_t = sum_{r >= t} dG_r
    float x = dG;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      if (lane + off < 64) x += y;
    }
    if (r < L) {
      const int64_t row = (b * a.T + t0 + r) * a.Hv + hv;
      a.dg[row] = x;
      a.dbeta[row] = dB;
    }
  }
}

// ---------------------------------------------------------------------------
// fp16-operand chains for bf16 io, Dk = Dv = 128, value slices of 64 columns,
// C in {32, 64}.  Wave w owns the 16-column strip j0 + 16w .. j0 + 16w + 15
// of every C x 64 and 128 x 64 tile of its workgroup, so a C x 16 product
// held in MFMA accumulators can be fed straight back as the operand of the
// next product that contracts over the chunk rows ("chained" operand): the
// k index of such a product is relabelled so that lane group g supplies rows
// {4g..4g+3, 16+4g..16+4g+3} of each 32-row block, exactly the rows its
// accumulators hold; the LDS-side operand is read with the same relabelling
// (two 8-byte reads per fragment).  The next chunk's inputs are prefetched
// into registers while the current chunk computes; all loads are
// branch-free (rows past the sequence end are clamped, then zeroed).
namespace f16c {

constexpr int DK = 128, BV = 64, LDK = DK + 8;
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ f16x8 ld8(const _Float16* p) { return *reinterpret_cast<const f16x8*>(p); }

// A fragment of A[m][k] (row-major, k contiguous) for the relabelled 32-row
// block kb: elements 0..3 <- k = 32kb + 4g + 0..3, 4..7 <- 32kb + 16 + 4g + 0..3.
__device__ __forceinline__ f16x8 perm_frag(const _Float16* A, int ld, int m, int kb) {
  const int g = lane_id() >> 4;
  const f16x4 lo = *reinterpret_cast<const f16x4*>(A + m * ld + 32 * kb + 4 * g);
  const f16x4 hi = *reinterpret_cast<const f16x4*>(A + m * ld + 32 * kb + 16 + 4 * g);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Chained B fragments of a C x 16 strip x[tr][e] (fp32 accumulators).
template <int NT>
__device__ __forceinline__ void chain_frags(f16x8 (&bf)[NT / 2], const f32x4 (&x)[NT]) {
#pragma unroll
  for (int kb = 0; kb < NT / 2; ++kb)
    bf[kb] = f16x8{static_cast<_Float16>(x[2 * kb][0]), static_cast<_Float16>(x[2 * kb][1]),
                   static_cast<_Float16>(x[2 * kb][2]), static_cast<_Float16>(x[2 * kb][3]),
                   static_cast<_Float16>(x[2 * kb + 1][0]), static_cast<_Float16>(x[2 * kb + 1][1]),
                   static_cast<_Float16>(x[2 * kb + 1][2]), static_cast<_Float16>(x[2 * kb + 1][3])};
}

// acc[t] += A[16t : 16t+16, 0:C] * X for t < NO (X chained as bf).
template <int NO, int NT>
__device__ __forceinline__ void mma_chain_rows(f32x4 (&acc)[NO], const _Float16* A, int ld, const f16x8 (&bf)[NT / 2]) {
  const int m = lane_id() & 15;
#pragma unroll
  for (int kb = 0; kb < NT / 2; ++kb) {
    f16x8 af[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t) af[t] = perm_frag(A, ld, 16 * t + m, kb);
#pragma unroll
    for (int t = 0; t < NO; ++t) acc[t] = F16Op::mma(af[t], bf[kb], acc[t]);
  }
}

// acc[t] += A[16t : 16t+16, 0:K] * B where B^T rows n0..n0+15 are read from
// Bt (k contiguous); K a multiple of 32.  k-outer so the NO accumulators are
// independent and the B fragment is shared.
template <int NO, int K>
__device__ __forceinline__ void mma_rows(f32x4 (&acc)[NO], const _Float16* A, int lda, const _Float16* Bt, int ldb,
                                         int n0) {
  const int r = lane_id() & 15, kl = (lane_id() >> 4) * 8;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const f16x8 bfr = ld8(Bt + (n0 + r) * ldb + k0 + kl);
    f16x8 af[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t) af[t] = ld8(A + (16 * t + r) * lda + k0 + kl);
#pragma unroll
    for (int t = 0; t < NO; ++t) acc[t] = F16Op::mma(af[t], bfr, acc[t]);
  }
}

// One C x C row block: acc[t] = Q[m0:m0+16] . K[16t : 16t+16]^T over DK.
template <int NT>
__device__ __forceinline__ void mma_qk_row(f32x4 (&acc)[NT], const _Float16* Qs, const _Float16* Ks, int m0) {
  const int r = lane_id() & 15, kl = (lane_id() >> 4) * 8;
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = zero4();
#pragma unroll
  for (int k0 = 0; k0 < DK; k0 += 32) {
    const f16x8 af = ld8(Qs + (m0 + r) * LDK + k0 + kl);
    f16x8 bfr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) bfr[t] = ld8(Ks + (16 * t + r) * LDK + k0 + kl);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = F16Op::mma(af, bfr[t], acc[t]);
  }
}

// Raw inputs of one chunk held in registers between the prefetch and the
// LDS staging.  K/Q rows: thread -> (row tid / TPR, EPT elements).
template <int C, bool WANT_Q>
struct Pre {
  static constexpr int TPR = 256 / C, EPT = DK / TPR, NV = EPT / 8;
  static constexpr int NTU = (C * C / 8 + 255) / 256;   // 16-byte units of T per thread
  uint4 k[NV], q[WANT_Q ? NV : 1];
  uint4 t[NTU], pm[NTU];
  float gv, bv;
  uint32_t v[C / 16][2];  // this lane's strip rows of v (forward) or dO (dh), bf16 pairs
};

__device__ __forceinline__ uint4 sel4(bool ok, uint4 x) {
  return ok ? x : uint4{0u, 0u, 0u, 0u};
}

template <int C, bool WANT_Q>
__device__ __forceinline__ void prefetch(Pre<C, WANT_Q>& p, const CArgs& a, int64_t b, int c, int kh, int hv,
                                         int jcol, const void* vsrc) {
  using P = Pre<C, WANT_Q>;
  const int tid = threadIdx.x, g = lane_id() >> 4;
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const int L = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
  const int r = tid / P::TPR, part = tid % P::TPR;
  const int rc = r < L ? r : L - 1;
  const bf16_t* kb = static_cast<const bf16_t*>(a.k) + ((b * a.T + t0) * a.Hk + kh) * DK;
  const bf16_t* qb = static_cast<const bf16_t*>(a.q) + ((b * a.T + t0) * a.Hk + kh) * DK;
  const int off = rc * a.Hk * DK + part * P::EPT;
#pragma unroll
  for (int u = 0; u < P::NV; ++u) {
    p.k[u] = sel4(r < L, *reinterpret_cast<const uint4*>(kb + off + 8 * u));
    if constexpr (WANT_Q) p.q[u] = sel4(r < L, *reinterpret_cast<const uint4*>(qb + off + 8 * u));
  }
  const uint4* tsrc = reinterpret_cast<const uint4*>(static_cast<const _Float16*>(a.tmat) +
                                                     ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(C * C));
  const uint4* psrc = reinterpret_cast<const uint4*>(static_cast<const _Float16*>(a.pmat) +
                                                     ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(C * C));
#pragma unroll
  for (int u = 0; u < P::NTU; ++u) {
    const int e = tid + 256 * u;
    if (P::NTU * 256 == C * C / 8 || e < C * C / 8) {
      p.t[u] = tsrc[e];
      p.pm[u] = psrc[e];
    }
  }
  if (tid < 64) {
    const int rr = tid < L ? tid : L - 1;
    const int64_t row = (b * a.T + t0 + rr) * a.Hv + hv;
    const float gv = a.g[row], bv = a.beta[row];
    p.gv = tid < L ? gv : 0.f;
    p.bv = tid < L ? bv : 0.f;
  }
  const bf16_t* vb = static_cast<const bf16_t*>(vsrc) + ((b * a.T + t0) * a.Hv + hv) * DK + jcol;
#pragma unroll
  for (int tr = 0; tr < C / 16; ++tr)
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int r0 = 16 * tr + 4 * g + 2 * e2, r1 = r0 + 1;
      const uint32_t x0 = vb[(r0 < L ? r0 : L - 1) * a.Hv * DK];
      const uint32_t x1 = vb[(r1 < L ? r1 : L - 1) * a.Hv * DK];
      p.v[tr][e2] = (r0 < L ? x0 : 0u) | ((r1 < L ? x1 : 0u) << 16);
    }
}

__device__ __forceinline__ void unpack_strip(float (&x)[4], const uint32_t (&w)[2]) {
  x[0] = __uint_as_float(w[0] << 16);
  x[1] = __uint_as_float(w[0] & 0xffff0000u);
  x[2] = __uint_as_float(w[1] << 16);
  x[3] = __uint_as_float(w[1] & 0xffff0000u);
}

__device__ __forceinline__ void unpack8(const uint4& u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Normalise the prefetched rows and write them as fp16: row-major
// dst[r][i] (16-byte stores) and, if TRANS, transposed dstT[i][r].
template <int C, int NV, bool TRANS, bool ROW = true>
__device__ __forceinline__ void stage_rows_pre(_Float16* dst, _Float16* dstT, const uint4 (&raw)[NV], int l2) {
  constexpr int TPR = 256 / C, EPT = DK / TPR, LDC = C + 8;
  const int tid = threadIdx.x, r = tid / TPR, part = tid % TPR;
  float x[NV][8];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    unpack8(raw[u], x[u]);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[u][i] * x[u][i];
  }
  ss = xsum<1, TPR>(ss);
  const float rn = l2 ? rsqrtf(ss + kL2Eps) : 1.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(x[u][i] * rn);
    if constexpr (ROW) *reinterpret_cast<f16x8*>(dst + r * LDK + part * EPT + 8 * u) = h;
    if constexpr (TRANS) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dstT[(part * EPT + 8 * u + i) * LDC + r] = h[i];
    }
  }
}

// T (row-major from the prep kernel) -> Ts[r][s] or, transposed, Ts[s][r].
template <int C, int NTU, bool TRANS>
__device__ __forceinline__ void stage_t_pre(_Float16* Ts, const uint4 (&raw)[NTU]) {
  constexpr int LDC = C + 8;
#pragma unroll
  for (int u = 0; u < NTU; ++u) {
    const int e = threadIdx.x + 256 * u;
    if (e < C * C / 8) {
      const int r = (8 * e) / C, s = (8 * e) % C;
      if constexpr (!TRANS) {
        *reinterpret_cast<uint4*>(Ts + r * LDC + s) = raw[u];
      } else {
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Ts[(s + 2 * i) * LDC + r] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xffffu));
          Ts[(s + 2 * i + 1) * LDC + r] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16));
        }
      }
    }
  }
}

// Gate scalars from the prefetched g, beta (wave 0; caller barriers):
// G2 = log2(e) * running sum of g (for exp2 of differences), gam, lam, beta,
// sc[0] = gam_C.
template <int C>
__device__ __forceinline__ void stage_gates_pre(float* G2, float* gam, float* lam, float* bet, float* sc, float gv,
                                                float bv, int L) {
  const int lane = threadIdx.x;
  if (lane >= 64) return;
  float x = gv;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  const float gc = __shfl(x, L - 1, 64);
  if (lane < C) {
    G2[lane] = x * kLog2e;
    gam[lane] = expf(x);
    lam[lane] = expf(gc - x);
    bet[lane] = bv;
  }
  if (lane == 0) sc[0] = expf(gc);
}

// P row block m0: exp(G_r - G_s) q_r.k_s for s <= r, else 0.
__device__ __forceinline__ float pmask(const float* G2, int r, int s, float qk) {
  return s <= r ? exp2f(G2[r] - G2[s]) * qk : 0.f;
}

}  // namespace f16c

// Forward chain, fp16 operands (see f16c).  Per chunk and wave:
// Y = K H0 and Z = Q H0 (16 MFMA each), a 16-row block of P (16), U = T RHS
// (8, chained), O += P U (8, chained), H = gam_C H + K^T (lam U) (16, chained).
template <int C, typename TO, bool WRITE_O, bool STORE_H>
__global__ __launch_bounds__(256) void chunk_fwd_f16_kernel(CArgs a) {
  using namespace f16c;
  constexpr int LDC = C + 8, NT = C / 16, NTK = DK / 16;
  __shared__ __align__(16) _Float16 Ks[C * LDK];
  __shared__ __align__(16) _Float16 KsT[DK * LDC];
  __shared__ __align__(16) _Float16 Qs[WRITE_O ? C * LDK : 8];
  __shared__ __align__(16) _Float16 Ts[C * LDC];
  __shared__ __align__(16) _Float16 Ps[WRITE_O ? C * LDC : 8];
  __shared__ __align__(16) _Float16 Hs[BV * LDK];   // Hs[j][i] = H[i][j]
  __shared__ float G2[C], gam[C], lam[C], bet[C], sc[1];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (a.Hv / a.Hk);
  const int j0 = blockIdx.x * BV;
  const int jw = 16 * w + c16;  // this lane's column in the slice
  const int64_t hbase = (b * a.Hv + hv) * DK * DK + j0 + jw;

  f32x4 h[NTK];
#pragma unroll
  for (int ti = 0; ti < NTK; ++ti) {
    h[ti] = zero4();
    if (a.h0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) h[ti][e] = a.h0[hbase + (16 * ti + 4 * g + e) * DK];
    }
  }
  auto write_hs = [&]() {
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti) {
      const f16x4 v4{static_cast<_Float16>(h[ti][0]), static_cast<_Float16>(h[ti][1]),
                     static_cast<_Float16>(h[ti][2]), static_cast<_Float16>(h[ti][3])};
      *reinterpret_cast<f16x4*>(Hs + jw * LDK + 16 * ti + 4 * g) = v4;
    }
  };
  Pre<C, WRITE_O> pre;
  uint32_t vcur[NT][2];
  int Lcur = 0;
  auto stage = [&](int c) {
    const int64_t t0 = static_cast<int64_t>(c) * C;
    const int L = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
    stage_rows_pre<C, Pre<C, WRITE_O>::NV, true>(Ks, KsT, pre.k, a.l2);
    if constexpr (WRITE_O) stage_rows_pre<C, Pre<C, WRITE_O>::NV, false>(Qs, nullptr, pre.q, a.l2);
    stage_t_pre<C, Pre<C, WRITE_O>::NTU, false>(Ts, pre.t);
    if constexpr (WRITE_O) stage_t_pre<C, Pre<C, WRITE_O>::NTU, false>(Ps, pre.pm);
    stage_gates_pre<C>(G2, gam, lam, bet, sc, pre.gv, pre.bv, L);
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) { vcur[tr][0] = pre.v[tr][0]; vcur[tr][1] = pre.v[tr][1]; }
    Lcur = L;
  };
  prefetch<C, WRITE_O>(pre, a, b, 0, kh, hv, j0 + jw, a.v);
  stage(0);
  write_hs();
  __syncthreads();

  for (int c = 0; c < a.NC; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * C;
    const int L = Lcur;
    if constexpr (STORE_H) {  // chunk entry state, natural [Dk][Dv] layout
      _Float16* dst = static_cast<_Float16*>(a.hst) + ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(DK * DK) + j0 + jw;
#pragma unroll
      for (int ti = 0; ti < NTK; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(16 * ti + 4 * g + e) * DK] = static_cast<_Float16>(h[ti][e]);
    }
    if (c + 1 < a.NC) prefetch<C, WRITE_O>(pre, a, b, c + 1, kh, hv, j0 + jw, a.v);

    // Y = K H0 -> RHS;  Z = Q H0 -> O
    f32x4 y[NT], o[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) y[tr] = zero4();
    mma_rows<NT, DK>(y, Ks, LDK, Hs, LDK, 16 * w);
    if constexpr (WRITE_O) {
#pragma unroll
      for (int tr = 0; tr < NT; ++tr) o[tr] = zero4();
      mma_rows<NT, DK>(o, Qs, LDK, Hs, LDK, 16 * w);
    }
    f32x4 rhs[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      float vv[4];
      unpack_strip(vv, vcur[tr]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * tr + 4 * g + e;
        rhs[tr][e] = bet[r] * (vv[e] - gam[r] * y[tr][e]);
        if constexpr (WRITE_O) o[tr][e] *= gam[r];
      }
    }
    // U = T RHS
    f16x8 bf[NT / 2];
    chain_frags<NT>(bf, rhs);
    f32x4 u[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) u[tr] = zero4();
    mma_chain_rows<NT, NT>(u, Ts, LDC, bf);

    if constexpr (WRITE_O) {
      chain_frags<NT>(bf, u);
      mma_chain_rows<NT, NT>(o, Ps, LDC, bf);
      TO* ob = static_cast<TO*>(a.o) + ((b * a.T + t0) * a.Hv + hv) * DK + j0 + jw;
#pragma unroll
      for (int tr = 0; tr < NT; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tr + 4 * g + e;
          if (r < L) st1<TO>(ob + static_cast<int64_t>(r) * a.Hv * DK, o[tr][e]);
        }
    }
    f32x4 lu[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr)
#pragma unroll
      for (int e = 0; e < 4; ++e) lu[tr][e] = lam[16 * tr + 4 * g + e] * u[tr][e];
    chain_frags<NT>(bf, lu);
    const float gc = sc[0];
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti) h[ti] = h[ti] * gc;
    mma_chain_rows<NTK, NT>(h, KsT, LDC, bf);
    __syncthreads();  // all reads of this chunk's LDS are done
    write_hs();
    if (c + 1 < a.NC) stage(c + 1);
    __syncthreads();
  }
  if (a.ht) {
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.ht[hbase + (16 * ti + 4 * g + e) * DK] = h[ti][e];
  }
}

// Reverse dH chain, fp16 operands.  Per chunk and wave: X = K dH (16 MFMA),
// a 16-row block of P (16), dU = lam X + P^T dO (8, chained), dRHS = T^T dU
// (8, chained), dH = gam_C dH + Q^T (gam dO) - K^T (beta gam dRHS) (32,
// chained).  Stores each chunk's incoming dH for the gradient kernel.
template <int C, typename TO>
__global__ __launch_bounds__(256) void chunk_dh_f16_kernel(CArgs a) {
  using namespace f16c;
  constexpr int LDC = C + 8, NT = C / 16, NTK = DK / 16;
  __shared__ __align__(16) _Float16 Ks[C * LDK];
  __shared__ __align__(16) _Float16 KsT[DK * LDC];
  __shared__ __align__(16) _Float16 QsT[DK * LDC];
  __shared__ __align__(16) _Float16 TsT[C * LDC];   // TsT[r][s] = T[s][r]
  __shared__ __align__(16) _Float16 PsT[C * LDC];   // PsT[s][r] = P[r][s]
  __shared__ __align__(16) _Float16 dHs[BV * LDK];  // dHs[j][i] = dH[i][j]
  __shared__ float G2[C], gam[C], lam[C], bet[C], sc[1];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (a.Hv / a.Hk);
  const int j0 = blockIdx.x * BV;
  const int jw = 16 * w + c16;
  const int64_t hbase = (b * a.Hv + hv) * DK * DK + j0 + jw;

  f32x4 dh[NTK];
#pragma unroll
  for (int ti = 0; ti < NTK; ++ti) {
    dh[ti] = zero4();
    if (a.dht) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dh[ti][e] = a.dht[hbase + (16 * ti + 4 * g + e) * DK];
    }
  }
  auto write_dhs = [&]() {
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti) {
      const f16x4 v4{static_cast<_Float16>(dh[ti][0]), static_cast<_Float16>(dh[ti][1]),
                     static_cast<_Float16>(dh[ti][2]), static_cast<_Float16>(dh[ti][3])};
      *reinterpret_cast<f16x4*>(dHs + jw * LDK + 16 * ti + 4 * g) = v4;
    }
  };
  Pre<C, true> pre;
  uint32_t docur[NT][2];
  int Lcur = 0;
  auto stage = [&](int c) {
    const int64_t t0 = static_cast<int64_t>(c) * C;
    const int L = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
    stage_rows_pre<C, Pre<C, true>::NV, true>(Ks, KsT, pre.k, a.l2);
    stage_rows_pre<C, Pre<C, true>::NV, true, false>(nullptr, QsT, pre.q, a.l2);
    stage_t_pre<C, Pre<C, true>::NTU, true>(TsT, pre.t);
    stage_t_pre<C, Pre<C, true>::NTU, true>(PsT, pre.pm);
    stage_gates_pre<C>(G2, gam, lam, bet, sc, pre.gv, pre.bv, L);
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) { docur[tr][0] = pre.v[tr][0]; docur[tr][1] = pre.v[tr][1]; }
    Lcur = L;
  };
  prefetch<C, true>(pre, a, b, a.NC - 1, kh, hv, j0 + jw, a.dout);
  stage(a.NC - 1);
  write_dhs();
  __syncthreads();

  for (int c = a.NC - 1; c >= 0; --c) {
    const int64_t t0 = static_cast<int64_t>(c) * C;
    const int L = Lcur;
    {  // gradient at this chunk's end, natural [Dk][Dv] layout
      _Float16* dst = static_cast<_Float16*>(a.dhst) + ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(DK * DK) + j0 + jw;
#pragma unroll
      for (int ti = 0; ti < NTK; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(16 * ti + 4 * g + e) * DK] = static_cast<_Float16>(dh[ti][e]);
    }
    if (c > 0) prefetch<C, true>(pre, a, b, c - 1, kh, hv, j0 + jw, a.dout);

    f32x4 du[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) du[tr] = zero4();
    mma_rows<NT, DK>(du, Ks, LDK, dHs, LDK, 16 * w);
#pragma unroll
    for (int tr = 0; tr < NT; ++tr)
#pragma unroll
      for (int e = 0; e < 4; ++e) du[tr][e] *= lam[16 * tr + 4 * g + e];
    f32x4 dof[NT], gdo[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      float x[4];
      unpack_strip(x, docur[tr]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dof[tr][e] = x[e];
        gdo[tr][e] = gam[16 * tr + 4 * g + e] * x[e];
      }
    }
    f16x8 bf[NT / 2];
    chain_frags<NT>(bf, dof);
    mma_chain_rows<NT, NT>(du, PsT, LDC, bf);
    chain_frags<NT>(bf, du);
    f32x4 dr[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) dr[tr] = zero4();
    mma_chain_rows<NT, NT>(dr, TsT, LDC, bf);
    TO* dvb = static_cast<TO*>(a.dv) + ((b * a.T + t0) * a.Hv + hv) * DK + j0 + jw;
#pragma unroll
    for (int tr = 0; tr < NT; ++tr)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * tr + 4 * g + e;
        if (r < L) st1<TO>(dvb + static_cast<int64_t>(r) * a.Hv * DK, bet[r] * dr[tr][e]);
        dr[tr][e] *= -bet[r] * gam[r];
      }
    const float gc = sc[0];
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti) dh[ti] = dh[ti] * gc;
    chain_frags<NT>(bf, gdo);
    mma_chain_rows<NTK, NT>(dh, QsT, LDC, bf);
    chain_frags<NT>(bf, dr);
    mma_chain_rows<NTK, NT>(dh, KsT, LDC, bf);
    __syncthreads();
    write_dhs();
    if (c > 0) stage(c - 1);
    __syncthreads();
  }
  if (a.dh0) {
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.dh0[hbase + (16 * ti + 4 * g + e) * DK] = dh[ti][e];
  }
}

namespace f16c {

// acc[t] += A[16t : 16t+16, 0:K] * B, B^T rows n0..n0+15 read through a
// row-contiguous view (element (n, k) at Bm[k * ldb + n]); B is shared.
template <int NO, int K>
__device__ __forceinline__ void mma_rows_bkmin(f32x4 (&acc)[NO], const _Float16* A, int lda, const _Float16* Bm,
                                               int ldb, int n0) {
  const int r = lane_id() & 15, kl = (lane_id() >> 4) * 8;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    f16x8 bfr;
#pragma unroll
    for (int i = 0; i < 8; ++i) bfr[i] = Bm[(k0 + kl + i) * ldb + n0 + r];
    f16x8 af[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t) af[t] = ld8(A + (16 * t + r) * lda + k0 + kl);
#pragma unroll
    for (int t = 0; t < NO; ++t) acc[t] = F16Op::mma(af[t], bfr, acc[t]);
  }
}

// acc[t] += A[m0 : m0+16, 0:K] * B[:, nb + 16t : nb + 16t + 16]; B^T rows
// from Bt (k contiguous); the A fragment is shared.
template <int NCOL, int K>
__device__ __forceinline__ void mma_cols(f32x4 (&acc)[NCOL], const _Float16* A, int lda, int m0, const _Float16* Bt,
                                         int ldb, int nb) {
  const int r = lane_id() & 15, kl = (lane_id() >> 4) * 8;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const f16x8 af = ld8(A + (m0 + r) * lda + k0 + kl);
    f16x8 bfr[NCOL];
#pragma unroll
    for (int t = 0; t < NCOL; ++t) bfr[t] = ld8(Bt + (nb + 16 * t + r) * ldb + k0 + kl);
#pragma unroll
    for (int t = 0; t < NCOL; ++t) acc[t] = F16Op::mma(af, bfr[t], acc[t]);
  }
}

// Branch-free load of this lane's strip rows (16tr + 4g + e) of a bf16
// [B,T,Hv,Dv] tensor at column jcol; rows >= L read as 0.
template <int NT>
__device__ __forceinline__ void load_strip(f32x4 (&x)[NT], const bf16_t* base, int64_t rstride, int L) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int tr = 0; tr < NT; ++tr)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * tr + 4 * g + e;
      const float v = bf16_to_f32(base[(r < L ? r : L - 1) * rstride]);
      x[tr][e] = r < L ? v : 0.f;
    }
}

}  // namespace f16c

// All gradients of one chunk except dv and dH (fp16 operands), given its
// entry state H0 and the gradient dH at its end, both [Dk][Dv] fp16.  The
// value dim is walked in two halves of 64 columns; wave w owns the 16-column
// strip 16w.. of a half, so Y = K H0, X = K dH, U = T RHS, dU = lam X + P^T dO
// and dRHS = T^T dU chain in registers.  The value-dim reductions
//   X1 = dRHS H0^T, X2 = dO H0^T, dP = dO U^T   (phase 1)
//   X3 = U dH^T, dT = dU RHS^T                  (phase 2)
// read row-contiguous copies written to LDS.  Then the C x C stage
// (dA = -T^T dT T^T) and dq / dk as in chunk_grad_kernel.
template <int C>
__global__ __launch_bounds__(256) void chunk_grad_f16_kernel(CArgs a) {
  using namespace f16c;
  constexpr int LDC = C + 8, NT = C / 16, LDJ = 64 + 8;
  constexpr int WPR = 4 / NT;   // waves per row tile in the reductions
  constexpr int NCK = 8 / WPR;  // Dk column tiles per wave
  constexpr int NCQ = NT / WPR; // C column tiles per wave
  constexpr int POOL_HALF = 2 * DK * LDJ + 3 * C * LDJ;
  constexpr int POOL_CC = 5 * C * LDC;
  constexpr int POOL = POOL_HALF > POOL_CC ? POOL_HALF : POOL_CC;
  __shared__ __align__(16) _Float16 Ks[C * LDK];
  __shared__ __align__(16) _Float16 KsT[DK * LDC];
  __shared__ __align__(16) _Float16 QsT[DK * LDC];
  __shared__ __align__(16) _Float16 Ts[C * LDC];
  __shared__ __align__(16) _Float16 TsT[C * LDC];
  __shared__ __align__(16) _Float16 PsT[C * LDC];
  __shared__ __align__(16) _Float16 pool[POOL];
  __shared__ float G2[C], gam[C], lam[C], bet[C], sc[1];
  __shared__ float sG[4][C], sGc[4][C], sB[4][C], red[2][4];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int c = blockIdx.x, hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (a.Hv / a.Hk);
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const int L = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
  const int64_t cbase = (b * a.Hv + hv) * a.NC + c;
  const int rt = w % NT, cq = w / NT;  // reduction tile ownership

  for (int e = tid; e < 4 * C; e += 256) {
    sG[e / C][e % C] = 0.f;
    sGc[e / C][e % C] = 0.f;
    sB[e / C][e % C] = 0.f;
  }
  {
    Pre<C, true> pre;
    prefetch<C, true>(pre, a, b, c, kh, hv, 0, a.v);
    stage_rows_pre<C, Pre<C, true>::NV, true>(Ks, KsT, pre.k, a.l2);
    stage_rows_pre<C, Pre<C, true>::NV, true, false>(nullptr, QsT, pre.q, a.l2);
    stage_t_pre<C, Pre<C, true>::NTU, false>(Ts, pre.t);
    stage_t_pre<C, Pre<C, true>::NTU, true>(TsT, pre.t);
    stage_t_pre<C, Pre<C, true>::NTU, true>(PsT, pre.pm);
    stage_gates_pre<C>(G2, gam, lam, bet, sc, pre.gv, pre.bv, L);
  }

  f32x4 x1[NCK], x2[NCK], x3[NCK], dP[NCQ], dT[NCQ];
#pragma unroll
  for (int t = 0; t < NCK; ++t) x1[t] = x2[t] = x3[t] = zero4();
#pragma unroll
  for (int t = 0; t < NCQ; ++t) dP[t] = dT[t] = zero4();
  float hh = 0.f;  // this thread's part of <dH, H0>
  f32x4 psb[NT], psy[NT];  // this lane's column parts of the phase-A row sums
#pragma unroll
  for (int t = 0; t < NT; ++t) psb[t] = psy[t] = zero4();
  _Float16* H0T = pool;               // H0T[i][j]  = H0[i][jh + j]
  _Float16* dHT = H0T + DK * LDJ;     // dHT[i][j]  = dH[i][jh + j]
  _Float16* X0 = dHT + DK * LDJ;      // [C][LDJ]: dRHS, then dU
  _Float16* X1b = X0 + C * LDJ;       // [C][LDJ]: dO, then RHS
  _Float16* X2b = X1b + C * LDJ;      // [C][LDJ]: U
  const _Float16* hsrc = static_cast<const _Float16*>(a.hst) + cbase * static_cast<int64_t>(DK * DK);
  const _Float16* dhsrc = static_cast<const _Float16*>(a.dhst) + cbase * static_cast<int64_t>(DK * DK);
  const int64_t rstride = static_cast<int64_t>(a.Hv) * DK;

  for (int jh = 0; jh < DK; jh += 64) {
    __syncthreads();  // previous users of the pool (and the staging above) are done
#pragma unroll
    for (int u = 0; u < DK * 8 / 256; ++u) {
      const int e = tid + 256 * u;
      const int i = e / 8, q8 = e % 8;
      const uint4 hv4 = *reinterpret_cast<const uint4*>(hsrc + i * DK + jh + 8 * q8);
      const uint4 dv4 = *reinterpret_cast<const uint4*>(dhsrc + i * DK + jh + 8 * q8);
      *reinterpret_cast<uint4*>(H0T + i * LDJ + 8 * q8) = hv4;
      *reinterpret_cast<uint4*>(dHT + i * LDJ + 8 * q8) = dv4;
      const _Float16* ph = reinterpret_cast<const _Float16*>(&hv4);
      const _Float16* pd = reinterpret_cast<const _Float16*>(&dv4);
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) hh += static_cast<float>(ph[k2]) * static_cast<float>(pd[k2]);
    }
    const int jcol = jh + 16 * w + c16;
    f32x4 vv[NT], dov[NT];
    load_strip<NT>(vv, static_cast<const bf16_t*>(a.v) + ((b * a.T + t0) * a.Hv + hv) * DK + jcol, rstride, L);
    load_strip<NT>(dov, static_cast<const bf16_t*>(a.dout) + ((b * a.T + t0) * a.Hv + hv) * DK + jcol, rstride, L);
    __syncthreads();

    f32x4 y[NT], du[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = du[t] = zero4();
    mma_rows_bkmin<NT, DK>(y, Ks, LDK, H0T, LDJ, 16 * w);
    mma_rows_bkmin<NT, DK>(du, Ks, LDK, dHT, LDJ, 16 * w);
    f32x4 rhs[NT], vmy[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * tr + 4 * g + e;
        vmy[tr][e] = vv[tr][e] - gam[r] * y[tr][e];
        rhs[tr][e] = bet[r] * vmy[tr][e];
        du[tr][e] *= lam[r];
      }
    f16x8 bf[NT / 2];
    f32x4 u[NT], dr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) u[t] = dr[t] = zero4();
    chain_frags<NT>(bf, rhs);
    mma_chain_rows<NT, NT>(u, Ts, LDC, bf);
    chain_frags<NT>(bf, dov);
    mma_chain_rows<NT, NT>(du, PsT, LDC, bf);
    chain_frags<NT>(bf, du);
    mma_chain_rows<NT, NT>(dr, TsT, LDC, bf);
    const int jl = 16 * w + c16;
#pragma unroll
    for (int tr = 0; tr < NT; ++tr)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * tr + 4 * g + e;
        psb[tr][e] += dr[tr][e] * vmy[tr][e];
        psy[tr][e] += dr[tr][e] * y[tr][e];
        X0[r * LDJ + jl] = static_cast<_Float16>(dr[tr][e]);
        X1b[r * LDJ + jl] = static_cast<_Float16>(dov[tr][e]);
        X2b[r * LDJ + jl] = static_cast<_Float16>(u[tr][e]);
      }
    __syncthreads();
    // phase 1: X1 += dRHS H0^T, X2 += dO H0^T, dP += dO U^T
    mma_cols<NCK, 64>(x1, X0, LDJ, 16 * rt, H0T, LDJ, 16 * cq * NCK);
    mma_cols<NCK, 64>(x2, X1b, LDJ, 16 * rt, H0T, LDJ, 16 * cq * NCK);
    mma_cols<NCQ, 64>(dP, X1b, LDJ, 16 * rt, X2b, LDJ, 16 * cq * NCQ);
    __syncthreads();
#pragma unroll
    for (int tr = 0; tr < NT; ++tr)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * tr + 4 * g + e;
        X0[r * LDJ + jl] = static_cast<_Float16>(du[tr][e]);
        X1b[r * LDJ + jl] = static_cast<_Float16>(rhs[tr][e]);
      }
    __syncthreads();
    // phase 2: X3 += U dH^T, dT += dU RHS^T
    mma_cols<NCK, 64>(x3, X2b, LDJ, 16 * rt, dHT, LDJ, 16 * cq * NCK);
    mma_cols<NCQ, 64>(dT, X0, LDJ, 16 * rt, X1b, LDJ, 16 * cq * NCQ);
  }
  // phase-A row sums: dbeta_r += sum_j dRHS (V - gam Y), dG_r -= beta gam sum_j dRHS Y
#pragma unroll
  for (int tr = 0; tr < NT; ++tr)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * tr + 4 * g + e;
      const float sb = row16_sum(psb[tr][e]);
      const float sy = row16_sum(psy[tr][e]);
      if (c16 == 0) {
        sB[w][r] += sb;
        sG[w][r] -= bet[r] * gam[r] * sy;
      }
    }
  __syncthreads();

  // ---- C x C stage
  _Float16* dTT = pool;             // dTT[s'][s] = dT[s][s']
  _Float16* M1s = dTT + C * LDC;
  _Float16* dPm = M1s + C * LDC;    // dPm[r][s]
  _Float16* dPmT = dPm + C * LDC;   // dPmT[s][r]
  _Float16* dAs = dPmT + C * LDC;   // symmetric dAm + dAm^T
  float rowG[4] = {0.f, 0.f, 0.f, 0.f}, rowB[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's row parts
#pragma unroll
  for (int cc = 0; cc < NCQ; ++cc) {
    const int s2 = 16 * (cq * NCQ + cc) + c16;
    f16x4 t4;
    float col = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + 4 * g + e;
      t4[e] = static_cast<_Float16>(dT[cc][e]);
      const float pv = static_cast<float>(PsT[s2 * LDC + r]);      // P_rs
      const float m = s2 <= r ? exp2f(G2[r] - G2[s2]) : 0.f;
      const float dpp = dP[cc][e] * pv;
      rowG[e] += dpp;
      col += dpp;
      dPm[r * LDC + s2] = static_cast<_Float16>(dP[cc][e] * m);
    }
    *reinterpret_cast<f16x4*>(dTT + s2 * LDC + 16 * rt + 4 * g) = t4;
    f16x4 p4;
#pragma unroll
    for (int e = 0; e < 4; ++e) p4[e] = dPm[(16 * rt + 4 * g + e) * LDC + s2];
    *reinterpret_cast<f16x4*>(dPmT + s2 * LDC + 16 * rt + 4 * g) = p4;
    col = xsum<16, 64>(col);
    if (lane < 16) sGc[w][s2] += col;
  }
  __syncthreads();
  f32x4 m1[NCQ];
#pragma unroll
  for (int cc = 0; cc < NCQ; ++cc) m1[cc] = zero4();
  mma_cols<NCQ, C>(m1, TsT, LDC, 16 * rt, dTT, LDC, 16 * cq * NCQ);
#pragma unroll
  for (int cc = 0; cc < NCQ; ++cc)
#pragma unroll
    for (int e = 0; e < 4; ++e) M1s[(16 * rt + 4 * g + e) * LDC + 16 * (cq * NCQ + cc) + c16] = static_cast<_Float16>(m1[cc][e]);
  __syncthreads();
  f32x4 da[NCQ], kk[NCQ];
#pragma unroll
  for (int cc = 0; cc < NCQ; ++cc) da[cc] = kk[cc] = zero4();
  mma_cols<NCQ, C>(da, M1s, LDC, 16 * rt, Ts, LDC, 16 * cq * NCQ);
  mma_cols<NCQ, DK>(kk, Ks, LDK, 16 * rt, Ks, LDK, 16 * cq * NCQ);
#pragma unroll
  for (int cc = 0; cc < NCQ; ++cc) {
    const int s2 = 16 * (cq * NCQ + cc) + c16;
    float col = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + 4 * g + e;
      const float ex = s2 < r ? exp2f(G2[r] - G2[s2]) : 0.f;
      const float dav = -da[cc][e] * ex;
      const float dam = dav * bet[r];
      const float ag = dam * kk[cc][e];
      rowB[e] += dav * kk[cc][e];
      rowG[e] += ag;
      col += ag;
      if (s2 < r) {
        dAs[r * LDC + s2] = static_cast<_Float16>(dam);
        dAs[s2 * LDC + r] = static_cast<_Float16>(dam);
      } else if (s2 == r) {
        dAs[r * LDC + r] = static_cast<_Float16>(0.f);
      }
    }
    col = xsum<16, 64>(col);
    if (lane < 16) sGc[w][s2] += col;
  }
  __syncthreads();

  // ---- dq, dk per v-head; X2 / X3 terms of dG
  f32x4 dq[NCK], dk[NCK];
#pragma unroll
  for (int t = 0; t < NCK; ++t) dq[t] = dk[t] = zero4();
  mma_cols<NCK, C>(dq, dPm, LDC, 16 * rt, KsT, LDC, 16 * cq * NCK);
  mma_cols<NCK, C>(dk, dPmT, LDC, 16 * rt, QsT, LDC, 16 * cq * NCK);
  mma_cols<NCK, C>(dk, dAs, LDC, 16 * rt, KsT, LDC, 16 * cq * NCK);
  float gcx = 0.f;
  float* pq = a.pdq + ((b * a.T + t0) * a.Hv + hv) * DK;
  float* pk = a.pdk + ((b * a.T + t0) * a.Hv + hv) * DK;
#pragma unroll
  for (int ct = 0; ct < NCK; ++ct) {
    const int i2 = 16 * (cq * NCK + ct) + c16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + 4 * g + e;
      const float qn = static_cast<float>(QsT[i2 * LDC + r]);
      const float kn = static_cast<float>(KsT[i2 * LDC + r]);
      const float t3 = lam[r] * kn * x3[ct][e];
      rowG[e] += gam[r] * qn * x2[ct][e] - t3;
      gcx += t3;
      const float dqv = dq[ct][e] + gam[r] * x2[ct][e];
      const float dkv = dk[ct][e] + lam[r] * x3[ct][e] - bet[r] * gam[r] * x1[ct][e];
      if (r < L) {
        pq[static_cast<int64_t>(r) * rstride + i2] = dqv;
        pk[static_cast<int64_t>(r) * rstride + i2] = dkv;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float rg = row16_sum(rowG[e]);
    const float rb = row16_sum(rowB[e]);
    if (c16 == 0) {
      sG[w][16 * rt + 4 * g + e] += rg;
      sB[w][16 * rt + 4 * g + e] += rb;
    }
  }
  hh = xsum<1, 64>(hh);
  gcx = xsum<1, 64>(gcx);
  if (lane == 0) {
    red[0][w] = hh;
    red[1][w] = gcx;
  }
  __syncthreads();
  if (w == 0) {
    const int r = lane;
    float dG = 0.f, dB = 0.f;
    if (r < C) {
      dG = sG[0][r] + sG[1][r] + sG[2][r] + sG[3][r] - (sGc[0][r] + sGc[1][r] + sGc[2][r] + sGc[3][r]);
      dB = sB[0][r] + sB[1][r] + sB[2][r] + sB[3][r];
    }
    if (r == L - 1)
      dG += sc[0] * (red[0][0] + red[0][1] + red[0][2] + red[0][3]) + (red[1][0] + red[1][1] + red[1][2] + red[1][3]);
    if (r >= L) dG = 0.f;
    float x = dG;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float yv = __shfl_down(x, off, 64);
      if (lane + off < 64) x += yv;
    }
    if (r < L) {
      const int64_t row = (b * a.T + t0 + r) * a.Hv + hv;
      a.dg[row] = x;
      a.dbeta[row] = dB;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.
template <typename CF, typename TI>
hipError_t prep(const CArgs& a, hipStream_t st) {
  ProfScope ps("chunk_prep", st);
  hipLaunchKernelGGL((chunk_prep_kernel<CF, TI>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(64), 0,
                     st, a);
  return hipGetLastError();
}

template <typename CF, typename TI, typename TO>
hipError_t dh(const CArgs& a, hipStream_t st) {
  ProfScope ps("chunk_dh", st);
  if constexpr (std::is_same_v<typename CF::OP, F16Op>) {
    hipLaunchKernelGGL((chunk_dh_f16_kernel<CF::C, TO>), dim3(f16c::DK / f16c::BV, a.Hv, static_cast<unsigned>(a.B)),
                       dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((chunk_dh_kernel<CF, TI, TO>), dim3(CF::DK / CF::BV, a.Hv, static_cast<unsigned>(a.B)),
                       dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <typename CF, typename TI>
hipError_t grad(const CArgs& a, hipStream_t st) {
  ProfScope ps("chunk_grad", st);
  if constexpr (std::is_same_v<typename CF::OP, F16Op>) {
    hipLaunchKernelGGL((chunk_grad_f16_kernel<CF::C>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(256), 0,
                       st, a);
  } else {
    hipLaunchKernelGGL((chunk_grad_kernel<CF, TI>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(256), 0,
                       st, a);
  }
  return hipGetLastError();
}

template <typename CF, typename TI, typename TO, bool WO, bool SH>
hipError_t fwd(const CArgs& a, hipStream_t st) {
  ProfScope ps(WO ? "chunk_fwd" : "chunk_states", st);
  if constexpr (std::is_same_v<typename CF::OP, F16Op>) {
    hipLaunchKernelGGL((chunk_fwd_f16_kernel<CF::C, TO, WO, SH>), dim3(f16c::DK / f16c::BV, a.Hv, static_cast<unsigned>(a.B)),
                       dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((chunk_fwd_kernel<CF, TI, TO, WO, SH>), dim3(CF::DK / CF::BV, a.Hv, static_cast<unsigned>(a.B)),
                       dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

CArgs base_args(const Shape& s, int C) {
  CArgs a{};
  a.B = s.B;
  a.T = s.T;
  a.Hk = s.Hk;
  a.Hv = s.Hv;
  a.NC = static_cast<int>((s.T + C - 1) / C);
  a.l2 = s.l2norm ? 1 : 0;
  return a;
}

// Calls f(cfg_tag, ti_tag, to_tag) for the configuration the shape maps to.
template <typename F>
hipError_t with_cfg(const Shape& s, int C, F&& f) {
  auto go = [&](auto cfg) -> hipError_t {
    using CF = decltype(cfg);
    auto by_out = [&](auto ti) -> hipError_t {
      return s.out_bf16 ? f(cfg, ti, std::common_type<bf16_t>{}) : f(cfg, ti, std::common_type<float>{});
    };
    return s.io_bf16 ? by_out(std::common_type<bf16_t>{}) : by_out(std::common_type<float>{});
  };
  if (chunk_uses_f16(s, C)) {
    if (C == 64) return go(Cfg<F16Op, 64, 128, 64, 64>{});
    if (C == 32) return go(Cfg<F16Op, 32, 128, 64, 64>{});
    return hipErrorInvalidValue;
  }
  if (s.D == 16) {
    if (C == 64) return go(Cfg<F32Op, 64, 16, 16, 16>{});
    if (C == 32) return go(Cfg<F32Op, 32, 16, 16, 16>{});
    if (C == 16) return go(Cfg<F32Op, 16, 16, 16, 16>{});
    return hipErrorInvalidValue;
  }
  if (C == 64) return go(Cfg<F32Op, 64, 128, 32, 16>{});
  if (C == 32) return go(Cfg<F32Op, 32, 128, 32, 16>{});
  if (C == 16) return go(Cfg<F32Op, 16, 128, 32, 16>{});
  return hipErrorInvalidValue;
}

}  // namespace

bool chunk_uses_f16(const Shape& s, int C) { return s.io_bf16 && s.D == 128 && C >= 32; }

size_t chunk_tmat_bytes(const Shape& s, int C) {
  const int64_t nc = (s.T + C - 1) / C;
  return static_cast<size_t>(s.B * s.Hv * nc) * C * C * (chunk_uses_f16(s, C) ? 2 : 4);
}

size_t chunk_state_bytes(const Shape& s, int C) {
  const int64_t nc = (s.T + C - 1) / C;
  return static_cast<size_t>(s.B * s.Hv * nc) * s.D * s.D * (chunk_uses_f16(s, C) ? 2 : 4);
}

hipError_t launch_chunk_fwd(const Shape& s, int C, const ChunkFwdArgs& x, hipStream_t st) {
  CArgs a = base_args(s, C);
  a.q = x.q; a.k = x.k; a.v = x.v; a.g = x.g; a.beta = x.beta; a.h0 = x.h0;
  a.o = x.o; a.ht = x.ht; a.tmat = x.tmat; a.pmat = x.pmat;
  return with_cfg(s, C, [&](auto cfg, auto ti, auto to) -> hipError_t {
    using CF = decltype(cfg);
    using TI = typename decltype(ti)::type;
    using TO = typename decltype(to)::type;
    hipError_t e = prep<CF, TI>(a, st);
    if (e != hipSuccess) return e;
    return fwd<CF, TI, TO, true, false>(a, st);
  });
}

hipError_t launch_chunk_bwd(const Shape& s, int C, const ChunkBwdArgs& x, hipStream_t st) {
  CArgs a = base_args(s, C);
  a.q = x.q; a.k = x.k; a.v = x.v; a.dout = x.dout; a.g = x.g; a.beta = x.beta; a.h0 = x.h0; a.dht = x.dht;
  a.dv = x.dv; a.dh0 = x.dh0; a.tmat = x.tmat; a.pmat = x.pmat; a.hst = x.hst; a.dhst = x.dhst;
  a.pdq = x.pdq; a.pdk = x.pdk; a.dg = x.dg; a.dbeta = x.dbeta;
  return with_cfg(s, C, [&](auto cfg, auto ti, auto to) -> hipError_t {
    using CF = decltype(cfg);
    using TI = typename decltype(ti)::type;
    using TO = typename decltype(to)::type;
    hipError_t e = prep<CF, TI>(a, st);
    if (e == hipSuccess) e = fwd<CF, TI, TO, false, true>(a, st);
    if (e == hipSuccess) e = dh<CF, TI, TO>(a, st);
    if (e == hipSuccess) e = grad<CF, TI>(a, st);
    return e;
  });
}

}  // namespace gdr
