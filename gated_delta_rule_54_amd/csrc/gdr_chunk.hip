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
  int fg;  // fused gate activation: g, beta hold pre-activations
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
  float x = 0.f, bt = 0.f;
  if (lane < L) {
    x = a.fg ? fg_log_alpha(a.g[row]) : a.g[row];
    bt = a.fg ? fg_beta(a.beta[row]) : a.beta[row];
  }
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
      a.dg[row] = a.fg ? x * fg_dlog_alpha(a.g[row]) : x;
      a.dbeta[row] = a.fg ? dB * fg_dbeta(a.beta[row]) : dB;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.
template <typename CF, typename TI>
hipError_t prep(const CArgs& a, hipStream_t st) {
  ProfScope ps("chunk_prep", st);
  hipLaunchKernelGGL((chunk_prep_kernel<CF, TI>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <typename CF, typename TI, typename TO>
hipError_t dh(const CArgs& a, hipStream_t st) {
  ProfScope ps("chunk_dh", st);
  hipLaunchKernelGGL((chunk_dh_kernel<CF, TI, TO>), dim3(CF::DK / CF::BV, a.Hv, static_cast<unsigned>(a.B)),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename CF, typename TI>
hipError_t grad(const CArgs& a, hipStream_t st) {
  ProfScope ps("chunk_grad", st);
  hipLaunchKernelGGL((chunk_grad_kernel<CF, TI>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename CF, typename TI, typename TO, bool WO, bool SH>
hipError_t fwd(const CArgs& a, hipStream_t st) {
  ProfScope ps(WO ? "chunk_fwd" : "chunk_states", st);
  hipLaunchKernelGGL((chunk_fwd_kernel<CF, TI, TO, WO, SH>), dim3(CF::DK / CF::BV, a.Hv, static_cast<unsigned>(a.B)),
                     dim3(256), 0, st, a);
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
  a.fg = s.fused_gates ? 1 : 0;
  return a;
}

// Calls f(cfg_tag, ti_tag, to_tag) for the fp32-operand configuration the
// shape maps to.
template <typename F>
hipError_t with_cfg(const Shape& s, int C, F&& f) {
  auto go = [&](auto cfg) -> hipError_t {
    auto by_out = [&](auto ti) -> hipError_t {
      return s.out_bf16 ? f(cfg, ti, std::common_type<bf16_t>{}) : f(cfg, ti, std::common_type<float>{});
    };
    return s.io_bf16 ? by_out(std::common_type<bf16_t>{}) : by_out(std::common_type<float>{});
  };
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

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace of the fp32-operand path: T and P per chunk (forward and VJP),
// then chunk-entry states, chunk-end gradients and per-v-head dq/dk (VJP).
struct Ws32 {
  size_t tmat, pmat, hst, dhst, pdq, pdk, total;
};

Ws32 plan32(const Shape& s, int C, bool bwd) {
  const size_t nv = static_cast<size_t>(s.B * s.Hv) * static_cast<size_t>((s.T + C - 1) / C);
  const size_t rows = static_cast<size_t>(s.B * s.T) * s.Hv;
  Ws32 w{};
  size_t off = 0;
  w.tmat = off; off = up(off + nv * C * C * 4);
  w.pmat = off; off = up(off + nv * C * C * 4);
  if (bwd) {
    w.hst = off;  off = up(off + nv * s.D * s.D * 4);
    w.dhst = off; off = up(off + nv * s.D * s.D * 4);
    w.pdq = off;  off = up(off + rows * s.D * 4);
    w.pdk = off;  off = up(off + rows * s.D * 4);
  }
  w.total = off;
  return w;
}

}  // namespace

bool chunk_uses_f16(const Shape& s, int C) { return s.io_bf16 && s.D == 128 && C >= 32; }

size_t chunk_fwd_workspace(const Shape& s, int C) {
  return chunk_uses_f16(s, C) ? chunk16_fwd_workspace(s, C) : plan32(s, C, false).total;
}

size_t chunk_bwd_workspace(const Shape& s, int C) {
  return chunk_uses_f16(s, C) ? chunk16_bwd_workspace(s, C) : plan32(s, C, true).total;
}

hipError_t launch_chunk_fwd(const Shape& s, int C, const ChunkFwdArgs& x, void* ws, hipStream_t st) {
  if (chunk_uses_f16(s, C)) return launch_chunk16_fwd(s, C, x, ws, st);
  const Ws32 w = plan32(s, C, false);
  char* base = static_cast<char*>(ws);
  CArgs a = base_args(s, C);
  a.q = x.q; a.k = x.k; a.v = x.v; a.g = x.g; a.beta = x.beta; a.h0 = x.h0;
  a.o = x.o; a.ht = x.ht; a.tmat = base + w.tmat; a.pmat = base + w.pmat;
  return with_cfg(s, C, [&](auto cfg, auto ti, auto to) -> hipError_t {
    using CF = decltype(cfg);
    using TI = typename decltype(ti)::type;
    using TO = typename decltype(to)::type;
    hipError_t e = prep<CF, TI>(a, st);
    if (e != hipSuccess) return e;
    return fwd<CF, TI, TO, true, false>(a, st);
  });
}

hipError_t launch_chunk_bwd(const Shape& s, int C, const ChunkBwdArgs& x, void* ws, hipStream_t st) {
  if (chunk_uses_f16(s, C)) return launch_chunk16_bwd(s, C, x, ws, st);
  const Ws32 w = plan32(s, C, true);
  char* base = static_cast<char*>(ws);
  CArgs a = base_args(s, C);
  a.q = x.q; a.k = x.k; a.v = x.v; a.dout = x.dout; a.g = x.g; a.beta = x.beta; a.h0 = x.h0; a.dht = x.dht;
  a.dv = x.dv; a.dh0 = x.dh0; a.tmat = base + w.tmat; a.pmat = base + w.pmat; a.hst = base + w.hst;
  a.dhst = base + w.dhst; a.pdq = reinterpret_cast<float*>(base + w.pdq);
  a.pdk = reinterpret_cast<float*>(base + w.pdk); a.dg = x.dg; a.dbeta = x.dbeta;
  hipError_t e = with_cfg(s, C, [&](auto cfg, auto ti, auto to) -> hipError_t {
    using CF = decltype(cfg);
    using TI = typename decltype(ti)::type;
    using TO = typename decltype(to)::type;
    hipError_t e2 = prep<CF, TI>(a, st);
    if (e2 == hipSuccess) e2 = fwd<CF, TI, TO, false, true>(a, st);
    if (e2 == hipSuccess) e2 = dh<CF, TI, TO>(a, st);
    if (e2 == hipSuccess) e2 = grad<CF, TI>(a, st);
    return e2;
  });
  if (e != hipSuccess) return e;
  EpiArgs ea{x.q, x.k, a.pdq, a.pdk, nullptr, nullptr, 1, x.dq, x.dk, nullptr, nullptr};
  return launch_bwd_epilogue(s, ea, st);
}

}  // namespace gdr
