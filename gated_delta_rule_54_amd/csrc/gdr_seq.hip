// Sequential (token-by-token) gated delta rule kernels for gfx950:
//   seq_fwd_kernel  - decode / sequential prefill forward
//   seq_bwd_kernel  - sequential VJP (checkpoint, replay, reverse sweep)
//   epilogue_kernel - partial sums, q/k L2-norm VJP, GQA group sums
//
// One wave (64 lanes) owns a Dk x BV slice of one head's fp32 state H = S^T
// and keeps it in registers for the whole sequence.  Value columns of H
// never mix (each column follows its own recurrence given k, q, alpha,
// beta), so slices of one head are independent workgroups.
//
// Per token the state is traversed twice, as on the page "Two-pass
// optimization for channelwise gated delta rule kernel" (pytorch/executorch
// pull request 21020, summary): pass one forms the decayed state D =
// diag(alpha) H and the prediction p = D^T k (and r = D^T q) with the decay
// folded in; pass two applies the rank-one update H = D + k u^T.  Unlike
// that page's second pass, the output needs no extra reduction here: with
// u = beta (v - p), o = H_t^T q = r + (k.q) u.
//
// Lane layout (Lay<D, BV>): lane = rg * NCG + cg; the lane holds rows
// rg*RPL .. rg*RPL+RPL-1 and columns cg*4 .. cg*4+3 of the slice.  A
// reduction over Dk is an xor-butterfly over the rg bits of the lane id, a
// reduction over the slice's columns one over the cg bits.  One load
// instruction of the state covers NRG rows x BV*4 contiguous bytes.

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef float f32x4n __attribute__((ext_vector_type(4)));  // native vector for non-temporal access

template <int D, int BV>
struct Lay {
  static constexpr int NCG = BV / 4;    // 4-column groups per slice
  static constexpr int NRG = 64 / NCG;  // row groups
  static constexpr int RPL = D / NRG;   // rows per lane
  static_assert(BV % 4 == 0 && 64 % NCG == 0 && D % NRG == 0, "layout");
};

struct Dims {
  int64_t B, T;
  int Hk, Hv;
  int l2;
  int fg;  // fused gate activation: g, beta hold pre-activations
};

template <int N, typename T>
__device__ __forceinline__ void ld_rows(const T* p, float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int m = 0; m < N; m += 4) {
      float t4[4];
      ld4<T>(p + m, t4);
      x[m] = t4[0]; x[m + 1] = t4[1]; x[m + 2] = t4[2]; x[m + 3] = t4[3];
    }
  } else {
#pragma unroll
    for (int m = 0; m < N; ++m) x[m] = ld1<T>(p + m);
  }
}

// Inputs of one token as seen by one lane.
template <int RPL, bool CW>
struct Tok {
  float k[RPL], q[RPL], v[4], a[CW ? RPL : 1], beta, dout[4];
};

template <int D, typename L, typename TI, bool CW, bool WANT_Q, bool WANT_DO>
__device__ __forceinline__ void load_tok(Tok<L::RPL, CW>& x, const Dims& d,
                                         const void* q, const void* k, const void* v,
                                         const void* dout, const float* g,
                                         const float* beta, int64_t row,
                                         int kh, int hv, int i0, int j0) {
  constexpr int RPL = L::RPL;
  const int64_t krow = (row * d.Hk + kh) * D + i0;
  const int64_t vrow = (row * d.Hv + hv) * D + j0;
  const int64_t grow = row * d.Hv + hv;
  ld_rows<RPL, TI>(static_cast<const TI*>(k) + krow, x.k);
  if constexpr (WANT_Q) ld_rows<RPL, TI>(static_cast<const TI*>(q) + krow, x.q);
  ld4<TI>(static_cast<const TI*>(v) + vrow, x.v);
  if constexpr (WANT_DO) ld4<TI>(static_cast<const TI*>(dout) + vrow, x.dout);
  if constexpr (CW) {
    ld_rows<RPL, float>(g + grow * D + i0, x.a);
#pragma unroll
    for (int m = 0; m < RPL; ++m) x.a[m] = d.fg ? fg_alpha(x.a[m]) : expf(x.a[m]);
  } else {
    x.a[0] = d.fg ? fg_alpha(g[grow]) : expf(g[grow]);
  }
  x.beta = d.fg ? fg_beta(beta[grow]) : beta[grow];
}

template <int RPL, bool CW>
__device__ __forceinline__ float alpha_of(const Tok<RPL, CW>& x, int m) {
  if constexpr (CW) return x.a[m]; else return x.a[0];
}

// Reciprocal L2 norm of the lane-distributed row vector (1 when disabled).
template <int NCG, int RPL>
__device__ __forceinline__ float rnorm(const float (&x)[RPL], int l2) {
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < RPL; ++m) s += x[m] * x[m];
  s = xsum<NCG, 64>(s);
  return l2 ? rsqrtf(s + kL2Eps) : 1.f;
}

// One forward token on the lane's state slice h.  Returns u (4 columns);
// when WANT_O also fills o.
template <typename L, bool CW, bool WANT_O>
__device__ __forceinline__ void fwd_step(float (&h)[L::RPL][4], const Tok<L::RPL, CW>& x,
                                         int l2, float (&u)[4], float (&o)[4]) {
  const float rk = rnorm<L::NCG, L::RPL>(x.k, l2);
  float rq = 1.f, kq = 0.f;
  if constexpr (WANT_O) {
    rq = rnorm<L::NCG, L::RPL>(x.q, l2);
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < L::RPL; ++m) s += x.k[m] * x.q[m];
    kq = xsum<L::NCG, 64>(s) * rk * rq;
  }
  // pass 1: D = diag(alpha) H, p = D^T k, r = D^T q
  float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < L::RPL; ++m) {
    const float am = alpha_of(x, m);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dme = am * h[m][e];
      h[m][e] = dme;
      p[e] += dme * x.k[m];
      if constexpr (WANT_O) r[e] += dme * x.q[m];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = xsum<L::NCG, 64>(p[e]) * rk;
    u[e] = x.beta * (x.v[e] - p[e]);
    if constexpr (WANT_O) o[e] = xsum<L::NCG, 64>(r[e]) * rq + kq * u[e];
  }
  // pass 2: H = D + k u^T
#pragma unroll
  for (int m = 0; m < L::RPL; ++m) {
    const float km = x.k[m] * rk;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[m][e] += km * u[e];
  }
}

template <int D, int BV, typename TI, typename TO, bool CW>
__global__ __launch_bounds__(64) void seq_fwd_kernel(Dims d, SeqFwdArgs a) {
  using L = Lay<D, BV>;
  const int lane = threadIdx.x;
  const int cg = lane % L::NCG, rg = lane / L::NCG;
  const int hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (d.Hv / d.Hk);
  const int j0 = blockIdx.x * BV + cg * 4;
  const int i0 = rg * L::RPL;
  const int64_t hbase = ((b * d.Hv + hv) * D + i0) * D + j0;

  float h[L::RPL][4];
#pragma unroll
  for (int m = 0; m < L::RPL; ++m) {
    if (a.h0) {  // streamed once: non-temporal
      const f32x4n t4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4n*>(a.h0 + hbase + m * D));
      h[m][0] = t4[0]; h[m][1] = t4[1]; h[m][2] = t4[2]; h[m][3] = t4[3];
    } else {
      h[m][0] = h[m][1] = h[m][2] = h[m][3] = 0.f;
    }
  }
  // sequence b: rows tb .. tb + len - 1 (a ragged batch gives offsets cu[0..B],
  // lengths clamped to [0, T])
  int64_t tb = b * d.T, len = d.T;
  if (a.cu) {
    tb = a.cu[b];
    len = a.cu[b + 1] - tb;
    len = len < 0 ? 0 : (len > d.T ? d.T : len);
  }
  Tok<L::RPL, CW> cur, nxt;
  if (len > 0) load_tok<D, L, TI, CW, true, false>(cur, d, a.q, a.k, a.v, nullptr, a.g, a.beta, tb, kh, hv, i0, j0);
  for (int64_t t = 0; t < len; ++t) {
    if (t + 1 < len)  // prefetch the next token while this one computes
      load_tok<D, L, TI, CW, true, false>(nxt, d, a.q, a.k, a.v, nullptr, a.g, a.beta, tb + t + 1, kh, hv, i0, j0);
    float u[4], o[4];
    fwd_step<L, CW, true>(h, cur, d.l2, u, o);
    if (rg == 0) st4<TO>(static_cast<TO*>(a.o) + ((tb + t) * d.Hv + hv) * D + j0, o);
    cur = nxt;
  }
  if (a.ht) {
#pragma unroll
    for (int m = 0; m < L::RPL; ++m)
      __builtin_nontemporal_store(f32x4n{h[m][0], h[m][1], h[m][2], h[m][3]}, reinterpret_cast<f32x4n*>(a.ht + hbase + m * D));
  }
}

// Decode step (T = 1, Dk = Dv = 128): NW waves per 128 x BV state slice,
// wave w owning rows (128/NW)w .. (128/NW)(w+1) - 1 (lanes: BV/4 column
// groups of 4 columns x 64/(BV/4) row groups of 128/NW/(64/(BV/4)) rows), so
// each wave issues 1/NW of the slice's state loads and stores; the sums over
// Dk (|k|^2, |q|^2, k.q, p, r) add the lanes' parts by butterfly and, with
// more than one wave, the waves' parts through LDS.
template <typename TI, typename TO, bool CW, int NW, int BV = 32>
__global__ __launch_bounds__(64 * NW) void decode_kernel(Dims d, SeqFwdArgs a) {
  constexpr int D = 128, NCG = BV / 4, RG = 64 / NCG, RPL = D / NW / RG, NV = 11;
  static_assert(RPL >= 1 && NCG * RG == 64, "slice shape");
  __shared__ float part[NW][NCG][NV + 1];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int cg = lane % NCG, rg = lane / NCG;
  const int hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (d.Hv / d.Hk);
  const int j0 = blockIdx.x * BV + cg * 4;
  const int i0 = (D / NW) * w + rg * RPL;
  const int64_t hbase = ((b * d.Hv + hv) * D + i0) * D + j0;
  int64_t tb = b * d.T, len = d.T;  // ragged batch: rows cu[b] .., length 0 or 1
  if (a.cu) {
    tb = a.cu[b];
    len = a.cu[b + 1] - tb;
    len = len < 0 ? 0 : (len > d.T ? d.T : len);
  }
  // The token's rows first: their loads are issued ahead of the state's,
  // so the sums that need no state (|k|^2, |q|^2, k.q) are formed while the
  // state is still arriving.
  const int64_t krow = (tb * d.Hk + kh) * D + i0;
  const int64_t vrow = (tb * d.Hv + hv) * D + j0;
  const int64_t grow = tb * d.Hv + hv;
  float k[RPL], q[RPL], v[4], al[CW ? RPL : 1], beta = 0.f;
  if (len > 0) {  // the same for every thread of the block
    ld_rows<RPL, TI>(static_cast<const TI*>(a.k) + krow, k);
    ld_rows<RPL, TI>(static_cast<const TI*>(a.q) + krow, q);
    ld4<TI>(static_cast<const TI*>(a.v) + vrow, v);
    if constexpr (CW) {
      ld_rows<RPL, float>(a.g + grow * D + i0, al);
    } else {
      al[0] = a.g[grow];
    }
    beta = a.beta[grow];
  }
  float h[RPL][4];
#pragma unroll
  for (int m = 0; m < RPL; ++m) {
    if (a.h0) {  // streamed once: non-temporal
      const f32x4n t4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4n*>(a.h0 + hbase + m * D));
      h[m][0] = t4[0]; h[m][1] = t4[1]; h[m][2] = t4[2]; h[m][3] = t4[3];
    } else {
      h[m][0] = h[m][1] = h[m][2] = h[m][3] = 0.f;
    }
  }
  if (len > 0) {
    if constexpr (CW) {
#pragma unroll
      for (int m = 0; m < RPL; ++m) al[m] = d.fg ? fg_alpha(al[m]) : expf(al[m]);
    } else {
      al[0] = d.fg ? fg_alpha(al[0]) : expf(al[0]);
    }
    beta = d.fg ? fg_beta(beta) : beta;
    // this wave's halves of the sums over Dk
    float x[NV] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // |k|^2 |q|^2 k.q p[4] r[4]
#pragma unroll
    for (int m = 0; m < RPL; ++m) {  // needs no state
      x[0] += k[m] * k[m];
      x[1] += q[m] * q[m];
      x[2] += k[m] * q[m];
    }
#pragma unroll
    for (int n = 0; n < 3; ++n) x[n] = xsum<NCG, 64>(x[n]);
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      const float am = CW ? al[CW ? m : 0] : al[0];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dme = am * h[m][e];
        h[m][e] = dme;
        x[3 + e] += dme * k[m];
        x[7 + e] += dme * q[m];
      }
    }
#pragma unroll
    for (int n = 3; n < NV; ++n) x[n] = xsum<NCG, 64>(x[n]);
    if constexpr (NW > 1) {
      if (rg == 0) {
#pragma unroll
        for (int n = 0; n < NV; ++n) part[w][cg][n] = x[n];
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < NV; ++n) {  // all waves' parts in one order (every wave gets the same sums)
        float t = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) t += part[w2][cg][n];
        x[n] = t;
      }
    }
    const float rk = d.l2 ? rsqrtf(x[0] + kL2Eps) : 1.f;
    const float rq = d.l2 ? rsqrtf(x[1] + kL2Eps) : 1.f;
    const float kq = x[2] * rk * rq;
    float u[4], o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] = beta * (v[e] - x[3 + e] * rk);
      o[e] = x[7 + e] * rq + kq * u[e];
    }
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      const float km = k[m] * rk;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[m][e] += km * u[e];
    }
    if (w == 0 && rg == 0) st4<TO>(static_cast<TO*>(a.o) + vrow, o);
  }
  if (a.ht) {
#pragma unroll
    for (int m = 0; m < RPL; ++m)
      __builtin_nontemporal_store(f32x4n{h[m][0], h[m][1], h[m][2], h[m][3]}, reinterpret_cast<f32x4n*>(a.ht + hbase + m * D));
  }
}

// ---------------------------------------------------------------------------
// Sequential VJP.  Phase 1 replays the forward and stores the state before
// every kSeqSeg-th token (lane-private layout).  Phase 2 walks the segments
// backwards: it reloads the segment's checkpoint, replays the segment while
// saving each state H_{t-1} to per-wave scratch, then runs the reverse
// recurrence over the segment, carrying dH in registers.  States are never
// recovered by inverting the update (the inverse is ill-conditioned).
//
// Reverse step for token t (dH = gradient arriving at H_t):
//   dHt = dH + q do^T;       dq  = H_t do
//   du  = dHt^T k;           dk  = dHt u - beta D du
//   dv  = beta du;           dbeta = <du, v - p>
//   dD  = dHt - beta k du^T; dg  = <dD, D> (per row when channelwise)
//   dH  = diag(alpha) dD
// dq, dk, dbeta, dg sum over value columns, so each slice writes partial
// sums that the epilogue adds in slice order.
template <int D, int BV, typename TI, typename TO, bool CW>
__global__ __launch_bounds__(64) void seq_bwd_kernel(Dims d, SeqBwdArgs a, int nck, int ns) {
  using L = Lay<D, BV>;
  constexpr int RPL = L::RPL;
  const int lane = threadIdx.x;
  const int cg = lane % L::NCG, rg = lane / L::NCG;
  const int slice = static_cast<int>(blockIdx.x), hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (d.Hv / d.Hk);
  const int j0 = slice * BV + cg * 4;
  const int i0 = rg * RPL;
  const int64_t hbase = ((b * d.Hv + hv) * D + i0) * D + j0;
  const int64_t wg = (b * d.Hv + hv) * ns + slice;
  float* ck = a.ckpt + wg * static_cast<int64_t>(nck) * D * BV;
  float* sc = a.scratch + wg * static_cast<int64_t>(kSeqSeg) * D * BV;
  auto lane_ptr = [&](float* base, int64_t idx, int m) {  // lane-private float4 slot
    return base + ((idx * RPL + m) * 64 + lane) * 4;
  };

  // sequence b: token rows tb .. tb + len - 1 (ragged: offsets cu, lengths
  // clamped to [0, T]); partial sums stay indexed by (b, t) as for B x T
  int64_t tb = b * d.T, slen = d.T;
  if (a.cu) {
    tb = a.cu[b];
    slen = a.cu[b + 1] - tb;
    slen = slen < 0 ? 0 : (slen > d.T ? d.T : slen);
  }
  const int64_t t_beg = 0, t_end = slen;  // tokens of this workgroup
  const int nckb = static_cast<int>((t_end - t_beg + kSeqSeg - 1) / kSeqSeg);
  float h[RPL][4];
#pragma unroll
  for (int m = 0; m < RPL; ++m) {
    if (a.h0) ld4<float>(a.h0 + hbase + m * D, h[m]);
    else h[m][0] = h[m][1] = h[m][2] = h[m][3] = 0.f;
  }
  // phase 1: checkpoints at the start of every segment (the tokens of the
  // last segment need no forward pass here: phase 2 replays them)
  for (int64_t t = t_beg; t < t_end; ++t) {
    if ((t - t_beg) % kSeqSeg == 0) {
#pragma unroll
      for (int m = 0; m < RPL; ++m) st4<float>(lane_ptr(ck, (t - t_beg) / kSeqSeg, m), h[m]);
      if ((t - t_beg) / kSeqSeg == nckb - 1) break;
    }
    Tok<RPL, CW> x;
    load_tok<D, L, TI, CW, false, false>(x, d, a.q, a.k, a.v, nullptr, a.g, a.beta, tb + t, kh, hv, i0, j0);
    float u[4], o[4];
    fwd_step<L, CW, false>(h, x, d.l2, u, o);
  }

  // phase 2: reverse
  float dH[RPL][4];
#pragma unroll
  for (int m = 0; m < RPL; ++m) {
    if (a.dht) ld4<float>(a.dht + hbase + m * D, dH[m]);
    else dH[m][0] = dH[m][1] = dH[m][2] = dH[m][3] = 0.f;
  }
  for (int c = nckb - 1; c >= 0; --c) {
    const int64_t t0 = t_beg + static_cast<int64_t>(c) * kSeqSeg;
    const int len = static_cast<int>(t_end - t0 < kSeqSeg ? t_end - t0 : kSeqSeg);
#pragma unroll
    for (int m = 0; m < RPL; ++m) ld4<float>(lane_ptr(ck, c, m), h[m]);
    for (int tau = 0; tau < len; ++tau) {
#pragma unroll
      for (int m = 0; m < RPL; ++m) st4<float>(lane_ptr(sc, tau, m), h[m]);
      Tok<RPL, CW> x;
      load_tok<D, L, TI, CW, false, false>(x, d, a.q, a.k, a.v, nullptr, a.g, a.beta, tb + t0 + tau, kh, hv, i0,
                                           j0);
      float u[4], o[4];
      fwd_step<L, CW, false>(h, x, d.l2, u, o);
    }
    for (int tau = len - 1; tau >= 0; --tau) {
      const int64_t t = t0 + tau;
      Tok<RPL, CW> x;
      load_tok<D, L, TI, CW, true, true>(x, d, a.q, a.k, a.v, a.dout, a.g, a.beta, tb + t, kh, hv, i0, j0);
      float Dm[RPL][4];
#pragma unroll
      for (int m = 0; m < RPL; ++m) {
        float hp[4];
        ld4<float>(lane_ptr(sc, tau, m), hp);
        const float am = alpha_of(x, m);
#pragma unroll
        for (int e = 0; e < 4; ++e) Dm[m][e] = am * hp[e];
      }
      const float rk = rnorm<L::NCG, RPL>(x.k, d.l2);
      const float rq = rnorm<L::NCG, RPL>(x.q, d.l2);
      float kn[RPL], qn[RPL];
#pragma unroll
      for (int m = 0; m < RPL; ++m) { kn[m] = x.k[m] * rk; qn[m] = x.q[m] * rq; }
      // recompute p, u
      float p[4] = {0.f, 0.f, 0.f, 0.f}, u[4];
#pragma unroll
      for (int m = 0; m < RPL; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] += Dm[m][e] * kn[m];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = xsum<L::NCG, 64>(p[e]);
        u[e] = x.beta * (x.v[e] - p[e]);
      }
      // dHt = dH + q do^T (in place), du = dHt^T k
      float du[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < RPL; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dH[m][e] += qn[m] * x.dout[e];
          du[e] += dH[m][e] * kn[m];
        }
#pragma unroll
      for (int e = 0; e < 4; ++e) du[e] = xsum<L::NCG, 64>(du[e]);
      // row partials over this slice's columns
      float dqr[RPL], dkr[RPL], dgr[RPL];
      float dgs = 0.f;
#pragma unroll
      for (int m = 0; m < RPL; ++m) {
        float sq = 0.f, sk = 0.f, sg = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ht = Dm[m][e] + kn[m] * u[e];
          sq += ht * x.dout[e];
          sk += dH[m][e] * u[e] - x.beta * Dm[m][e] * du[e];
          const float dD = dH[m][e] - x.beta * kn[m] * du[e];
          sg += dD * Dm[m][e];
          dH[m][e] = alpha_of(x, m) * dD;
        }
        dqr[m] = xsum<1, L::NCG>(sq);
        dkr[m] = xsum<1, L::NCG>(sk);
        if constexpr (CW) dgr[m] = xsum<1, L::NCG>(sg);
        else dgs += sg;
      }
      float dbs = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) dbs += du[e] * (x.v[e] - p[e]);
      dbs = xsum<1, L::NCG>(dbs);
      if constexpr (!CW) dgs = xsum<1, 64>(dgs);

      const int64_t row = (tb + t) * d.Hv + hv;                    // token row, v-head
      const int64_t prow = (static_cast<int64_t>(slice) * d.B * d.T + b * d.T + t) * d.Hv + hv;  // (slice, b, t, hv)
      if (cg == 0) {
        float* pq = a.part_dq + prow * D + i0;
        float* pk = a.part_dk + prow * D + i0;
#pragma unroll
        for (int m = 0; m < RPL; ++m) { pq[m] = dqr[m]; pk[m] = dkr[m]; }
        if constexpr (CW) {
          float* pg = a.part_dg + prow * D + i0;
#pragma unroll
          for (int m = 0; m < RPL; ++m) pg[m] = dgr[m];
        }
      }
      if (rg == 0) {
        float dvv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dvv[e] = x.beta * du[e];
        st4<TO>(static_cast<TO*>(a.dv) + row * D + j0, dvv);
      }
      if (lane == 0) {
        a.part_db[prow] = dbs;
        if constexpr (!CW) a.part_dg[prow] = dgs;
      }
    }
  }
  if (a.dh0) {
#pragma unroll
    for (int m = 0; m < RPL; ++m) st4<float>(a.dh0 + hbase + m * D, dH[m]);
  }
}

// ---------------------------------------------------------------------------
// Epilogue: one wave per (b, t, kh).  dq_hat = sum over the group's v-heads
// (in order) of the sum over slices (in order) of the partials; then
// dq = r (dq_hat - q_hat <q_hat, dq_hat>) when q was normalised in-kernel.
template <int D, typename TI, typename TO, bool CW>
__global__ __launch_bounds__(64) void epilogue_kernel(Dims d, EpiArgs a) {
  constexpr int EPT = (D + 63) / 64;
  const int lane = threadIdx.x;
  const int64_t pid = blockIdx.x;         // (b*T + t)*Hk + kh
  const int kh = static_cast<int>(pid % d.Hk);
  const int64_t bt = pid / d.Hk;
  int64_t io = bt;                        // token row (ragged: cu[b] + t)
  if (a.cu) {
    const int64_t b = bt / d.T, t = bt % d.T, s0 = a.cu[b];
    if (t >= a.cu[b + 1] - s0) return;   // past the end of sequence b
    io = s0 + t;
  }
  const int64_t id = io * d.Hk + kh;
  const int grp = d.Hv / d.Hk;
  const int64_t pstride = d.B * d.T * d.Hv;  // rows per slice
  for (int which = 0; which < 2; ++which) {
    const float* part = which == 0 ? a.part_dq : a.part_dk;
    const void* xin = which == 0 ? a.q : a.k;
    void* xout = which == 0 ? a.dq : a.dk;
    float s[EPT], x[EPT];
    float ss = 0.f, sx = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = lane + 64 * e;
      s[e] = 0.f; x[e] = 0.f;
      if (i < D) {
        for (int gi = 0; gi < grp; ++gi) {
          const int64_t row = bt * d.Hv + static_cast<int64_t>(kh) * grp + gi;
          for (int sl = 0; sl < a.nslices; ++sl) s[e] += part[(sl * pstride + row) * D + i];
        }
        x[e] = ld1<TI>(static_cast<const TI*>(xin) + id * D + i);
      }
      ss += x[e] * x[e];
    }
    if (d.l2) {
      ss = xsum<1, 64>(ss);
      const float r = rsqrtf(ss + kL2Eps);
#pragma unroll
      for (int e = 0; e < EPT; ++e) sx += x[e] * r * s[e];
      sx = xsum<1, 64>(sx);
#pragma unroll
      for (int e = 0; e < EPT; ++e) s[e] = r * (s[e] - x[e] * r * sx);
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = lane + 64 * e;
      if (i < D) st1<TO>(static_cast<TO*>(xout) + id * D + i, s[e]);
    }
  }
  // dbeta, dg for the group's v-heads
  for (int gi = 0; gi < grp; ++gi) {
    const int64_t row = bt * d.Hv + static_cast<int64_t>(kh) * grp + gi;  // partials
    const int64_t orow = io * d.Hv + static_cast<int64_t>(kh) * grp + gi;  // outputs, gates
    if (a.part_db && lane == 0) {
      float s = 0.f;
      for (int sl = 0; sl < a.nslices; ++sl) s += a.part_db[sl * pstride + row];
      a.dbeta[orow] = d.fg ? s * fg_dbeta(a.beta[orow]) : s;
    }
    if (a.part_dg) {
      if constexpr (CW) {
        for (int i = lane; i < D; i += 64) {
          float s = 0.f;
          for (int sl = 0; sl < a.nslices; ++sl) s += a.part_dg[(sl * pstride + row) * D + i];
          a.dg[orow * D + i] = d.fg ? s * fg_dlog_alpha(a.g[orow * D + i]) : s;
        }
      } else if (lane == 0) {
        float s = 0.f;
        for (int sl = 0; sl < a.nslices; ++sl) s += a.part_dg[sl * pstride + row];
        a.dg[orow] = d.fg ? s * fg_dlog_alpha(a.g[orow]) : s;
      }
    }
  }
}

// Dk = 128 epilogue: one 16-lane DPP row per (row (b, t, kh), dq or dk),
// eight consecutive elements per lane (16-byte input loads, 32-byte partial
// loads), so a 256-thread block covers 8 rows; the row reductions of the
// L2-norm VJP are DPP row sums.  dbeta / dg partials (sequential path) are
// summed by the dq groups.
template <typename T> __device__ __forceinline__ void ld8f(const T* p, float (&x)[8]);
template <> __device__ __forceinline__ void ld8f<float>(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <> __device__ __forceinline__ void ld8f<bf16_t>(const bf16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
template <typename T> __device__ __forceinline__ void st8(T* p, const float (&x)[8]);
template <> __device__ __forceinline__ void st8<float>(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}
template <> __device__ __forceinline__ void st8<bf16_t>(bf16_t* p, const float (&x)[8]) {
  uint4 u;
  uint32_t* w = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = static_cast<uint32_t>(f32_to_bf16(x[2 * k])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * k + 1])) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}

template <typename TI, typename TO, bool CW>
__global__ __launch_bounds__(256) void epilogue128_kernel(Dims d, EpiArgs a) {
  constexpr int D = 128;
  const int sub = threadIdx.x & 15;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int64_t rows = d.B * d.T * d.Hk;
  if (item >= 2 * rows) return;  // whole 16-lane groups leave together
  const int which = static_cast<int>(item & 1);
  const int64_t pid = item >> 1;  // (b*T + t)*Hk + kh
  const int kh = static_cast<int>(pid % d.Hk);
  const int64_t bt = pid / d.Hk;
  int64_t io = bt;                // token row (ragged: cu[b] + t)
  if (a.cu) {
    const int64_t b = bt / d.T, t = bt % d.T, s0 = a.cu[b];
    if (t >= a.cu[b + 1] - s0) return;  // past the end of sequence b (the whole 16-lane group)
    io = s0 + t;
  }
  const int64_t id = io * d.Hk + kh;
  const int grp = d.Hv / d.Hk;
  const int64_t pstride = d.B * d.T * d.Hv;
  const int i = 8 * sub;
  const float* part = which == 0 ? a.part_dq : a.part_dk;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int gi = 0; gi < grp; ++gi) {
    const int64_t row = bt * d.Hv + static_cast<int64_t>(kh) * grp + gi;
    for (int sl = 0; sl < a.nslices; ++sl) {
      float pv[8];
      ld8f<float>(part + (sl * pstride + row) * D + i, pv);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += pv[e];
    }
  }
  if (d.l2) {
    float x[8];
    ld8f<TI>(static_cast<const TI*>(which == 0 ? a.q : a.k) + id * D + i, x);
    float ss = 0.f, sx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss += x[e] * x[e];
      sx += x[e] * s[e];
    }
    ss = row16_sum(ss);
    sx = row16_sum(sx);
    const float r = rsqrtf(ss + kL2Eps);
    sx *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = r * (s[e] - x[e] * r * sx);
  }
  st8<TO>(static_cast<TO*>(which == 0 ? a.dq : a.dk) + id * D + i, s);
  if (which != 0) return;
  for (int gi = 0; gi < grp; ++gi) {
    const int64_t row = bt * d.Hv + static_cast<int64_t>(kh) * grp + gi;  // partials
    const int64_t orow = io * d.Hv + static_cast<int64_t>(kh) * grp + gi;  // outputs, gates
    if (a.part_db && sub == 0) {
      float sb = 0.f;
      for (int sl = 0; sl < a.nslices; ++sl) sb += a.part_db[sl * pstride + row];
      a.dbeta[orow] = d.fg ? sb * fg_dbeta(a.beta[orow]) : sb;
    }
    if (a.part_dg) {
      if constexpr (CW) {
        float gsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int sl = 0; sl < a.nslices; ++sl) {
          float pv[8];
          ld8f<float>(a.part_dg + (sl * pstride + row) * D + i, pv);
#pragma unroll
          for (int e = 0; e < 8; ++e) gsum[e] += pv[e];
        }
        if (d.fg) {
#pragma unroll
          for (int e = 0; e < 8; ++e) gsum[e] *= fg_dlog_alpha(a.g[orow * D + i + e]);
        }
        st8<float>(a.dg + orow * D + i, gsum);
      } else if (sub == 0) {
        float sg = 0.f;
        for (int sl = 0; sl < a.nslices; ++sl) sg += a.part_dg[sl * pstride + row];
        a.dg[orow] = d.fg ? sg * fg_dlog_alpha(a.g[orow]) : sg;
      }
    }
  }
}

Dims dims_of(const Shape& s) { return Dims{s.B, s.T, s.Hk, s.Hv, s.l2norm ? 1 : 0, s.fused_gates ? 1 : 0}; }

template <int D> constexpr int fwd_bv() { return D == 16 ? 16 : 32; }
// Decode slices at B=8, Hv=32 (rocprofv3 kernel durations on rotated state
// buffers, us): 32 columns x 2 waves 8.36 (chosen); 32 x 1: 8.64, 32 x 4:
// 8.87; 64 x 2: 8.57, 64 x 4: 8.58, 64 x 8: 8.69; 128 x 4: 8.90, 128 x 8:
// 8.93, 128 x 16: 8.90; 16 columns (half a 128-byte line per row) x 1, 2, 4:
// 12.2 - 13.3.
constexpr int kDecWaves = 2, kDecCols = 32;
// with fewer slices than CUs (B=1, Hv=32: 3.45 vs 3.66 us per step with 2 waves, 3.82 with 8)
constexpr int kDecSmallGrid = 256, kDecWavesSmall = 4;
template <int D> constexpr int bwd_bv() { return D == 16 ? 16 : 32; }

template <int D, typename TI, typename TO, bool CW>
hipError_t fwd_go(const Shape& s, const SeqFwdArgs& a, hipStream_t st) {
  constexpr int BV = fwd_bv<D>();
  dim3 grid(D / BV, s.Hv, static_cast<unsigned>(s.B));
  ProfScope ps("seq_fwd", st);
  if constexpr (D == 128) {
    if (s.T == 1) {  // decode step
      if (s.B * s.Hv * (D / BV) < kDecSmallGrid) {  // fewer slices than CUs: shorter waves
        hipLaunchKernelGGL((decode_kernel<TI, TO, CW, kDecWavesSmall>), grid, dim3(64 * kDecWavesSmall), 0, st,
                           dims_of(s), a);
        return hipGetLastError();
      }
      hipLaunchKernelGGL((decode_kernel<TI, TO, CW, kDecWaves, kDecCols>),
                         dim3(D / kDecCols, s.Hv, static_cast<unsigned>(s.B)), dim3(64 * kDecWaves), 0, st, dims_of(s), a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((seq_fwd_kernel<D, BV, TI, TO, CW>), grid, dim3(64), 0, st, dims_of(s), a);
  return hipGetLastError();
}

template <int D, typename TI, typename TO, bool CW>
hipError_t bwd_go(const Shape& s, const SeqBwdArgs& a, hipStream_t st) {
  constexpr int BV = bwd_bv<D>();
  const int nck = static_cast<int>((s.T + kSeqSeg - 1) / kSeqSeg);
  dim3 grid(D / BV, s.Hv, static_cast<unsigned>(s.B));
  ProfScope ps("seq_bwd", st);
  hipLaunchKernelGGL((seq_bwd_kernel<D, BV, TI, TO, CW>), grid, dim3(64), 0, st, dims_of(s), a, nck, D / BV);
  return hipGetLastError();
}

template <int D, typename TI, typename TO, bool CW>
hipError_t epi_go(const Shape& s, const EpiArgs& a, hipStream_t st) {
  const int64_t rows = s.B * s.T * s.Hk;
  ProfScope ps("bwd_epilogue", st);
  if constexpr (D == 128) {
    hipLaunchKernelGGL((epilogue128_kernel<TI, TO, CW>), dim3(static_cast<unsigned>((2 * rows + 15) / 16)), dim3(256), 0,
                       st, dims_of(s), a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((epilogue_kernel<D, TI, TO, CW>), dim3(static_cast<unsigned>(rows)), dim3(64), 0, st,
                     dims_of(s), a);
  return hipGetLastError();
}

// Instantiate F over (D, io, out, channelwise) and call it.
template <template <int, typename, typename, bool> class F, typename... A>
hipError_t dispatch(const Shape& s, A&&... args) {
  auto by_cw = [&](auto dtag, auto itag, auto otag) -> hipError_t {
    constexpr int D = decltype(dtag)::value;
    using TI = typename decltype(itag)::type;
    using TO = typename decltype(otag)::type;
    return s.channelwise ? F<D, TI, TO, true>::run(s, args...) : F<D, TI, TO, false>::run(s, args...);
  };
  auto by_out = [&](auto dtag, auto itag) -> hipError_t {
    return s.out_bf16 ? by_cw(dtag, itag, std::common_type<bf16_t>{}) : by_cw(dtag, itag, std::common_type<float>{});
  };
  auto by_in = [&](auto dtag) -> hipError_t {
    return s.io_bf16 ? by_out(dtag, std::common_type<bf16_t>{}) : by_out(dtag, std::common_type<float>{});
  };
  if (s.D == 16) return by_in(std::integral_constant<int, 16>{});
  if (s.D == 128) return by_in(std::integral_constant<int, 128>{});
  return hipErrorInvalidValue;
}

template <int D, typename TI, typename TO, bool CW> struct FwdF {
  static hipError_t run(const Shape& s, const SeqFwdArgs& a, hipStream_t st) { return fwd_go<D, TI, TO, CW>(s, a, st); }
};
template <int D, typename TI, typename TO, bool CW> struct BwdF {
  static hipError_t run(const Shape& s, const SeqBwdArgs& a, hipStream_t st) { return bwd_go<D, TI, TO, CW>(s, a, st); }
};
template <int D, typename TI, typename TO, bool CW> struct EpiF {
  static hipError_t run(const Shape& s, const EpiArgs& a, hipStream_t st) { return epi_go<D, TI, TO, CW>(s, a, st); }
};

}  // namespace

int seq_bwd_slices(const Shape& s) { return s.D == 16 ? 1 : s.D / 32; }

size_t seq_bwd_ckpt_floats(const Shape& s) {
  const int64_t nck = (s.T + kSeqSeg - 1) / kSeqSeg;
  return static_cast<size_t>(s.B * s.Hv * nck) * s.D * s.D;
}

size_t seq_bwd_scratch_floats(const Shape& s) {
  return static_cast<size_t>(s.B * s.Hv) * kSeqSeg * s.D * s.D;
}

hipError_t launch_seq_fwd(const Shape& s, const SeqFwdArgs& a, hipStream_t st) {
  return dispatch<FwdF>(s, a, st);
}
hipError_t launch_seq_bwd(const Shape& s, const SeqBwdArgs& a, hipStream_t st) {
  return dispatch<BwdF>(s, a, st);
}
hipError_t launch_bwd_epilogue(const Shape& s, const EpiArgs& a, hipStream_t st) {
  return dispatch<EpiF>(s, a, st);
}

}  // namespace gdr
