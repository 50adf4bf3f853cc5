// Chunked gated delta rule for bf16 io at Dk = Dv = 128 on gfx950: fp16
// matrix-core operands (v_mfma_f32_16x16x32_f16), fp32 accumulation, fp32
// carried state.  The chunk algebra is the one stated at the top of
// gdr_chunk.hip (the chunk-parallel form behind the "chunked" VJP of the page
// "Adding VJP for gated delta net", ml-explore/mlx pull request 4565).
//
// Work split:
//   prep16   per (b, v-head, chunk), parallel.  Normalises the chunk's q / k
//            rows, forms A and P on the matrix cores, inverts I + A, and
//            writes the chunk's operands as fp16 "images": byte-exact copies
//            of the padded LDS tiles the other kernels read.
//              key image   per (b, k-head, chunk):  Kn [C][136] | Qn [C][136]
//                          (columns in chained-fragment order: see key_unit)
//              chunk image per (b, v-head, chunk):  gam | lam | beta | log2(e) G
//                          (4 x C fp32) | T | P, each C x C tile [C][C+8]
//            Normalisation and gate math thus happen once per chunk instead
//            of once per consumer workgroup.  Products that need a tile
//            transposed (Kn^T, Qn^T, T^T, P^T) read it from the row-major
//            copy with ds_read_b64_tr_b16, so the images hold each tile once
//            and forward and VJP share one image format.
//   chain16  per (b, v-head, value slice of 16, 32 or 64 columns): the
//            sequential pass over chunks.  Wave w owns a 16-column strip of the state in MFMA
//            accumulators.  Each chunk's images are copied into one of two LDS
//            buffers by buffer_load_dwordx4 ... lds (no registers, no ALU)
//            while the previous chunk computes; one barrier per chunk.
//   dh16     the reverse pass carrying dH, same structure.
//   grad16   per (b, k-head, chunk), parallel: every remaining gradient, the
//            k-head's v-heads in turn.
//
// Chained operands: a C x 16 (or 128 x 16) strip held in accumulators is fed
// back as the B operand of the next product that contracts over its rows by
// relabelling that product's k index, so that lane group g supplies rows
// {4g..4g+3, 16+4g..16+4g+3} of each 32-row block - exactly the rows its
// accumulators hold.  The LDS-side A operand is read with the same
// relabelling: one 16-byte read per fragment from the key images, which are
// stored in that order, two 8-byte reads from T and P.
//
// Global traffic of the chain kernels goes through buffer resources whose
// extent ends at the chunk's last valid row: loads past it return 0 and
// stores past it are dropped, so ragged last chunks need no branches.

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_mma.h"

namespace gdr {
namespace {

constexpr int DK = 128;       // key dim == value dim
constexpr int LDK = DK + 8;   // pitch (halves) of [*][DK] tiles
constexpr int NTK = DK / 16;  // 16-row tiles of a state strip
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void;
// LDS address of a generic pointer into a __shared__ array: its low 32 bits
// (the shared aperture's base is 4 GB aligned), with no null check.
__device__ __forceinline__ lds_void lds_addr(const void* p) {
  return (lds_void)(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Byte sizes of the images (all multiples of 16).
template <int C>
struct Img {
  static constexpr int LDC = C + 8;                // pitch (halves) of [*][C] tiles
  static constexpr uint32_t KN = C * LDK * 2;      // Kn or Qn    [C][LDK]
  static constexpr uint32_t KEY = 2 * KN;          // Kn | Qn
  static constexpr uint32_t GT = 4 * C * 4;        // gam | lam | beta | G2
  static constexpr uint32_t TM = C * LDC * 2;      // one C x C tile
  static constexpr uint32_t CHK = GT + 2 * TM;     // gates | T | P
};

struct K16 {
  const bf16_t *q, *k, *v, *dout;
  const float *g, *beta, *h0, *dht;
  void* o;
  float* ht;
  void* dv;
  float* dh0;
  char *kimg, *cimg;       // [B][Hk][NC] key images, [B][Hv][NC] chunk images
  char* pkimg;             // channelwise VJP: [B][Hk][NC] unscaled key images (K_hat | Q_hat, norm factors)
  _Float16 *hst, *dhst;    // [B][Hv][NC][DK][DK]: chunk-entry H, chunk-end dH
  float *pdq, *pdk;        // dq_hat / dk_hat over a group's v-heads: running-sum tiles per (b, chunk, k-head)
                           // in the gradient kernel's lane order, or, split launch, rows [B][T][Hv][DK]
  void *dq, *dk;           // [B][T][Hk][DK] out dtype
  float *dg, *dbeta;       // [B][T][Hv]
  int64_t B, T;
  int Hk, Hv, NC, l2;
  int fg;                  // fused gate activation: g, beta hold pre-activations
  const int64_t* cu;       // ragged batch: sequence b is rows cu[b] .. cu[b+1) (null: rows b*T .. b*T+T)
};

// Sequence b of the batch: its first token row and its length.  A ragged
// batch gives row offsets cu[0..B] (each length clamped to [0, T]: the
// workspace holds ceil(T / C) chunks per sequence); otherwise sequence b is
// rows b * T .. b * T + T - 1.
struct SeqSpan {
  int64_t t0, len;
};
__device__ __forceinline__ SeqSpan seq_span(const K16& a, int64_t b) {
  if (!a.cu) return SeqSpan{b * a.T, a.T};
  const int64_t s0 = a.cu[b], n = a.cu[b + 1] - s0;
  return SeqSpan{s0, n < 0 ? 0 : (n > a.T ? a.T : n)};
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// Wave index as a scalar (wave-uniform by construction).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(nbytes), 0x00020000);
}

__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// Copy by NTH threads (thread tid of the group, in its wave wq) of NBYTES
// from buffer r (byte offset off) into LDS at dst, without registers:
// 16-byte unit e travels in lane e % 64 of wave (e / 64) % (NTH / 64) during
// round e / NTH (buffer_load_dwordx4 ... lds writes the wave's 64 units to
// consecutive LDS addresses).  Completion is observed by wait_all() followed
// by a barrier.
template <int NBYTES, int NTH>
__device__ __forceinline__ void dma(rsrc_t r, uint32_t off, char* dst, int tid, int w) {
  static_assert(NBYTES % 16 == 0, "images are made of 16-byte units");
  constexpr int N16 = NBYTES / 16;
#pragma unroll
  for (int u = 0; u < (N16 + NTH - 1) / NTH; ++u) {
    if (N16 % NTH == 0 || NTH * u + tid < N16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_addr(dst + 16 * (NTH * u + 64 * w)), 16, off + 16 * tid,
                                               16 * NTH * u, 0, 0);
  }
}

__device__ __forceinline__ f16x8 ld8(const _Float16* p) { return *reinterpret_cast<const f16x8*>(p); }

// Eight consecutive fp32 values at p (16-byte aligned).
__device__ __forceinline__ void ld8f(float (&x)[8], const float* p) {
  const float4 a0 = *reinterpret_cast<const float4*>(p), a1 = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
  x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
}

// A fragment of A[m][k] (k contiguous) for the relabelled 32-column block kb:
// elements 0..3 <- k = 32kb + 4g + 0..3, 4..7 <- 32kb + 16 + 4g + 0..3.
__device__ __forceinline__ f16x8 perm_frag(const _Float16* A, int ld, int m, int kb) {
  const int g = lane_id() >> 4;
  const f16x4 lo = *reinterpret_cast<const f16x4*>(A + m * ld + 32 * kb + 4 * g);
  const f16x4 hi = *reinterpret_cast<const f16x4*>(A + m * ld + 32 * kb + 16 + 4 * g);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Transposed reads.  ds_read_b64_tr_b16 treats each 16-lane group as one
// unit: lane p of the group names 4 consecutive halves (its row of a 16 x 4
// block D[p][0..3]) and receives D[p/4 + 4i][p%4], i = 0..3.  Pointing lane p
// at row k0 + p/4, columns n0 + 4(p%4) .. +3 of a row-major M[k][n] thus
// hands lane p the column n0 + p of rows k0 .. k0+3: a k-run of M^T.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f16x4 tr4(const _Float16* M, int ld, int k0, int n0) {
  const int p = lane_id() & 15;
  const _Float16* src = M + (k0 + (p >> 2)) * ld + n0 + 4 * (p & 3);
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src));
}

// perm_frag of A = M^T (A[m][k] = M[k][m], M row-major) for rows m0 + (lane & 15).
__device__ __forceinline__ f16x8 perm_frag_t(const _Float16* M, int ld, int m0, int kb) {
  const int g = lane_id() >> 4;
  const f16x4 lo = tr4(M, ld, 32 * kb + 4 * g, m0);
  const f16x4 hi = tr4(M, ld, 32 * kb + 16 + 4 * g, m0);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Plain-order fragment (k = k0 + 8g .. k0 + 8g + 7) of column n0 + (lane & 15)
// of a row-major M[k][n]: the A fragment of M^T, or the B fragment of M.
__device__ __forceinline__ f16x8 frag_t(const _Float16* M, int ld, int k0, int n0) {
  const int g = lane_id() >> 4;
  const f16x4 lo = tr4(M, ld, k0 + 8 * g, n0);
  const f16x4 hi = tr4(M, ld, k0 + 8 * g + 4, n0);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Key-ordered tiles.  The key images store each row's columns in the order
// the chained fragments consume them: 16-byte unit 4kb + g of a row holds
// the columns 32kb + 4g .. +3 and 32kb + 16 + 4g .. +3 (the row pad, unit
// DK / 8, is unchanged).  An A fragment of a chained product is then one
// 16-byte read (plain 8-byte pairs read at half the rate), and a transposed
// read names its four columns from the unit order.
__device__ __forceinline__ f16x8 key_unit(const _Float16* row, int u) {  // unit u < DK / 8 of a natural row
  const int kb = u >> 2, g = u & 3;
  const f16x4 lo = *reinterpret_cast<const f16x4*>(row + 32 * kb + 4 * g);
  const f16x4 hi = *reinterpret_cast<const f16x4*>(row + 32 * kb + 16 + 4 * g);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// perm_frag of a key-ordered A.
__device__ __forceinline__ f16x8 kfrag(const _Float16* A, int ld, int m, int kb) {
  return ld8(A + m * ld + 32 * kb + 8 * (lane_id() >> 4));
}
// tr4 of a key-ordered M (n0 a multiple of 16): lane p of the group names
// the unit half holding natural columns n0 + 4(p % 4) .. +3, so it receives
// natural column n0 + p of rows k0 .. k0 + 3, as tr4 does on a natural M.
__device__ __forceinline__ f16x4 tr4k(const _Float16* M, int ld, int k0, int n0) {
  const int p = lane_id() & 15;
  const _Float16* src = M + (k0 + (p >> 2)) * ld + (n0 & ~31) + 8 * (p & 3) + 4 * ((n0 >> 4) & 1);
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src));
}
__device__ __forceinline__ f16x8 perm_frag_tk(const _Float16* M, int ld, int m0, int kb) {
  const int g = lane_id() >> 4;
  const f16x4 lo = tr4k(M, ld, 32 * kb + 4 * g, m0);
  const f16x4 hi = tr4k(M, ld, 32 * kb + 16 + 4 * g, m0);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ f16x8 frag_tk(const _Float16* M, int ld, int k0, int n0) {
  const int g = lane_id() >> 4;
  const f16x4 lo = tr4k(M, ld, k0 + 8 * g, n0);
  const f16x4 hi = tr4k(M, ld, k0 + 8 * g + 4, n0);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Four bf16 values carried as the 16-bit halves of a transpose-read result,
// widened to fp32.  The halves are taken from the two 32-bit words: a
// bit_cast of a single vector element would read the vector's first element.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void bf16x4_to_f32(float (&x)[4], f16x4 h) {
  const u32x2 u = __builtin_bit_cast(u32x2, h);
  x[0] = __uint_as_float(u[0] << 16);
  x[1] = __uint_as_float(u[0] & 0xffff0000u);
  x[2] = __uint_as_float(u[1] << 16);
  x[3] = __uint_as_float(u[1] & 0xffff0000u);
}

// Chained B fragments of a strip x[t][e] (rows 16t + 4g + e of this lane).
template <int NT>
__device__ __forceinline__ void chain_frags(f16x8 (&bf)[NT / 2], const f32x4 (&x)[NT]) {
#pragma unroll
  for (int kb = 0; kb < NT / 2; ++kb)
    bf[kb] = f16x8{static_cast<_Float16>(x[2 * kb][0]), static_cast<_Float16>(x[2 * kb][1]),
                   static_cast<_Float16>(x[2 * kb][2]), static_cast<_Float16>(x[2 * kb][3]),
                   static_cast<_Float16>(x[2 * kb + 1][0]), static_cast<_Float16>(x[2 * kb + 1][1]),
                   static_cast<_Float16>(x[2 * kb + 1][2]), static_cast<_Float16>(x[2 * kb + 1][3])};
}

// Zero pattern of a square C x C operand by 16-row blocks: products of
// row tile t with the k-block pair kb (columns 32kb .. 32kb + 31) that only
// meet zero blocks are skipped.  kLower: A is zero above its diagonal blocks
// (T, P, the masked dP); kUpper: zero below them (their transposes).
enum Tri { kFull = 0, kLower = 1, kUpper = 2 };
template <int TRI>
__device__ __forceinline__ constexpr bool tri_skip(int t, int kb) {
  return (TRI == kLower && 2 * kb > t) || (TRI == kUpper && 2 * kb + 1 < t);
}

// acc[t] += A[16t : 16t+16, 0 : 16 NT] X for t < NO, X chained as bf.
template <int NO, int NT, int TRI = kFull, bool KP = false>
__device__ __forceinline__ void mma_chain_rows(f32x4 (&acc)[NO], const _Float16* A, int ld, const f16x8 (&bf)[NT / 2]) {
  const int m = lane_id() & 15;
#pragma unroll
  for (int kb = 0; kb < NT / 2; ++kb) {
    f16x8 af[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t)
      if (!tri_skip<TRI>(t, kb)) af[t] = KP ? kfrag(A, ld, 16 * t + m, kb) : perm_frag(A, ld, 16 * t + m, kb);
#pragma unroll
    for (int t = 0; t < NO; ++t)
      if (!tri_skip<TRI>(t, kb)) acc[t] = F16Op::mma(af[t], bf[kb], acc[t]);
  }
}

// mma_chain_rows for two chained operands sharing A: acc1 += A X1, acc2 += A X2.
template <int NO, int NT, bool KP = false>
__device__ __forceinline__ void mma_chain_rows2(f32x4 (&acc1)[NO], f32x4 (&acc2)[NO], const _Float16* A, int ld,
                                                const f16x8 (&bf1)[NT / 2], const f16x8 (&bf2)[NT / 2]) {
  const int m = lane_id() & 15;
#pragma unroll
  for (int kb = 0; kb < NT / 2; ++kb) {
    f16x8 af[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t) af[t] = KP ? kfrag(A, ld, 16 * t + m, kb) : perm_frag(A, ld, 16 * t + m, kb);
#pragma unroll
    for (int t = 0; t < NO; ++t) {
      acc1[t] = F16Op::mma(af[t], bf1[kb], acc1[t]);
      acc2[t] = F16Op::mma(af[t], bf2[kb], acc2[t]);
    }
  }
}

// mma_chain_rows with A = M^T, M row-major [16 NT][ld] (TRI describes A; KP: M key-ordered).
template <int NO, int NT, int TRI = kFull, bool KP = false>
__device__ __forceinline__ void mma_chain_rows_t(f32x4 (&acc)[NO], const _Float16* M, int ld,
                                                 const f16x8 (&bf)[NT / 2]) {
#pragma unroll
  for (int kb = 0; kb < NT / 2; ++kb) {
    f16x8 af[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t)
      if (!tri_skip<TRI>(t, kb)) af[t] = KP ? perm_frag_tk(M, ld, 16 * t, kb) : perm_frag_t(M, ld, 16 * t, kb);
#pragma unroll
    for (int t = 0; t < NO; ++t)
      if (!tri_skip<TRI>(t, kb)) acc[t] = F16Op::mma(af[t], bf[kb], acc[t]);
  }
}

// acc[t] += A[m0 : m0+16, 0:K] B[:, nb + 16t : nb + 16t + 16]; B^T rows from
// Bt (k contiguous); the A fragment is shared.
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

// mma_cols with A = M^T (A[m][k] = M[k][m], M row-major).
template <int NCOL, int K>
__device__ __forceinline__ void mma_cols_t(f32x4 (&acc)[NCOL], const _Float16* M, int ldm, int m0, const _Float16* Bt,
                                           int ldb, int nb) {
  const int r = lane_id() & 15, kl = (lane_id() >> 4) * 8;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const f16x8 af = frag_t(M, ldm, k0, m0);
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

// With ON, x passes through an empty asm statement, so the compiler cannot
// treat what is derived from it as loop invariant: addresses built from the
// lane index inside a loop are rebuilt there instead of being held in
// registers across the whole loop body.
template <bool ON>
__device__ __forceinline__ int opaque_v(int x) {
  if constexpr (ON) asm volatile("" : "+v"(x));
  return x;
}
template <bool ON>
__device__ __forceinline__ int opaque_s(int x) {
  if constexpr (ON) asm volatile("" : "+s"(x));
  return x;
}

// Stores this lane's strip rows 16tr + 4g + e as TO through buffer r (rows
// rowb bytes apart, voff = byte offset of row 4g at the lane's column);
// rows past the buffer end are dropped.  voff is held as is, so each store
// adds one uniform row offset to it (left free, the compiler folds the
// lane's row into a multiply by rowb at every store).
template <typename TO, int NT>
__device__ __forceinline__ void store_strip_buf(rsrc_t r, uint32_t voff, uint32_t rowb, const f32x4 (&x)[NT]) {
  const uint32_t v0 = static_cast<uint32_t>(opaque_v<true>(static_cast<int>(voff)));
#pragma unroll
  for (int tr = 0; tr < NT; ++tr)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t off = v0 + (16 * tr + e) * rowb;
      if constexpr (std::is_same_v<TO, float>) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[tr][e]), r, off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[tr][e])), r, off, 0,
                                              0);
      }
    }
}

// The sequence of rank r when the sequences of a ragged batch of at most 64
// are ordered by decreasing length (equal lengths by index).  Lane j holds
// sequence j's length; each lane counts the sequences ahead of its own.
constexpr int kMaxRankedSeqs = 64;
__device__ __forceinline__ int64_t seq_by_length(const K16& a, int r) {
  const int lane = lane_id(), nb = static_cast<int>(a.B);
  const int len = lane < nb ? static_cast<int>(seq_span(a, lane).len) : -1;
  int rank = 0;
  for (int j = 0; j < nb; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
  }
  const unsigned long long m = __ballot(lane < nb && rank == r);
  return m ? __builtin_ctzll(m) : r;  // exactly one lane matches for 0 <= r < B
}

// Chunk c of sequence b for the workgroup of an (NC, heads, B) grid.
// Without a ragged batch, or with more than 64 sequences, block (x, z) is
// chunk x of sequence z (possibly past its end).  A ragged batch of at most
// 64 numbers its chunks in sequence order and block (x, z) takes chunk
// x + NC z of that list: the blocks past the batch's last chunk are then
// the last ones dispatched (they get c = NC, past every sequence's end)
// instead of holding a CU between real chunks, which costs the gradient
// kernels (one workgroup per CU) about 15% on a ragged batch of half-empty
// rows; the prep kernels, four and two workgroups per CU, keep the plain
// order, which measured slightly faster for them.
struct ChunkPos {
  int c;
  int64_t b;
};
__device__ __forceinline__ ChunkPos chunk_pos(const K16& a, int C) {
  ChunkPos p{static_cast<int>(blockIdx.x), static_cast<int64_t>(blockIdx.z)};
  if (!a.cu || a.B > kMaxRankedSeqs) return p;
  const int lane = lane_id(), nb = static_cast<int>(a.B);
  const int nch = lane < nb ? static_cast<int>((seq_span(a, lane).len + C - 1) / C) : 0;
  const int incl = wave_prefix_sum(nch);  // chunks of sequences 0 .. lane
  const int excl = incl - nch;
  const int idx = static_cast<int>(blockIdx.x) + a.NC * static_cast<int>(blockIdx.z);
  const unsigned long long m = __ballot(lane < nb && excl <= idx && idx < incl);
  if (!m) {
    p.c = a.NC;
    p.b = 0;
    return p;
  }
  const int bb = __builtin_ctzll(m);
  p.b = bb;
  p.c = idx - __builtin_amdgcn_readlane(excl, bb);
  return p;
}

// Chain workgroup -> (b, v-head, value slice), nsl slices per v-head.
// Workgroups are dealt to the eight XCDs round robin.  The remap keeps the
// gs = nsl * Hv / Hk workgroups of a (b, k-head) group, which read one key
// image (and the nsl that read one chunk image), on one XCD, so they share
// its L2, and deals the groups to the XCDs in turn, so every XCD holds an
// eighth of every sequence's groups (a ragged batch's long sequences do not
// pile onto one XCD).  A ragged batch of at most 64 sequences takes them
// longest first (the dispatch order follows the block index), so the chains
// that end last are short ones.
struct ChainPos {
  int slice, hv, kh;
  int64_t b;
};
__device__ __forceinline__ ChainPos chain_pos(const K16& a, int nsl) {
  const int nb = gridDim.x, l0 = blockIdx.x;
  const int gs = nsl * (a.Hv / a.Hk);
  int lg = l0;
  if (nb % (8 * gs) == 0) {
    const int x = l0 % 8, slot = l0 / 8;  // XCD, and the workgroup's place in its list
    lg = (x + 8 * (slot / gs)) * gs + slot % gs;
  }
  ChainPos p;
  p.slice = lg % nsl;
  p.hv = (lg / nsl) % a.Hv;
  p.b = (lg / nsl) / a.Hv;
  if (a.cu && a.B <= kMaxRankedSeqs) p.b = seq_by_length(a, static_cast<int>(p.b));
  p.kh = p.hv / (a.Hv / a.Hk);
  return p;
}

// ---------------------------------------------------------------------------
// prep16: one workgroup (4 waves) per (chunk, v-head, b).
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint4 sel4(bool ok, uint4 x) { return ok ? x : uint4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ void unpack8(const uint4& u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Rows of q or k (thread -> row tid / TPR, elements part * EPT ..), each
// scaled by r = (sum x^2 + eps)^(-1/2) over Dk when l2 is set (the L2 norm
// the Megatron-LM page folds into the kernel), written as fp16 to
// dst[r][LDK]; the row's pad (halves DK .. DK+7) holds r as fp32 bits, then
// zeros (r = 1 when l2 is not set).
template <int C, int NV, int NTH = 256>
__device__ __forceinline__ void norm_rows(_Float16* dst, const uint4 (&raw)[NV], int l2) {
  constexpr int TPR = NTH / C, EPT = DK / TPR;
  const int tid = threadIdx.x, r = tid / TPR, part = tid % TPR;
  float x[NV][8];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    unpack8(raw[u], x[u]);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[u][i] * x[u][i];
  }
  if constexpr (TPR == 8 || TPR == 16) {
    ss = group_sum_dpp<TPR>(ss);
  } else {
    ss = xsum<1, TPR>(ss);
  }
  const float rn = l2 ? rsqrtf(ss + kL2Eps) : 1.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(x[u][i] * rn);
    *reinterpret_cast<f16x8*>(dst + r * LDK + part * EPT + 8 * u) = h;
  }
  if (part == 0) *reinterpret_cast<uint4*>(dst + r * LDK + DK) = uint4{__float_as_uint(rn), 0u, 0u, 0u};
}

// Writes an image tile of ROWS rows of UPR 16-byte units (the last unit of a
// row is its pad: zeros, or f's values with KEEP_PAD) to global memory;
// f(row, unit) gives the 8 values.
template <int ROWS, int UPR, int NTH = 256, bool KEEP_PAD = false, typename F>
__device__ __forceinline__ void write_tile(char* dst, F&& f) {
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int e = threadIdx.x; e < ROWS * UPR; e += NTH) {
    const int r = e / UPR, u = e % UPR;
    d[e] = (u == UPR - 1 && !KEEP_PAD) ? uint4{0u, 0u, 0u, 0u} : __builtin_bit_cast(uint4, f(r, u));
  }
}

// T = (I + A)^-1 and P for one chunk and v-head; A (strictly lower) and P
// from K K^T and Q K^T on the matrix cores.  The inverse is blocked in
// 16 x 16 tiles: wave w inverts diagonal block w by forward substitution
// (lane = column), then the blocks below the diagonal follow level by level,
//     T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj),
// on fp32 matrix cores; everything is fp32 until the images are written.
template <int C>
__global__ __launch_bounds__(512) void prep16_kernel(K16 a) {
  using IM = Img<C>;
  constexpr int NTH = 512, NW = NTH / 64;
  constexpr int NT = C / 16, LDA = C + 4, LDC = IM::LDC;
  constexpr int TPR = NTH / C, EPT = DK / TPR, NV = EPT / 8;
  static_assert(C * LDC <= C * LDK, "an fp16 [C][LDC] tile fits a key tile's space");
  static_assert(C * LDA * 4 <= C * LDK * 2, "an fp32 [C][LDA] tile fits a key tile's space");
  // 35 KB in all, so four workgroups share a CU.  Two key-tile spaces:
  // Kn, then A (fp32), then the fp16 P tile [C][LDC]; Qn, then the fp32 T
  // (its image is converted to fp16 as it is written).  A and P wait in
  // registers until the spaces are free.
  __shared__ __align__(16) _Float16 Ks[C * LDK];
  __shared__ __align__(16) _Float16 Qs[C * LDK];
  float* A = reinterpret_cast<float*>(Ks);
  float* Tf = reinterpret_cast<float*>(Qs);
  _Float16* Pst = Ks;
  // zeroes the 16-byte units of a [C][LDC] fp16 tile that lie above its
  // 16 x 16 diagonal blocks (no other thread writes them)
  auto zero_upper = [&](_Float16* M) {
    constexpr int UR = LDC / 8;
    for (int e = threadIdx.x; e < C * UR; e += NTH) {
      const int r = e / UR, u = e % UR;
      if (u < C / 8 && u / 2 > r / 16) reinterpret_cast<uint4*>(M)[e] = uint4{0u, 0u, 0u, 0u};
    }
  };
  __shared__ __align__(16) float gates[4 * C];  // gam | lam | beta | G2
  float* gam = gates;
  float* lam = gates + C;
  float* bet = gates + 2 * C;
  float* G2 = gates + 3 * C;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int c = blockIdx.x, hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int grp = a.Hv / a.Hk, kh = hv / grp;
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const SeqSpan sp = seq_span(a, b);
  if (t0 >= sp.len) return;  // past the end of a shorter sequence of a ragged batch
  const int L = static_cast<int>(sp.len - t0 < C ? sp.len - t0 : C);
  {
    const int r = tid / TPR, part = tid % TPR;
    const int rc = r < L ? r : L - 1;
    const int64_t off = ((sp.t0 + t0 + rc) * a.Hk + kh) * DK + part * EPT;
    uint4 kr[NV], qr[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      kr[u] = sel4(r < L, *reinterpret_cast<const uint4*>(a.k + off + 8 * u));
      qr[u] = sel4(r < L, *reinterpret_cast<const uint4*>(a.q + off + 8 * u));
    }
    float gv = 0.f, bv = 0.f;
    if (tid < 64) {
      const int rr = tid < L ? tid : L - 1;
      const int64_t row = (sp.t0 + t0 + rr) * a.Hv + hv;
      gv = a.fg ? fg_log_alpha(a.g[row]) : a.g[row];
      bv = a.fg ? fg_beta(a.beta[row]) : a.beta[row];
      gv = tid < L ? gv : 0.f;
      bv = tid < L ? bv : 0.f;
    }
    norm_rows<C, NV, NTH>(Ks, kr, a.l2);
    norm_rows<C, NV, NTH>(Qs, qr, a.l2);
    if (tid < 64) {  // running sum G over the chunk (g = 0 past the end), then G at the last row
      const float x = wave_prefix_sum(gv);
      const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), L - 1));
      if (lane < C) {
        G2[lane] = x * kLog2e;
        gam[lane] = expf(x);
        lam[lane] = expf(gc - x);
        bet[lane] = bv;
      }
    }
  }
  __syncthreads();
  // A (fp32) and P (fp16), kept in registers, on the NT(NT+1)/2 tiles on or
  // below the diagonal, at most two per wave; each tile's fragments are read
  // before its products
  constexpr int NL = NT * (NT + 1) / 2, KS = DK / 32;
  static_assert(NL <= 2 * NW, "two lower tiles per wave at most");
  auto tile_rc = [](int t, int& tr, int& tc) {
    tr = 0;
    while ((tr + 1) * (tr + 2) / 2 <= t) ++tr;
    tc = t - tr * (tr + 1) / 2;
  };
  f16x4 preg[2];
  f32x4 areg[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int t = w + it * NW;
    if (t >= NL) continue;
    int tr, tc;
    tile_rc(t, tr, tc);
    f16x8 ka[KS], qa[KS], kb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ka[ks] = ld8(Ks + (16 * tr + c16) * LDK + 32 * ks + 8 * g);
      qa[ks] = ld8(Qs + (16 * tr + c16) * LDK + 32 * ks + 8 * g);
      kb[ks] = ld8(Ks + (16 * tc + c16) * LDK + 32 * ks + 8 * g);
    }
    f32x4 kk = zero4(), qk = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kk = F16Op::mma(ka[ks], kb[ks], kk);
      qk = F16Op::mma(qa[ks], kb[ks], qk);
    }
    const int s2 = 16 * tc + c16;
    const float g2s = G2[s2];
    const f32x4 g2r = *reinterpret_cast<const f32x4*>(G2 + 16 * tr + 4 * g);  // rows 16tr + 4g + e
    const f32x4 btr = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * tr + 4 * g + e;
      const float ex = s2 <= r ? __builtin_amdgcn_exp2f(g2r[e] - g2s) : 0.f;
      areg[it][e] = s2 < r ? btr[e] * ex * kk[e] : 0.f;
      preg[it][e] = static_cast<_Float16>(ex * qk[e]);
    }
  }
  // ---- key image (one v-head of each k-head group writes it), while Kn / Qn
  // are intact; each row's pad keeps its norm factor r for the L2-norm VJP
  constexpr int UK = DK / 8 + 1;  // 16-byte units per [*][LDK] row
  if (hv % grp == 0) {
    char* kim = a.kimg + ((b * a.Hk + kh) * a.NC + c) * static_cast<int64_t>(IM::KEY);
    write_tile<C, UK, NTH, true>(kim, [&](int r, int u) { return u < DK / 8 ? key_unit(Ks + r * LDK, u) : ld8(Ks + r * LDK + 8 * u); });
    write_tile<C, UK, NTH, true>(kim + IM::KN, [&](int r, int u) { return u < DK / 8 ? key_unit(Qs + r * LDK, u) : ld8(Qs + r * LDK + 8 * u); });
  }
  __syncthreads();
  // A from registers into the Kn space (only its lower tiles are read)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int t = w + it * NW;
    if (t >= NL) continue;
    int tr, tc;
    tile_rc(t, tr, tc);
#pragma unroll
    for (int e = 0; e < 4; ++e) A[(16 * tr + 4 * g + e) * LDA + 16 * tc + c16] = areg[it][e];
  }
  __syncthreads();
  if (w < NT && lane < 16) {  // diagonal blocks (entries above the diagonal come out 0)
    const int o = 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc[2] = {r == lane ? 1.f : 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2) acc[s2 & 1] -= A[(o + r) * LDA + o + s2] * x[s2];
      x[r] = acc[0] + acc[1];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tf[(o + r) * LDA + o + lane] = x[r];
  }
  __syncthreads();
  for (int d = 1; d < NT; ++d) {  // blocks below the diagonal, one distance at a time
    const int i = d + w;
    if (i < NT) {
      const int j = i - d;
      f32x4 m = zero4();
      for (int k = j; k < i; ++k) {
        // product q takes k = 16k + 4g + q: this lane's four A values are one
        // 16-byte read
        const f32x4 av = *reinterpret_cast<const f32x4*>(A + (16 * i + c16) * LDA + 16 * k + 4 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float bv = Tf[(16 * k + 4 * g + q) * LDA + 16 * j + c16];
          m = F32Op::mma(av[q], bv, m);
        }
      }
      // T_ij = -T_ii m; m's accumulators supply B(k = 4g + e, n) directly
      f32x4 tij = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) tij = F32Op::mma(Tf[(16 * i + c16) * LDA + 16 * i + 4 * g + e], m[e], tij);
#pragma unroll
      for (int e = 0; e < 4; ++e) Tf[(16 * i + 4 * g + e) * LDA + 16 * j + c16] = -tij[e];
    }
    __syncthreads();
  }
  // P from registers into the A space (A is no longer read), zero above its
  // diagonal blocks
  zero_upper(Pst);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int t = w + it * NW;
    if (t >= NL) continue;
    int tr, tc;
    tile_rc(t, tr, tc);
#pragma unroll
    for (int e = 0; e < 4; ++e) Pst[(16 * tr + 4 * g + e) * LDC + 16 * tc + c16] = preg[it][e];
  }
  __syncthreads();

  // ---- chunk image
  char* cim = a.cimg + ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(IM::CHK);
  for (int e = tid; e < C; e += NTH)
    reinterpret_cast<float4*>(cim)[e] = reinterpret_cast<const float4*>(gates)[e];
  constexpr int UC = C / 8 + 1;  // 16-byte units per [*][LDC] row
  // T from the fp32 tile, zero above its diagonal blocks (never written there)
  write_tile<C, UC, NTH>(cim + IM::GT, [&](int r, int u) {
    f16x8 v;
    if (u / 2 > r / 16) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = static_cast<_Float16>(0.f);
    } else {
      float x[8];
      ld8f(x, Tf + r * LDA + 8 * u);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = static_cast<_Float16>(x[q]);
    }
    return v;
  });
  write_tile<C, UC, NTH>(cim + IM::GT + IM::TM, [&](int r, int u) { return ld8(Pst + r * LDC + 8 * u); });
}

// ---------------------------------------------------------------------------
// Chain kernels: NCW compute waves (16 value columns each: a value slice of
// BV = 16 NCW columns) and one producer wave per workgroup, one workgroup
// per (b, v-head, slice).  The compute waves own the state in MFMA
// accumulators and touch only LDS; the producer wave issues all bulk global
// traffic of the chunk loop: it copies the next chunk's images and the rows
// of v / dO for this slice (C x BV bf16) into LDS by buffer_load ... lds,
// and stores the previous chunk's o from an LDS tile [C][LDO] (written from
// the accumulators) as 16-byte rows.  One barrier per chunk; a wave stalled
// on memory issue never holds up the matrix cores.  Chunk states (H for the
// VJP, dH) leave the compute waves as four 16-byte stores per lane in
// chained-fragment order (see frag_off).  The launch takes the widest slice
// whose grid still covers every CU (NCW = 4 from B Hv >= CUs / 2, e.g. B = 4,
// Hv = 32 on 256 CUs; 1 at B = 1): a workgroup's time per chunk is set by its compute
// waves' own chain of products, so narrower slices finish a small batch
// sooner, and by the copy of the next chunk when every CU is copying, so a
// full grid keeps the widest slices (fewest copies of each image).
// ---------------------------------------------------------------------------

// Workgroup barrier that orders LDS accesses only (global stores in flight
// stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Chunk states (H entering a chunk, dH at a chunk's end; fp16) are stored
// per (b, v-head, chunk) as [8][NTK / 2][64][8] halves: entry (wg, kb, lane,
// i) is row 32kb + 16(i / 4) + 4(lane / 16) + i % 4, column 16wg + lane % 16
// of the state, i.e. the chained fragment kb of that lane's 16-column strip.
// Byte offset of this lane's fragment kb of column group wg:
__device__ __forceinline__ uint32_t frag_off(int wg, int kb) {
  return static_cast<uint32_t>(((wg * (NTK / 2) + kb) * 64 + lane_id()) * 16);
}

// Copy by NTH threads (as dma) of rows 0 .. ROWS-1 (RB bytes each, rows rowb
// bytes apart from byte col0 of buffer r) into LDS at dst as a packed
// [ROWS][RB] tile; rows >= L repeat row L - 1 (finite values that the chunk
// algebra multiplies by zero).
template <int ROWS, int RB, int NTH>
__device__ __forceinline__ void dma_rows(rsrc_t r, uint32_t rowb, uint32_t col0, int L, char* dst, int tid, int w) {
  constexpr int UPR = RB / 16, N16 = ROWS * UPR;
  static_assert(N16 % NTH == 0, "whole rounds");
#pragma unroll
  for (int u = 0; u < N16 / NTH; ++u) {
    const int e = NTH * u + tid;
    const int row = e / UPR, cu = e % UPR;
    const int rr = row < L ? row : L - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_addr(dst + 16 * (NTH * u + 64 * w)), 16,
                                             rr * rowb + col0 + 16 * cu, 0, 0, 0);
  }
}

// Rows r0 .. r0+3 of column c0 + (lane & 15) of a packed bf16 [*][ld] tile,
// as fp32, by one transpose read (tr4's lane addressing; the bits are moved,
// not converted).  r0 is the same for the lanes of a 16-lane group, and the
// calling wave has no LDS copies in flight.
__device__ __forceinline__ void tile_col4_bf16(float (&x)[4], const uint16_t* M, int ld, int r0, int c0) {
  bf16x4_to_f32(x, tr4(reinterpret_cast<const _Float16*>(M), ld, r0, c0));
}

// Output tile of one chunk and value slice of BVX columns: [C][LDO] elements of TO.
template <typename TO, int BVX>
struct OutTile {
  static constexpr int LDO = std::is_same_v<TO, float> ? BVX + 4 : BVX + 8;
  static constexpr int UPR = BVX * static_cast<int>(sizeof(TO)) / 16;  // 16-byte units per row
  template <int C>
  static constexpr uint32_t bytes() { return C * LDO * sizeof(TO); }
};

// This lane's strip rows 16tr + 4g + e of column col into the output tile.
template <typename TO, int NT, int BVX>
__device__ __forceinline__ void put_strip(char* os, int col, const f32x4 (&x)[NT]) {
  constexpr int LDO = OutTile<TO, BVX>::LDO;
  const int g = lane_id() >> 4;
#pragma unroll
  for (int tr = 0; tr < NT; ++tr)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = (16 * tr + 4 * g + e) * LDO + col;
      if constexpr (std::is_same_v<TO, float>)
        reinterpret_cast<float*>(os)[i] = x[tr][e];
      else
        reinterpret_cast<uint16_t*>(os)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[tr][e]));
    }
}

// One wave stores the output tile's rows to buffer r (rows rowb bytes apart
// from byte col0); rows past the buffer end are dropped.
template <typename TO, int C, int BVX>
__device__ __forceinline__ void flush_tile(const char* os, rsrc_t r, uint32_t rowb, uint32_t col0) {
  constexpr int LDO = OutTile<TO, BVX>::LDO, UPR = OutTile<TO, BVX>::UPR, N16 = C * UPR;
  static_assert(N16 % 64 == 0, "whole wave rounds");
  const int lane = lane_id();
#pragma unroll
  for (int u = 0; u < N16 / 64; ++u) {
    const int e = 64 * u + lane, row = e / UPR, cu = e % UPR;
    const u32x4 val = *reinterpret_cast<const u32x4*>(os + row * LDO * sizeof(TO) + 16 * cu);
    __builtin_amdgcn_raw_buffer_store_b128(val, r, row * rowb + col0 + 16 * cu, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// chain16: forward pass over chunks (WRITE_O: outputs; STORE_H: every
// chunk's entry state for the VJP).  Per chunk and compute wave:
//   Y = Kn H, Z = Qn H          (16 MFMA each, H chained)
//   U = T (beta (V - gam Y))    (8, chained)
//   O = gam Z + P U             (8, chained)
//   H = gam_C H + Kn^T (lam U)  (16, chained)
// ---------------------------------------------------------------------------
template <int C, typename TO, bool WRITE_O, bool STORE_H, int NCW>
__global__ __launch_bounds__(64 * (NCW + 1)) void chain16_kernel(K16 a) {
  constexpr int BV = 16 * NCW, NSL = DK / BV;  // value columns of a workgroup, workgroups per v-head
  using IM = Img<C>;
  constexpr int NT = C / 16, LDC = IM::LDC;
  constexpr uint32_t CB = WRITE_O ? IM::CHK : IM::GT + IM::TM;  // gates | T (| P)
  constexpr uint32_t KB = WRITE_O ? IM::KEY : IM::KN;           // Kn (| Qn)
  constexpr uint32_t VB = C * BV * 2;                           // v tile [C][BV] bf16
  constexpr uint32_t OB = WRITE_O ? OutTile<TO, BV>::template bytes<C>() : 16;
  __shared__ __align__(16) char bufA[CB + KB + VB];
  __shared__ __align__(16) char bufB[CB + KB + VB];
  __shared__ __align__(16) char osA[OB];
  __shared__ __align__(16) char osB[OB];

  const int w = wave_id(), lane = lane_id(), g = lane >> 4, c16 = lane & 15;
  const ChainPos p = chain_pos(a, NSL);
  const SeqSpan sp = seq_span(a, p.b);
  const int nc = static_cast<int>((sp.len + C - 1) / C);
  if (nc == 0) {  // empty sequence of a ragged batch: the state passes through
    if (w < NCW && a.ht) {
      const int64_t base = (p.b * a.Hv + p.hv) * DK * DK + p.slice * BV + 16 * w + c16;
      for (int i = 0; i < DK; ++i) a.ht[base + i * DK] = a.h0 ? a.h0[base + i * DK] : 0.f;
    }
    return;
  }
  auto rows_of = [&](int c) { return static_cast<int>(sp.len - static_cast<int64_t>(c) * C < C ? sp.len - static_cast<int64_t>(c) * C : C); };
  auto seq_rsrc = [&](const void* base, int esize, int c, uint32_t rowb) {
    const char* p0 = static_cast<const char*>(base) + (sp.t0 + static_cast<int64_t>(c) * C) * a.Hv * DK * esize;
    return make_rsrc(p0, static_cast<uint32_t>(rows_of(c)) * rowb);
  };
  const uint32_t rowv = static_cast<uint32_t>(a.Hv) * DK * 2;         // bf16 row pitch of v
  const uint32_t rowo = static_cast<uint32_t>(a.Hv) * DK * sizeof(TO);  // row pitch of o

  if (w == NCW) {  // ---- producer wave
    const char* kim0 = a.kimg + (p.b * a.Hk + p.kh) * a.NC * static_cast<int64_t>(IM::KEY);
    const char* cim0 = a.cimg + (p.b * a.Hv + p.hv) * a.NC * static_cast<int64_t>(IM::CHK);
    const uint32_t colv = (p.hv * DK + p.slice * BV) * 2;
    const uint32_t colo = (p.hv * DK + p.slice * BV) * static_cast<uint32_t>(sizeof(TO));
    auto stage = [&](int c, char* buf) {
      dma<CB, 64>(make_rsrc(cim0 + c * static_cast<int64_t>(IM::CHK), CB), 0, buf, lane, 0);
      dma<KB, 64>(make_rsrc(kim0 + c * static_cast<int64_t>(IM::KEY), KB), 0, buf + CB, lane, 0);
      dma_rows<C, BV * 2, 64>(seq_rsrc(a.v, 2, c, rowv), rowv, colv, rows_of(c), buf + CB + KB, lane, 0);
    };
    auto pstep = [&](int c, char* nxt, const char* os_prev) __attribute__((always_inline)) {
      if (c + 1 < nc) stage(c + 1, nxt);
      if constexpr (WRITE_O) {
        if (c > 0) flush_tile<TO, C, BV>(os_prev, seq_rsrc(a.o, sizeof(TO), c - 1, rowo), rowo, colo);
      }
      wait_all();
      lds_barrier();
    };
    stage(0, bufA);
    wait_all();
    lds_barrier();
    for (int c = 0; c < nc; c += 2) {
      pstep(c, bufB, osB);
      if (c + 1 < nc) pstep(c + 1, bufA, osA);
    }
    if constexpr (WRITE_O)
      flush_tile<TO, C, BV>(((nc - 1) & 1) ? osB : osA, seq_rsrc(a.o, sizeof(TO), nc - 1, rowo), rowo, colo);
    return;
  }

  // ---- compute waves
  const int jcol = p.slice * BV + 16 * w + c16;  // this lane's state column
  const int wg = p.slice * NCW + w;              // column group of the chunk-state layout
  const int64_t hbase = (p.b * a.Hv + p.hv) * DK * DK + jcol;
  f32x4 h[NTK];
#pragma unroll
  for (int ti = 0; ti < NTK; ++ti) {
    h[ti] = zero4();
    if (a.h0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) h[ti][e] = a.h0[hbase + (16 * ti + 4 * g + e) * DK];
    }
  }
  lds_barrier();

  auto step = [&](int c, const char* cur, char* os) __attribute__((always_inline)) {
    const float* gam = reinterpret_cast<const float*>(cur);
    const float* lam = gam + C;
    const float* bet = gam + 2 * C;
    const _Float16* Tm = reinterpret_cast<const _Float16*>(cur + IM::GT);
    const _Float16* Pm = Tm + C * LDC;
    const _Float16* Kn = reinterpret_cast<const _Float16*>(cur + CB);
    const _Float16* Qn = Kn + C * LDK;
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(cur + CB + KB);

    f16x8 hf[NTK / 2];
    chain_frags<NTK>(hf, h);
    f32x4 y[NT], u[NT], o[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = u[t] = zero4();
    mma_chain_rows<NT, NTK, kFull, true>(y, Kn, LDK, hf);
    if constexpr (WRITE_O) {
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] = zero4();
      mma_chain_rows<NT, NTK, kFull, true>(o, Qn, LDK, hf);
    }
    if constexpr (STORE_H) {  // entry state of chunk c
      const rsrc_t hr = make_rsrc(a.hst + ((p.b * a.Hv + p.hv) * a.NC + c) * static_cast<int64_t>(DK * DK), DK * DK * 2);
#pragma unroll
      for (int kb = 0; kb < NTK / 2; ++kb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hf[kb]), hr, frag_off(wg, kb), 0, 0);
    }
    f32x4 rhs[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gam + 16 * tr + 4 * g);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
      float vv[4];
      tile_col4_bf16(vv, Vs, BV, 16 * tr + 4 * g, 16 * w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rhs[tr][e] = bv[e] * (vv[e] - gv[e] * y[tr][e]);
        if constexpr (WRITE_O) o[tr][e] *= gv[e];
      }
    }
    f16x8 bf[NT / 2];
    chain_frags<NT>(bf, rhs);
    mma_chain_rows<NT, NT, kLower>(u, Tm, LDC, bf);
    if constexpr (WRITE_O) {
      chain_frags<NT>(bf, u);
      mma_chain_rows<NT, NT, kLower>(o, Pm, LDC, bf);
    }
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const f32x4 lv = *reinterpret_cast<const f32x4*>(lam + 16 * tr + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[tr][e] *= lv[e];
    }
    chain_frags<NT>(bf, u);
    const float gc = gam[rows_of(c) - 1];
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti) h[ti] = h[ti] * gc;
    mma_chain_rows_t<NTK, NT, kFull, true>(h, Kn, LDK, bf);
    if constexpr (WRITE_O) put_strip<TO, NT, BV>(os, 16 * w + c16, o);
    lds_barrier();
  };
  for (int c = 0; c < nc; c += 2) {
    step(c, bufA, osA);
    if (c + 1 < nc) step(c + 1, bufB, osB);
  }
  if (a.ht) {
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.ht[hbase + (16 * ti + 4 * g + e) * DK] = h[ti][e];
  }
}

// ---------------------------------------------------------------------------
// dh16: reverse pass carrying dH.  Per chunk and compute wave:
//   dU   = lam (Kn dH) + P^T dO           (16 + 8 MFMA, chained)
//   dRHS = T^T dU                         (8, chained)
//   dH   = gam_C dH + Qn^T (gam dO) - Kn^T (beta gam dRHS)   (16 + 16, chained)
// Every chunk's incoming dH (the gradient at its end) is stored for grad16,
// which also forms dv = beta dRHS.
// ---------------------------------------------------------------------------
template <int C, typename TO, int NCW>
__global__ __launch_bounds__(64 * (NCW + 1)) void dh16_kernel(K16 a) {
  constexpr int BV = 16 * NCW, NSL = DK / BV;
  using IM = Img<C>;
  constexpr int NT = C / 16, LDC = IM::LDC;
  constexpr uint32_t CB = IM::CHK;  // gates | T | P
  constexpr uint32_t KB = IM::KEY;  // Kn | Qn
  constexpr uint32_t VB = C * BV * 2;
  __shared__ __align__(16) char bufA[CB + KB + VB];
  __shared__ __align__(16) char bufB[CB + KB + VB];

  const int w = wave_id(), lane = lane_id(), g = lane >> 4, c16 = lane & 15;
  const ChainPos p = chain_pos(a, NSL);
  const SeqSpan sp = seq_span(a, p.b);
  const int nc = static_cast<int>((sp.len + C - 1) / C);
  if (nc == 0) {  // empty sequence of a ragged batch: the state passes through
    if (w < NCW && a.dh0) {
      const int64_t base = (p.b * a.Hv + p.hv) * DK * DK + p.slice * BV + 16 * w + c16;
      for (int i = 0; i < DK; ++i) a.dh0[base + i * DK] = a.dht ? a.dht[base + i * DK] : 0.f;
    }
    return;
  }
  auto rows_of = [&](int c) { return static_cast<int>(sp.len - static_cast<int64_t>(c) * C < C ? sp.len - static_cast<int64_t>(c) * C : C); };
  auto seq_rsrc = [&](const void* base, int esize, int c, uint32_t rowb) {
    const char* p0 = static_cast<const char*>(base) + (sp.t0 + static_cast<int64_t>(c) * C) * a.Hv * DK * esize;
    return make_rsrc(p0, static_cast<uint32_t>(rows_of(c)) * rowb);
  };
  const uint32_t rowv = static_cast<uint32_t>(a.Hv) * DK * 2;

  if (w == NCW) {  // ---- producer wave: chunks NC-1, NC-2, ...
    const char* kim0 = a.kimg + (p.b * a.Hk + p.kh) * a.NC * static_cast<int64_t>(IM::KEY);
    const char* cim0 = a.cimg + (p.b * a.Hv + p.hv) * a.NC * static_cast<int64_t>(IM::CHK);
    const uint32_t colv = (p.hv * DK + p.slice * BV) * 2;
    auto stage = [&](int c, char* buf) {
      dma<CB, 64>(make_rsrc(cim0 + c * static_cast<int64_t>(IM::CHK), CB), 0, buf, lane, 0);
      dma<KB, 64>(make_rsrc(kim0 + c * static_cast<int64_t>(IM::KEY), KB), 0, buf + CB, lane, 0);
      dma_rows<C, BV * 2, 64>(seq_rsrc(a.dout, 2, c, rowv), rowv, colv, rows_of(c), buf + CB + KB, lane, 0);
    };
    auto pstep = [&](int c, char* nxt) __attribute__((always_inline)) {
      if (c > 0) stage(c - 1, nxt);
      wait_all();
      lds_barrier();
    };
    stage(nc - 1, bufA);
    wait_all();
    lds_barrier();
    for (int i = 0; i < nc; i += 2) {
      pstep(nc - 1 - i, bufB);
      if (i + 1 < nc) pstep(nc - 2 - i, bufA);
    }
    return;
  }

  // ---- compute waves
  const int jcol = p.slice * BV + 16 * w + c16;
  const int wg = p.slice * NCW + w;
  const int64_t hbase = (p.b * a.Hv + p.hv) * DK * DK + jcol;
  f32x4 dh[NTK];
#pragma unroll
  for (int ti = 0; ti < NTK; ++ti) {
    dh[ti] = zero4();
    if (a.dht) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dh[ti][e] = a.dht[hbase + (16 * ti + 4 * g + e) * DK];
    }
  }
  lds_barrier();

  auto step = [&](int c, const char* cur) __attribute__((always_inline)) {
    const float* gam = reinterpret_cast<const float*>(cur);
    const float* lam = gam + C;
    const float* bet = gam + 2 * C;
    const _Float16* Tm = reinterpret_cast<const _Float16*>(cur + IM::GT);
    const _Float16* Pm = Tm + C * LDC;
    const _Float16* Kn = reinterpret_cast<const _Float16*>(cur + CB);
    const _Float16* Qn = Kn + C * LDK;
    const uint16_t* Ds = reinterpret_cast<const uint16_t*>(cur + CB + KB);

    f16x8 hf[NTK / 2];
    chain_frags<NTK>(hf, dh);
    f32x4 du[NT], dr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) du[t] = dr[t] = zero4();
    mma_chain_rows<NT, NTK, kFull, true>(du, Kn, LDK, hf);
    {  // gradient at this chunk's end
      const rsrc_t hr = make_rsrc(a.dhst + ((p.b * a.Hv + p.hv) * a.NC + c) * static_cast<int64_t>(DK * DK), DK * DK * 2);
#pragma unroll
      for (int kb = 0; kb < NTK / 2; ++kb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hf[kb]), hr, frag_off(wg, kb), 0, 0);
    }
    f32x4 dof[NT], gdo[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const f32x4 lv = *reinterpret_cast<const f32x4*>(lam + 16 * tr + 4 * g);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gam + 16 * tr + 4 * g);
      float x[4];
      tile_col4_bf16(x, Ds, BV, 16 * tr + 4 * g, 16 * w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        du[tr][e] *= lv[e];
        dof[tr][e] = x[e];
        gdo[tr][e] = gv[e] * x[e];
      }
    }
    f16x8 bf[NT / 2];
    chain_frags<NT>(bf, dof);
    mma_chain_rows_t<NT, NT, kUpper>(du, Pm, LDC, bf);
    chain_frags<NT>(bf, du);
    mma_chain_rows_t<NT, NT, kUpper>(dr, Tm, LDC, bf);
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gam + 16 * tr + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) dr[tr][e] = -gv[e] * bv[e] * dr[tr][e];
    }
    const float gc = gam[rows_of(c) - 1];
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti) dh[ti] = dh[ti] * gc;
    chain_frags<NT>(bf, gdo);
    mma_chain_rows_t<NTK, NT, kFull, true>(dh, Qn, LDK, bf);
    chain_frags<NT>(bf, dr);
    mma_chain_rows_t<NTK, NT, kFull, true>(dh, Kn, LDK, bf);
    lds_barrier();
  };
  // chunks NC-1, NC-2, ... alternate between the two buffers
  for (int i = 0; i < nc; i += 2) {
    step(nc - 1 - i, bufA);
    if (i + 1 < nc) step(nc - 2 - i, bufB);
  }
  if (a.dh0) {
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.dh0[hbase + (16 * ti + 4 * g + e) * DK] = dh[ti][e];
  }
}

// ---------------------------------------------------------------------------
// grad16: all gradients of one chunk except dH, given its entry state
// H0 and the gradient dH at its end (both [Dk][Dv] fp16).  Eight waves.  One
// workgroup per (chunk, k-head, b) walks the v-heads of the k-head group one
// after the other (GROUP; ONLY when the group has one v-head): the key image
// is loaded once, each v-head's dq_hat / dk_hat share is added in fp32 to
// sums held in registers, and after the last v-head the L2-norm VJP is
// applied and dq, dk are written.  The sum order is fixed, so results are
// reproducible.  With fewer such workgroups than CUs, SPLIT runs one
// workgroup per (chunk, v-head, b) and stores each v-head's share for the
// epilogue kernel, which sums the group and applies the norm VJP.
//   Phase A  wave w owns the 16-column value strip jw = 16w .. 16w+15 and
//            chains in registers Y = K H0, X = K dH, U = T RHS,
//            dU = lam X + P^T dO, dRHS = T^T dU; it stores dv = beta dRHS
//            and writes dRHS, dO and U (then dU, RHS) as row-major [C][Dv]
//            copies to LDS.
//   Phase 1  X1 = dRHS H0^T, X2 = dO H0^T (wave w: Dk tile w, all rows),
//            dP = dO U^T (C x C tiles dealt to the waves).
//   Phase 2  X3 = U dH^T, dT = dU RHS^T.
//   Then the C x C stage (dA = -T^T dT T^T), dq_hat / dk_hat of this v-head
//   (wave w: Dk tile w), dbeta and dg.  H0 / dH come from global memory
//   once, as the chained strips the chain kernels store (phase A operands);
//   phases 1 and 2 take their row fragments from a transposed LDS copy Hs
//   written from those strips (H0 first, then dH).
// ---------------------------------------------------------------------------
// acc[t] += A[16t : 16t+16, 0:K] Bm[0:K, n0 : n0+16], Bm row-major; the B
// fragment is shared.
template <int NO, int K, int TRI = kFull, bool KP = false>
__device__ __forceinline__ void mma_rows(f32x4 (&acc)[NO], const _Float16* A, int lda, const _Float16* Bm, int ldb,
                                         int n0) {
  const int r = lane_id() & 15, kl = (lane_id() >> 4) * 8;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const f16x8 bfr = KP ? frag_tk(Bm, ldb, k0, n0) : frag_t(Bm, ldb, k0, n0);
    f16x8 af[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t)
      if (!tri_skip<TRI>(t, k0 / 32)) af[t] = ld8(A + (16 * t + r) * lda + k0 + kl);
#pragma unroll
    for (int t = 0; t < NO; ++t)
      if (!tri_skip<TRI>(t, k0 / 32)) acc[t] = F16Op::mma(af[t], bfr, acc[t]);
  }
}

// mma_rows with A = M^T (A[m][k] = M[k][m], M row-major; transposed reads).
template <int NO, int K, int TRI = kFull, bool KP = false>
__device__ __forceinline__ void mma_rows_ta(f32x4 (&acc)[NO], const _Float16* M, int ldm, const _Float16* Bm, int ldb,
                                            int n0) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const f16x8 bfr = KP ? frag_tk(Bm, ldb, k0, n0) : frag_t(Bm, ldb, k0, n0);
    f16x8 af[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t)
      if (!tri_skip<TRI>(t, k0 / 32)) af[t] = frag_t(M, ldm, k0, 16 * t);
#pragma unroll
    for (int t = 0; t < NO; ++t)
      if (!tri_skip<TRI>(t, k0 / 32)) acc[t] = F16Op::mma(af[t], bfr, acc[t]);
  }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum GradMode { kOnly = 0, kSplit = 1, kGroup = 2 };

template <int C, typename TO, int MODE>
__global__ __launch_bounds__(512) void grad16_kernel(K16 a) {
  using IM = Img<C>;
  constexpr int NW = 8;
  constexpr int LDC = IM::LDC, NT = C / 16;
  constexpr int LDR = C + 8;                     // pitch of the transposed strip tiles X[j][r]
  constexpr int XT = DK * LDR;                   // halves per strip tile
  constexpr int XB = 3 * XT;
  constexpr int LDQ = DK + 8;                    // pitch of the dq / dk output tiles
  constexpr int NQ = NT * NT;                    // C x C tiles
  constexpr int DPW = NQ >= NW ? NQ / NW : 1;    // C x C tiles per wave, all in one row tile
  static_assert(4 * C * LDC <= XB, "C x C stage buffers alias the strip buffers");
  static_assert(2 * C * DK <= DK * LDK, "raw v / dO tiles fit the state buffer");
  static_assert(2 * C * LDQ * 2 + 4 * NW * C * 4 <= XB * 2, "dq / dk tiles and norm partials fit the strip buffers");
  __shared__ __align__(16) char img[IM::CHK + IM::KEY];
  __shared__ __align__(16) _Float16 xb[XB];
  __shared__ __align__(16) _Float16 Hs[DK * LDK];  // H0, then dH, as Hs[j][i]
  __shared__ __align__(16) float sG[NW][C];
  __shared__ __align__(16) float sB[NW][C];
  __shared__ float sGc[NW][C], red[2][NW];
  __shared__ __align__(16) float sDot[2][C];
  // L2-norm VJP row partials q_hat . dq_hat, k_hat . dk_hat, after the dq / dk output tiles
  float (*sN)[NW][C] = reinterpret_cast<float (*)[NW][C]>(xb + 2 * C * LDQ);

  const int tid0 = threadIdx.x, w0 = wave_id();
  // kSplit: blockIdx.y = v-head, each storing its own dq_hat / dk_hat rows
  // for the epilogue kernel; otherwise blockIdx.y = k-head
  const ChunkPos cp = chunk_pos(a, C);
  const int c = cp.c, yy = blockIdx.y;
  const int64_t b = cp.b;
  // kGroup: one workgroup walks all v-heads of its k-head in order, with
  // the group sums of dq_hat / dk_hat kept in registers and the key image
  // loaded once
  constexpr bool GROUP = MODE == kGroup;
  const int ngi = GROUP ? a.Hv / a.Hk : 1;
  const int kh = MODE == kSplit ? yy / (a.Hv / a.Hk) : yy;
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const SeqSpan sp = seq_span(a, b);
  if (t0 >= sp.len) return;  // past the end of a shorter sequence of a ragged batch
  const int L = static_cast<int>(sp.len - t0 < C ? sp.len - t0 : C);

  dma<IM::KEY, 512>(make_rsrc(a.kimg + ((b * a.Hk + kh) * a.NC + c) * static_cast<int64_t>(IM::KEY), IM::KEY), 0,
                    img + IM::CHK, tid0, w0);
  const _Float16* Ks = reinterpret_cast<const _Float16*>(img + IM::CHK);
  const _Float16* Qs = Ks + C * LDK;
  // raw v / dO rows of a v-head's chunk, packed [C][DK] bf16, in the state
  // buffer Hs, which holds them until phase A has taken its strips; the next
  // v-head's rows are requested as soon as phase 2 has read dH from Hs
  const uint32_t rowv = static_cast<uint32_t>(a.Hv) * DK * 2;
  const int64_t seq0 = (sp.t0 + t0) * a.Hv * DK;
  auto load_vdo = [&](int hvx, int tid, int w) {
    dma_rows<C, DK * 2, 512>(make_rsrc(a.v + seq0, static_cast<uint32_t>(L) * rowv), rowv, hvx * DK * 2, L,
                             reinterpret_cast<char*>(Hs), tid, w);
    dma_rows<C, DK * 2, 512>(make_rsrc(a.dout + seq0, static_cast<uint32_t>(L) * rowv), rowv, hvx * DK * 2, L,
                             reinterpret_cast<char*>(Hs + C * DK), tid, w);
  };
  // a v-head's chunk image (into img) and this lane's chained strips of its
  // H0 / dH (rows 16ti + 4g + e, column jw, as the chain kernels store them;
  // the row fragments of phases 1 / 2 come from the transposed copy Hs
  // written from these strips); the next v-head's are requested once its
  // predecessor's last products are done
  auto load_cimg = [&](int hvx, int tid, int w) {
    const int64_t cb = (b * a.Hv + hvx) * a.NC + c;
    dma<IM::CHK, 512>(make_rsrc(a.cimg + cb * static_cast<int64_t>(IM::CHK), IM::CHK), 0, img, tid, w);
  };
  auto load_states = [&](f16x8 (&h0f)[NTK / 2], f16x8 (&dhf)[NTK / 2], int hvx, int w) {
    const int64_t cb = (b * a.Hv + hvx) * a.NC + c;
    const rsrc_t hr = make_rsrc(a.hst + cb * static_cast<int64_t>(DK * DK), DK * DK * 2);
    const rsrc_t dhr = make_rsrc(a.dhst + cb * static_cast<int64_t>(DK * DK), DK * DK * 2);
#pragma unroll
    for (int kb = 0; kb < NTK / 2; ++kb) {
      h0f[kb] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(hr, frag_off(w, kb), 0, 0));
      dhf[kb] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(dhr, frag_off(w, kb), 0, 0));
    }
  };
  const int hv0 = MODE == kSplit ? yy : kh * (a.Hv / a.Hk);
  load_vdo(hv0, tid0, w0);
  load_cimg(hv0, tid0, w0);
  float dqv[NT][4], dkv[NT][4];  // this v-head's (kGroup: the group's) dq_hat / dk_hat, rows 16rt + 4g + e, column i2
  f32x4 kk[DPW];  // K_hat K_hat^T on this wave's C x C tiles, the same for every v-head of the group
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) dqv[rt][e] = dkv[rt][e] = 0.f;
#pragma unroll 1
  for (int gi = 0; gi < ngi; ++gi) {
    const int tid = opaque_v<GROUP>(tid0), w = opaque_s<GROUP>(w0), lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int jw = 16 * w + c16;         // phase A value column
    const int i2 = 16 * w + c16;         // phase 1/2 and dq/dk key row
    const bool qact = w * DPW < NQ;      // this wave owns C x C tiles
    const int qr = (w * DPW) / NT, qc0 = (w * DPW) % NT;
    const int hv = hv0 + gi;
    f16x8 h0f[NTK / 2], dhf[NTK / 2];
    load_states(h0f, dhf, hv, w);
    // fused gates: wave 0's lane 63 - r takes row r's pre-activation g and
    // beta now, for the dg / dbeta it forms at the end of this v-head
    float fgg = 0.f, fgb = 0.f;
    if (a.fg && w == 0 && 63 - lane < L) {
      const int64_t row = (sp.t0 + t0 + 63 - lane) * a.Hv + hv;
      fgg = a.g[row];
      fgb = a.beta[row];
    }
    // Hs[j][i] <- strips (rows i of column j = jw)
    auto put_state = [&](const f16x8 (&f)[NTK / 2]) {
#pragma unroll
      for (int kb = 0; kb < NTK / 2; ++kb) {
        *reinterpret_cast<f16x4*>(Hs + jw * LDK + 32 * kb + 4 * g) = f16x4{f[kb][0], f[kb][1], f[kb][2], f[kb][3]};
        *reinterpret_cast<f16x4*>(Hs + jw * LDK + 32 * kb + 16 + 4 * g) = f16x4{f[kb][4], f[kb][5], f[kb][6], f[kb][7]};
      }
    };
    wait_all();
    __syncthreads();
    // column sums of this v-head: each wave clears its own row (wave 0 reads
    // all rows for the previous v-head's dg before it passes the barrier above)
    if (lane < C) sGc[w][lane] = 0.f;
    const float* gam = reinterpret_cast<const float*>(img);
    const float* lam = gam + C;
    const float* bet = gam + 2 * C;
    const float* G2 = gam + 3 * C;
    const _Float16* Ts = reinterpret_cast<const _Float16*>(img + IM::GT);
    const _Float16* Ps = Ts + C * LDC;
    const float gamC = gam[L - 1];
    // strip tiles, transposed (X[j][r]): dRHS then dU | dO then RHS | U
    _Float16* X0 = xb;
    _Float16* X1b = xb + XT;
    _Float16* X2b = xb + 2 * XT;
    // this lane's strip rows 16tr + 4g .. +3 of column jw into X[jw][.]
    auto put_strip_t = [&](_Float16* X, const f32x4 (&x)[NT]) {
#pragma unroll
      for (int tr = 0; tr < NT; ++tr)
        *reinterpret_cast<f16x4*>(X + jw * LDR + 16 * tr + 4 * g) =
            f16x4{static_cast<_Float16>(x[tr][0]), static_cast<_Float16>(x[tr][1]), static_cast<_Float16>(x[tr][2]),
                  static_cast<_Float16>(x[tr][3])};
    };
    // the same from the strip's chained fragments (already fp16)
    auto put_frags_t = [&](_Float16* X, const f16x8 (&f)[NT / 2]) {
#pragma unroll
      for (int kb = 0; kb < NT / 2; ++kb) {
        *reinterpret_cast<f16x4*>(X + jw * LDR + 32 * kb + 4 * g) = f16x4{f[kb][0], f[kb][1], f[kb][2], f[kb][3]};
        *reinterpret_cast<f16x4*>(X + jw * LDR + 32 * kb + 16 + 4 * g) = f16x4{f[kb][4], f[kb][5], f[kb][6], f[kb][7]};
      }
    };

    // ---- phase A
    float hh = 0.f;  // this lane's part of <dH, H0>
#pragma unroll
    for (int kb = 0; kb < NTK / 2; ++kb) {
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2)
        hh = __builtin_amdgcn_fdot2(f16x2{h0f[kb][2 * p2], h0f[kb][2 * p2 + 1]},
                                    f16x2{dhf[kb][2 * p2], dhf[kb][2 * p2 + 1]}, hh, false);
    }
    f32x4 y[NT], du[NT], u[NT], dr[NT], rhs[NT], dov[NT];
    f16x4 vraw[NT], draw[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      vraw[tr] = tr4(Hs, DK, 16 * tr + 4 * g, 16 * w);
      draw[tr] = tr4(Hs + C * DK, DK, 16 * tr + 4 * g, 16 * w);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = du[t] = u[t] = dr[t] = zero4();
    mma_chain_rows2<NT, NTK, true>(y, du, Ks, LDK, h0f, dhf);
    lds_barrier();  // every wave holds its v / dO strips: Hs may take H0
    put_state(h0f);
    f32x4 psb[NT], psy[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gam + 16 * tr + 4 * g);
      const f32x4 lv = *reinterpret_cast<const f32x4*>(lam + 16 * tr + 4 * g);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
      float vv[4], dd[4];
      bf16x4_to_f32(vv, vraw[tr]);
      bf16x4_to_f32(dd, draw[tr]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float vmy = vv[e] - gv[e] * y[tr][e];
        psb[tr][e] = vmy;  // completed below once dRHS is known
        rhs[tr][e] = bv[e] * vmy;
        du[tr][e] *= lv[e];
        dov[tr][e] = dd[e];
      }
    }
    // RHS, dO and dU as chained fragments, kept (fp16) for the strip tiles
    f16x8 frhs[NT / 2], fdo[NT / 2], fdu[NT / 2];
    chain_frags<NT>(frhs, rhs);
    mma_chain_rows<NT, NT, kLower>(u, Ts, LDC, frhs);
    chain_frags<NT>(fdo, dov);
    mma_chain_rows_t<NT, NT, kUpper>(du, Ps, LDC, fdo);
    chain_frags<NT>(fdu, du);
    mma_chain_rows_t<NT, NT, kUpper>(dr, Ts, LDC, fdu);
    {  // dv = beta dRHS; rows past the sequence's end are dropped by the buffer extent
      const uint32_t rowo = static_cast<uint32_t>(a.Hv) * DK * sizeof(TO);
      const rsrc_t ovr = make_rsrc(static_cast<char*>(a.dv) + (sp.t0 + t0) * rowo, static_cast<uint32_t>(L) * rowo);
      f32x4 dvs[NT];
#pragma unroll
      for (int tr = 0; tr < NT; ++tr) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) dvs[tr][e] = bv[e] * dr[tr][e];
      }
      store_strip_buf<TO, NT>(ovr, 4 * g * rowo + (hv * DK + jw) * static_cast<uint32_t>(sizeof(TO)), rowo, dvs);
    }
#pragma unroll
    for (int tr = 0; tr < NT; ++tr)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        psb[tr][e] *= dr[tr][e];
        psy[tr][e] = dr[tr][e] * y[tr][e];
      }
    put_strip_t(X0, dr);
    put_frags_t(X1b, fdo);
    put_strip_t(X2b, u);
    // This wave's shares of dbeta_r and dG_r (summed over its 16 value
    // columns) start the per-wave row sums sB / sG:
    // dbeta_r = sum_j dRHS (V - gam Y);  dG_r = -beta gam sum_j dRHS Y + ...
    // Lane c16 of group g sums row rs = 16 (k / 4) + 4 g + k % 4, its value
    // k = 4 tr + e of the row sums below (k = c16 NT / 4).
    const int ks = c16 * NT / 4, rs = 16 * (ks >> 2) + 4 * g + (ks & 3);
    {
      float vb[4 * NT], vy[4 * NT];
#pragma unroll
      for (int tr = 0; tr < NT; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vb[4 * tr + e] = psb[tr][e];
          vy[4 * tr + e] = psy[tr][e];
        }
      const float sb = row16_scatter(vb), sy = row16_scatter(vy);
      sB[w][rs] = sb;
      sG[w][rs] = -bet[rs] * gam[rs] * sy;
    }
    __syncthreads();

    // ---- phase 1: X1 = dRHS H0^T, X2 = dO H0^T, dP = dO U^T
    f32x4 x1[NT], x2[NT], x3[NT], dP[DPW], dT[DPW];
#pragma unroll
    for (int t = 0; t < NT; ++t) x1[t] = x2[t] = x3[t] = zero4();
#pragma unroll
    for (int t = 0; t < DPW; ++t) dP[t] = dT[t] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const f16x8 bfr = frag_t(Hs, LDK, 32 * ks, 16 * w);  // H0[i2][32ks + 8g ..]
      f16x8 a1[NT], a2[NT];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        a1[rt] = frag_t(X0, LDR, 32 * ks, 16 * rt);
        a2[rt] = frag_t(X1b, LDR, 32 * ks, 16 * rt);
      }
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        x1[rt] = F16Op::mma(a1[rt], bfr, x1[rt]);
        x2[rt] = F16Op::mma(a2[rt], bfr, x2[rt]);
      }
    }
    if (qact) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const f16x8 af = frag_t(X1b, LDR, 32 * ks, 16 * qr);
#pragma unroll
        for (int t = 0; t < DPW; ++t) dP[t] = F16Op::mma(af, frag_t(X2b, LDR, 32 * ks, 16 * (qc0 + t)), dP[t]);
      }
    }
    __syncthreads();
    put_frags_t(X0, fdu);
    put_frags_t(X1b, frhs);
    put_state(dhf);
    __syncthreads();
    // ---- phase 2: X3 = U dH^T, dT = dU RHS^T
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const f16x8 bfr = frag_t(Hs, LDK, 32 * ks, 16 * w);  // dH[i2][32ks + 8g ..]
      f16x8 a3[NT];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) a3[rt] = frag_t(X2b, LDR, 32 * ks, 16 * rt);
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) x3[rt] = F16Op::mma(a3[rt], bfr, x3[rt]);
    }
    if (qact) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const f16x8 af = frag_t(X0, LDR, 32 * ks, 16 * qr);
#pragma unroll
        for (int t = 0; t < DPW; ++t) dT[t] = F16Op::mma(af, frag_t(X1b, LDR, 32 * ks, 16 * (qc0 + t)), dT[t]);
      }
    }
    __syncthreads();
    if (gi + 1 < ngi) load_vdo(hv + 1, tid, w);  // Hs is free until the next v-head's phase A

    // ---- C x C stage on the tiles (qr, qc0 + t)
    // [C][LDC] fp16 tiles, each stored transposed by 8-byte rows of four
    // (a lane's four rows 16qr + 4g + e of one column) and read transposed
    // where the products want the untransposed matrix
    _Float16* dTT = xb;              // dTT[s'][s] = dT[s][s']
    _Float16* M1T = dTT + C * LDC;   // M1T[s][r] = M1[r][s], M1 = T^T dT
    _Float16* dPmT = M1T + C * LDC;  // dPmT[s][r] = dPm[r][s]
    _Float16* dAmT = dPmT + C * LDC; // dAmT[s][r] = dAm[r][s] (strictly upper)
    float rgc[4] = {0.f, 0.f, 0.f, 0.f}, rbc[4] = {0.f, 0.f, 0.f, 0.f};
    // this lane's rows 16qr + 4g + e: their log2 gates and betas
    const f32x4 g2q = *reinterpret_cast<const f32x4*>(G2 + 16 * qr + 4 * g);
    const f32x4 btq = *reinterpret_cast<const f32x4*>(bet + 16 * qr + 4 * g);
    float colp[DPW];  // this lane's share of column s2's sum of dP * P, finished in the dA stage
    float mx[DPW][4];  // exp2(G2_r - G2_s) on and below the diagonal, kept for the dA stage
    if (qact) {
#pragma unroll
      for (int t = 0; t < DPW; ++t) {
        const int s2 = 16 * (qc0 + t) + c16;
        const float g2s = G2[s2];
        const f16x4 p4s = tr4(Ps, LDC, 16 * qr + 4 * g, 16 * (qc0 + t));  // P_rs, rows r of column s2
        f16x4 t4, p4;
        float col = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * qr + 4 * g + e;
          t4[e] = static_cast<_Float16>(dT[t][e]);
          const float pv = static_cast<float>(p4s[e]);
          const float m = s2 <= r ? __builtin_amdgcn_exp2f(g2q[e] - g2s) : 0.f;
          mx[t][e] = m;
          const float dpp = dP[t][e] * pv;
          rgc[e] += dpp;
          col += dpp;
          p4[e] = static_cast<_Float16>(dP[t][e] * m);
        }
        *reinterpret_cast<f16x4*>(dTT + s2 * LDC + 16 * qr + 4 * g) = t4;
        *reinterpret_cast<f16x4*>(dPmT + s2 * LDC + 16 * qr + 4 * g) = p4;
        colp[t] = col;  // reduced over the rows with the dA stage's share
      }
    }
    __syncthreads();
    if (qact) {
      f32x4 m1[DPW];
#pragma unroll
      for (int t = 0; t < DPW; ++t) m1[t] = zero4();
      mma_cols_t<DPW, C>(m1, Ts, LDC, 16 * qr, dTT, LDC, 16 * qc0);
#pragma unroll
      for (int t = 0; t < DPW; ++t)
        *reinterpret_cast<f16x4*>(M1T + (16 * (qc0 + t) + c16) * LDC + 16 * qr + 4 * g) =
            f16x4{static_cast<_Float16>(m1[t][0]), static_cast<_Float16>(m1[t][1]), static_cast<_Float16>(m1[t][2]),
                  static_cast<_Float16>(m1[t][3])};
    }
    __syncthreads();
    if (qact) {
      f32x4 da[DPW];
#pragma unroll
      for (int t = 0; t < DPW; ++t) da[t] = zero4();
      mma_cols_t<DPW, C>(da, M1T, LDC, 16 * qr, Ts, LDC, 16 * qc0);
      if (gi == 0) {
#pragma unroll
        for (int t = 0; t < DPW; ++t) kk[t] = zero4();
        mma_cols<DPW, DK>(kk, Ks, LDK, 16 * qr, Ks, LDK, 16 * qc0);
      }
#pragma unroll
      for (int t = 0; t < DPW; ++t) {
        const int s2 = 16 * (qc0 + t) + c16;
        float col = colp[t];
        f16x4 a4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * qr + 4 * g + e;
          const float ex = s2 < r ? mx[t][e] : 0.f;
          const float dav = -da[t][e] * ex;
          const float dam = dav * btq[e];
          const float ag = dam * kk[t][e];
          rbc[e] += dav * kk[t][e];
          rgc[e] += ag;
          col += ag;
          a4[e] = static_cast<_Float16>(s2 < r ? dam : 0.f);
        }
        *reinterpret_cast<f16x4*>(dAmT + s2 * LDC + 16 * qr + 4 * g) = a4;
        col = rows4_sum(col);
        if (lane < 16) sGc[w][s2] += col;
      }
      f32x4 rg, rb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rg[e] = row16_sum(rgc[e]);
        rb[e] = row16_sum(rbc[e]);
      }
      if (c16 == 0) {
        f32x4* pg = reinterpret_cast<f32x4*>(&sG[w][16 * qr + 4 * g]);
        f32x4* pb = reinterpret_cast<f32x4*>(&sB[w][16 * qr + 4 * g]);
        *pg = *pg + rg;
        *pb = *pb + rb;
      }
    }
    __syncthreads();

    // ---- dq_hat, dk_hat on Dk tile w; X2 / X3 terms of dG
    f32x4 dq[NT], dk[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) dq[t] = dk[t] = zero4();
    mma_rows_ta<NT, C, kLower, true>(dq, dPmT, LDC, Ks, LDK, 16 * w);   // dPm K
    mma_rows<NT, C, kUpper, true>(dk, dPmT, LDC, Qs, LDK, 16 * w);      // dPm^T Q
    mma_rows_ta<NT, C, kLower, true>(dk, dAmT, LDC, Ks, LDK, 16 * w);   // dAm K
    mma_rows<NT, C, kUpper, true>(dk, dAmT, LDC, Ks, LDK, 16 * w);      // dAm^T K
    float gcx = 0.f;
    float vx[4 * NT];  // this lane's terms of dG_r (rows 16rt + 4g + e), summed over the wave's 16 keys below
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gam + 16 * rt + 4 * g);
      const f32x4 lv = *reinterpret_cast<const f32x4*>(lam + 16 * rt + 4 * g);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * rt + 4 * g);
      const f16x4 qn4 = tr4k(Qs, LDK, 16 * rt + 4 * g, 16 * w);  // Qn[16rt + 4g + e][i2]
      const f16x4 kn4 = tr4k(Ks, LDK, 16 * rt + 4 * g, 16 * w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float qn = static_cast<float>(qn4[e]);
        const float kn = static_cast<float>(kn4[e]);
        const float t3 = lv[e] * kn * x3[rt][e];
        gcx += t3;
        vx[4 * rt + e] = gv[e] * qn * x2[rt][e] - t3;
        dqv[rt][e] += dq[rt][e] + gv[e] * x2[rt][e];
        dkv[rt][e] += dk[rt][e] + lv[e] * x3[rt][e] - bv[e] * gv[e] * x1[rt][e];
      }
    }
    sG[w][rs] += row16_scatter(vx);
    if constexpr (MODE == kSplit) {  // rows (b * T + t) * Hv + hv of [B * T * Hv][DK]; rows >= L dropped
      const uint32_t rowp = static_cast<uint32_t>(a.Hv) * DK * 4;
      const int64_t prow = (b * a.T + t0) * a.Hv + hv;
      const rsrc_t sq = make_rsrc(a.pdq + prow * DK, static_cast<uint32_t>(L) * rowp);
      const rsrc_t sk = make_rsrc(a.pdk + prow * DK, static_cast<uint32_t>(L) * rowp);
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = (16 * rt + 4 * g + e) * rowp + i2 * 4;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dqv[rt][e]), sq, off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dkv[rt][e]), sk, off, 0, 0);
        }
    }
    hh = rows4_sum(row16_sum(hh));
    gcx = rows4_sum(row16_sum(gcx));
    if (lane == 0) {
      red[0][w] = hh;
      red[1][w] = gcx;
    }
    __syncthreads();
    // every wave is past its last read of the chunk image and of h0f / dhf
    if (gi + 1 < ngi) load_cimg(hv + 1, tid, w);
    if (w == 0) {  // lane 63 - r takes row r, so that a prefix sum in lane order sums rows >= r
      const int r = 63 - lane;
      float dG = 0.f, dB = 0.f;
      if (r < C) {
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
          dG += sG[w2][r] - sGc[w2][r];
          dB += sB[w2][r];
        }
      }
      if (r == L - 1) {
        float hs = 0.f, xs = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
          hs += red[0][w2];
          xs += red[1][w2];
        }
        dG += gamC * hs + xs;
      }
      if (r >= L) dG = 0.f;
      const float x = wave_prefix_sum(dG);  // dg_t = sum_{r >= t} dG_r
      if (r < L) {
        const int64_t row = (sp.t0 + t0 + r) * a.Hv + hv;
        a.dg[row] = a.fg ? x * fg_dlog_alpha(fgg) : x;
        a.dbeta[row] = a.fg ? dB * fg_dbeta(fgb) : dB;
      }
    }
  }
  if constexpr (MODE != kSplit) {
    const int tid = tid0, w = w0, lane = tid & 63, g = lane >> 4, c16 = lane & 15, i2 = 16 * w + c16;
    // L2-norm VJP of the group's sums: with x_hat = r x and
    // r = (|x|^2 + eps)^(-1/2), dx = r (dx_hat - x_hat (x_hat . dx_hat)) (the
    // Megatron-LM page's fold of the norm into the kernel, differentiated);
    // x_hat from the key image, r from its rows' pads
    if (a.l2) {
      float xq[NT][4], xk[NT][4];  // q_hat / k_hat at this lane's rows 16rt + 4g + e, column i2
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        const f16x4 q4 = tr4k(Qs, LDK, 16 * rt + 4 * g, 16 * w);
        const f16x4 k4 = tr4k(Ks, LDK, 16 * rt + 4 * g, 16 * w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xq[rt][e] = static_cast<float>(q4[e]);
          xk[rt][e] = static_cast<float>(k4[e]);
        }
      }
      {
        float v1[4 * NT], v3[4 * NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v1[4 * rt + e] = xq[rt][e] * dqv[rt][e];
            v3[4 * rt + e] = xk[rt][e] * dkv[rt][e];
          }
        const int ks = c16 * NT / 4, rs = 16 * (ks >> 2) + 4 * g + (ks & 3);  // the row lane c16 of group g sums
        sN[0][w][rs] = row16_scatter(v1);
        sN[1][w][rs] = row16_scatter(v3);
      }
      __syncthreads();
      if (tid < 2 * C) {
        const int m = tid / C, r = tid % C;
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) sum += sN[m][w2][r];
        sDot[m][r] = sum;
      }
      __syncthreads();
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        const f32x4 qd = *reinterpret_cast<const f32x4*>(&sDot[0][16 * rt + 4 * g]);
        const f32x4 kd = *reinterpret_cast<const f32x4*>(&sDot[1][16 * rt + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * g + e;
          const float rq = *reinterpret_cast<const float*>(Qs + r * LDK + DK);
          const float rk = *reinterpret_cast<const float*>(Ks + r * LDK + DK);
          dqv[rt][e] = rq * (dqv[rt][e] - xq[rt][e] * qd[e]);
          dkv[rt][e] = rk * (dkv[rt][e] - xk[rt][e] * kd[e]);
        }
      }
    }
    const uint32_t rowo = static_cast<uint32_t>(a.Hk) * DK * sizeof(TO);
    const int64_t seqo = (sp.t0 + t0) * a.Hk * DK * static_cast<int64_t>(sizeof(TO));
    const rsrc_t oqr = make_rsrc(static_cast<char*>(a.dq) + seqo, static_cast<uint32_t>(L) * rowo);
    const rsrc_t okr = make_rsrc(static_cast<char*>(a.dk) + seqo, static_cast<uint32_t>(L) * rowo);
    f32x4 oq[NT], ok[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oq[rt][e] = dqv[rt][e];
        ok[rt][e] = dkv[rt][e];
      }
    if constexpr (std::is_same_v<TO, float>) {
      const uint32_t voffo = 4 * g * rowo + (kh * DK + i2) * 4;
      store_strip_buf<TO, NT>(oqr, voffo, rowo, oq);
      store_strip_buf<TO, NT>(okr, voffo, rowo, ok);
    } else {  // through [C][LDQ] tiles in the strip buffers, stored as 16-byte rows
      uint16_t* Oq = reinterpret_cast<uint16_t*>(xb);
      uint16_t* Ok = Oq + C * LDQ;
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * g + e;
          Oq[r * LDQ + i2] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(oq[rt][e]));
          Ok[r * LDQ + i2] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(ok[rt][e]));
        }
      lds_barrier();
#pragma unroll
      for (int u2 = 0; u2 < C * DK * 2 / 16 / 512; ++u2) {
        const int e = 512 * u2 + tid, row = e / 16, cu = e % 16;
        const uint32_t off = row * rowo + kh * DK * 2 + 16 * cu;
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(Oq + row * LDQ + 8 * cu), oqr, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(Ok + row * LDQ + 8 * cu), okr, off, 0, 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Channelwise gates (the per-key-channel decay of the page "Two-pass
// optimization for channelwise gated delta rule kernel") on the chunked
// path, forward only.  With G_r the per-channel running sum of g over the
// chunk, the chunk algebra of the scalar gate holds with each key and query
// row scaled per channel:
//   Y = (K o e^G) H0,  RHS = beta (V - Y),  U = T RHS,
//   O = (Q o e^G) H0 + P U,  H_C = diag(e^{G_C}) H0 + (K o e^{G_C - G})^T U,
//   A_rs = beta_r sum_i k_ri k_si e^{G_ri - G_si}  (s < r),
//   P_rs = sum_i q_ri k_si e^{G_ri - G_si}          (s <= r).
// Blocks of A / P below the 16-row diagonal blocks run on the matrix cores
// with both factors taken relative to the first row b of the row block
// (k_r e^{G_r - G_b} and k_s e^{G_b - G_s}, each <= 1 because g <= 0); the
// diagonal blocks are summed exactly in fp32 with one exponential per pair
// and channel, so no gate value can overflow a factor.
// ---------------------------------------------------------------------------
template <int C>
struct ImgCW {
  static constexpr int LDC = C + 8;
  static constexpr uint32_t KN = C * LDK * 2;       // one [C][LDK] fp16 tile
  static constexpr uint32_t KEY = 3 * KN;           // K o e^G | Q o e^G | K o e^{G_C - G}
  static constexpr uint32_t GT = (C + DK) * 4;      // beta [C] | e^{G_C} [DK]
  static constexpr uint32_t TM = C * LDC * 2;
  static constexpr uint32_t CHK = GT + 2 * TM;      // gates | T | P
};

// T = (I + A)^-1 of one chunk (A strictly lower, fp32 [C][LDA]) into Tf
// (fp32) and Tst (fp16 [C][LDC], whose blocks above the diagonal blocks the
// caller has zeroed): wave w inverts diagonal block w by substitution, the
// blocks below follow one distance at a time on fp32 matrix cores.  Called by
// every thread of the workgroup (4 waves or more); ends with a barrier.
template <int C, int LDA, int LDC>
__device__ __forceinline__ void unit_lower_inverse(const float* A, float* Tf, _Float16* Tst) {
  constexpr int NT = C / 16;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  if (w < NT && lane < 16) {
    const int o = 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc[2] = {r == lane ? 1.f : 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2) acc[s2 & 1] -= A[(o + r) * LDA + o + s2] * x[s2];
      x[r] = acc[0] + acc[1];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      Tf[(o + r) * LDA + o + lane] = x[r];
      Tst[(o + r) * LDC + o + lane] = static_cast<_Float16>(x[r]);
    }
  }
  __syncthreads();
  for (int d = 1; d < NT; ++d) {
    const int i = d + w;
    if (i < NT) {
      const int j = i - d;
      f32x4 m = zero4();
      for (int k = j; k < i; ++k) {
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float av = A[(16 * i + c16) * LDA + 16 * k + k0 + g];
          const float bv = Tf[(16 * k + k0 + g) * LDA + 16 * j + c16];
          m = F32Op::mma(av, bv, m);
        }
      }
      f32x4 tij = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) tij = F32Op::mma(Tf[(16 * i + c16) * LDA + 16 * i + 4 * g + e], m[e], tij);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Tf[(16 * i + 4 * g + e) * LDA + 16 * j + c16] = -tij[e];
        Tst[(16 * i + 4 * g + e) * LDC + 16 * j + c16] = static_cast<_Float16>(-tij[e]);
      }
    }
    __syncthreads();
  }
}


// Rows of the 16-row diagonal blocks that 16-lane group grp (0..31) of a
// cwprep workgroup sums: C = 64: block grp & 3, local rows {w, 15 - w} of
// wave w = grp / 4 (17 pairs per group; all groups of a wave run the same
// loop bounds); C = 32: block grp & 1, local row w or 15 - w.
template <int C>
__device__ __forceinline__ int diag_row(int grp, int j) {
  const int w = grp >> 2;
  if constexpr (C == 64) {
    return 16 * (grp & 3) + (j == 0 ? w : 15 - w);
  } else {
    return 16 * (grp & 1) + (((grp >> 1) & 1) == 0 ? w : 15 - w);
  }
}

template <int C>
__global__ __launch_bounds__(512) void cwprep16_kernel(K16 a) {
  using IM = ImgCW<C>;
  constexpr int NTH = 512, NT = C / 16, LDA = C + 4, LDC = IM::LDC, LDG = DK + 4;
  constexpr int TPR = NTH / C, EPT = DK / TPR, NV = EPT / 8;
  static_assert(C == 64 || C == 32, "chunk of 32 or 64 rows");
  // 79 KB of LDS, so two workgroups share a CU: one space holds Kn, Qn and
  // the running gate sums G2 until the images are written, then A, the fp32
  // and fp16 T and the fp16 P tiles (A and P wait in registers meanwhile)
  constexpr int KSZ = C * LDK * 2, GSZ = C * LDG * 4, ASZ = C * LDA * 4, CSZ = C * LDC * 2;
  static_assert(2 * ASZ + 2 * CSZ <= 2 * KSZ + GSZ, "A, T and P fit the Kn / Qn / G2 space");
  __shared__ __align__(16) char U[2 * KSZ + GSZ];
  _Float16* Ks = reinterpret_cast<_Float16*>(U);
  _Float16* Qs = reinterpret_cast<_Float16*>(U + KSZ);
  float* G2 = reinterpret_cast<float*>(U + 2 * KSZ);  // log2(e) * G[r][i]
  float* A = reinterpret_cast<float*>(U);
  float* Tf = reinterpret_cast<float*>(U + ASZ);
  _Float16* Tst = reinterpret_cast<_Float16*>(U + 2 * ASZ);
  _Float16* Pst = reinterpret_cast<_Float16*>(U + 2 * ASZ + CSZ);
  __shared__ __align__(16) float dpart[4 * 64 * 8];  // factored diagonal blocks: second channel half's sums
  __shared__ float bet[C];
  __shared__ float part_sum[4 * DK];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int c = blockIdx.x, hv = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int kh = hv / (a.Hv / a.Hk);
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const SeqSpan sp = seq_span(a, b);
  if (t0 >= sp.len) return;  // past the end of a shorter sequence of a ragged batch
  const int L = static_cast<int>(sp.len - t0 < C ? sp.len - t0 : C);
  // gates: thread -> channel tid % DK, rows of quarter tid / DK, running sum
  // in registers (g = 0 past the end)
  constexpr int RQ = C / 4;
  const int gi = tid & (DK - 1), gq = tid >> 7;
  float gr[RQ];
  {
    const float* gp = a.g + ((sp.t0 + t0 + gq * RQ) * a.Hv + hv) * DK + gi;
    const int64_t rs = static_cast<int64_t>(a.Hv) * DK;
#pragma unroll
    for (int j = 0; j < RQ; ++j) gr[j] = gq * RQ + j < L ? gp[j * rs] : 0.f;
  }
  {  // q / k rows (normalised, fp16) and beta
    const int r = tid / TPR, part = tid % TPR;
    const int rc = r < L ? r : L - 1;
    const int64_t off = ((sp.t0 + t0 + rc) * a.Hk + kh) * DK + part * EPT;
    uint4 kr[NV], qr[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      kr[u] = sel4(r < L, *reinterpret_cast<const uint4*>(a.k + off + 8 * u));
      qr[u] = sel4(r < L, *reinterpret_cast<const uint4*>(a.q + off + 8 * u));
    }
    norm_rows<C, NV, NTH>(Ks, kr, a.l2);
    norm_rows<C, NV, NTH>(Qs, qr, a.l2);
    if (tid < C) {
      float bv = 0.f;
      if (tid < L) {
        bv = a.beta[(sp.t0 + t0 + tid) * a.Hv + hv];
        if (a.fg) bv = fg_beta(bv);
      }
      bet[tid] = bv;
    }
  }
  float run = 0.f, tv = 0.f;
#pragma unroll
  for (int j = 0; j < RQ; ++j) {
    const float gj = a.fg && gq * RQ + j < L ? fg_log_alpha(gr[j]) : gr[j];
    run += gj;
    tv += fabsf(gj);
    gr[j] = run;
  }
  part_sum[gq * DK + gi] = run;
  // the factored diagonal blocks need every factor e^{+-(G_r - G_o)} of a
  // block inside the fp32 range: a total |g| over a block of at most
  // kSpan (log2 units) bounds them by 2^kSpan; else the exact sums
  constexpr float kSpan = 96.f;
  const bool exact = __syncthreads_or(tv * kLog2e > kSpan * RQ / 16);
  {
    float base = 0.f;
    for (int q2 = 0; q2 < gq; ++q2) base += part_sum[q2 * DK + gi];
#pragma unroll
    for (int j = 0; j < RQ; ++j) G2[(gq * RQ + j) * LDG + gi] = (gr[j] + base) * kLog2e;
  }
  __syncthreads();

  // ---- A and P on and below the 16 x 16 diagonal blocks, into registers.
  // Diagonal block o (rows o .. o+15), factored about its first row:
  //   e^{G_r - G_s} = e^{G_r - G_o} e^{G_o - G_s},
  // on fp32 matrix cores, wave w taking block w % 4 and channel half w / 4
  // (the lane's 16 channels are a relabelling of the contraction index,
  // the same for both operands).
  f32x4 dkk = zero4(), dqk = zero4();
  float ea[C / 32], ep[C / 32];  // exact diagonal sums: row diag_row(tid / 16, j), column block start + c16
  if (!exact) {
    if ((w & 3) < NT) {
      const int o = 16 * (w & 3), h = w >> 2, row = o + c16;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i0 = 32 * g + 16 * h + 8 * u;
        float gx[8], go[8];
        ld8f(gx, G2 + row * LDG + i0);
        ld8f(go, G2 + o * LDG + i0);
        const f16x8 kv = ld8(Ks + row * LDK + i0), qv = ld8(Qs + row * LDK + i0);
#pragma unroll
        for (int q2 = 0; q2 < 8; ++q2) {
          const float x = gx[q2] - go[q2];
          const float fa = __builtin_amdgcn_exp2f(x), fb = __builtin_amdgcn_exp2f(-x);
          const float kf = static_cast<float>(kv[q2]);
          dkk = F32Op::mma(kf * fa, kf * fb, dkk);
          dqk = F32Op::mma(static_cast<float>(qv[q2]) * fa, kf * fb, dqk);
        }
      }
      if (h == 1) {  // the second channel half hands its sums to the first
        float4* pp = reinterpret_cast<float4*>(dpart + ((w & 3) * 64 + lane) * 8);
        pp[0] = make_float4(dkk[0], dkk[1], dkk[2], dkk[3]);
        pp[1] = make_float4(dqk[0], dqk[1], dqk[2], dqk[3]);
      }
    }
  } else {  // exact: a 16-lane group per row, eight channels per lane, one
            // exponential per pair and channel, four pairs in flight, DPP row
            // sums; lane c16 keeps the entry of column (row block start) + c16
    const int grp = tid >> 4, i0 = 8 * c16;
#pragma unroll
    for (int j = 0; j < C / 32; ++j) {
      ea[j] = ep[j] = 0.f;
      const int rr = diag_row<C>(grp, j), s0 = rr & ~15;
      float gr8[8], kr8[8], qr8[8];
      ld8f(gr8, G2 + rr * LDG + i0);
      {
        const f16x8 kv = ld8(Ks + rr * LDK + i0), qv = ld8(Qs + rr * LDK + i0);
#pragma unroll
        for (int q2 = 0; q2 < 8; ++q2) {
          kr8[q2] = static_cast<float>(kv[q2]);
          qr8[q2] = static_cast<float>(qv[q2]);
        }
      }
#pragma unroll 1
      for (int sb = s0; sb <= rr; sb += 4) {
        float kk[4], qk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ss = sb + u <= rr ? sb + u : rr;
          float gs8[8];
          ld8f(gs8, G2 + ss * LDG + i0);
          const f16x8 ks = ld8(Ks + ss * LDK + i0);
          kk[u] = qk[u] = 0.f;
#pragma unroll
          for (int q2 = 0; q2 < 8; ++q2) {
            const float x = static_cast<float>(ks[q2]) * __builtin_amdgcn_exp2f(gr8[q2] - gs8[q2]);
            kk[u] += kr8[q2] * x;
            qk[u] += qr8[q2] * x;
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kk[u] = row16_sum(kk[u]);
          qk[u] = row16_sum(qk[u]);
          const int ss = sb + u;
          if (ss <= rr && ss - s0 == c16) {
            ea[j] = ss < rr ? bet[rr] * kk[u] : 0.f;
            ep[j] = qk[u];
          }
        }
      }
    }
  }
  // Tiles (R, S), S < R, below the diagonal blocks, about the first row
  // b = 16R of row block R (both factors <= 1 for g <= 0):
  //   (k_r e^{G_r - G_b}) . (k_s e^{G_b - G_s}), fp16 matrix cores, one tile
  // (both products) per wave, operands built in registers.
  constexpr int NOFF = NT * (NT - 1) / 2;
  static_assert(NOFF <= 8, "one lower tile per wave");
  f32x4 okk = zero4(), oqk = zero4();
  int oR = 1, oS = 0;
  if (w < NOFF) {
    while (oR * (oR + 1) / 2 <= w) ++oR;
    oS = w - oR * (oR - 1) / 2;
    const int bref = 16 * oR, r = bref + c16, sr = 16 * oS + c16;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const int i0 = 32 * ks + 8 * g;
      float gb[8], gx[8], gs[8];
      ld8f(gb, G2 + bref * LDG + i0);
      ld8f(gx, G2 + r * LDG + i0);
      ld8f(gs, G2 + sr * LDG + i0);
      const f16x8 kv = ld8(Ks + r * LDK + i0), qv = ld8(Qs + r * LDK + i0), sv = ld8(Ks + sr * LDK + i0);
      f16x8 ak, aq, bs;
#pragma unroll
      for (int q2 = 0; q2 < 8; ++q2) {
        const float fr = __builtin_amdgcn_exp2f(gx[q2] - gb[q2]);
        const float fs = __builtin_amdgcn_exp2f(gb[q2] - gs[q2]);
        ak[q2] = static_cast<_Float16>(static_cast<float>(kv[q2]) * fr);
        aq[q2] = static_cast<_Float16>(static_cast<float>(qv[q2]) * fr);
        bs[q2] = static_cast<_Float16>(static_cast<float>(sv[q2]) * fs);
      }
      okk = F16Op::mma(ak, bs, okk);
      oqk = F16Op::mma(aq, bs, oqk);
    }
  }

  // ---- images of this (b, v-head, chunk) that need Kn, Qn, G2: the gates
  // (beta, e^{G_C}) and the three scaled key tiles
  char* cim = a.cimg + ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(IM::CHK);
  float* cg = reinterpret_cast<float*>(cim);
  for (int e = tid; e < C + DK; e += NTH)
    cg[e] = e < C ? bet[e] : __builtin_amdgcn_exp2f(G2[(C - 1) * LDG + e - C]);
  char* kim = a.kimg + ((b * a.Hv + hv) * a.NC + c) * static_cast<int64_t>(IM::KEY);
  constexpr int UK = LDK / 8;  // 16-byte units per [*][LDK] row, the last one the zero pad
  // The three scaled key tiles in one pass: unit u of row r of K o e^G,
  // Q o e^G and K o e^{G_C - G} share the row's reads of G and K.
  {
    uint4* dkg = reinterpret_cast<uint4*>(kim);
    uint4* dqg = reinterpret_cast<uint4*>(kim + IM::KN);
    uint4* dkl = reinterpret_cast<uint4*>(kim + 2 * IM::KN);
    for (int e = tid; e < C * UK; e += NTH) {
      const int r = e / UK, u = e % UK;
      if (u == UK - 1) {
        dkg[e] = dqg[e] = dkl[e] = uint4{0u, 0u, 0u, 0u};
        continue;
      }
      // key-ordered unit u: natural columns n .. n + 3 and n + 16 .. n + 19
      const int n = 32 * (u >> 2) + 4 * (u & 3);
      float gx[8], ge[8];
      {
        const float4 a0 = *reinterpret_cast<const float4*>(G2 + r * LDG + n);
        const float4 a1 = *reinterpret_cast<const float4*>(G2 + r * LDG + n + 16);
        const float4 b0 = *reinterpret_cast<const float4*>(G2 + (C - 1) * LDG + n);
        const float4 b1 = *reinterpret_cast<const float4*>(G2 + (C - 1) * LDG + n + 16);
        gx[0] = a0.x; gx[1] = a0.y; gx[2] = a0.z; gx[3] = a0.w; gx[4] = a1.x; gx[5] = a1.y; gx[6] = a1.z; gx[7] = a1.w;
        ge[0] = b0.x; ge[1] = b0.y; ge[2] = b0.z; ge[3] = b0.w; ge[4] = b1.x; ge[5] = b1.y; ge[6] = b1.z; ge[7] = b1.w;
      }
      const f16x8 kv = key_unit(Ks + r * LDK, u), qv = key_unit(Qs + r * LDK, u);
      f16x8 okg, oqg, okl;
#pragma unroll
      for (int q2 = 0; q2 < 8; ++q2) {
        const float f = __builtin_amdgcn_exp2f(gx[q2]), fl = __builtin_amdgcn_exp2f(ge[q2] - gx[q2]);
        okg[q2] = static_cast<_Float16>(static_cast<float>(kv[q2]) * f);
        oqg[q2] = static_cast<_Float16>(static_cast<float>(qv[q2]) * f);
        okl[q2] = static_cast<_Float16>(static_cast<float>(kv[q2]) * fl);
      }
      dkg[e] = __builtin_bit_cast(uint4, okg);
      dqg[e] = __builtin_bit_cast(uint4, oqg);
      dkl[e] = __builtin_bit_cast(uint4, okl);
    }
  }
  if (a.pkimg && hv % (a.Hv / a.Hk) == 0) {  // the k-head's unscaled key image, for the VJP
    char* pim = a.pkimg + ((b * a.Hk + kh) * a.NC + c) * static_cast<int64_t>(Img<C>::KEY);
    write_tile<C, UK, NTH, true>(pim, [&](int r, int u) { return ld8(Ks + r * LDK + 8 * u); });
    write_tile<C, UK, NTH, true>(pim + Img<C>::KN, [&](int r, int u) { return ld8(Qs + r * LDK + 8 * u); });
  }
  __syncthreads();  // Kn, Qn and G2 are no longer read: their space takes A, T and P

  for (int e = tid; e < 2 * CSZ / 16; e += NTH)  // fp16 T and P tiles start at zero
    reinterpret_cast<uint4*>(Tst)[e] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();
  if (w < NOFF) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = 16 * oR + 4 * g + e, ss = 16 * oS + c16;
      A[rr * LDA + ss] = bet[rr] * okk[e];
      Pst[rr * LDC + ss] = static_cast<_Float16>(oqk[e]);
    }
  }
  if (!exact) {
    if (w < 4 && w < NT) {  // diagonal blocks: both halves, lower triangle
      const float4* pp = reinterpret_cast<const float4*>(dpart + (w * 64 + lane) * 8);
      const float4 pk = pp[0], pq = pp[1];
      dkk[0] += pk.x; dkk[1] += pk.y; dkk[2] += pk.z; dkk[3] += pk.w;
      dqk[0] += pq.x; dqk[1] += pq.y; dqk[2] += pq.z; dqk[3] += pq.w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 16 * w + 4 * g + e, ss = 16 * w + c16;
        if (ss <= rr) {
          A[rr * LDA + ss] = ss < rr ? bet[rr] * dkk[e] : 0.f;
          Pst[rr * LDC + ss] = static_cast<_Float16>(dqk[e]);
        }
      }
    }
  } else {
    const int grp = tid >> 4;
#pragma unroll
    for (int j = 0; j < C / 32; ++j) {
      const int rr = diag_row<C>(grp, j), ss = (rr & ~15) + c16;
      if (ss <= rr) {
        A[rr * LDA + ss] = ea[j];
        Pst[rr * LDC + ss] = static_cast<_Float16>(ep[j]);
      }
    }
  }
  __syncthreads();
  unit_lower_inverse<C, LDA, LDC>(A, Tf, Tst);

  // ---- T and P images
  constexpr int UC = LDC / 8;
  write_tile<C, UC, NTH>(cim + IM::GT, [&](int r, int u) { return ld8(Tst + r * LDC + 8 * u); });
  write_tile<C, UC, NTH>(cim + IM::GT + IM::TM, [&](int r, int u) { return ld8(Pst + r * LDC + 8 * u); });
}

// Channelwise forward chain: as chain16, using the scaled key rows of the
// channelwise images and decaying H's rows by e^{G_C}:
//   Y = Kg H, Z = Qg H, U = T (beta (V - Y)), O = Z + P U,
//   H = diag(e^{G_C}) H + Kl^T U.
// The chunk's o leaves the compute waves as 2-byte stores (their LDS share
// holds the three key tiles).  STORE_H: every chunk's entry state is stored
// for the VJP (fp16, chained-fragment order); WRITE_O false: no outputs.
template <int C, typename TO, bool WRITE_O, bool STORE_H, int NCW>
__global__ __launch_bounds__(64 * (NCW + 1)) void cwchain16_kernel(K16 a) {
  constexpr int BV = 16 * NCW, NSL = DK / BV;
  using IM = ImgCW<C>;
  constexpr int NT = C / 16, LDC = IM::LDC;
  constexpr uint32_t CB = IM::CHK, KB = IM::KEY, VB = C * BV * 2;
  __shared__ __align__(16) char bufA[CB + KB + VB];
  __shared__ __align__(16) char bufB[CB + KB + VB];

  const int w = wave_id(), lane = lane_id(), g = lane >> 4, c16 = lane & 15;
  const ChainPos p = chain_pos(a, NSL);
  const SeqSpan sp = seq_span(a, p.b);
  const int nc = static_cast<int>((sp.len + C - 1) / C);
  if (nc == 0) {  // empty sequence of a ragged batch: the state passes through
    if (w < NCW && a.ht) {
      const int64_t base = (p.b * a.Hv + p.hv) * DK * DK + p.slice * BV + 16 * w + c16;
      for (int i = 0; i < DK; ++i) a.ht[base + i * DK] = a.h0 ? a.h0[base + i * DK] : 0.f;
    }
    return;
  }
  auto rows_of = [&](int c) { return static_cast<int>(sp.len - static_cast<int64_t>(c) * C < C ? sp.len - static_cast<int64_t>(c) * C : C); };
  auto seq_rsrc = [&](const void* base, int esize, int c, uint32_t rowb) {
    const char* p0 = static_cast<const char*>(base) + (sp.t0 + static_cast<int64_t>(c) * C) * a.Hv * DK * esize;
    return make_rsrc(p0, static_cast<uint32_t>(rows_of(c)) * rowb);
  };
  const uint32_t rowv = static_cast<uint32_t>(a.Hv) * DK * 2;
  const uint32_t rowo = static_cast<uint32_t>(a.Hv) * DK * sizeof(TO);

  if (w == NCW) {  // ---- producer wave
    const char* kim0 = a.kimg + (p.b * a.Hv + p.hv) * a.NC * static_cast<int64_t>(IM::KEY);
    const char* cim0 = a.cimg + (p.b * a.Hv + p.hv) * a.NC * static_cast<int64_t>(IM::CHK);
    const uint32_t colv = (p.hv * DK + p.slice * BV) * 2;
    auto stage = [&](int c, char* buf) {
      dma<CB, 64>(make_rsrc(cim0 + c * static_cast<int64_t>(IM::CHK), CB), 0, buf, lane, 0);
      dma<KB, 64>(make_rsrc(kim0 + c * static_cast<int64_t>(IM::KEY), KB), 0, buf + CB, lane, 0);
      dma_rows<C, BV * 2, 64>(seq_rsrc(a.v, 2, c, rowv), rowv, colv, rows_of(c), buf + CB + KB, lane, 0);
    };
    stage(0, bufA);
    wait_all();
    lds_barrier();
    for (int c = 0; c < nc; c += 2) {
      if (c + 1 < nc) stage(c + 1, bufB);
      wait_all();
      lds_barrier();
      if (c + 1 < nc) {
        if (c + 2 < nc) stage(c + 2, bufA);
        wait_all();
        lds_barrier();
      }
    }
    return;
  }

  // ---- compute waves
  const int jcol = p.slice * BV + 16 * w + c16;
  const int wg = p.slice * NCW + w;  // column group of the chunk-state layout
  const int64_t hbase = (p.b * a.Hv + p.hv) * DK * DK + jcol;
  const uint32_t voffo = 4 * g * rowo + (p.hv * DK + jcol) * static_cast<uint32_t>(sizeof(TO));
  f32x4 h[NTK];
#pragma unroll
  for (int ti = 0; ti < NTK; ++ti) {
    h[ti] = zero4();
    if (a.h0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) h[ti][e] = a.h0[hbase + (16 * ti + 4 * g + e) * DK];
    }
  }
  lds_barrier();
  f32x4 o[NT];
  auto step = [&](int c, const char* cur) __attribute__((always_inline)) {
    if constexpr (WRITE_O) {
      if (c > 0) store_strip_buf<TO, NT>(seq_rsrc(a.o, sizeof(TO), c - 1, rowo), voffo, rowo, o);
    }
    const float* bet = reinterpret_cast<const float*>(cur);
    const float* gC = bet + C;
    const _Float16* Tm = reinterpret_cast<const _Float16*>(cur + IM::GT);
    const _Float16* Pm = Tm + C * LDC;
    const _Float16* Kg = reinterpret_cast<const _Float16*>(cur + CB);
    const _Float16* Qg = Kg + C * LDK;
    const _Float16* Kl = Qg + C * LDK;
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(cur + CB + KB);

    f16x8 hf[NTK / 2];
    chain_frags<NTK>(hf, h);
    if constexpr (STORE_H) {  // entry state of chunk c
      const rsrc_t hr = make_rsrc(a.hst + ((p.b * a.Hv + p.hv) * a.NC + c) * static_cast<int64_t>(DK * DK), DK * DK * 2);
#pragma unroll
      for (int kb = 0; kb < NTK / 2; ++kb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hf[kb]), hr, frag_off(wg, kb), 0, 0);
    }
    f32x4 y[NT], u[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = u[t] = o[t] = zero4();
    mma_chain_rows<NT, NTK, kFull, true>(y, Kg, LDK, hf);
    if constexpr (WRITE_O) mma_chain_rows<NT, NTK, kFull, true>(o, Qg, LDK, hf);
    f32x4 rhs[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
      float vv[4];
      tile_col4_bf16(vv, Vs, BV, 16 * tr + 4 * g, 16 * w);
#pragma unroll
      for (int e = 0; e < 4; ++e) rhs[tr][e] = bv[e] * (vv[e] - y[tr][e]);
    }
    f16x8 bf[NT / 2];
    chain_frags<NT>(bf, rhs);
    mma_chain_rows<NT, NT, kLower>(u, Tm, LDC, bf);
    chain_frags<NT>(bf, u);
    if constexpr (WRITE_O) mma_chain_rows<NT, NT, kLower>(o, Pm, LDC, bf);
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti) {
      const f32x4 dec = *reinterpret_cast<const f32x4*>(gC + 16 * ti + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) h[ti][e] *= dec[e];
    }
    mma_chain_rows_t<NTK, NT, kFull, true>(h, Kl, LDK, bf);
    lds_barrier();
  };
  for (int c = 0; c < nc; c += 2) {
    step(c, bufA);
    if (c + 1 < nc) step(c + 1, bufB);
  }
  if constexpr (WRITE_O) store_strip_buf<TO, NT>(seq_rsrc(a.o, sizeof(TO), nc - 1, rowo), voffo, rowo, o);
  if (a.ht) {
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.ht[hbase + (16 * ti + 4 * g + e) * DK] = h[ti][e];
  }
}

// Channelwise reverse chain: carries dH backwards over the chunks with the
// channelwise images and stores every chunk's end gradient for the per-chunk
// VJP; writes dh0.  Per chunk and compute wave:
//   dU = Kl dH + P^T dO,  dRHS = T^T dU,
//   dH = diag(e^{G_C}) dH + Qg^T dO - Kg^T (beta dRHS).
// (dv and the other gradients come from the per-chunk VJP.)
template <int C, int NCW>
__global__ __launch_bounds__(64 * (NCW + 1)) void cwdh16_kernel(K16 a) {
  constexpr int BV = 16 * NCW, NSL = DK / BV;
  using IM = ImgCW<C>;
  constexpr int NT = C / 16, LDC = IM::LDC;
  constexpr uint32_t CB = IM::CHK, KB = IM::KEY, VB = C * BV * 2;
  __shared__ __align__(16) char bufA[CB + KB + VB];
  __shared__ __align__(16) char bufB[CB + KB + VB];

  const int w = wave_id(), lane = lane_id(), g = lane >> 4, c16 = lane & 15;
  const ChainPos p = chain_pos(a, NSL);
  const SeqSpan sp = seq_span(a, p.b);
  const int nc = static_cast<int>((sp.len + C - 1) / C);
  if (nc == 0) {  // empty sequence of a ragged batch: the gradient passes through
    if (w < NCW && a.dh0) {
      const int64_t base = (p.b * a.Hv + p.hv) * DK * DK + p.slice * BV + 16 * w + c16;
      for (int i = 0; i < DK; ++i) a.dh0[base + i * DK] = a.dht ? a.dht[base + i * DK] : 0.f;
    }
    return;
  }
  auto rows_of = [&](int c) { return static_cast<int>(sp.len - static_cast<int64_t>(c) * C < C ? sp.len - static_cast<int64_t>(c) * C : C); };
  const uint32_t rowv = static_cast<uint32_t>(a.Hv) * DK * 2;

  if (w == NCW) {  // ---- producer wave: chunks nc-1, nc-2, ...
    const char* kim0 = a.kimg + (p.b * a.Hv + p.hv) * a.NC * static_cast<int64_t>(IM::KEY);
    const char* cim0 = a.cimg + (p.b * a.Hv + p.hv) * a.NC * static_cast<int64_t>(IM::CHK);
    const uint32_t colv = (p.hv * DK + p.slice * BV) * 2;
    auto stage = [&](int c, char* buf) {
      const char* p0 = reinterpret_cast<const char*>(a.dout) + (sp.t0 + static_cast<int64_t>(c) * C) * rowv;
      dma<CB, 64>(make_rsrc(cim0 + c * static_cast<int64_t>(IM::CHK), CB), 0, buf, lane, 0);
      dma<KB, 64>(make_rsrc(kim0 + c * static_cast<int64_t>(IM::KEY), KB), 0, buf + CB, lane, 0);
      dma_rows<C, BV * 2, 64>(make_rsrc(p0, static_cast<uint32_t>(rows_of(c)) * rowv), rowv, colv, rows_of(c),
                              buf + CB + KB, lane, 0);
    };
    stage(nc - 1, bufA);
    wait_all();
    lds_barrier();
    for (int i = 0; i < nc; i += 2) {
      if (nc - 2 - i >= 0) stage(nc - 2 - i, bufB);
      wait_all();
      lds_barrier();
      if (i + 1 < nc) {
        if (nc - 3 - i >= 0) stage(nc - 3 - i, bufA);
        wait_all();
        lds_barrier();
      }
    }
    return;
  }

  // ---- compute waves
  const int jcol = p.slice * BV + 16 * w + c16;
  const int wg = p.slice * NCW + w;
  const int64_t hbase = (p.b * a.Hv + p.hv) * DK * DK + jcol;
  f32x4 dh[NTK];
#pragma unroll
  for (int ti = 0; ti < NTK; ++ti) {
    dh[ti] = zero4();
    if (a.dht) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dh[ti][e] = a.dht[hbase + (16 * ti + 4 * g + e) * DK];
    }
  }
  lds_barrier();

  auto step = [&](int c, const char* cur) __attribute__((always_inline)) {
    const float* bet = reinterpret_cast<const float*>(cur);
    const float* gC = bet + C;
    const _Float16* Tm = reinterpret_cast<const _Float16*>(cur + IM::GT);
    const _Float16* Pm = Tm + C * LDC;
    const _Float16* Kg = reinterpret_cast<const _Float16*>(cur + CB);
    const _Float16* Qg = Kg + C * LDK;
    const _Float16* Kl = Qg + C * LDK;
    const uint16_t* Ds = reinterpret_cast<const uint16_t*>(cur + CB + KB);

    f16x8 hf[NTK / 2];
    chain_frags<NTK>(hf, dh);
    {  // gradient at this chunk's end
      const rsrc_t hr = make_rsrc(a.dhst + ((p.b * a.Hv + p.hv) * a.NC + c) * static_cast<int64_t>(DK * DK), DK * DK * 2);
#pragma unroll
      for (int kb = 0; kb < NTK / 2; ++kb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hf[kb]), hr, frag_off(wg, kb), 0, 0);
    }
    f32x4 du[NT], dr[NT], dof[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) du[t] = dr[t] = zero4();
    mma_chain_rows<NT, NTK, kFull, true>(du, Kl, LDK, hf);
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      float x[4];
      tile_col4_bf16(x, Ds, BV, 16 * tr + 4 * g, 16 * w);
#pragma unroll
      for (int e = 0; e < 4; ++e) dof[tr][e] = x[e];
    }
    f16x8 bf[NT / 2], bo[NT / 2];
    chain_frags<NT>(bo, dof);
    mma_chain_rows_t<NT, NT, kUpper>(du, Pm, LDC, bo);
    chain_frags<NT>(bf, du);
    mma_chain_rows_t<NT, NT, kUpper>(dr, Tm, LDC, bf);
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) dr[tr][e] = -bv[e] * dr[tr][e];
    }
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti) {
      const f32x4 dec = *reinterpret_cast<const f32x4*>(gC + 16 * ti + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) dh[ti][e] *= dec[e];
    }
    mma_chain_rows_t<NTK, NT, kFull, true>(dh, Qg, LDK, bo);
    chain_frags<NT>(bf, dr);
    mma_chain_rows_t<NTK, NT, kFull, true>(dh, Kg, LDK, bf);
    lds_barrier();
  };
  // chunks nc-1, nc-2, ... alternate between the two buffers
  for (int i = 0; i < nc; i += 2) {
    step(nc - 1 - i, bufA);
    if (i + 1 < nc) step(nc - 2 - i, bufB);
  }
  if (a.dh0) {
#pragma unroll
    for (int ti = 0; ti < NTK; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) a.dh0[hbase + (16 * ti + 4 * g + e) * DK] = dh[ti][e];
  }
}

// ---------------------------------------------------------------------------
// cwgrad16: all gradients of one chunk except dH for the channelwise gate
// (the per-key-channel decay of the page "Two-pass optimization for
// channelwise gated delta rule kernel"), one workgroup of eight waves per
// (chunk, k-head, b) walking the group's v-heads in order (as grad16's group
// walk: dq_hat / dk_hat summed in registers, the L2-norm VJP after the last
// v-head).  With G_r the per-channel running sum of g over the chunk,
// W_rs = e^{G_r - G_s} per channel (<= 1 for s <= r), Kg = K o e^G and
// Kl = K o e^{G_C - G}, per v-head:
//   Phase A  Y = Kg H0, RHS = beta (V - Y), U = T RHS,
//            dU = Kl dH + P^T dO, dRHS = T^T dU; dv = beta dRHS;
//            dbeta_r gets dRHS_r . (V - Y)_r
//   Phase 1  X1 = dRHS H0^T, X2 = dO H0^T, dP = dO U^T
//   Phase 2  X3 = U dH^T, dT = dU RHS^T
//   C x C    dA = -T^T dT T^T (s < r); dP masked to s <= r
//   then per channel (the decay differs per channel, so the chunk-local
//   sums carry W inside them):
//     dq_r   = e^{G_r} X2_r + sum_{s<=r} dP_rs W_rs k_s
//     dk+_r  = beta_r (-e^{G_r} X1_r + a_r),  a_r = sum_{s<r} dA_rs W_rs k_s
//     dk-_s  = e^{G_C - G_s} X3_s + sum_{r>=s} dP_rs W_rs q_r
//              + sum_{r>s} dA_rs beta_r W_rs k_r
//     dk = dk+ + dk-,  dbeta_r += k_r . a_r,
//     dG = q o dq + k o (dk+ - dk-), and at the last valid row also
//       sum_r k_r o (e^{G_C - G_r} X3_r) + e^{G_C} o rowsum(H0 o dH),
//     dg_t = sum_{r >= t} dG_r.
//   Blocks of these sums below the 16-row diagonal blocks run as 16x16x16
//   fp16 matrix-core products with W split at a block boundary, both
//   factors <= 1: about the last row l of the column block for the row
//   sums (k_s e^{G_l - G_s}, then e^{G_r - G_l}), about the first row b of
//   the row block for the column sums (q_r e^{G_r - G_b}, then
//   e^{G_b - G_s}).  Diagonal blocks are summed in fp32 with W split about
//   their first row o (e^{G_r - G_o} e^{G_o - G_s}) when the chunk's gates
//   keep every such factor within 2^96, else with one exponential per pair.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma16x16x16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

template <int C, typename TO>
__global__ __launch_bounds__(512) void cwgrad16_kernel(K16 a) {
  using IM = ImgCW<C>;
  using IP = Img<C>;
  constexpr int NW = 8, LDC = IM::LDC, NT = C / 16;
  constexpr int LDR = C + 8;                   // pitch of the transposed strip tiles X[j][r]
  constexpr int XT = DK * LDR, XB = 3 * XT;
  constexpr int LDQ = DK + 8;                  // pitch of the dq / dk output tiles
  constexpr int NQ = NT * NT;
  constexpr int DPW = NQ >= NW ? NQ / NW : 1;  // C x C tiles per wave, all in one row tile
  constexpr int LDG = C + 4;                   // pitch (floats) of G2T[i][r]
  constexpr uint32_t KXB = 2 * IM::KN > DK * LDG * 4 ? 2 * IM::KN : DK * LDG * 4;
  static_assert(6 * C * LDC <= XB, "C x C buffers alias the strip buffers");
  static_assert(IP::KEY <= DK * LDK * 2, "the plain key image fits the state buffer");
  static_assert(2 * C * DK <= DK * LDK, "raw v / dO tiles fit the state buffer");
  static_assert(2 * C * LDQ * 2 + 4 * NW * C * 4 <= XB * 2, "dq / dk tiles and norm partials fit the strip buffers");
  __shared__ __align__(16) char cimg[IM::CHK];     // beta | e^{G_C} | T | P
  __shared__ __align__(16) char kx[KXB];           // Kg | Kl (phase A), then G2T
  __shared__ __align__(16) _Float16 xb[XB];
  __shared__ __align__(16) _Float16 Hs[DK * LDK];  // v / dO rows, H0, dH as Hs[j][i], then K_hat | Q_hat
  __shared__ __align__(16) float sB[NW][C];        // per-wave parts of dbeta
  __shared__ __align__(16) float sQ[4][DK];        // running gate sums of the row quarters
  __shared__ __align__(16) float sDot[2][C];
  float (*sN)[NW][C] = reinterpret_cast<float (*)[NW][C]>(xb + 2 * C * LDQ);

  const int tid0 = threadIdx.x, w0 = wave_id();
  const ChunkPos cp = chunk_pos(a, C);
  const int c = cp.c, kh = blockIdx.y;
  const int64_t b = cp.b;
  const int grp = a.Hv / a.Hk;
  const int64_t t0 = static_cast<int64_t>(c) * C;
  const SeqSpan sp = seq_span(a, b);
  if (t0 >= sp.len) return;  // past the end of a shorter sequence of a ragged batch
  const int L = static_cast<int>(sp.len - t0 < C ? sp.len - t0 : C);
  const uint32_t rowv = static_cast<uint32_t>(a.Hv) * DK * 2;
  const int64_t seq0 = (sp.t0 + t0) * a.Hv * DK;
  const float* bet = reinterpret_cast<const float*>(cimg);
  const float* eGC = bet + C;
  const _Float16* Ts = reinterpret_cast<const _Float16*>(cimg + IM::GT);
  const _Float16* Ps = Ts + C * LDC;
  const _Float16* Kg = reinterpret_cast<const _Float16*>(kx);
  const _Float16* Kl = Kg + C * LDK;
  float* G2T = reinterpret_cast<float*>(kx);  // log2(e) G[r][i] at G2T[i * LDG + r]
  const _Float16* Ks = Hs;                    // plain key image: K_hat | Q_hat, norm factors in the row pads
  const _Float16* Qs = Hs + C * LDK;
  _Float16* X0 = xb;
  _Float16* X1b = xb + XT;
  _Float16* X2b = xb + 2 * XT;
  _Float16* dTT = xb;  // C x C tiles, after phase 2
  _Float16* M1s = dTT + C * LDC;
  _Float16* dPm = M1s + C * LDC;   // dP, s <= r            [r][s]
  _Float16* dPmT = dPm + C * LDC;  //                       [s][r]
  _Float16* dAm = dPmT + C * LDC;  // dA, s < r             [r][s]
  _Float16* dAmT = dAm + C * LDC;  //                       [s][r]

  float dqv[NT][4], dkv[NT][4];  // the group's dq_hat / dk_hat, rows 16rt + 4g + e, column i2
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) dqv[rt][e] = dkv[rt][e] = 0.f;
#pragma unroll 1
  for (int gi = 0; gi < grp; ++gi) {
    const int tid = opaque_v<true>(tid0), w = opaque_s<true>(w0), lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int jw = 16 * w + c16;  // phase A value column
    const int i2 = 16 * w + c16;  // key channel of phases 1 / 2 and of the per-channel sums
    const bool qact = w * DPW < NQ;
    const int qr = (w * DPW) / NT, qc0 = (w * DPW) % NT;
    const int hv = kh * grp + gi;
    const int64_t cb = (b * a.Hv + hv) * a.NC + c;
    {
      const char* kim = a.kimg + cb * static_cast<int64_t>(IM::KEY);  // Kg | Qg | Kl
      dma<IM::CHK, 512>(make_rsrc(a.cimg + cb * static_cast<int64_t>(IM::CHK), IM::CHK), 0, cimg, tid, w);
      dma<IM::KN, 512>(make_rsrc(kim, IM::KN), 0, kx, tid, w);
      dma<IM::KN, 512>(make_rsrc(kim + 2 * IM::KN, IM::KN), 0, kx + IM::KN, tid, w);
      dma_rows<C, DK * 2, 512>(make_rsrc(a.v + seq0, static_cast<uint32_t>(L) * rowv), rowv, hv * DK * 2, L,
                               reinterpret_cast<char*>(Hs), tid, w);
      dma_rows<C, DK * 2, 512>(make_rsrc(a.dout + seq0, static_cast<uint32_t>(L) * rowv), rowv, hv * DK * 2, L,
                               reinterpret_cast<char*>(Hs + C * DK), tid, w);
    }
    // this lane's chained strips of H0 / dH (rows 16ti + 4g + e, column jw)
    f16x8 h0f[NTK / 2], dhf[NTK / 2];
    {
      const rsrc_t hr = make_rsrc(a.hst + cb * static_cast<int64_t>(DK * DK), DK * DK * 2);
      const rsrc_t dhr = make_rsrc(a.dhst + cb * static_cast<int64_t>(DK * DK), DK * DK * 2);
#pragma unroll
      for (int kb = 0; kb < NTK / 2; ++kb) {
        h0f[kb] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(hr, frag_off(w, kb), 0, 0));
        dhf[kb] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(dhr, frag_off(w, kb), 0, 0));
      }
    }
    auto put_state = [&](const f16x8 (&f)[NTK / 2]) {  // Hs[j][i] <- strips
#pragma unroll
      for (int kb = 0; kb < NTK / 2; ++kb) {
        *reinterpret_cast<f16x4*>(Hs + jw * LDK + 32 * kb + 4 * g) = f16x4{f[kb][0], f[kb][1], f[kb][2], f[kb][3]};
        *reinterpret_cast<f16x4*>(Hs + jw * LDK + 32 * kb + 16 + 4 * g) = f16x4{f[kb][4], f[kb][5], f[kb][6], f[kb][7]};
      }
    };
    auto put_strip_t = [&](_Float16* X, const f32x4 (&x)[NT]) {  // rows 16tr + 4g .. +3 of column jw
#pragma unroll
      for (int tr = 0; tr < NT; ++tr)
        *reinterpret_cast<f16x4*>(X + jw * LDR + 16 * tr + 4 * g) =
            f16x4{static_cast<_Float16>(x[tr][0]), static_cast<_Float16>(x[tr][1]), static_cast<_Float16>(x[tr][2]),
                  static_cast<_Float16>(x[tr][3])};
    };
    // the same from the strip's chained fragments (already fp16)
    auto put_frags_t = [&](_Float16* X, const f16x8 (&f)[NT / 2]) {
#pragma unroll
      for (int kb = 0; kb < NT / 2; ++kb) {
        *reinterpret_cast<f16x4*>(X + jw * LDR + 32 * kb + 4 * g) = f16x4{f[kb][0], f[kb][1], f[kb][2], f[kb][3]};
        *reinterpret_cast<f16x4*>(X + jw * LDR + 32 * kb + 16 + 4 * g) = f16x4{f[kb][4], f[kb][5], f[kb][6], f[kb][7]};
      }
    };
    wait_all();
    __syncthreads();

    // ---- phase A
    f32x4 y[NT], du[NT], u[NT], dr[NT], rhs[NT], dov[NT];
    f16x4 vraw[NT], draw[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      vraw[tr] = tr4(Hs, DK, 16 * tr + 4 * g, 16 * w);
      draw[tr] = tr4(Hs + C * DK, DK, 16 * tr + 4 * g, 16 * w);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = du[t] = u[t] = dr[t] = zero4();
    mma_chain_rows<NT, NTK, kFull, true>(y, Kg, LDK, h0f);
    mma_chain_rows<NT, NTK, kFull, true>(du, Kl, LDK, dhf);
    lds_barrier();  // every wave holds its v / dO strips: Hs may take H0
    put_state(h0f);
    f32x4 psb[NT];
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
      float vv[4], dd[4];
      bf16x4_to_f32(vv, vraw[tr]);
      bf16x4_to_f32(dd, draw[tr]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float vmy = vv[e] - y[tr][e];
        psb[tr][e] = vmy;
        rhs[tr][e] = bv[e] * vmy;
        dov[tr][e] = dd[e];
      }
    }
    // RHS, dO and dU as chained fragments, kept (fp16) for the strip tiles
    f16x8 frhs[NT / 2], fdo[NT / 2], fdu[NT / 2];
    chain_frags<NT>(frhs, rhs);
    mma_chain_rows<NT, NT, kLower>(u, Ts, LDC, frhs);
    chain_frags<NT>(fdo, dov);
    mma_chain_rows_t<NT, NT, kUpper>(du, Ps, LDC, fdo);
    chain_frags<NT>(fdu, du);
    mma_chain_rows_t<NT, NT, kUpper>(dr, Ts, LDC, fdu);
    {  // dv = beta dRHS; rows past the sequence's end are dropped by the buffer extent
      const uint32_t rowo = static_cast<uint32_t>(a.Hv) * DK * sizeof(TO);
      const rsrc_t ovr = make_rsrc(static_cast<char*>(a.dv) + (sp.t0 + t0) * rowo, static_cast<uint32_t>(L) * rowo);
      f32x4 dvs[NT];
#pragma unroll
      for (int tr = 0; tr < NT; ++tr) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * tr + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) dvs[tr][e] = bv[e] * dr[tr][e];
      }
      store_strip_buf<TO, NT>(ovr, 4 * g * rowo + (hv * DK + jw) * static_cast<uint32_t>(sizeof(TO)), rowo, dvs);
    }
    // lane c16 of group g sums row rs = 16 (k / 4) + 4 g + k % 4 of the
    // row sums over the wave's 16 columns, its value k = 4 tr + e (k = c16 NT / 4)
    const int ks = c16 * NT / 4, rs = 16 * (ks >> 2) + 4 * g + (ks & 3);
    {
      float vb[4 * NT];
#pragma unroll
      for (int tr = 0; tr < NT; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) vb[4 * tr + e] = psb[tr][e] * dr[tr][e];
      sB[w][rs] = row16_scatter(vb);
    }
    put_strip_t(X0, dr);
    put_frags_t(X1b, fdo);
    put_strip_t(X2b, u);
    __syncthreads();

    // ---- phase 1: X1 = dRHS H0^T, X2 = dO H0^T, dP = dO U^T; the H0 row
    // fragments stay for rowsum(H0 o dH) in phase 2
    f32x4 x1[NT], x2[NT], x3[NT], dP[DPW], dT[DPW];
#pragma unroll
    for (int t = 0; t < NT; ++t) x1[t] = x2[t] = x3[t] = zero4();
#pragma unroll
    for (int t = 0; t < DPW; ++t) dP[t] = dT[t] = zero4();
    f16x8 h0k[DK / 32];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const f16x8 bfr = frag_t(Hs, LDK, 32 * ks, 16 * w);  // H0[i2][32ks + 8g ..]
      h0k[ks] = bfr;
      f16x8 a1[NT], a2[NT];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        a1[rt] = frag_t(X0, LDR, 32 * ks, 16 * rt);
        a2[rt] = frag_t(X1b, LDR, 32 * ks, 16 * rt);
      }
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        x1[rt] = F16Op::mma(a1[rt], bfr, x1[rt]);
        x2[rt] = F16Op::mma(a2[rt], bfr, x2[rt]);
      }
    }
    if (qact) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const f16x8 af = frag_t(X1b, LDR, 32 * ks, 16 * qr);
#pragma unroll
        for (int t = 0; t < DPW; ++t) dP[t] = F16Op::mma(af, frag_t(X2b, LDR, 32 * ks, 16 * (qc0 + t)), dP[t]);
      }
    }
    __syncthreads();
    put_frags_t(X0, fdu);
    put_frags_t(X1b, frhs);
    put_state(dhf);
    __syncthreads();
    // ---- phase 2: X3 = U dH^T, dT = dU RHS^T
    float hd = 0.f;  // this lane's part of sum_j H0[i2][j] dH[i2][j]
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const f16x8 bfr = frag_t(Hs, LDK, 32 * ks, 16 * w);  // dH[i2][32ks + 8g ..]
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2)
        hd = __builtin_amdgcn_fdot2(f16x2{h0k[ks][2 * p2], h0k[ks][2 * p2 + 1]}, f16x2{bfr[2 * p2], bfr[2 * p2 + 1]},
                                    hd, false);
      f16x8 a3[NT];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) a3[rt] = frag_t(X2b, LDR, 32 * ks, 16 * rt);
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) x3[rt] = F16Op::mma(a3[rt], bfr, x3[rt]);
    }
    if (qact) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const f16x8 af = frag_t(X0, LDR, 32 * ks, 16 * qr);
#pragma unroll
        for (int t = 0; t < DPW; ++t) dT[t] = F16Op::mma(af, frag_t(X1b, LDR, 32 * ks, 16 * (qc0 + t)), dT[t]);
      }
    }
    hd = rows4_sum(hd);
    __syncthreads();

    // ---- Kg / Kl and the states are done: the plain key image goes to Hs,
    // the running gate sums (log2 units, channel-major) to kx
    dma<IP::KEY, 512>(make_rsrc(a.pkimg + ((b * a.Hk + kh) * a.NC + c) * static_cast<int64_t>(IP::KEY), IP::KEY), 0,
                      reinterpret_cast<char*>(Hs), tid, w);
    constexpr int RQ = C / 4;  // rows per quarter; thread -> channel tid % DK, quarter tid / DK
    const int gch = tid & (DK - 1), gq = tid >> 7;
    float grun[RQ], gspan = 0.f;
    {
      const float* gp = a.g + ((sp.t0 + t0 + gq * RQ) * a.Hv + hv) * DK + gch;
      const int64_t rs = static_cast<int64_t>(a.Hv) * DK;
      float run = 0.f;
#pragma unroll
      for (int j = 0; j < RQ; ++j) {
        float gj = 0.f;
        if (gq * RQ + j < L) gj = a.fg ? fg_log_alpha(gp[j * rs]) : gp[j * rs];
        run += gj;
        gspan += fabsf(gj);
        grun[j] = run;
      }
      sQ[gq][gch] = run;
      gspan *= kLog2e;  // bound on the span of G over this quarter of the rows, log2 units
    }
    // C x C stage, part 1: dT transposed, dP masked (and transposed)
    if (qact) {
#pragma unroll
      for (int t = 0; t < DPW; ++t) {
        const int s2 = 16 * (qc0 + t) + c16;
        f16x4 t4, p4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * qr + 4 * g + e;
          t4[e] = static_cast<_Float16>(dT[t][e]);
          p4[e] = static_cast<_Float16>(s2 <= r ? dP[t][e] : 0.f);
          dPm[r * LDC + s2] = p4[e];
        }
        *reinterpret_cast<f16x4*>(dTT + s2 * LDC + 16 * qr + 4 * g) = t4;
        *reinterpret_cast<f16x4*>(dPmT + s2 * LDC + 16 * qr + 4 * g) = p4;
      }
    }
    // The diagonal blocks split W about their first row o when every factor
    // e^{G_o - G_s} of the chunk stays within 2^96 (a quarter of the rows is
    // at most one 16-row block); else one exponential per pair.
    constexpr float kSpan = 96.f;
    const bool exact = __syncthreads_or(gspan > kSpan * RQ / 16);
    {
      float base = 0.f;
      for (int q2 = 0; q2 < gq; ++q2) base += sQ[q2][gch];
#pragma unroll
      for (int j = 0; j < RQ; j += 4)
        *reinterpret_cast<f32x4*>(G2T + gch * LDG + gq * RQ + j) =
            f32x4{(grun[j] + base) * kLog2e, (grun[j + 1] + base) * kLog2e, (grun[j + 2] + base) * kLog2e,
                  (grun[j + 3] + base) * kLog2e};
    }
    if (qact) {
      f32x4 m1[DPW];
#pragma unroll
      for (int t = 0; t < DPW; ++t) m1[t] = zero4();
      mma_cols_t<DPW, C>(m1, Ts, LDC, 16 * qr, dTT, LDC, 16 * qc0);
#pragma unroll
      for (int t = 0; t < DPW; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          M1s[(16 * qr + 4 * g + e) * LDC + 16 * (qc0 + t) + c16] = static_cast<_Float16>(m1[t][e]);
    }
    __syncthreads();
    // ---- the per-channel sums start from the products with the states
    float G2r[NT][4];  // log2(e) G at this lane's rows, channel i2
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(G2T + i2 * LDG + 16 * rt + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) G2r[rt][e] = gv[e];
    }
    const float G2C = G2T[i2 * LDG + L - 1];
    float dq[NT][4], dkp[NT][4], dkm[NT][4], ta[NT][4];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * rt + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float eg = __builtin_amdgcn_exp2f(G2r[rt][e]);
        dq[rt][e] = eg * x2[rt][e];
        dkp[rt][e] = -bv[e] * eg * x1[rt][e];
        dkm[rt][e] = __builtin_amdgcn_exp2f(G2C - G2r[rt][e]) * x3[rt][e];
        ta[rt][e] = 0.f;
      }
    }
    // C x C stage, part 2: dA = -T^T dT T^T below the diagonal
    if (qact) {
      f32x4 da[DPW];
#pragma unroll
      for (int t = 0; t < DPW; ++t) da[t] = zero4();
      mma_cols<DPW, C>(da, M1s, LDC, 16 * qr, Ts, LDC, 16 * qc0);
#pragma unroll
      for (int t = 0; t < DPW; ++t) {
        const int s2 = 16 * (qc0 + t) + c16;
        f16x4 a4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * qr + 4 * g + e;
          a4[e] = static_cast<_Float16>(s2 < r ? -da[t][e] : 0.f);
          dAm[r * LDC + s2] = a4[e];
        }
        *reinterpret_cast<f16x4*>(dAmT + s2 * LDC + 16 * qr + 4 * g) = a4;
      }
    }
    wait_all();  // the plain key image
    __syncthreads();

    // ---- row sums: dq += sum_{s<=r} dP_rs W_rs k_s, a += sum_{s<r} dA_rs W_rs k_s
#pragma unroll
    for (int S = 0; S + 1 < NT; ++S) {  // blocks below the diagonal, about the last row of column block S
      const float g2l = G2T[i2 * LDG + 16 * S + 15];
      const f16x4 kq = tr4(Ks, LDK, 16 * S + 4 * g, 16 * w);
      const f32x4 g2s = *reinterpret_cast<const f32x4*>(G2T + i2 * LDG + 16 * S + 4 * g);
      f16x4 bk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bk[i] = static_cast<_Float16>(static_cast<float>(kq[i]) * __builtin_amdgcn_exp2f(g2l - g2s[i]));
#pragma unroll
      for (int R = S + 1; R < NT; ++R) {
        const f16x4 ap = *reinterpret_cast<const f16x4*>(dPm + (16 * R + c16) * LDC + 16 * S + 4 * g);
        const f16x4 aa = *reinterpret_cast<const f16x4*>(dAm + (16 * R + c16) * LDC + 16 * S + 4 * g);
        const f32x4 tp = mma16x16x16(ap, bk, zero4());
        const f32x4 tq = mma16x16x16(aa, bk, zero4());
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sc = __builtin_amdgcn_exp2f(G2r[R][e] - g2l);
          dq[R][e] += sc * tp[e];
          ta[R][e] += sc * tq[e];
        }
      }
    }
    if (!exact) {
#pragma unroll
      for (int R = 0; R < NT; ++R) {  // diagonal blocks about their first row o: W = e^{G_r - G_o} e^{G_o - G_s},
        // the second factor (up to 2^96) inside fp32 matrix-core products; product kk
        // of lane group g sums over s = 16R + 4g + kk, the rows this lane holds
        const float g2o = G2T[i2 * LDG + 16 * R];
        const f16x4 kq = tr4(Ks, LDK, 16 * R + 4 * g, 16 * w);
        const f16x4 ap = *reinterpret_cast<const f16x4*>(dPm + (16 * R + c16) * LDC + 16 * R + 4 * g);
        const f16x4 aa = *reinterpret_cast<const f16x4*>(dAm + (16 * R + c16) * LDC + 16 * R + 4 * g);
        f32x4 tp = zero4(), tq = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float kb = static_cast<float>(kq[kk]) * __builtin_amdgcn_exp2f(g2o - G2r[R][kk]);
          tp = F32Op::mma(static_cast<float>(ap[kk]), kb, tp);
          tq = F32Op::mma(static_cast<float>(aa[kk]), kb, tq);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ar = __builtin_amdgcn_exp2f(G2r[R][e] - g2o);
          dq[R][e] += ar * tp[e];
          ta[R][e] += ar * tq[e];
        }
      }
    } else {
#pragma unroll
    for (int R = 0; R < NT; ++R) {  // diagonal blocks, one exponential per pair
#pragma unroll 1
      for (int sq = 0; sq < 4; ++sq) {
        const f16x4 kq = tr4(Ks, LDK, 16 * R + 4 * sq, 16 * w);
        const f32x4 g2s = *reinterpret_cast<const f32x4*>(G2T + i2 * LDG + 16 * R + 4 * sq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * g + e;
          const f16x4 pq = *reinterpret_cast<const f16x4*>(dPm + r * LDC + 16 * R + 4 * sq);
          const f16x4 aq = *reinterpret_cast<const f16x4*>(dAm + r * LDC + 16 * R + 4 * sq);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float wk = 4 * sq + i <= 4 * g + e
                                 ? static_cast<float>(kq[i]) * __builtin_amdgcn_exp2f(G2r[R][e] - g2s[i])
                                 : 0.f;
            dq[R][e] += static_cast<float>(pq[i]) * wk;
            ta[R][e] += static_cast<float>(aq[i]) * wk;
          }
        }
      }
    }
    }
    // ---- the last row's sum_r k_r o (e^{G_C - G_r} X3_r), before the column sums join dk-
    float kl3 = 0.f;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const f16x4 k4 = tr4(Ks, LDK, 16 * rt + 4 * g, 16 * w);
#pragma unroll
      for (int e = 0; e < 4; ++e) kl3 += static_cast<float>(k4[e]) * dkm[rt][e];
    }
    kl3 = rows4_sum(kl3);
    // ---- column sums: dk- += sum_{r>=s} dP_rs W_rs q_r + sum_{r>s} dA_rs beta_r W_rs k_r
#pragma unroll
    for (int R = 1; R < NT; ++R) {  // blocks below the diagonal, about the first row of row block R
      const float g2b = G2T[i2 * LDG + 16 * R];
      const f16x4 q4 = tr4(Qs, LDK, 16 * R + 4 * g, 16 * w);
      const f16x4 k4 = tr4(Ks, LDK, 16 * R + 4 * g, 16 * w);
      const f32x4 g2v = *reinterpret_cast<const f32x4*>(G2T + i2 * LDG + 16 * R + 4 * g);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * R + 4 * g);
      f16x4 bq, bkb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = __builtin_amdgcn_exp2f(g2v[i] - g2b);
        bq[i] = static_cast<_Float16>(static_cast<float>(q4[i]) * f);
        bkb[i] = static_cast<_Float16>(bv[i] * static_cast<float>(k4[i]) * f);
      }
#pragma unroll
      for (int S = 0; S < R; ++S) {
        const f16x4 ap = *reinterpret_cast<const f16x4*>(dPmT + (16 * S + c16) * LDC + 16 * R + 4 * g);
        const f16x4 aa = *reinterpret_cast<const f16x4*>(dAmT + (16 * S + c16) * LDC + 16 * R + 4 * g);
        f32x4 tp = mma16x16x16(ap, bq, zero4());
        tp = mma16x16x16(aa, bkb, tp);
#pragma unroll
        for (int e = 0; e < 4; ++e) dkm[S][e] += __builtin_amdgcn_exp2f(g2b - G2r[S][e]) * tp[e];
      }
    }
    if (!exact) {
#pragma unroll
      for (int R = 0; R < NT; ++R) {  // diagonal blocks about their first row o, as fp32 products over
        // r = 16R + 4g + kk with e^{G_r - G_o} on the right operand, e^{G_o - G_s} after
        const float g2o = G2T[i2 * LDG + 16 * R];
        const f16x4 q4 = tr4(Qs, LDK, 16 * R + 4 * g, 16 * w);
        const f16x4 k4 = tr4(Ks, LDK, 16 * R + 4 * g, 16 * w);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * R + 4 * g);
        const f16x4 ap = *reinterpret_cast<const f16x4*>(dPmT + (16 * R + c16) * LDC + 16 * R + 4 * g);
        const f16x4 aa = *reinterpret_cast<const f16x4*>(dAmT + (16 * R + c16) * LDC + 16 * R + 4 * g);
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float f = __builtin_amdgcn_exp2f(G2r[R][kk] - g2o);
          acc = F32Op::mma(static_cast<float>(ap[kk]), static_cast<float>(q4[kk]) * f, acc);
          acc = F32Op::mma(static_cast<float>(aa[kk]), bv[kk] * static_cast<float>(k4[kk]) * f, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dkm[R][e] += __builtin_amdgcn_exp2f(g2o - G2r[R][e]) * acc[e];
      }
    } else {
#pragma unroll
    for (int R = 0; R < NT; ++R) {  // diagonal blocks, one exponential per pair
#pragma unroll 1
      for (int rq = 0; rq < 4; ++rq) {
        const f16x4 q4 = tr4(Qs, LDK, 16 * R + 4 * rq, 16 * w);
        const f16x4 k4 = tr4(Ks, LDK, 16 * R + 4 * rq, 16 * w);
        const f32x4 g2v = *reinterpret_cast<const f32x4*>(G2T + i2 * LDG + 16 * R + 4 * rq);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * R + 4 * rq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = 16 * R + 4 * g + e;
          const f16x4 pq = *reinterpret_cast<const f16x4*>(dPmT + s * LDC + 16 * R + 4 * rq);
          const f16x4 aq = *reinterpret_cast<const f16x4*>(dAmT + s * LDC + 16 * R + 4 * rq);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float f = 4 * rq + i >= 4 * g + e ? __builtin_amdgcn_exp2f(g2v[i] - G2r[R][e]) : 0.f;
            dkm[R][e] += f * (static_cast<float>(pq[i]) * static_cast<float>(q4[i]) +
                              static_cast<float>(aq[i]) * bv[i] * static_cast<float>(k4[i]));
          }
        }
      }
    }
    }

    // ---- dk, dG, dg, dbeta of this v-head
    float dG[NT][4];
    float vb[4 * NT];  // this lane's terms of dbeta_r, summed over the wave's 16 keys below
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bet + 16 * rt + 4 * g);
      const f16x4 q4 = tr4(Qs, LDK, 16 * rt + 4 * g, 16 * w);
      const f16x4 k4 = tr4(Ks, LDK, 16 * rt + 4 * g, 16 * w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * g + e;
        const float qn = static_cast<float>(q4[e]), kn = static_cast<float>(k4[e]);
        vb[4 * rt + e] = kn * ta[rt][e];
        dkp[rt][e] += bv[e] * ta[rt][e];
        float x = qn * dq[rt][e] + kn * (dkp[rt][e] - dkm[rt][e]);
        if (r == L - 1) x += kl3 + eGC[i2] * hd;
        dG[rt][e] = r < L ? x : 0.f;
        dqv[rt][e] += dq[rt][e];
        dkv[rt][e] += dkp[rt][e] + dkm[rt][e];
      }
    }
    sB[w][rs] += row16_scatter(vb);
    {  // dg_t = sum_{r >= t} dG_r per channel: rows 16rt + 4g + e live in
       // lanes c16 + 16g; suffix within the lane, across the lane groups,
       // then across the row tiles
      float tot[NT];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        float s = 0.f;
#pragma unroll
        for (int e = 3; e >= 0; --e) {
          s += dG[rt][e];
          dG[rt][e] = s;
        }
        // the lane groups above g: the odd neighbour (row swap), then the
        // upper pair of groups (half swap); each swap's two results hold the
        // lane's own value and its partner's (the even row, or the lower
        // half, finds its partner's in the second)
        const unsigned su = __float_as_uint(s);
        const auto pa = __builtin_amdgcn_permlane16_swap(su, su, false, false);
        const unsigned pa0 = pa[0], pa1 = pa[1];
        const float pair = __uint_as_float(pa0) + __uint_as_float(pa1);
        const unsigned pu = __float_as_uint(pair);
        const auto pb = __builtin_amdgcn_permlane32_swap(pu, pu, false, false);
        const unsigned pb0 = pb[0], pb1 = pb[1];
        const float after = ((g & 1) == 0 ? __uint_as_float(pa1) : 0.f) + (g < 2 ? __uint_as_float(pb1) : 0.f);
#pragma unroll
        for (int e = 0; e < 4; ++e) dG[rt][e] += after;
        tot[rt] = __uint_as_float(pb0) + __uint_as_float(pb1);  // all four groups
      }
      float later = 0.f;
#pragma unroll
      for (int rt = NT - 1; rt >= 0; --rt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * g + e;
          if (r < L) {
            const int64_t idx = ((sp.t0 + t0 + r) * a.Hv + hv) * DK + i2;
            const float x = dG[rt][e] + later;
            a.dg[idx] = a.fg ? x * fg_dlog_alpha(a.g[idx]) : x;
          }
        }
        later += tot[rt];
      }
    }
    __syncthreads();
    if (w == 0) {
      const int r = lane;
      if (r < L) {
        float dB = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) dB += sB[w2][r];
        const int64_t row = (sp.t0 + t0 + r) * a.Hv + hv;
        a.dbeta[row] = a.fg ? dB * fg_dbeta(a.beta[row]) : dB;
      }
    }
  }
  {  // L2-norm VJP of the group's sums (x_hat and the norm factors from the plain key image), dq, dk
    const int tid = tid0, w = w0, lane = tid & 63, g = lane >> 4, c16 = lane & 15, i2 = 16 * w + c16;
    if (a.l2) {
      float xq[NT][4], xk[NT][4];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        const f16x4 q4 = tr4(Qs, LDK, 16 * rt + 4 * g, 16 * w);
        const f16x4 k4 = tr4(Ks, LDK, 16 * rt + 4 * g, 16 * w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xq[rt][e] = static_cast<float>(q4[e]);
          xk[rt][e] = static_cast<float>(k4[e]);
        }
      }
      {
        float v1[4 * NT], v3[4 * NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v1[4 * rt + e] = xq[rt][e] * dqv[rt][e];
            v3[4 * rt + e] = xk[rt][e] * dkv[rt][e];
          }
        const int ks = c16 * NT / 4, rs = 16 * (ks >> 2) + 4 * g + (ks & 3);  // the row lane c16 of group g sums
        sN[0][w][rs] = row16_scatter(v1);
        sN[1][w][rs] = row16_scatter(v3);
      }
      __syncthreads();
      if (tid < 2 * C) {
        const int m = tid / C, r = tid % C;
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) sum += sN[m][w2][r];
        sDot[m][r] = sum;
      }
      __syncthreads();
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        const f32x4 qd = *reinterpret_cast<const f32x4*>(&sDot[0][16 * rt + 4 * g]);
        const f32x4 kd = *reinterpret_cast<const f32x4*>(&sDot[1][16 * rt + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * g + e;
          const float rq = *reinterpret_cast<const float*>(Qs + r * LDK + DK);
          const float rk = *reinterpret_cast<const float*>(Ks + r * LDK + DK);
          dqv[rt][e] = rq * (dqv[rt][e] - xq[rt][e] * qd[e]);
          dkv[rt][e] = rk * (dkv[rt][e] - xk[rt][e] * kd[e]);
        }
      }
    }
    const uint32_t rowo = static_cast<uint32_t>(a.Hk) * DK * sizeof(TO);
    const int64_t seqo = (sp.t0 + t0) * a.Hk * DK * static_cast<int64_t>(sizeof(TO));
    const rsrc_t oqr = make_rsrc(static_cast<char*>(a.dq) + seqo, static_cast<uint32_t>(L) * rowo);
    const rsrc_t okr = make_rsrc(static_cast<char*>(a.dk) + seqo, static_cast<uint32_t>(L) * rowo);
    f32x4 oq[NT], ok[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oq[rt][e] = dqv[rt][e];
        ok[rt][e] = dkv[rt][e];
      }
    const uint32_t voffo = 4 * g * rowo + (kh * DK + i2) * static_cast<uint32_t>(sizeof(TO));
    store_strip_buf<TO, NT>(oqr, voffo, rowo, oq);
    store_strip_buf<TO, NT>(okr, voffo, rowo, ok);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Ws16 {
  size_t kimg, cimg, hst, dhst, pdq, pdk, total;  // pdq / pdk: per-v-head dq_hat / dk_hat rows (split gradient)
};

// A k-head group's v-heads share one gradient workgroup per (chunk, k-head,
// b) when that gives at least one workgroup per CU; with fewer, the gradient
// launch runs one workgroup per v-head and the epilogue kernel sums the
// group and applies the norm VJP.
constexpr int kCUs = 256;
bool grad_split(const Shape& s, int C) {
  const int64_t nc = (s.T + C - 1) / C;
  return s.Hv > s.Hk && nc * s.Hk * s.B < kCUs;
}

template <int C>
Ws16 plan16(const Shape& s, bool bwd) {
  using IM = Img<C>;
  const size_t nc = static_cast<size_t>((s.T + C - 1) / C);
  const size_t nk = static_cast<size_t>(s.B) * s.Hk * nc, nv = static_cast<size_t>(s.B) * s.Hv * nc;
  Ws16 w{};
  size_t off = 0;
  w.kimg = off; off = up(off + nk * IM::KEY);
  w.cimg = off; off = up(off + nv * IM::CHK);
  if (bwd) {
    // with a split gradient launch, the dq_hat / dk_hat rows of every v-head
    // ([B * T * Hv][DK] <= B * nc * C * Hv rows)
    const size_t rows = static_cast<size_t>(s.B) * nc * C * s.Hv;
    w.hst = off;  off = up(off + nv * DK * DK * 2);
    w.dhst = off; off = up(off + nv * DK * DK * 2);
    if (grad_split(s, C)) {
      w.pdq = off;  off = up(off + rows * DK * 4);
      w.pdk = off;  off = up(off + rows * DK * 4);
    }
  }
  w.total = off;
  return w;
}

Ws16 plan_any(const Shape& s, int C, bool bwd) { return C == 64 ? plan16<64>(s, bwd) : plan16<32>(s, bwd); }

K16 args16(const Shape& s, int C, void* ws, const Ws16& w) {
  K16 a{};
  a.B = s.B;
  a.T = s.T;
  a.Hk = s.Hk;
  a.Hv = s.Hv;
  a.NC = static_cast<int>((s.T + C - 1) / C);
  a.l2 = s.l2norm ? 1 : 0;
  a.fg = s.fused_gates ? 1 : 0;
  char* base = static_cast<char*>(ws);
  a.kimg = base + w.kimg;
  a.cimg = base + w.cimg;
  if (w.hst || w.dhst) {
    a.hst = reinterpret_cast<_Float16*>(base + w.hst);
    a.dhst = reinterpret_cast<_Float16*>(base + w.dhst);
    if (w.pdq) {
      a.pdq = reinterpret_cast<float*>(base + w.pdq);
      a.pdk = reinterpret_cast<float*>(base + w.pdk);
    }
  }
  return a;
}

// Compute waves per chain workgroup (16 value columns each): the widest
// slice whose grid of (b, v-head, slice) workgroups still covers every CU
// of the current device.
int chain_waves(const K16& a) {
  static int ncu[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 4;
  if (ncu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    ncu[dev] = n;
  }
  const int64_t heads = static_cast<int64_t>(a.Hv) * a.B;
  if (heads * (DK / 64) >= ncu[dev]) return 4;
  if (heads * (DK / 32) >= ncu[dev]) return 2;
  return 1;
}

// Calls f(std::integral_constant<int, NW>) for the chain workgroup shape nw.
template <typename F>
void with_chain_waves(int nw, F&& f) {
  if (nw == 4)
    f(std::integral_constant<int, 4>{});
  else if (nw == 2)
    f(std::integral_constant<int, 2>{});
  else
    f(std::integral_constant<int, 1>{});
}

// Grid of a chain launch with NW compute waves per workgroup.
dim3 chain_grid(const K16& a, int nw) { return dim3(static_cast<unsigned>(DK / (16 * nw) * a.Hv * a.B)); }

template <int C>
hipError_t prep16(const K16& a, hipStream_t st) {
  ProfScope ps("chunk_prep", st);
  hipLaunchKernelGGL((prep16_kernel<C>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(512), 0, st, a);
  return hipGetLastError();
}

template <int C, typename TO, bool WO, bool SH>
hipError_t chain16(const K16& a, hipStream_t st) {
  ProfScope ps(WO ? (SH ? "chunk_fwd_save" : "chunk_fwd") : "chunk_states", st);
  with_chain_waves(chain_waves(a), [&](auto nw) {
    constexpr int NW = decltype(nw)::value;
    hipLaunchKernelGGL((chain16_kernel<C, TO, WO, SH, NW>), chain_grid(a, NW), dim3(64 * (NW + 1)), 0, st, a);
  });
  return hipGetLastError();
}

template <int C, typename TO>
hipError_t dh16(const K16& a, hipStream_t st) {
  ProfScope ps("chunk_dh", st);
  with_chain_waves(chain_waves(a), [&](auto nw) {
    constexpr int NW = decltype(nw)::value;
    hipLaunchKernelGGL((dh16_kernel<C, TO, NW>), chain_grid(a, NW), dim3(64 * (NW + 1)), 0, st, a);
  });
  return hipGetLastError();
}

template <int C, typename TO>
hipError_t grad16(const Shape& s, K16 a, hipStream_t st) {
  const int grp = a.Hv / a.Hk;
  if (grad_split(s, C)) {
    {
      ProfScope ps("chunk_grad", st);
      hipLaunchKernelGGL((grad16_kernel<C, TO, kSplit>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(512), 0, st,
                         a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    EpiArgs ea{a.q, a.k, a.pdq, a.pdk, nullptr, nullptr, 1, a.dq, a.dk, a.dbeta, a.dg, a.g, a.beta, a.cu};
    return launch_bwd_epilogue(s, ea, st);
  }
  ProfScope ps("chunk_grad", st);
  const dim3 grid(a.NC, a.Hk, static_cast<unsigned>(a.B));
  if (grp == 1)
    hipLaunchKernelGGL((grad16_kernel<C, TO, kOnly>), grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((grad16_kernel<C, TO, kGroup>), grid, dim3(512), 0, st, a);
  return hipGetLastError();
}

template <int C, typename TO>
hipError_t fwd_all(const Shape& s, const ChunkFwdArgs& x, void* ws, hipStream_t st) {
  K16 a = args16(s, C, ws, plan16<C>(s, s.save_chunks));
  a.cu = x.cu;
  a.q = static_cast<const bf16_t*>(x.q);
  a.k = static_cast<const bf16_t*>(x.k);
  a.v = static_cast<const bf16_t*>(x.v);
  a.g = x.g;
  a.beta = x.beta;
  a.h0 = x.h0;
  a.o = x.o;
  a.ht = x.ht;
  hipError_t e = prep16<C>(a, st);
  if (e != hipSuccess) return e;
  return s.save_chunks ? chain16<C, TO, true, true>(a, st) : chain16<C, TO, true, false>(a, st);
}

template <int C, typename TO>
hipError_t bwd_all(const Shape& s, const ChunkBwdArgs& x, void* ws, hipStream_t st) {
  K16 a = args16(s, C, ws, plan16<C>(s, true));
  a.cu = x.cu;
  a.q = static_cast<const bf16_t*>(x.q);
  a.k = static_cast<const bf16_t*>(x.k);
  a.v = static_cast<const bf16_t*>(x.v);
  a.dout = static_cast<const bf16_t*>(x.dout);
  a.g = x.g;
  a.beta = x.beta;
  a.h0 = x.h0;
  a.dht = x.dht;
  a.dv = x.dv;
  a.dh0 = x.dh0;
  a.dg = x.dg;
  a.dbeta = x.dbeta;
  a.dq = x.dq;
  a.dk = x.dk;
  hipError_t e = hipSuccess;
  if (!s.save_chunks) {  // else the forward left the images and chunk states in ws
    e = prep16<C>(a, st);
    if (e == hipSuccess) e = chain16<C, TO, false, true>(a, st);
  }
  if (e == hipSuccess) e = dh16<C, TO>(a, st);
  if (e == hipSuccess) e = grad16<C, TO>(s, a, st);
  return e;
}

// Channelwise forward: per-v-head key and chunk images, prep then chain.
template <int C>
Ws16 plan_cw(const Shape& s) {
  using IM = ImgCW<C>;
  const size_t nv = static_cast<size_t>(s.B) * s.Hv * static_cast<size_t>((s.T + C - 1) / C);
  Ws16 w{};
  size_t off = 0;
  w.kimg = off; off = up(off + nv * IM::KEY);
  w.cimg = off; off = up(off + nv * IM::CHK);
  w.total = off;
  return w;
}

template <int C, typename TO>
hipError_t fwd_cw(const Shape& s, const ChunkFwdArgs& x, void* ws, hipStream_t st) {
  K16 a = args16(s, C, ws, plan_cw<C>(s));
  a.cu = x.cu;
  a.q = static_cast<const bf16_t*>(x.q);
  a.k = static_cast<const bf16_t*>(x.k);
  a.v = static_cast<const bf16_t*>(x.v);
  a.g = x.g;
  a.beta = x.beta;
  a.h0 = x.h0;
  a.o = x.o;
  a.ht = x.ht;
  {
    ProfScope ps("chunk_prep_cw", st);
    hipLaunchKernelGGL((cwprep16_kernel<C>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(512), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps("chunk_fwd_cw", st);
  with_chain_waves(chain_waves(a), [&](auto nw) {
    constexpr int NW = decltype(nw)::value;
    hipLaunchKernelGGL((cwchain16_kernel<C, TO, true, false, NW>), chain_grid(a, NW), dim3(64 * (NW + 1)), 0, st, a);
  });
  return hipGetLastError();
}

// Channelwise VJP: the chunk images (and each k-head's unscaled key image),
// every chunk's entry state (forward chain), every chunk's end gradient and
// dh0 (reverse chain), then every chunk's gradients from those two states
// (cwgrad16: dq, dk, dv, dg, dbeta).
struct WsCW {
  size_t kimg, cimg, hst, dhst, pkimg, total;
};

template <int C>
WsCW plan_cw_bwd(const Shape& s) {
  using IM = ImgCW<C>;
  const size_t nv = static_cast<size_t>(s.B) * s.Hv * static_cast<size_t>((s.T + C - 1) / C);
  WsCW w{};
  size_t off = 0;
  w.kimg = off;    off = up(off + nv * IM::KEY);
  w.cimg = off;    off = up(off + nv * IM::CHK);
  w.hst = off;     off = up(off + nv * DK * DK * 2);
  w.dhst = off;    off = up(off + nv * DK * DK * 2);
  w.pkimg = off;   off = up(off + static_cast<size_t>(s.B) * s.Hk * ((s.T + C - 1) / C) * Img<C>::KEY);
  w.total = off;
  return w;
}

template <int C>
hipError_t bwd_cw(const Shape& s, const ChunkBwdArgs& x, void* ws, hipStream_t st) {
  const WsCW w = plan_cw_bwd<C>(s);
  Ws16 w16{};
  w16.kimg = w.kimg;
  w16.cimg = w.cimg;
  w16.hst = w.hst;
  w16.dhst = w.dhst;
  K16 a = args16(s, C, ws, w16);
  a.cu = x.cu;
  a.q = static_cast<const bf16_t*>(x.q);
  a.k = static_cast<const bf16_t*>(x.k);
  a.v = static_cast<const bf16_t*>(x.v);
  a.dout = static_cast<const bf16_t*>(x.dout);
  a.g = x.g;
  a.beta = x.beta;
  a.h0 = x.h0;
  a.dht = x.dht;
  a.dh0 = x.dh0;
  a.pkimg = static_cast<char*>(ws) + w.pkimg;
  const int nw = chain_waves(a);
  {
    ProfScope ps("chunk_prep_cw", st);
    hipLaunchKernelGGL((cwprep16_kernel<C>), dim3(a.NC, a.Hv, static_cast<unsigned>(a.B)), dim3(512), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("chunk_states_cw", st);
    with_chain_waves(nw, [&](auto w) {
      constexpr int NW = decltype(w)::value;
      hipLaunchKernelGGL((cwchain16_kernel<C, bf16_t, false, true, NW>), chain_grid(a, NW), dim3(64 * (NW + 1)), 0, st, a);
    });
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("chunk_dh_cw", st);
    with_chain_waves(nw, [&](auto w) {
      constexpr int NW = decltype(w)::value;
      hipLaunchKernelGGL((cwdh16_kernel<C, NW>), chain_grid(a, NW), dim3(64 * (NW + 1)), 0, st, a);
    });
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.dq = x.dq;
  a.dk = x.dk;
  a.dv = x.dv;
  a.dg = x.dg;
  a.dbeta = x.dbeta;
  ProfScope ps("chunk_grad_cw", st);
  const dim3 grid(a.NC, a.Hk, static_cast<unsigned>(a.B));
  if (s.out_bf16)
    hipLaunchKernelGGL((cwgrad16_kernel<C, bf16_t>), grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((cwgrad16_kernel<C, float>), grid, dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace

size_t chunk16_fwd_workspace(const Shape& s, int C) {
  if (s.channelwise) return C == 64 ? plan_cw<64>(s).total : plan_cw<32>(s).total;
  return plan_any(s, C, s.save_chunks).total;
}
size_t chunk16_bwd_workspace(const Shape& s, int C) {
  if (s.channelwise) return C == 64 ? plan_cw_bwd<64>(s).total : plan_cw_bwd<32>(s).total;
  return plan_any(s, C, true).total;
}

hipError_t launch_chunk16_fwd(const Shape& s, int C, const ChunkFwdArgs& x, void* ws, hipStream_t st) {
  if (s.channelwise) {
    if (C == 64) return s.out_bf16 ? fwd_cw<64, bf16_t>(s, x, ws, st) : fwd_cw<64, float>(s, x, ws, st);
    if (C == 32) return s.out_bf16 ? fwd_cw<32, bf16_t>(s, x, ws, st) : fwd_cw<32, float>(s, x, ws, st);
    return hipErrorInvalidValue;
  }
  if (C == 64) return s.out_bf16 ? fwd_all<64, bf16_t>(s, x, ws, st) : fwd_all<64, float>(s, x, ws, st);
  if (C == 32) return s.out_bf16 ? fwd_all<32, bf16_t>(s, x, ws, st) : fwd_all<32, float>(s, x, ws, st);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk16_bwd(const Shape& s, int C, const ChunkBwdArgs& x, void* ws, hipStream_t st) {
  if (s.channelwise) {
    if (C == 64) return bwd_cw<64>(s, x, ws, st);
    if (C == 32) return bwd_cw<32>(s, x, ws, st);
    return hipErrorInvalidValue;
  }
  if (C == 64) return s.out_bf16 ? bwd_all<64, bf16_t>(s, x, ws, st) : bwd_all<64, float>(s, x, ws, st);
  if (C == 32) return s.out_bf16 ? bwd_all<32, bf16_t>(s, x, ws, st) : bwd_all<32, float>(s, x, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace gdr
