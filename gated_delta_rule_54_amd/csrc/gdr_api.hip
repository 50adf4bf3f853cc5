// C ABI of libgdr (declared in include/gdr.h): argument validation,
// workspace sizing and carving, algorithm choice, kernel launches.
// Nothing here allocates, frees or synchronises.

#include <gdr.h>

#include <string.h>

#include <mutex>
#include <string>

#include "gdr_internal.h"

namespace {

thread_local std::string g_last_hip_error;

using gdr::Shape;

constexpr size_t kWsAlign = 256;

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool misaligned(const void* p, uintptr_t a = 16) {
  return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) != 0;
}

gdr_status check_problem(const gdr_problem* p) {
  if (!p) return GDR_ERR_NULL_ARG;
  if (p->B < 0 || p->T < 0 || p->Hk <= 0 || p->Hv <= 0 || p->Dk <= 0 || p->Dv <= 0)
    return GDR_ERR_BAD_SHAPE;
  if (p->Hv % p->Hk != 0) return GDR_ERR_BAD_SHAPE;
  if (p->Dk != p->Dv || (p->Dk != 16 && p->Dk != 128)) return GDR_ERR_UNSUPPORTED;
  if ((p->io_dtype != GDR_F32 && p->io_dtype != GDR_BF16) ||
      (p->out_dtype != GDR_F32 && p->out_dtype != GDR_BF16))
    return GDR_ERR_UNSUPPORTED;
  if (p->flags & ~static_cast<uint32_t>(GDR_USE_QK_L2NORM | GDR_CHANNELWISE | GDR_FUSED_GATES | GDR_SAVE_CHUNKS))
    return GDR_ERR_UNSUPPORTED;
  if (p->algo < GDR_ALGO_AUTO || p->algo > GDR_ALGO_CHUNKED) return GDR_ERR_UNSUPPORTED;
  if (p->chunk_size != 0 && p->chunk_size != 16 && p->chunk_size != 32 && p->chunk_size != 64)
    return GDR_ERR_UNSUPPORTED;
  // grid limits: B is a grid dimension, B*T*Hk rows in the epilogue
  if (p->B > 65535 || p->Hv > 65535) return GDR_ERR_UNSUPPORTED;
  if (p->B * p->T * p->Hk > 0x7fffffffLL) return GDR_ERR_UNSUPPORTED;
  return GDR_OK;
}

Shape shape_of(const gdr_problem* p) {
  Shape s;
  s.B = p->B;
  s.T = p->T;
  s.Hk = p->Hk;
  s.Hv = p->Hv;
  s.D = p->Dk;
  s.io_bf16 = p->io_dtype == GDR_BF16;
  s.out_bf16 = p->out_dtype == GDR_BF16;
  s.l2norm = (p->flags & GDR_USE_QK_L2NORM) != 0;
  s.channelwise = (p->flags & GDR_CHANNELWISE) != 0;
  s.fused_gates = (p->flags & GDR_FUSED_GATES) != 0;
  s.save_chunks = (p->flags & GDR_SAVE_CHUNKS) != 0 && !s.channelwise;
  return s;
}

// Chunk size actually used (0 means 64).
int chunk_of(const gdr_problem* p) { return p->chunk_size ? p->chunk_size : 64; }

constexpr bool kChunkedBackward = true;

// Shortest T at which AUTO takes the chunked kernels: below it the
// sequential kernels' per-token cost is under the chunked pipeline's fixed
// cost.  Measured on MI355X (HIP events, B in {1, 4, 8}, Hv = 32, D = 128):
// on the fp16 path the forward takes 16 vs 19-26 us sequential against
// chunked at T = 8 and 26-32 vs 19-27 at T = 16; the scalar VJP 34-50 vs
// 39-57 at T = 4 and 54-78 vs 38-59 at T = 8; the channelwise VJP 66-76 vs
// 68-78 at T = 8 and 117-134 vs 69-79 at T = 16.  On the fp32 path (fp32 io
// or D = 16) the chunked pipeline costs more: forward 43 vs 63 us at T = 32,
// 82-98 vs 64-94 at T = 64; VJP 182-205 vs 206-260 at T = 32, 368-405 vs
// 214-276 at T = 64.
constexpr int kAutoChunkedFwdT = 12, kAutoChunkedBwdT = 6, kAutoChunkedBwdTChannelwise = 10, kAutoChunkedF32T = 64;

// SEQUENTIAL or CHUNKED for this call.
gdr_status resolve_algo(const gdr_problem* p, bool backward, int* algo, bool ragged = false) {
  // channelwise gates: chunked kernels on the fp16 matrix-core path only
  // (bf16 io, Dk = 128, C >= 32).  Ragged batches: the chunked kernels on
  // that path, and the sequential ones.
  const bool f16 = gdr::chunk_uses_f16(shape_of(p), chunk_of(p));
  const bool chunk_ok = (p->flags & GDR_CHANNELWISE) ? f16
                                                     : (!backward || kChunkedBackward) && (!ragged || f16);
  const bool seq_ok = true;
  if (p->algo == GDR_ALGO_CHUNKED) {
    if (!chunk_ok) return GDR_ERR_UNSUPPORTED;
    *algo = GDR_ALGO_CHUNKED;
  } else if (p->algo == GDR_ALGO_AUTO) {
    const int64_t t_min = !f16                          ? kAutoChunkedF32T
                          : !backward                    ? kAutoChunkedFwdT
                          : (p->flags & GDR_CHANNELWISE) ? kAutoChunkedBwdTChannelwise
                                                         : kAutoChunkedBwdT;
    if (chunk_ok && (p->T >= t_min || !seq_ok)) *algo = GDR_ALGO_CHUNKED;
    else if (seq_ok) *algo = GDR_ALGO_SEQUENTIAL;
    else return GDR_ERR_UNSUPPORTED;
  } else {
    if (!seq_ok) return GDR_ERR_UNSUPPORTED;
    *algo = GDR_ALGO_SEQUENTIAL;
  }
  return GDR_OK;
}

// Whether gdr_forward with GDR_SAVE_CHUNKS leaves its chunks for the VJP of
// problem p: the forward's algorithm is the chunked one on its fp16 path with
// a scalar gate.  AUTO's forward and backward can choose different
// algorithms for one T, so the backward honours the flag only where this
// holds (elsewhere both calls ignore it).
bool forward_keeps_chunks(const gdr_problem* p, bool ragged = false) {
  int algo;
  if (resolve_algo(p, false, &algo, ragged) != GDR_OK) return false;
  const Shape s = shape_of(p);
  return algo == GDR_ALGO_CHUNKED && !s.channelwise && gdr::chunk_uses_f16(s, chunk_of(p));
}

// The shape of a backward call: GDR_SAVE_CHUNKS only where the forward keeps chunks.
Shape backward_shape(const gdr_problem* p, bool ragged = false) {
  Shape s = shape_of(p);
  if (s.save_chunks && !forward_keeps_chunks(p, ragged)) s.save_chunks = false;
  return s;
}

// ---- workspace plans: byte offsets of each carved buffer -----------------
struct BwdPlan {
  size_t ckpt, scratch, pdq, pdk, pdb, pdg, total;
};

BwdPlan plan_seq_bwd(const Shape& s) {
  BwdPlan w{};
  const size_t ns = static_cast<size_t>(gdr::seq_bwd_slices(s));
  const size_t rows = static_cast<size_t>(s.B * s.T * s.Hv);
  size_t off = 0;
  w.ckpt = off;    off = align_up(off + gdr::seq_bwd_ckpt_floats(s) * 4);
  w.scratch = off; off = align_up(off + gdr::seq_bwd_scratch_floats(s) * 4);
  w.pdq = off;     off = align_up(off + ns * rows * s.D * 4);
  w.pdk = off;     off = align_up(off + ns * rows * s.D * 4);
  w.pdb = off;     off = align_up(off + ns * rows * 4);
  w.pdg = off;     off = align_up(off + ns * rows * (s.channelwise ? s.D : 1) * 4);
  w.total = off;
  return w;
}

gdr_status hip_fail(hipError_t e) { return gdr::record_hip_error(e); }

template <typename T> T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

// ---- fixed device scratch for gdr_forward_noalloc -------------------------
// A file-scope device array holds the workspace of the allocation-free
// forward.  Every GPU the library runs on keeps its own copy until the
// process ends.  Host code never passes the array's name (a host-side
// stand-in) to a kernel or copy: it uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on that device's first call.
namespace {

constexpr size_t kScratchBytes = size_t(GDR_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address (looked up once per device, with that
// device current).
gdr_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gdr::record_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return GDR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return gdr::record_hip_error(e);
    if (!p) return GDR_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDR_OK;
}

}  // namespace

gdr_status gdr::record_hip_error(hipError_t e) {
  g_last_hip_error = hipGetErrorString(e);
  return GDR_ERR_HIP;
}

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char* gdr_status_str(gdr_status s) {
  switch (s) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL_ARG: return "required pointer argument is NULL";
    case GDR_ERR_BAD_SHAPE: return "invalid shape (negative size or Hv % Hk != 0)";
    case GDR_ERR_UNSUPPORTED: return "unsupported problem (dims, dtype, flags, algo or chunk size)";
    case GDR_ERR_BAD_ALIGNMENT: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case GDR_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the size query returned";
    case GDR_ERR_HIP: return "HIP error (see gdr_last_hip_error)";
    case GDR_STATUS_MAX_ENUM: break;
  }
  return "unknown gdr_status";
}

const char* gdr_last_hip_error(void) { return g_last_hip_error.c_str(); }

gdr_status gdr_forward_workspace(const gdr_problem* p, size_t* bytes) {
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  if (!bytes) return GDR_ERR_NULL_ARG;
  int algo;
  if ((st = resolve_algo(p, false, &algo)) != GDR_OK) return st;
  const Shape s = shape_of(p);
  *bytes = (algo == GDR_ALGO_CHUNKED && s.B > 0 && s.T > 0) ? gdr::chunk_fwd_workspace(s, chunk_of(p)) : 0;
  return GDR_OK;
}

gdr_status gdr_keeps_chunks(const gdr_problem* p, int* keeps) {
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  if (!keeps) return GDR_ERR_NULL_ARG;
  int algo;
  if ((st = resolve_algo(p, false, &algo)) != GDR_OK) return st;
  *keeps = forward_keeps_chunks(p) ? 1 : 0;
  return GDR_OK;
}

gdr_status gdr_backward_workspace(const gdr_problem* p, size_t* bytes) {
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  if (!bytes) return GDR_ERR_NULL_ARG;
  int algo;
  if ((st = resolve_algo(p, true, &algo)) != GDR_OK) return st;
  const Shape s = backward_shape(p);
  *bytes = (s.B == 0 || s.T == 0) ? 0
           : algo == GDR_ALGO_CHUNKED ? gdr::chunk_bwd_workspace(s, chunk_of(p)) : plan_seq_bwd(s).total;
  return GDR_OK;
}

namespace {

// gdr_forward / gdr_forward_varlen (cu: ragged-batch row offsets or null).
gdr_status forward_impl(const gdr_problem* p, const int64_t* cu, bool ragged, const void* q, const void* k,
                        const void* v, const float* g, const float* beta, const float* h0, void* o, float* ht,
                        void* ws, size_t ws_bytes, void* hip_stream) {
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  const Shape s = shape_of(p);
  const bool empty = s.B == 0 || s.T == 0;
  if (!empty && (!q || !k || !v || !g || !beta || !o)) return GDR_ERR_NULL_ARG;
  if (ragged && !empty && !cu) return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, g, beta, h0, o, ht};
  for (const void* ptr : ptrs)
    if (misaligned(ptr)) return GDR_ERR_BAD_ALIGNMENT;
  if (misaligned(ws, kWsAlign) || misaligned(cu, 8)) return GDR_ERR_BAD_ALIGNMENT;
  int algo;
  if ((st = resolve_algo(p, false, &algo, ragged)) != GDR_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (s.B == 0) return GDR_OK;
  const size_t state_bytes = static_cast<size_t>(s.B * s.Hv) * s.D * s.D * sizeof(float);
  if (s.T == 0) {
    if (!ht) return GDR_OK;
    hipError_t e = h0 ? (h0 == ht ? hipSuccess : hipMemcpyAsync(ht, h0, state_bytes, hipMemcpyDeviceToDevice, stream))
                      : hipMemsetAsync(ht, 0, state_bytes, stream);
    return e == hipSuccess ? GDR_OK : hip_fail(e);
  }
  if (algo == GDR_ALGO_CHUNKED) {
    if (!ws) return GDR_ERR_NULL_ARG;
    if (ws_bytes < gdr::chunk_fwd_workspace(s, chunk_of(p))) return GDR_ERR_WORKSPACE_TOO_SMALL;
    gdr::ChunkFwdArgs a{q, k, v, g, beta, h0, o, ht, cu};
    hipError_t e = gdr::launch_chunk_fwd(s, chunk_of(p), a, ws, stream);
    return e == hipSuccess ? GDR_OK : hip_fail(e);
  }
  gdr::SeqFwdArgs a{q, k, v, g, beta, h0, o, ht, cu};
  hipError_t e = gdr::launch_seq_fwd(s, a, stream);
  return e == hipSuccess ? GDR_OK : hip_fail(e);
}

// gdr_backward / gdr_backward_varlen.
gdr_status backward_impl(const gdr_problem* p, const int64_t* cu, bool ragged, const void* q, const void* k,
                         const void* v, const float* g, const float* beta, const float* h0, const void* dout,
                         const float* dht, void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                         void* ws, size_t ws_bytes, void* hip_stream) {
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  const Shape s = backward_shape(p, ragged);
  const bool empty = s.B == 0 || s.T == 0;
  if (!empty && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
    return GDR_ERR_NULL_ARG;
  if (ragged && !empty && !cu) return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, g, beta, h0, dout, dht, dq, dk, dv, dg, dbeta, dh0};
  for (const void* ptr : ptrs)
    if (misaligned(ptr)) return GDR_ERR_BAD_ALIGNMENT;
  if (misaligned(ws, kWsAlign) || misaligned(cu, 8)) return GDR_ERR_BAD_ALIGNMENT;
  int algo;
  if ((st = resolve_algo(p, true, &algo, ragged)) != GDR_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (s.B == 0) return GDR_OK;
  const size_t state_bytes = static_cast<size_t>(s.B * s.Hv) * s.D * s.D * sizeof(float);
  if (s.T == 0) {
    if (!dh0) return GDR_OK;
    hipError_t e = dht ? hipMemcpyAsync(dh0, dht, state_bytes, hipMemcpyDeviceToDevice, stream)
                       : hipMemsetAsync(dh0, 0, state_bytes, stream);
    return e == hipSuccess ? GDR_OK : hip_fail(e);
  }
  if (algo == GDR_ALGO_CHUNKED) {
    const int C = chunk_of(p);
    if (!ws) return GDR_ERR_NULL_ARG;
    if (ws_bytes < gdr::chunk_bwd_workspace(s, C)) return GDR_ERR_WORKSPACE_TOO_SMALL;
    gdr::ChunkBwdArgs a{q, k, v, dout, g, beta, h0, dht, dq, dk, dv, dg, dbeta, dh0, cu};
    hipError_t e = gdr::launch_chunk_bwd(s, C, a, ws, stream);
    return e == hipSuccess ? GDR_OK : hip_fail(e);
  }
  const BwdPlan w = plan_seq_bwd(s);
  if (!ws) return GDR_ERR_NULL_ARG;
  if (ws_bytes < w.total) return GDR_ERR_WORKSPACE_TOO_SMALL;
  gdr::SeqBwdArgs a{q, k, v, dout, g, beta, h0, dht, dv, dh0,
                    at<float>(ws, w.ckpt), at<float>(ws, w.scratch), at<float>(ws, w.pdq),
                    at<float>(ws, w.pdk), at<float>(ws, w.pdb), at<float>(ws, w.pdg), cu};
  hipError_t e = gdr::launch_seq_bwd(s, a, stream);
  if (e != hipSuccess) return hip_fail(e);
  gdr::EpiArgs ea{q, k, a.part_dq, a.part_dk, a.part_db, a.part_dg, gdr::seq_bwd_slices(s), dq, dk, dbeta, dg, g, beta,
                  cu};
  e = gdr::launch_bwd_epilogue(s, ea, stream);
  return e == hipSuccess ? GDR_OK : hip_fail(e);
}

}  // namespace

gdr_status gdr_forward(const gdr_problem* p, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* h0, void* o, float* ht,
                       void* ws, size_t ws_bytes, void* hip_stream) {
  return forward_impl(p, nullptr, false, q, k, v, g, beta, h0, o, ht, ws, ws_bytes, hip_stream);
}

gdr_status gdr_forward_noalloc(const gdr_problem* p, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const float* h0, void* o, float* ht,
                               void* hip_stream) {
  gdr_status st = check_problem(p);
  if (st != GDR_OK) return st;
  if (p->flags & GDR_SAVE_CHUNKS) return GDR_ERR_UNSUPPORTED;  // the scratch is not the caller's to keep
  size_t need = 0;
  if ((st = gdr_forward_workspace(p, &need)) != GDR_OK) return st;
  if (need > kScratchBytes) return GDR_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0 && (st = device_scratch(&ws)) != GDR_OK) return st;
  return forward_impl(p, nullptr, false, q, k, v, g, beta, h0, o, ht, ws, need, hip_stream);
}

gdr_status gdr_forward_varlen(const gdr_problem* p, const int64_t* cu_seqlens, const void* q, const void* k,
                              const void* v, const float* g, const float* beta, const float* h0, void* o,
                              float* ht, void* ws, size_t ws_bytes, void* hip_stream) {
  return forward_impl(p, cu_seqlens, true, q, k, v, g, beta, h0, o, ht, ws, ws_bytes, hip_stream);
}

gdr_status gdr_backward(const gdr_problem* p, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* h0, const void* dout,
                        const float* dht, void* dq, void* dk, void* dv, float* dg, float* dbeta,
                        float* dh0, void* ws, size_t ws_bytes, void* hip_stream) {
  return backward_impl(p, nullptr, false, q, k, v, g, beta, h0, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws,
                       ws_bytes, hip_stream);
}

gdr_status gdr_backward_varlen(const gdr_problem* p, const int64_t* cu_seqlens, const void* q, const void* k,
                               const void* v, const float* g, const float* beta, const float* h0,
                               const void* dout, const float* dht, void* dq, void* dk, void* dv, float* dg,
                               float* dbeta, float* dh0, void* ws, size_t ws_bytes, void* hip_stream) {
  return backward_impl(p, cu_seqlens, true, q, k, v, g, beta, h0, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws,
                       ws_bytes, hip_stream);
}

}  // extern "C"
