// Host-side interface between the C ABI (gdr_api.hip) and the kernel
// translation units.  Shapes here are already validated.
#pragma once

#include <gdr.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// Keeps the text of a failed HIP call for gdr_last_hip_error() (this
// thread) and returns GDR_ERR_HIP.
gdr_status record_hip_error(hipError_t e);

// Brackets one kernel launch with profiling events when gdr_profile_enable
// is on for this thread (no-op otherwise).
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t st);
  ~ProfScope();
 private:
  hipStream_t stream_;
  bool active_;
};

struct Shape {
  int64_t B, T;
  int Hk, Hv, D;      // Dk == Dv == D
  bool io_bf16, out_bf16, l2norm, channelwise, fused_gates;
  bool save_chunks;  // fp16 chunked path: forward keeps images and chunk states, backward reuses them
};

// ---- sequential (token-by-token) path ------------------------------------
struct SeqFwdArgs {
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  void* o;
  float* ht;
  const int64_t* cu;  // ragged batch row offsets [B + 1], or null
};
hipError_t launch_seq_fwd(const Shape& s, const SeqFwdArgs& a, hipStream_t st);

// Checkpoint every kSeqSeg tokens; per-WG replay scratch of kSeqSeg states.
constexpr int kSeqSeg = 16;
int seq_bwd_slices(const Shape& s);            // value slices per head
size_t seq_bwd_ckpt_floats(const Shape& s);    // checkpoint buffer
size_t seq_bwd_scratch_floats(const Shape& s); // replay buffer

struct SeqBwdArgs {
  const void *q, *k, *v, *dout;
  const float *g, *beta, *h0, *dht;
  void* dv;
  float* dh0;
  float* ckpt;       // seq_bwd_ckpt_floats
  float* scratch;    // seq_bwd_scratch_floats
  float* part_dq;    // [NS][B][T][Hv][D] partial dq_hat per value slice
  float* part_dk;    // [NS][B][T][Hv][D]
  float* part_db;    // [NS][B][T][Hv]
  float* part_dg;    // [NS][B][T][Hv] or [NS][B][T][Hv][D]
  const int64_t* cu; // ragged batch row offsets [B + 1], or null (partials stay [B][T])
};
hipError_t launch_seq_bwd(const Shape& s, const SeqBwdArgs& a, hipStream_t st);

// ---- backward epilogue (shared by both paths) ------------------------------
// Sums per-slice / per-v-head partials in a fixed order, applies the L2-norm
// VJP and writes dq, dk (out dtype); sums dbeta / dg partials when given.
struct EpiArgs {
  const void *q, *k;
  const float *part_dq, *part_dk, *part_db, *part_dg;  // part_db/dg may be null
  int nslices;
  void *dq, *dk;
  float *dbeta, *dg;
  const float *g, *beta;  // gate inputs (pre-activations with fused gates)
  const int64_t* cu;      // ragged batch row offsets [B + 1], or null
};
hipError_t launch_bwd_epilogue(const Shape& s, const EpiArgs& a, hipStream_t st);

// ---- chunked (matrix-core) path --------------------------------------------
// fp16 matrix-core operands are used for bf16 io with Dk = 128 and C >= 32
// (gdr_chunk16.hip); every other supported shape uses fp32 operands
// (gdr_chunk.hip).  Each implementation sizes and carves its own workspace.
bool chunk_uses_f16(const Shape& s, int C);
size_t chunk_fwd_workspace(const Shape& s, int C);
size_t chunk_bwd_workspace(const Shape& s, int C);

struct ChunkFwdArgs {
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  void* o;
  float* ht;
  const int64_t* cu;  // ragged batch row offsets [B + 1] (fp16 path only), or null
};
hipError_t launch_chunk_fwd(const Shape& s, int C, const ChunkFwdArgs& a, void* ws, hipStream_t st);

// VJP: recomputes every chunk's entry state, runs the reverse dH pass
// (writes dv, dh0), the per-chunk gradient pass (dg, dbeta, per-v-head
// dq_hat / dk_hat) and the epilogue (dq, dk).
struct ChunkBwdArgs {
  const void *q, *k, *v, *dout;
  const float *g, *beta, *h0, *dht;
  void *dq, *dk, *dv;
  float *dg, *dbeta, *dh0;
  const int64_t* cu;  // ragged batch row offsets [B + 1] (fp16 path only), or null
};
hipError_t launch_chunk_bwd(const Shape& s, int C, const ChunkBwdArgs& a, void* ws, hipStream_t st);

size_t chunk16_fwd_workspace(const Shape& s, int C);
size_t chunk16_bwd_workspace(const Shape& s, int C);
hipError_t launch_chunk16_fwd(const Shape& s, int C, const ChunkFwdArgs& a, void* ws, hipStream_t st);
hipError_t launch_chunk16_bwd(const Shape& s, int C, const ChunkBwdArgs& a, void* ws, hipStream_t st);

}  // namespace gdr
