/*
 * gdr.h - C ABI of libgdr: the gated delta rule (forward and VJP) on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The pages this library follows all turn on the gated
 * delta rule ("Adding VJP for gated delta net", ml-explore/mlx pull request
 * 4565; "Two-pass optimization for channelwise gated delta rule kernel",
 * pytorch/executorch pull request 21020; "perf(gated_delta_net): fold q/k
 * L2-norm into the gated_delta_rule kernel", NVIDIA/Megatron-LM pull request
 * 5396).  Per batch b and value head h, a state S (Dv x Dk) evolves per
 * token t as
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * the published gated delta rule (Yang, Kautz & Hatamizadeh, ICLR 2025).
 *   - alpha_t = exp(g_t).  g is a scalar per (b, t, h), or, with
 *     GDR_CHANNELWISE, one value per key channel (the ExecuTorch page's
 *     channelwise kernel): then the decay diag(alpha_t) is applied to the
 *     state before the prediction, S_{t-1} diag(alpha_t) (I - beta k k^T).
 *   - With GDR_USE_QK_L2NORM, q_t and k_t are replaced by
 *     x * (sum x^2 + 1e-6)^(-1/2) over the key dim inside the kernels (the
 *     Megatron-LM page, "What"/"Why"); without it they are used as given.
 *   - GQA: q and k have Hk heads; value head h reads k/q head h / (Hv/Hk).
 *   - No output scale is applied.
 *
 * Memory.  The state is stored as H = S^T with layout [B, Hv, Dk, Dv]
 * (Dv contiguous), always fp32.  All tensors are dense, row-major and
 * contiguous:
 *   q, k          [B, T, Hk, Dk]     io_dtype
 *   v, dout       [B, T, Hv, Dv]     io_dtype
 *   g             [B, T, Hv] (scalar gate) or [B, T, Hv, Dk] (channelwise), fp32
 *   beta          [B, T, Hv]         fp32
 *   h0, ht, dh0, dht  [B, Hv, Dk, Dv] fp32
 *   o, dv         [B, T, Hv, Dv]     out_dtype
 *   dq, dk        [B, T, Hk, Dk]     out_dtype
 *   dg            same shape as g, fp32;  dbeta [B, T, Hv] fp32
 *
 * Ownership and threading.  Every tensor pointer, including the workspace,
 * is a DEVICE pointer owned by the caller.  The library never allocates,
 * frees or synchronises: calls validate, then enqueue kernels on
 * `hip_stream` (a hipStream_t; NULL = the default stream) and return.  Calls
 * on different streams may run concurrently if their buffers are disjoint.
 *
 * Errors.  All arguments are checked before anything is launched; on any
 * error nothing is written and a status other than GDR_OK is returned.  A
 * failed kernel launch returns GDR_ERR_HIP and the HIP error text is kept in
 * a thread-local string read by gdr_last_hip_error().  No exception or abort
 * crosses this boundary.  NaN/Inf inputs propagate and never trap.
 *
 * Supported sizes.  Dk == Dv, with Dk in {16, 128}; Hv % Hk == 0; T >= 0
 * (T == 0: forward copies h0, or zeros, into ht; backward copies dht, or
 * zeros, into dh0).  Every pointer must be 16-byte aligned, the workspace
 * 256-byte aligned.  Results are bitwise reproducible from run to run
 * (fixed reduction orders, no floating-point atomics).
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 4

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_ERR_NULL_ARG = 1,            /* a required pointer is NULL            */
  GDR_ERR_BAD_SHAPE = 2,           /* negative/zero sizes, Hv % Hk != 0     */
  GDR_ERR_UNSUPPORTED = 3,         /* a valid problem this build cannot run */
  GDR_ERR_BAD_ALIGNMENT = 4,       /* pointer not 16 B (workspace 256 B)    */
  GDR_ERR_WORKSPACE_TOO_SMALL = 5, /* ws_bytes below the *_workspace size   */
  GDR_ERR_HIP = 6,                 /* a HIP launch or copy failed           */
  /* Never returned.  Widens the type's range to every non-negative int, so
   * any status value a caller passes back (gdr_status_str) is a value of
   * the type in C++ as in C. */
  GDR_STATUS_MAX_ENUM = 0x7fffffff
} gdr_status;

typedef enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

/* How the time axis is processed.  Both are HIP kernels.
 *   SEQUENTIAL: one token after another, fp32 state on chip (the decode
 *     kernel; the MLX page's "sequential" VJP).  Every shape is supported.
 *   CHUNKED: tokens grouped in chunks of chunk_size; the work inside a chunk
 *     runs as dense matrix-core products (the MLX page's "chunked" VJP).
 *     Scalar gate: bf16 io uses fp16 matrix-core operands with fp32
 *     accumulation (Dk = 128, chunk_size 32 or 64), every other shape fp32
 *     matrix-core operands.  Channelwise gate: bf16 io, Dk = 128,
 *     chunk_size 32 or 64 only (see below).
 *   AUTO: CHUNKED when supported and T is at least 12 (gdr_forward), 6
 *     (gdr_backward) or 10 (gdr_backward with GDR_CHANNELWISE) on the fp16
 *     matrix-core path, 64 on the fp32 one, else SEQUENTIAL: below those
 *     lengths the sequential kernels are the faster of the two on MI355X.
 *
 * Range of the fp16 chunked path.  Its matrix-core operands (normalised
 * q / k, v and dout rows, T = (I + A)^-1, the chunk states it keeps) are
 * fp16, whose finite range is +-65504; accumulation and the carried state
 * are fp32.  bf16 inputs convert to fp16 exactly inside that range.  A
 * v or dout element beyond it (or a T entry beyond it, possible only with
 * beta outside (0, 1)) overflows to +-Inf in its operand, and the outputs
 * that depend on it come out non-finite (Inf or NaN), never finite and
 * wrong.  Inputs of that size need the SEQUENTIAL algorithm or fp32 io. */
typedef enum gdr_algo {
  GDR_ALGO_AUTO = 0,
  GDR_ALGO_SEQUENTIAL = 1,
  GDR_ALGO_CHUNKED = 2
} gdr_algo;

/* GDR_FUSED_GATES: g and beta carry pre-activations a and b; the kernels
 * use g = -softplus(a) = -log(1 + e^a) (so alpha = 1 / (1 + e^a)) and
 * beta = sigmoid(b), and gdr_backward returns dg = dL/da and dbeta = dL/db.
 * This folds the caller's gate preparation into the kernels, in the spirit
 * of the Megatron-LM page's L2-norm fold ("What"/"Why"); the activations are
 * this library's choice (the pages name none).  Works with every algorithm
 * and with GDR_CHANNELWISE (then a has g's per-channel shape). */
/* GDR_SAVE_CHUNKS: keep the forward's per-chunk work for the VJP (what a
 * training step's autograd saves), on the chunked algorithm with bf16 io,
 * Dk = Dv = 128, chunk_size 32 or 64 and a scalar gate; elsewhere (the
 * SEQUENTIAL algorithm, also when AUTO picks it; fp32 io; Dk = 16; the
 * channelwise gate) both calls ignore the flag, and gdr_keeps_chunks tells
 * which case a problem is.  gdr_forward then needs gdr_backward_workspace(p) bytes
 * of workspace (gdr_forward_workspace reports that size) and leaves the
 * chunk images (normalised q/k, gates, T = (I + A)^-1, P) and every
 * chunk's entry state there; gdr_backward with the same problem, the same
 * inputs and that workspace, untouched in between, reads them instead of
 * recomputing them (it skips the prep and the chunk-state pass).  The
 * library cannot check that contract: a workspace not written by such a
 * forward gives wrong gradients (never an out-of-bounds access). */
enum { GDR_USE_QK_L2NORM = 1u, GDR_CHANNELWISE = 2u, GDR_FUSED_GATES = 4u, GDR_SAVE_CHUNKS = 8u };

typedef struct gdr_problem {
  int64_t B, T;       /* batch, tokens                                      */
  int32_t Hk, Hv;     /* k/q heads, v heads (Hv % Hk == 0)                  */
  int32_t Dk, Dv;     /* key and value head dims                            */
  int32_t io_dtype;   /* gdr_dtype of q, k, v, dout                         */
  int32_t out_dtype;  /* gdr_dtype of o, dq, dk, dv                         */
  uint32_t flags;     /* GDR_USE_QK_L2NORM | GDR_CHANNELWISE | GDR_FUSED_GATES
                         | GDR_SAVE_CHUNKS                                    */
  int32_t algo;       /* gdr_algo                                           */
  int32_t chunk_size; /* CHUNKED only: 16, 32 or 64; 0 means 64             */
} gdr_problem;
/* With GDR_CHANNELWISE, GDR_ALGO_CHUNKED is supported with bf16 io,
 * Dk = Dv = 128 and chunk_size 32 or 64 (else GDR_ERR_UNSUPPORTED); its VJP
 * forms each chunk's gradients from the chunk states the chunk chains store,
 * the per-channel decay carried inside the chunk-local sums (matrix cores
 * below the diagonal blocks, matrix cores or exact fp32 sums on them).
 * AUTO picks the chunked kernels there from the lengths given above. */

/* *keeps = 1 when GDR_SAVE_CHUNKS takes effect for problem *p (whether or
 * not the flag is set in p->flags), i.e. when gdr_forward with the flag
 * leaves its chunks in the workspace for gdr_backward; else 0, and both
 * calls ignore the flag.  Returns the validation status of the problem;
 * *keeps is written only on GDR_OK. */
gdr_status gdr_keeps_chunks(const gdr_problem* p, int* keeps);

/* Workspace bytes the call needs for problem *p (0 is possible).  Returns
 * the same validation status gdr_forward/gdr_backward would for the shape
 * part of the problem; *bytes is written only on GDR_OK. */
gdr_status gdr_forward_workspace(const gdr_problem* p, size_t* bytes);
gdr_status gdr_backward_workspace(const gdr_problem* p, size_t* bytes);

/* Forward pass.  h0 may be NULL (zero initial state).  ht may be NULL (final
 * state not wanted) and may alias h0 exactly (in-place decode: each kernel
 * reads its whole part of the state before writing it).  o must not alias
 * any input.  ws may be NULL when the workspace size is 0. */
gdr_status gdr_forward(const gdr_problem* p, const void* q, const void* k,
                       const void* v, const float* g, const float* beta,
                       const float* h0, void* o, float* ht, void* ws,
                       size_t ws_bytes, void* hip_stream);

/* VJP of gdr_forward for the loss <dout, o> + <dht, ht>.  Without
 * GDR_SAVE_CHUNKS the backward is stateless: it takes the forward's raw
 * inputs (q, k unnormalised when the flag is set) and recomputes what it
 * needs.  h0 and dht may be NULL (zeros); dh0 may be NULL (not wanted).
 * dq, dk, dv, dg, dbeta are required and must not alias inputs. */
gdr_status gdr_backward(const gdr_problem* p, const void* q, const void* k,
                        const void* v, const float* g, const float* beta,
                        const float* h0, const void* dout, const float* dht,
                        void* dq, void* dk, void* dv, float* dg, float* dbeta,
                        float* dh0, void* ws, size_t ws_bytes,
                        void* hip_stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): gdr_forward with the workspace taken from a fixed scratch
 * array of GDR_NOALLOC_SCRATCH_BYTES (64 MiB) that the library keeps on
 * every GPU it runs on until the process ends.  The call allocates and
 * frees nothing; the caller still owns q .. ht.  Limits: problems whose
 * gdr_forward_workspace exceeds the scratch return
 * GDR_ERR_WORKSPACE_TOO_SMALL before anything is launched (the chunked path
 * needs about 1.1 MiB per 64 tokens of each sequence at Hk = 16, Hv = 32,
 * D = 128; the sequential path needs none); GDR_SAVE_CHUNKS returns
 * GDR_ERR_UNSUPPORTED.  All calls on one GPU share that GPU's scratch, so
 * calls that overlap on one GPU (concurrent streams, threads) race: order
 * them on one stream.  The stream must belong to the current device. */
#define GDR_NOALLOC_SCRATCH_BYTES (64u << 20)
gdr_status gdr_forward_noalloc(const gdr_problem* p, const void* q, const void* k,
                               const void* v, const float* g, const float* beta,
                               const float* h0, void* o, float* ht, void* hip_stream);

/* Ragged (packed) batches: p->B sequences of different lengths laid end to
 * end along the token axis, for prefill of a batch of prompts.  cu_seqlens
 * (device memory, int64, B + 1 entries, 8-byte aligned) holds the row
 * offsets: sequence b is token rows cu_seqlens[b] .. cu_seqlens[b+1] - 1 of
 * q, k [rows, Hk, Dk], v, o, dout, dv [rows, Hv, Dv], g [rows, Hv] or
 * [rows, Hv, Dk], beta [rows, Hv], dq, dk, dg, dbeta likewise; h0, ht, dht,
 * dh0 stay [B, Hv, Dk, Dv], one state per sequence.  p->T is an upper bound
 * on every length: workspace sizes (gdr_forward_workspace /
 * gdr_backward_workspace of the same p) hold ceil(T / C) chunks per
 * sequence.  The library reads the offsets only on the device, so it cannot
 * check them: it clamps each length to [0, T] (tokens past T are neither
 * read nor written) and reads and writes only the rows the offsets name,
 * which must lie inside the caller's buffers.  A sequence of length 0
 * passes its state through (ht = h0, dh0 = dht).  Each sequence gives
 * exactly what a separate call on it would (this is not a feature of the
 * pages: an interface variant for batches of unequal prompts).
 * Supported: GDR_ALGO_SEQUENTIAL (every shape, both passes) and
 * GDR_ALGO_CHUNKED on its fp16 path (bf16 io, Dk = Dv = 128, chunk_size 32
 * or 64; scalar or channelwise gate; GDR_SAVE_CHUNKS with a scalar gate).
 * The fp32 chunked path (fp32 io or Dk = 16) returns GDR_ERR_UNSUPPORTED;
 * AUTO picks as for gdr_forward / gdr_backward. */
gdr_status gdr_forward_varlen(const gdr_problem* p, const int64_t* cu_seqlens,
                              const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              const float* h0, void* o, float* ht, void* ws,
                              size_t ws_bytes, void* hip_stream);
gdr_status gdr_backward_varlen(const gdr_problem* p, const int64_t* cu_seqlens,
                               const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const float* h0, const void* dout,
                               const float* dht, void* dq, void* dk, void* dv,
                               float* dg, float* dbeta, float* dh0, void* ws,
                               size_t ws_bytes, void* hip_stream);

/* Per-kernel timing for benchmarks (not for use under graph capture).
 * While enabled, every kernel that gdr_forward / gdr_backward launch from the
 * calling thread is bracketed by a pair of HIP events recorded on the call's
 * stream (events are created on first use and recycled).  gdr_profile_read
 * waits for all recorded events, writes up to `cap` per-kernel entries
 * (static kernel name, summed milliseconds, launch count) to `out`, stores
 * the number of kernels seen in *n and clears the record.  Disabling drops
 * any unread record. */
typedef struct gdr_kernel_time {
  const char* name;
  double total_ms;
  int64_t launches;
} gdr_kernel_time;
gdr_status gdr_profile_enable(int on);
gdr_status gdr_profile_read(gdr_kernel_time* out, int cap, int* n);

const char* gdr_status_str(gdr_status s); /* static string, never NULL      */
const char* gdr_last_hip_error(void);     /* this thread's last HIP error   */
int gdr_abi_version(void);                /* GDR_ABI_VERSION                */

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
