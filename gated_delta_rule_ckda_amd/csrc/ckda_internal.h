// Internal declarations shared by the host API and the kernel translation
// units of libckda.so.  Not installed; the public interface is include/ckda.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <cstdint>

#include "ckda.h"

namespace ckda {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Launch status of an internal launcher: hipSuccess or the HIP error seen by
// hipGetLastError() right after the launch.
using launch_result = hipError_t;

// Decode step (the recurrent form, one token per sequence).
struct StepArgs {
  int32_t N, H, dk, dv;
  int32_t Hk;          // q/k heads; value head h reads q/k head h / (H / Hk)
  int32_t use_l2norm;
  int32_t gate_range;  // ckda_gate_t
  int32_t gate_input;  // ckda_gate_input_t
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* beta;
  const float* h0;
  float* ht;
  void* o;
};
bool step_supported(int32_t dk, int32_t dv);
launch_result launch_step(const StepArgs& a, int32_t io_dtype, hipStream_t stream);

// Row normalisation test export.
launch_result launch_l2norm_debug(const void* x, float* y, int64_t rows,
                                  int32_t d, int32_t dtype, hipStream_t stream);

// Chunked forward: two passes over a workspace.  The transform pass runs one
// workgroup per (chunk, head) and writes that chunk's operands as one block;
// the state pass walks each (sequence, head) chain over its chunks' blocks.
//
// Block layout (elements of the handoff type: bf16 for bf16 io, f32 for f32
// io; C = chunk size):
//   X'   [C][C]   X Diag(beta),  X = (I + A)^{-1}          (lower triangular)
//   -W   [C][dk]  -X Diag(beta) Kt
//   Qt'  [C][dk]  scale rq . Qt
//   P'   [C][C]   scale Diag(rq) P Diag(rk)   (zero above the diagonal)
//   Kh'^T [dk][C] (Diag(rk) Kh)^T
//   g    [dk]     float32, the chunk's total gate product
// X' and P' are packed when tri_packed(C, es) (bf16 at C = 64): their first
// C/2 rows, zero past column C/2 - 1, keep only their first C/2 stored
// elements (in the perm32 storage order logical columns 0..31 are the first
// 32 positions of a row), so each of the two matrices takes 3/4 of C x C and
// every 128-byte line of it is written whole.  tri_row(r) is the element
// offset of row r inside either matrix.
// Blocks are 256-byte aligned; block (h, c) starts at (h * maxc + c) * blk_bytes.
__host__ __device__ constexpr bool tri_packed(int C, int es) { return C == 64 && es == 2; }
__host__ __device__ constexpr int64_t tri_elems(int C, int es) {
  return tri_packed(C, es) ? int64_t(C / 2) * (C / 2) + int64_t(C / 2) * C : int64_t(C) * C;
}
__host__ __device__ constexpr int64_t tri_row(int C, int es, int r) {
  return !tri_packed(C, es) ? int64_t(r) * C
         : (r < C / 2 ? int64_t(r) * (C / 2) : int64_t(C / 2) * (C / 2) + int64_t(r - C / 2) * C);
}
// element (r, stored position p) of a packed matrix is not stored
__host__ __device__ constexpr bool tri_dead(int C, int es, int r, int p) {
  return tri_packed(C, es) && r < C / 2 && p >= C / 2;
}
__host__ __device__ constexpr int64_t blk_off_W(int C, int dk, int es) { return tri_elems(C, es); }
__host__ __device__ constexpr int64_t blk_off_Q(int C, int dk, int es) { return tri_elems(C, es) + int64_t(C) * dk; }
__host__ __device__ constexpr int64_t blk_off_P(int C, int dk, int es) { return tri_elems(C, es) + 2 * int64_t(C) * dk; }
__host__ __device__ constexpr int64_t blk_off_K(int C, int dk, int es) { return 2 * tri_elems(C, es) + 2 * int64_t(C) * dk; }
__host__ __device__ constexpr int64_t blk_g_byte(int C, int dk, int es) {
  return (2 * tri_elems(C, es) + 3 * int64_t(C) * dk) * es;
}
__host__ __device__ constexpr int64_t blk_bytes(int C, int dk, int es) {
  return (blk_g_byte(C, dk, es) + 4 * int64_t(dk) + 255) & ~int64_t(255);
}

struct FwdArgs {
  int32_t B, T, H, dk, dv, num_seqs, chunk;
  int32_t Hk;  // q/k heads; value head h reads q/k head h / (H / Hk)
  int32_t use_l2norm;
  int32_t gate_range;  // ckda_gate_t
  int32_t gate_input;  // ckda_gate_input_t
  int32_t sign_absorb; // 1: run as a KDA forward on |alpha| with the signs folded into q, k
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* beta;
  const int32_t* cu_seqlens;
  const float* h0;
  void* o;
  float* ht;
  // workspace, laid out by the launcher
  unsigned char* blocks;  // [H][maxc] blocks of blk_bytes
  int32_t* first;         // [num_seqs + 1] first chunk of each sequence (packed batches)
  int32_t* chunk_seq;     // [maxc] sequence owning each chunk slot, -1 if unused (packed)
  int32_t* seq_order;     // [num_seqs] packed sequences by chunk count, most first (state pass)
  int2* chunk_geo;        // [maxc] first token and length of each chunk slot, length 0 if unused (packed)
  int32_t* irregular;     // [H][maxc] 1 where the transform pass left a chunk to its second launch
  int32_t maxc;           // chunk slots per head
  int32_t nc;             // chunks per sequence (dense batches)
  int64_t blk_bytes;
  // sign absorption buffers (sign_absorb = 1), laid out by the launcher
  uint32_t* cmask;        // [H][maxc][ceil(dk/32)] sign parity of each chunk
  uint32_t* tmask;        // [num_seqs][H][ceil(dk/32)] final parity of each sequence
  void* sq;               // [B*T][H][dk] Sigma q (io type)
  void* sk;               // [B*T][H][dk] Sigma k (io type)
  float* sa;              // [B*T][H][dk] |alpha|
  float* sb;              // [B*T][H] beta
  // records kept for the backward (null in a plain forward)
  float* xout;            // [H][maxc][C][C] X = (I + A)^{-1} of every chunk, fp32
  void* hc;               // [H][maxc][dk][dv] state entering every chunk (io type)
};
bool fwd_supported(int32_t chunk, int32_t dk, int32_t dv, int32_t io_dtype);
// Workspace bytes ckda_chunk_fwd needs for these sizes (0 for an empty call).
size_t fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t num_seqs,
                           int32_t chunk, int32_t io_dtype, bool packed, bool sign_absorb);
// Lays out the workspace in `a` and enqueues the transform pass (with the
// chunk map of a packed batch) and/or the state pass.
launch_result launch_fwd(FwdArgs a, int32_t io_dtype, void* ws, hipStream_t stream,
                         bool prepare, bool finish);
// The passes (one translation unit each).
bool prep_supported(int32_t chunk, int32_t dk, int32_t io_dtype);
launch_result launch_prep(const FwdArgs& a, int32_t io_dtype, hipStream_t stream);
launch_result launch_chunk_map(const FwdArgs& a, hipStream_t stream);
bool state_supported(int32_t chunk, int32_t dk, int32_t dv, int32_t io_dtype);
launch_result launch_state(const FwdArgs& a, int32_t io_dtype, hipStream_t stream);
// Sign absorption (sign_absorb.hip): workspace bytes beyond the plain
// forward's, their layout from `base`, the passes before the transform pass
// and the row flips of ht after the state pass.
int64_t sign_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t num_seqs,
                             int64_t maxc, int32_t io_dtype);
void sign_layout(FwdArgs& a, unsigned char* base, int32_t io_dtype);
launch_result launch_sign_absorb(const FwdArgs& a, int32_t io_dtype, hipStream_t stream);
launch_result launch_sign_fix(const FwdArgs& a, hipStream_t stream);

// Backward (chunk_bwd.hip).  The forward's arguments plus the gradients.
struct BwdArgs {
  FwdArgs f;
  const void* dout;  // [B,T,H,dv] io type
  const float* dht;  // [N,H,dk,dv] or null
  float* dq;         // [B,T,H,dk]
  float* dk;         // [B,T,H,dk]
  float* dv;         // [B,T,H,dv]
  float* dalpha;     // [B,T,H,dk]
  float* dbeta;      // [B,T,H]
  float* dh0;        // [N,H,dk,dv] or null
  // workspace
  // records in the io type (bf16 inputs: bf16, consumed as bf16 matrix-core
  // operands; fp32 inputs: fp32)
  void* dS;          // [H][maxc][dk][dv] state adjoint at each chunk's exit
  void* dU;          // [H][maxc][C][dv]
  int32_t* bflag;    // [H][maxc] 1: chunk left to the token-level kernel
  float* scratch;    // [grid3][14][C * max(dk, dv, C)] (f32 inputs)
  int32_t grid3;
};
// Workspace bytes of the backward beyond the forward's, their layout from
// `base` (sets b.f.xout and b.f.hc too), and the backward's own passes.
int64_t bwd_extra_bytes(int32_t H, int64_t maxc, int32_t C, int32_t dk, int32_t dv, int32_t io_dtype);
void bwd_layout(BwdArgs& b, unsigned char* base, int32_t io_dtype);
launch_result launch_bwd_passes(const BwdArgs& b, int32_t io_dtype, hipStream_t stream);
// All of ckda_chunk_bwd: the forward with records, then the backward passes.
size_t bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                           int32_t num_seqs, int32_t chunk, int32_t io_dtype, bool packed);
launch_result launch_bwd(BwdArgs b, int32_t io_dtype, void* ws, hipStream_t stream);
// The same split in two for training steps: the forward (o and ht written)
// that leaves the records in the backward's workspace layout, and the
// backward passes that read them there instead of recomputing them.
launch_result launch_fwd_save(FwdArgs a, int32_t io_dtype, void* ws, hipStream_t stream);
launch_result launch_bwd_saved(BwdArgs b, int32_t io_dtype, void* ws, hipStream_t stream);
// The backward for gate logits and grouped value heads (bwd_gates.hip): the
// workspace beyond the backward's own `core_bytes`, and the passes around
// launch_bwd that prepare float32 gates and one q/k head per value head and
// finish the gradients of the logits and of the shared q/k heads.
size_t bwd_gates_extra_bytes(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t dk,
                             int32_t io_dtype, bool logits);
launch_result launch_bwd_full(BwdArgs b, int32_t io_dtype, void* ws, size_t core_bytes,
                              hipStream_t stream, bool recompute = true);

// ---- small device helpers shared by the kernels --------------------------

// bf16 <-> f32.  Conversion to bf16 rounds to nearest even (finite inputs).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element types of the io tensors.
struct io_bf16 {
  using storage = uint16_t;
  static __device__ __forceinline__ float load(const storage* p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(storage* p, int64_t i, float x) {
    p[i] = f32_to_bf16(x);
  }
  // 4 consecutive values at p (8-byte aligned)
  static __device__ __forceinline__ void store4(storage* p, f32x4 x) {
    const uint32_t lo = f32_to_bf16(x[0]) | (static_cast<uint32_t>(f32_to_bf16(x[1])) << 16);
    const uint32_t hi = f32_to_bf16(x[2]) | (static_cast<uint32_t>(f32_to_bf16(x[3])) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
  }
};
struct io_f32 {
  using storage = float;
  static __device__ __forceinline__ float load(const storage* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(storage* p, int64_t i, float x) { p[i] = x; }
  static __device__ __forceinline__ void store4(storage* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
  }
};

constexpr float kL2Eps = 1e-6f;

// ---- gates -----------------------------------------------------------------
// The gate buffers hold either the gates (float32) or logits (float32 or
// bf16) that are activated on load (ckda_gate_input_t).  CKDA range (picx.dev
// summary, section "CKDA Definition"): alpha = 2 sigmoid(a) - 1 and
// beta = 2 sigmoid(b); KDA range: alpha = sigmoid(a), beta = sigmoid(b).
// 2 sigmoid(a) - 1 equals sign(a) tanh(|a|/2), formed as (1 - e) / (1 + e)
// with e = exp(-|a|) for |a| >= 1/2 and by the odd Taylor polynomial of
// tanh (through degree 9, error below 1e-8 relative) under 1/2, where 1 - e
// would cancel: a logit of 1e-9 gives a gate of 5e-10, not 0.  So alpha is 0
// exactly for a logit of 0 only, and +-1 once e underflows.  exp is v_exp_f32
// on a * log2(e) and the divisions are v_rcp_f32 (about 1 ulp each).
struct gate_f32 {  // gates as given
  using storage = float;
  static constexpr bool logits = false;
};
struct gate_logit_f32 {
  using storage = float;
  static constexpr bool logits = true;
};
struct gate_logit_bf16 {
  using storage = uint16_t;
  static constexpr bool logits = true;
};

__device__ __forceinline__ float exp_neg(float x) {  // e^-x
  return __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
}
// Both ranges share one exp and one reciprocal; the range only selects
// operands (no branch, so unrolled loads and activations stay interleaved).
__device__ __forceinline__ float alpha_from_logit(float a, bool ckda) {
  const float x = ckda ? fabsf(a) : a;
  const float e = exp_neg(x);
  const float r = __builtin_amdgcn_rcpf(1.f + e);
  const float y = 0.5f * x, y2 = y * y;
  const float poly =
      y * (1.f + y2 * (-1.f / 3 + y2 * (2.f / 15 + y2 * (-17.f / 315 + y2 * (62.f / 2835)))));
  const float m = (x < 0.5f) ? poly : (1.f - e) * r;  // tanh(|a|/2)
  return ckda ? copysignf(m, a) : r;
}
__device__ __forceinline__ float beta_from_logit(float b, bool ckda) {
  return (ckda ? 2.f : 1.f) * __builtin_amdgcn_rcpf(1.f + exp_neg(b));
}
template <class G>
__device__ __forceinline__ float gate_raw(const void* p, int64_t i) {
  const typename G::storage x = static_cast<const typename G::storage*>(p)[i];
  if constexpr (sizeof(typename G::storage) == 2)
    return bf16_to_f32(x);
  else
    return x;
}
// alpha (or beta) element i of a gate buffer of kind G
template <class G>
__device__ __forceinline__ float load_alpha(const void* p, int64_t i, bool ckda) {
  const float x = gate_raw<G>(p, i);
  if constexpr (G::logits) return alpha_from_logit(x, ckda);
  return x;
}
template <class G>
__device__ __forceinline__ float load_beta(const void* p, int64_t i, bool ckda) {
  const float x = gate_raw<G>(p, i);
  if constexpr (G::logits) return beta_from_logit(x, ckda);
  return x;
}
// the same with the kind chosen at run time (ckda_gate_input_t)
__device__ __forceinline__ float load_alpha_rt(const void* p, int64_t i, int gi, bool ckda) {
  if (gi == CKDA_GATES_LOGITS_BF16) return load_alpha<gate_logit_bf16>(p, i, ckda);
  if (gi == CKDA_GATES_LOGITS_F32) return load_alpha<gate_logit_f32>(p, i, ckda);
  return load_alpha<gate_f32>(p, i, ckda);
}
__device__ __forceinline__ float load_beta_rt(const void* p, int64_t i, int gi, bool ckda) {
  if (gi == CKDA_GATES_LOGITS_BF16) return load_beta<gate_logit_bf16>(p, i, ckda);
  if (gi == CKDA_GATES_LOGITS_F32) return load_beta<gate_logit_f32>(p, i, ckda);
  return load_beta<gate_f32>(p, i, ckda);
}

}  // namespace ckda
