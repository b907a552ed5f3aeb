/*
 * ckda.h -- C ABI of libckda.so: the (Complex) Kimi Delta Attention
 * recurrence on AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every sequence n and head h the library runs
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * over the sequence's tokens in order, starting from S_0 = h0[n,h] (or 0).
 * The transition A_t = (I - beta k k^T) Diag(alpha) is the gated delta-rule
 * transition of the picx.dev summary of the Complex KDA paper (section
 * "Background", transition-matrix equation); the rank-one write beta k v^T and
 * the read-out after the update complete it.  S is dk x dv; Diag(alpha)
 * scales its rows, so alpha holds one gate per key channel.  With
 * use_qk_l2norm set, q and k are first normalised per (token, head) over the
 * dk channels, x / sqrt(sum x^2 + 1e-6), inside the kernels (dormouse review
 * "RoPE into the KDA q/k path", section 2: the norm is an in-op step that the
 * layer switches on).
 *
 * Gate ranges (same summary, section "CKDA Definition"): CKDA takes
 * alpha in [-1,1] per channel and beta in [0,2]; KDA keeps alpha in (0,1].
 * Both are computed exactly as written, including alpha = 0 and negative
 * alpha; values outside the range are computed as written too, but then the
 * transition may expand and the results are not covered by the tests.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory: scratch space comes in as a
 *    caller-owned workspace argument, except for ckda_chunk_fwd_noalloc,
 *    which uses a static device array the library holds per GPU.  Apart from
 *    that array and its per-device address, it keeps no global mutable state
 *    but a thread-local error message.
 *  - Layouts are row-major and contiguous (last index fastest).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *    default stream).  The library never synchronises the host and never
 *    reads device memory on the host.  It enqueues kernel launches only (no
 *    memsets, copies or allocations), so a call made once outside a capture
 *    (one-time set-up) can then be captured into a HIP graph and replayed.
 *  - All argument validation happens on the host before any HIP call; a
 *    non-OK status means nothing was enqueued.  A failed launch returns
 *    CKDA_ERR_HIP.  Nothing crosses the ABI as an exception.
 *  - Data-dependent preconditions are documented, not checked: gate ranges,
 *    and cu_seqlens being non-decreasing with cu_seqlens[0] = 0.
 *  - Base pointers must be 16-byte aligned.
 */
#ifndef CKDA_H_
#define CKDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CKDA_ABI_VERSION 9

typedef enum {
  CKDA_OK = 0,
  CKDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment, aliasing */
  CKDA_ERR_UNSUPPORTED = 2,      /* valid arguments this build has no kernel for */
  CKDA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the size the query returns */
  CKDA_ERR_HIP = 4               /* the HIP runtime reported an error at launch */
} ckda_status_t;

typedef enum {
  CKDA_DTYPE_BF16 = 0, /* q, k, v, o in bfloat16 (o rounded to nearest even) */
  CKDA_DTYPE_F32 = 1   /* q, k, v, o in float32 */
} ckda_dtype_t;

typedef enum {
  CKDA_GATE_KDA = 0,  /* alpha in (0,1], beta in [0,1] */
  CKDA_GATE_CKDA = 1  /* alpha in [-1,1], beta in [0,2] */
} ckda_gate_t;

/*
 * What the alpha and beta buffers hold.
 *   CKDA_GATES_F32: the gates themselves, float32.
 *   CKDA_GATES_LOGITS_F32 / CKDA_GATES_LOGITS_BF16: pre-activation logits a
 *     (shaped like alpha) and b (shaped like beta), float32 or bfloat16; the
 *     kernels form the gates on load, in float32.  CKDA range (picx.dev
 *     summary, section "CKDA Definition"): alpha = 2 sigmoid(a) - 1 and
 *     beta = 2 sigmoid(b).  KDA range: alpha = sigmoid(a), beta = sigmoid(b)
 *     (the same activation without the shift and doubling that widen the
 *     range).  a = 0 gives alpha = 0 exactly in the CKDA range; logits of
 *     +-inf give the limits; a NaN logit gives NaN results.
 * Logits in bfloat16 halve the gate bytes the transform pass reads.
 */
typedef enum {
  CKDA_GATES_F32 = 0,
  CKDA_GATES_LOGITS_F32 = 1,
  CKDA_GATES_LOGITS_BF16 = 2
} ckda_gate_input_t;

/*
 * Descriptor of one chunked forward call.
 *   Dense batch (cu_seqlens == NULL): num_seqs == B sequences of T tokens;
 *     q, k : [B][T][Hk][dk]   alpha : [B][T][H][dk]   v, o : [B][T][H][dv]
 *     beta : [B][T][H]        (alpha and beta in the type gate_input names)
 *   H counts the value heads (those of v, o, alpha, beta and the state) and
 *   Hk = qk_heads the query/key heads (0 means Hk = H).  With Hk < H (grouped
 *   value heads) H must be a multiple of Hk and value head h reads query/key
 *   head h / (H / Hk), each q/k head serving H / Hk consecutive value heads
 *   (dormouse review "RoPE into the KDA q/k path", section 7: q and k sit on
 *   the key-head axis and are repeated over the value heads).
 *   Packed variable-length batch (cu_seqlens != NULL): B must be 1, T is the
 *     total token count, sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1
 *     (empty sequences allowed; then ht[n] = h0[n]).
 *   h0, ht : [num_seqs][H][dk][dv] float32.
 * chunk_size is the number of tokens handled as one block of the chunked
 * algorithm; the result does not depend on it beyond rounding.
 */
typedef struct {
  int32_t B, T, H, dk, dv;
  int32_t num_seqs;
  int32_t chunk_size;    /* 16, 32 or 64 */
  int32_t io_dtype;      /* ckda_dtype_t */
  int32_t gate_range;    /* ckda_gate_t */
  int32_t use_qk_l2norm; /* 0 or 1 */
  float scale;           /* o = scale * S^T q_hat */
  int32_t gate_input;    /* ckda_gate_input_t (0: float32 gate values) */
  int32_t qk_heads;      /* Hk, heads of q and k; 0 = H */
  int32_t sign_absorb;   /* 0: native signed gates; 1: global sign absorption */
} ckda_fwd_desc_t;

/*
 * sign_absorb = 1 selects a second strategy for signed gates, kept for
 * comparison (picx.dev summary, section "Implementation": cumulative signs
 * folded into the keys and queries, then an unmodified KDA kernel on
 * |alpha|).  Before the transform pass, two extra passes compute every key
 * channel's cumulative sign since the start of its sequence and write
 * sign * q, sign * k, |alpha| and beta (float32) into the workspace; the
 * unchanged passes then run on those, and a last pass negates the rows of ht
 * whose channel ended with a negative sign.  Sign flips are exact, so the
 * result equals the native one (bit for bit on regular chunks); the extra
 * passes cost one more read of q, k, alpha and a write of their absorbed
 * copies.  The default, 0, carries the signs inside the transform pass's
 * running gate products at no extra cost.
 */

/*
 * Bytes of device workspace ckda_chunk_fwd needs for this descriptor; 0 for
 * an invalid descriptor or an empty call.  `packed` is 1 when the call will
 * pass cu_seqlens (a packed batch), else 0.  The size depends only on the
 * sizes, never on data: one block of chunk operands and one int32 flag per
 * (head, chunk), with at most ceil(T / chunk_size) * B chunks for a dense
 * batch and ceil(T / chunk_size) + num_seqs for a packed one, plus the chunk
 * map of a packed batch, plus (sign_absorb = 1) the absorbed q, k, |alpha|,
 * beta for every value head and two sign masks.  At B=8, T=4096, H=16,
 * dk=128, chunk 64, bf16: 484 MiB (0.97 GiB with sign_absorb).
 */
size_t ckda_chunk_fwd_workspace_size(const ckda_fwd_desc_t* desc, int32_t packed);

/*
 * Chunked prefill.  Computes o for every token and, if ht != NULL, the final
 * state of every sequence.  h0 == NULL means a zero initial state.  h0 and ht
 * may be the same buffer (the state is read before it is written).  o must not
 * overlap any input.
 *
 * The chunked form computes exactly the recurrence above (up to rounding): a
 * chunk of C tokens entered with state S0 is one UT/WY step, the form of the
 * chunked KDA arm the dormouse review names (section 1: the layer's chunk
 * arm; section 6: the chunked WY comparison, whose zero-padded partial last
 * chunk this equals, padding tokens being identity transitions).
 *
 * Two passes run on `stream`: a transform pass over all chunks in parallel
 * (gate prefix, norms, the chunk's UT/WY transform), which writes each chunk's
 * operands into `workspace`, then a state pass that walks every
 * (sequence, head) over its chunks.  The transform pass is two launches: the
 * MFMA form for every chunk whose running gate products stay within
 * [2^-100, 2^10], then a short launch that redoes the other chunks (exact
 * zero gates, products that underflow) with direct products.  `workspace` is a device buffer of at
 * least ckda_chunk_fwd_workspace_size(desc, cu_seqlens != NULL) bytes,
 * 256-byte aligned, owned by the caller, not overlapping any argument; its
 * contents are scratch (undefined before and after the call).  Calls that
 * share a workspace must be ordered on one stream.  A workspace_bytes below
 * the query's size returns CKDA_ERR_WORKSPACE_TOO_SMALL; a NULL, misaligned
 * or overlapping workspace returns CKDA_ERR_INVALID_ARGUMENT.
 *
 * Supported shapes (others return CKDA_ERR_UNSUPPORTED):
 *   bf16 : dk = dv = 128 with chunk_size 16, 32 or 64; dk = dv = 64 with 16, 32, 64
 *   f32  : dk = dv in {16, 32, 64} with chunk_size 16 or 32 (<= 64 for dk <= 32)
 * ckda_fwd_supported() reports whether a descriptor has a kernel.
 */
ckda_status_t ckda_chunk_fwd(const ckda_fwd_desc_t* desc, const void* q,
                             const void* k, const void* v, const void* alpha,
                             const void* beta, const int32_t* cu_seqlens,
                             const float* h0, void* o, float* ht,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * ckda_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: the library keeps a static device scratch of
 * CKDA_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU it runs on, for the life of
 * the process, and runs the same two passes on it.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up that device's scratch address once.
 * Arguments, layouts, supported shapes and validation are those of
 * ckda_chunk_fwd.  A call whose workspace (ckda_chunk_fwd_workspace_size)
 * would exceed the scratch returns CKDA_ERR_WORKSPACE_TOO_SMALL before any
 * HIP call: at dk = dv = 128, chunk 64, bf16 that is about 2,160
 * (head, chunk) pairs, e.g. 16 heads of 8,000 tokens.  Every call on one GPU
 * shares that GPU's scratch, and each call rewrites all of it that it reads
 * (nothing needs to start at zero), so calls on one GPU must not overlap:
 * order them on one stream, or otherwise one after the other.  Calls that
 * overlap on one GPU race and give undefined results.
 */
#define CKDA_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
ckda_status_t ckda_chunk_fwd_noalloc(const ckda_fwd_desc_t* desc, const void* q,
                                     const void* k, const void* v, const void* alpha,
                                     const void* beta, const int32_t* cu_seqlens,
                                     const float* h0, void* o, float* ht, void* stream);

/*
 * The two passes of ckda_chunk_fwd as separate calls, for callers that time
 * them, or that let the transform pass of one batch run ahead of the state
 * pass of another.  The split is the chunked form's own: everything that does
 * not depend on the state entering a chunk (gate products, norms, the UT/WY
 * inverse of the chunked WY form, dormouse review section 6) is the prepare step,
 * and the walk of the state over the chunks (the recurrence of section
 * "Background", one chunk at a time) is the finish step.  ckda_chunk_fwd_prepare runs the transform pass and leaves
 * every chunk's operands in `workspace`; ckda_chunk_fwd_finish runs the state
 * pass from a workspace that a prepare call with the same descriptor and
 * cu_seqlens filled (on the same stream, or otherwise ordered before it), and
 * may run any number of times on it (each run recomputes o and ht from h0).
 * Arguments mean what they mean for ckda_chunk_fwd; validation is the same for
 * the arguments each call takes.  That the workspace was prepared for the same
 * descriptor is a precondition, not checked.
 */
ckda_status_t ckda_chunk_fwd_prepare(const ckda_fwd_desc_t* desc, const void* q,
                                     const void* k, const void* alpha,
                                     const void* beta, const int32_t* cu_seqlens,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream);
ckda_status_t ckda_chunk_fwd_finish(const ckda_fwd_desc_t* desc, const void* v,
                                    const int32_t* cu_seqlens, const float* h0,
                                    void* o, float* ht, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* 1 if ckda_chunk_fwd has a kernel for this descriptor's (chunk_size, dk, dv,
 * io_dtype), 0 if not (other fields are not inspected). */
int32_t ckda_fwd_supported(const ckda_fwd_desc_t* desc);

/*
 * Gradients of ckda_chunk_fwd (reverse mode of the recurrence the forward
 * computes; picx.dev summary of the Complex KDA paper, section "Background",
 * transition and update; the in-op L2 norm of the dormouse review "RoPE into
 * the KDA q/k path", section 2, is differentiated too).  Given the same
 * descriptor and inputs as the forward, dout = dL/do (io dtype, shaped like o)
 * and dht = dL/dht ([N][H][dk][dv] float32, NULL for zero), writes float32
 * gradients:
 *   dq, dk : [B*T][Hk][dk]   dalpha : [B*T][H][dk]   dv : [B*T][H][dv]
 *   dbeta  : [B*T][H]        dh0 : [N][H][dk][dv]  (NULL: not written)
 * in the forward's token layout (dense or packed).  h0 is the forward's
 * initial state (NULL for zero).  With gate logits (gate_input 1 or 2) dalpha
 * and dbeta are the gradients of the logits a and b, through the activation
 * of "CKDA Definition" (the sigmoid itself in the KDA range).  With grouped
 * value heads (Hk < H) dq and dk of a q/k head sum the gradients of the value
 * heads that read it (dormouse review, section 7).
 *
 * It recomputes the forward (keeping each chunk's X = (I + A)^{-1} and entry
 * state in the workspace), runs the state adjoint backwards over each
 * sequence's chunks, then the chunk-local gradients in parallel over chunks:
 * from the forward's running gate products where they lie in [2^-100, 2^10],
 * token by token elsewhere.  dalpha is formed with no division by a gate:
 * it sums the pairs of positions that straddle the gate, each times the
 * partial gate products on either side of it, so gates near zero are as
 * accurate as the others.  Every reduction runs in a fixed order: two calls
 * on the same inputs give the same bits.  With logits or grouped heads, extra
 * passes before and after prepare float32 gates and one q/k head per value
 * head in the workspace and finish the gradients.
 *
 * Requirements beyond the forward's: sign_absorb = 0 (else
 * CKDA_ERR_UNSUPPORTED).  Outputs must be 16-byte aligned and overlap no
 * input, each other or the workspace.  `workspace`: at least
 * ckda_chunk_bwd_workspace_size(desc, cu_seqlens != NULL) bytes, 256-byte
 * aligned, scratch (CKDA_ERR_WORKSPACE_TOO_SMALL below that size).
 * Asynchronous on `stream`.
 */
size_t ckda_chunk_bwd_workspace_size(const ckda_fwd_desc_t* desc, int32_t packed);
ckda_status_t ckda_chunk_bwd(const ckda_fwd_desc_t* desc, const void* q, const void* k,
                             const void* v, const void* alpha, const void* beta,
                             const int32_t* cu_seqlens, const float* h0, const void* dout,
                             const float* dht, float* dq, float* dk, float* dv,
                             float* dalpha, float* dbeta, float* dh0, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * The forward and the backward of a training step, with the backward's
 * records kept in between instead of recomputed (same chunked form and
 * gradients as ckda_chunk_fwd and ckda_chunk_bwd; picx.dev summary of the
 * Complex KDA paper, section "Background").
 *
 * ckda_chunk_fwd_save is ckda_chunk_fwd (same arguments, validation, o and
 * ht) that also leaves in `saved` what ckda_chunk_bwd would recompute: every
 * chunk's transform-pass block, X = (I + A)^{-1} in float32 and the state
 * entering the chunk (io dtype).  `saved`: at least
 * ckda_chunk_bwd_workspace_size(desc, cu_seqlens != NULL) bytes, 256-byte
 * aligned, overlapping no input or output (CKDA_ERR_WORKSPACE_TOO_SMALL
 * below that size); sign_absorb = 0 (else CKDA_ERR_UNSUPPORTED).
 *
 * ckda_chunk_bwd_saved is ckda_chunk_bwd with `saved` in the place of the
 * workspace, from which it reads the records rather than running the
 * forward again.  Precondition, not checked: `saved` was filled by
 * ckda_chunk_fwd_save with the same descriptor, cu_seqlens and forward
 * inputs, on the same stream or ordered before, and left untouched since.
 * The call only reads the records (it writes its own passes' data to the
 * rest of `saved`), so it may run any number of times on one save.  The
 * gradients are ckda_chunk_bwd's: the records are the same kernels' output
 * on the same inputs.
 *
 * For a layer of B=8, T=4096, H=16, d=128 in bf16, `saved` is 1.31 GB, of
 * which the records take 0.91 GB; the backward call no longer runs the
 * forward's two passes.
 */
ckda_status_t ckda_chunk_fwd_save(const ckda_fwd_desc_t* desc, const void* q, const void* k,
                                  const void* v, const void* alpha, const void* beta,
                                  const int32_t* cu_seqlens, const float* h0, void* o,
                                  float* ht, void* saved, size_t saved_bytes, void* stream);
ckda_status_t ckda_chunk_bwd_saved(const ckda_fwd_desc_t* desc, const void* q, const void* k,
                                   const void* v, const void* alpha, const void* beta,
                                   const int32_t* cu_seqlens, const float* h0,
                                   const void* dout, const float* dht, float* dq, float* dk,
                                   float* dv, float* dalpha, float* dbeta, float* dh0,
                                   void* saved, size_t saved_bytes, void* stream);

/*
 * Fused single-token decode step for N sequences: the recurrent form of the
 * same recurrence, one token per sequence (picx.dev summary, section
 * "Background", the transition A_t applied to the cached state, then the
 * write and the read-out; the dormouse review, section 1, describes the
 * recurrent arm beside the chunked one and its returned recurrent state):
 *   S <- (I - beta k^ k^T) Diag(alpha) S + beta k^ v^T,   o = scale S^T q^
 *   q, k : [N][Hk][dk]   alpha : [N][H][dk]   v, o : [N][H][dv]   beta : [N][H]
 *   h0, ht      : [N][H][dk][dv] float32; h0 == ht (in place) is allowed,
 *                 other partial overlaps are not.
 * Hk = qk_heads (0 means H) as for ckda_chunk_fwd: value head h reads
 * query/key head h / (H / Hk).  alpha and beta hold what gate_input (a
 * ckda_gate_input_t) says.
 * Supported: dk, dv in {16, 32, 64, 128}, both io dtypes, every gate input,
 * N * H up to 2^21 (one launch; larger returns CKDA_ERR_UNSUPPORTED).
 */
ckda_status_t ckda_recurrent_step(int32_t N, int32_t H, int32_t qk_heads, int32_t dk,
                                  int32_t dv, int32_t io_dtype, int32_t gate_range,
                                  int32_t gate_input, int32_t use_qk_l2norm,
                                  float scale, const void* q, const void* k,
                                  const void* v, const void* alpha, const void* beta,
                                  const float* h0, float* ht, void* o,
                                  void* stream);

/*
 * Test export of the in-kernel normalisation of q and k (dormouse review
 * "RoPE into the KDA q/k path", section 2: per head over the key channels):
 * y[r][:] = x[r][:] * (1 / sqrt(sum_c x[r][c]^2 + 1e-6)), in float32, with
 * IEEE sqrt and division and the same order of operations as the chunked and
 * decode kernels (one reciprocal per row, then a multiply per element), for
 * `rows` rows of d values (x in io dtype `dtype`, y float32).  d <= 1024.
 * Returns CKDA_ERR_INVALID_ARGUMENT for d outside [1, 1024], a NULL or
 * misaligned pointer, or y overlapping x.
 */
ckda_status_t ckda_l2norm_debug(const void* x, float* y, int64_t rows,
                                int32_t d, int32_t dtype, void* stream);

/* Static description of a status code. */
const char* ckda_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none): which argument failed validation, or the HIP error string. */
const char* ckda_last_error(void);

/* CKDA_ABI_VERSION of the library. */
int32_t ckda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CKDA_H_ */
