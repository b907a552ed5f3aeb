// Backward with gate logits and with grouped value heads.  The chunked
// backward (chunk_bwd.hip) runs on float32 gates and on q, k with one head
// per value head.  For a call with logits (picx.dev summary of the Complex
// KDA paper, section "CKDA Definition": alpha = 2 sigmoid(a) - 1,
// beta = 2 sigmoid(b); the sigmoid itself in the KDA range) or with fewer
// q/k heads than value heads (dormouse review "RoPE into the KDA q/k path",
// section 7: q, k on the key-head axis, repeated over the value heads), the
// passes here prepare those inputs in the workspace before it and finish the
// gradients after it:
//   before: the gates activated exactly as the forward activates them;
//           q, k copied out to one head per value head
//   after:  dL/da = dL/dalpha * f s(a) (1 - s(a)), dL/db likewise (f = 2 in
//           the CKDA range, 1 in the KDA range; s the sigmoid), in place;
//           dq, dk of a q/k head = the sum of its value heads' dq, dk, added
//           in head order.
#include "ckda_internal.h"

namespace ckda {
namespace {

constexpr int kNTg = 256;

unsigned grid_for(int64_t n, int per_thread) {
  const int64_t b = (n + static_cast<int64_t>(kNTg) * per_thread - 1) / (static_cast<int64_t>(kNTg) * per_thread);
  return static_cast<unsigned>(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

// alpha, beta (float32) from logits of kind G
template <class G>
__global__ __launch_bounds__(kNTg) void gates_activate_kernel(const void* a, const void* b,
                                                              bool ckda, float* alpha,
                                                              float* beta, int64_t na,
                                                              int64_t nb) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNTg;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kNTg + threadIdx.x; i < na; i += stride)
    alpha[i] = load_alpha<G>(a, i, ckda);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kNTg + threadIdx.x; i < nb; i += stride)
    beta[i] = load_beta<G>(b, i, ckda);
}

// dL/d(logit) = dL/dgate * f s (1 - s), in place; s (1 - s) = e / (1 + e)^2
// with e = exp(-|x|), accurate for logits of either sign
template <class G>
__global__ __launch_bounds__(kNTg) void gates_chain_kernel(const void* a, const void* b,
                                                           float f, float* dalpha, float* dbeta,
                                                           int64_t na, int64_t nb) {
  auto dsig = [](float x) {
    const float e = exp_neg(fabsf(x));
    const float r = __builtin_amdgcn_rcpf(1.f + e);
    return e * r * r;
  };
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNTg;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kNTg + threadIdx.x; i < na; i += stride)
    dalpha[i] *= f * dsig(gate_raw<G>(a, i));
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kNTg + threadIdx.x; i < nb; i += stride)
    dbeta[i] *= f * dsig(gate_raw<G>(b, i));
}

// q, k [rows][Hk][dk] -> [rows][H][dk]: value head h gets q/k head h / G.
// One thread per 16-byte piece of a destination row.
__global__ __launch_bounds__(kNTg) void qk_expand_kernel(const void* q, const void* k, void* qx,
                                                         void* kx, int64_t rows, int H, int Hk,
                                                         int row_bytes) {
  const int P = row_bytes / 16, G = H / Hk;
  const int64_t n = rows * H * P;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNTg;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kNTg + threadIdx.x; i < n; i += stride) {
    const int p = static_cast<int>(i % P);
    const int64_t th = i / P;
    const int h = static_cast<int>(th % H);
    const int64_t t = th / H;
    const int64_t src = (t * Hk + h / G) * P + p;
    reinterpret_cast<uint4*>(qx)[i] = reinterpret_cast<const uint4*>(q)[src];
    reinterpret_cast<uint4*>(kx)[i] = reinterpret_cast<const uint4*>(k)[src];
  }
}

// dq, dk [rows][Hk][dk] = sums over each q/k head's G value heads of
// dqx, dkx [rows][H][dk], in head order.  One thread per 4 channels.
__global__ __launch_bounds__(kNTg) void qk_group_sum_kernel(const float* dqx, const float* dkx,
                                                            float* dq, float* dk, int64_t rows,
                                                            int H, int Hk, int d) {
  const int P = d / 4, G = H / Hk;
  const int64_t n = rows * Hk * P;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNTg;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kNTg + threadIdx.x; i < n; i += stride) {
    const int p = static_cast<int>(i % P);
    const int64_t th = i / P;
    const int hk = static_cast<int>(th % Hk);
    const int64_t t = th / Hk;
    f32x4 sq = {0.f, 0.f, 0.f, 0.f}, sk = sq;
    for (int g = 0; g < G; ++g) {
      const int64_t s = (t * H + hk * G + g) * P + p;
      sq += reinterpret_cast<const f32x4*>(dqx)[s];
      sk += reinterpret_cast<const f32x4*>(dkx)[s];
    }
    reinterpret_cast<f32x4*>(dq)[i] = sq;
    reinterpret_cast<f32x4*>(dk)[i] = sk;
  }
}

int64_t up256(int64_t x) { return (x + 255) & ~int64_t(255); }

}  // namespace

size_t bwd_gates_extra_bytes(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t dk,
                             int32_t io_dtype, bool logits) {
  const int64_t tok = static_cast<int64_t>(B) * T;
  const int64_t es = io_dtype == CKDA_DTYPE_BF16 ? 2 : 4;
  int64_t b = 0;
  if (logits) b += up256(4 * tok * H * dk) + up256(4 * tok * H);
  if (Hk != H) b += 2 * up256(es * tok * H * dk) + 2 * up256(4 * tok * H * dk);
  return static_cast<size_t>(b);
}

launch_result launch_bwd_full(BwdArgs b, int32_t io_dtype, void* ws, size_t core_bytes,
                              hipStream_t stream, bool recompute) {
  FwdArgs& a = b.f;
  const bool logits = a.gate_input != CKDA_GATES_F32;
  const bool grouped = a.Hk != a.H;
  auto core = [&]() {
    return recompute ? launch_bwd(b, io_dtype, ws, stream) : launch_bwd_saved(b, io_dtype, ws, stream);
  };
  if (!logits && !grouped) return core();
  const int64_t tok = static_cast<int64_t>(a.B) * a.T;
  const int64_t es = io_dtype == CKDA_DTYPE_BF16 ? 2 : 4;
  const int64_t na = tok * a.H * a.dk, nb = tok * a.H;
  unsigned char* base = static_cast<unsigned char*>(ws) + up256(static_cast<int64_t>(core_bytes));
  const void* a_logit = a.alpha;
  const void* b_logit = a.beta;
  const int gi = a.gate_input;
  const bool ckda = a.gate_range == CKDA_GATE_CKDA;
  if (logits) {
    float* al = reinterpret_cast<float*>(base);
    base += up256(4 * na);
    float* be = reinterpret_cast<float*>(base);
    base += up256(4 * nb);
    if (tok > 0) {
      const unsigned g = grid_for(na, 1);
      if (gi == CKDA_GATES_LOGITS_BF16)
        hipLaunchKernelGGL(gates_activate_kernel<gate_logit_bf16>, dim3(g), dim3(kNTg), 0, stream,
                           a_logit, b_logit, ckda, al, be, na, nb);
      else
        hipLaunchKernelGGL(gates_activate_kernel<gate_logit_f32>, dim3(g), dim3(kNTg), 0, stream,
                           a_logit, b_logit, ckda, al, be, na, nb);
      const launch_result r = hipGetLastError();
      if (r != hipSuccess) return r;
    }
    a.alpha = al;
    a.beta = be;
    a.gate_input = CKDA_GATES_F32;
  }
  float* dq_out = b.dq;
  float* dk_out = b.dk;
  const int Hk = a.Hk;
  if (grouped) {
    void* qx = base;
    base += up256(es * na);
    void* kx = base;
    base += up256(es * na);
    float* dqx = reinterpret_cast<float*>(base);
    base += up256(4 * na);
    float* dkx = reinterpret_cast<float*>(base);
    base += up256(4 * na);
    if (tok > 0) {
      const int rb = static_cast<int>(a.dk * es);
      hipLaunchKernelGGL(qk_expand_kernel, dim3(grid_for(tok * a.H * (rb / 16), 1)), dim3(kNTg), 0,
                         stream, a.q, a.k, qx, kx, tok, a.H, Hk, rb);
      const launch_result r = hipGetLastError();
      if (r != hipSuccess) return r;
    }
    a.q = qx;
    a.k = kx;
    a.Hk = a.H;
    b.dq = dqx;
    b.dk = dkx;
  }
  {
    const launch_result r = core();
    if (r != hipSuccess) return r;
  }
  if (tok == 0) return hipSuccess;
  if (grouped) {
    hipLaunchKernelGGL(qk_group_sum_kernel, dim3(grid_for(tok * Hk * (a.dk / 4), 1)), dim3(kNTg), 0,
                       stream, b.dq, b.dk, dq_out, dk_out, tok, a.H, Hk, a.dk);
    const launch_result r = hipGetLastError();
    if (r != hipSuccess) return r;
  }
  if (logits) {
    const float f = ckda ? 2.f : 1.f;
    const unsigned g = grid_for(na, 1);
    if (gi == CKDA_GATES_LOGITS_BF16)
      hipLaunchKernelGGL(gates_chain_kernel<gate_logit_bf16>, dim3(g), dim3(kNTg), 0, stream, a_logit,
                         b_logit, f, b.dalpha, b.dbeta, na, nb);
    else
      hipLaunchKernelGGL(gates_chain_kernel<gate_logit_f32>, dim3(g), dim3(kNTg), 0, stream, a_logit,
                         b_logit, f, b.dalpha, b.dbeta, na, nb);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace ckda
