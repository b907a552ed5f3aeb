// Fused single-token recurrent step (decode) and the row-normalisation test
// export.
//
// One workgroup owns one (sequence, head) state S (dk x dv fp32, contiguous).
// The step reads S once and writes it once:
//
//   S~ = Diag(alpha) S                      (gate, per key channel = row)
//   w  = S~^T k_hat,  y = S~^T q_hat        (two column reductions, one pass)
//   S' = S~ + beta k_hat (v - w)^T          (delta-rule write)
//   o  = scale (y + beta (k_hat . q_hat) (v - w))   (= scale S'^T q_hat)
//
// alpha and beta are read as gates or as logits activated on load (the gate
// helpers of ckda_internal.h).
//
// The transition (I - beta k k^T) Diag(alpha) is the gated delta-rule
// transition of the picx.dev summary of the Complex KDA paper (section
// "Background"); q_hat, k_hat are the in-op L2-normalised query and key
// (dormouse review "RoPE into the KDA q/k path", section 2).
//
// The op is HBM-bound: 8 * dk * dv bytes of state traffic per (sequence,
// head) against ~7 dk dv flops.  Threads hold float4 column groups of
// several rows in registers between the read and the write, so every state
// byte crosses HBM exactly once per direction, with 16-byte accesses that are
// contiguous across a wavefront.
#include "ckda_internal.h"

namespace ckda {
namespace {

template <int DK, int DV>
struct StepShape {
  static constexpr int CG = DV / 4;                                 // float4 columns
  static constexpr int RG = (DK < 256 / CG) ? DK : 256 / CG;        // row groups
  static constexpr int RPT = DK / RG;                               // rows per thread
  static constexpr int NT = RG * CG;                                // threads
  static_assert(DV % 4 == 0 && DK % RG == 0, "bad decode shape");
  static_assert(NT >= 64 && NT <= 256, "decode block must hold one to four waves");
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <class IO, int DK, int DV>
__global__ __launch_bounds__((StepShape<DK, DV>::NT)) void step_kernel(StepArgs a) {
  using SH = StepShape<DK, DV>;
  constexpr int CG = SH::CG, RG = SH::RG, RPT = SH::RPT, NT = SH::NT;
  using T = typename IO::storage;

  __shared__ float s_q[DK], s_k[DK], s_a[DK], s_v[DV];
  __shared__ f32x4 s_pw[RG][CG], s_py[RG][CG];
  __shared__ float s_scal[3];

  const int64_t nh = blockIdx.x;
  const int t = threadIdx.x;
  const int cg = t % CG, rg = t / CG;

  const f32x4* S0 = reinterpret_cast<const f32x4*>(a.h0 + nh * DK * DV);
  f32x4* S1 = reinterpret_cast<f32x4*>(a.ht + nh * DK * DV);

  // State loads go out first so their latency overlaps the small loads and
  // the normalisation below.
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&S0[(rg + RG * i) * CG + cg]);

  // query/key head of this value head (grouped value heads share one)
  const int64_t nhk = (nh / a.H) * a.Hk + (nh % a.H) / (a.H / a.Hk);
  const T* q = static_cast<const T*>(a.q) + nhk * DK;
  const T* k = static_cast<const T*>(a.k) + nhk * DK;
  const T* v = static_cast<const T*>(a.v) + nh * DV;
  const bool ckda = a.gate_range == CKDA_GATE_CKDA;
  for (int i = t; i < DK; i += NT) {
    s_q[i] = IO::load(q, i);
    s_k[i] = IO::load(k, i);
    s_a[i] = load_alpha_rt(a.alpha, nh * DK + i, a.gate_input, ckda);
  }
  for (int i = t; i < DV; i += NT) s_v[i] = IO::load(v, i);
  __syncthreads();

  if (t < 64) {
    float qq = 0.f, kk = 0.f, kq = 0.f;
    for (int i = t; i < DK; i += 64) {
      const float x = s_q[i], y = s_k[i];
      qq += x * x;
      kk += y * y;
      kq += x * y;
    }
    qq = wave_sum(qq);
    kk = wave_sum(kk);
    kq = wave_sum(kq);
    if (t == 0) {
      const float rq = a.use_l2norm ? __fdiv_rn(1.f, __fsqrt_rn(qq + kL2Eps)) : 1.f;
      const float rk = a.use_l2norm ? __fdiv_rn(1.f, __fsqrt_rn(kk + kL2Eps)) : 1.f;
      s_scal[0] = rq;
      s_scal[1] = rk;
      s_scal[2] = (kq * rq) * rk;
    }
  }
  __syncthreads();
  const float rq = s_scal[0], rk = s_scal[1], kq = s_scal[2];
  const float bt = load_beta_rt(a.beta, nh, a.gate_input, ckda);

  f32x4 pw = {0.f, 0.f, 0.f, 0.f}, py = pw;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float al = s_a[r], kh = s_k[r] * rk, qh = s_q[r] * rq;
    s[i] *= al;
    pw += s[i] * kh;
    py += s[i] * qh;
  }
  s_pw[rg][cg] = pw;
  s_py[rg][cg] = py;
  __syncthreads();

  f32x4 w = s_pw[0][cg], y = s_py[0][cg];
#pragma unroll
  for (int g = 1; g < RG; ++g) {
    w += s_pw[g][cg];
    y += s_py[g][cg];
  }
  const f32x4 d = reinterpret_cast<const f32x4*>(s_v)[cg] - w;

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float bk = bt * (s_k[r] * rk);
    const f32x4 u = s[i] + bk * d;
    __builtin_nontemporal_store(u, &S1[r * CG + cg]);
  }
  if (rg == 0) {
    const float bkq = bt * kq;
    T* o = static_cast<T*>(a.o) + nh * DV + 4 * cg;
    IO::store(o, 0, a.scale * (y.x + bkq * d.x));
    IO::store(o, 1, a.scale * (y.y + bkq * d.y));
    IO::store(o, 2, a.scale * (y.z + bkq * d.z));
    IO::store(o, 3, a.scale * (y.w + bkq * d.w));
  }
}

template <class IO>
__global__ __launch_bounds__(64) void l2norm_debug_kernel(const void* xv, float* y,
                                                         int64_t rows, int d) {
  using T = typename IO::storage;
  const T* x = static_cast<const T*>(xv);
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    float ss = 0.f;
    for (int i = threadIdx.x; i < d; i += 64) {
      const float e = IO::load(x, r * d + i);
      ss += e * e;
    }
    ss = wave_sum(ss);
    const float n = __fsqrt_rn(ss + kL2Eps);
    for (int i = threadIdx.x; i < d; i += 64) y[r * d + i] = __fdiv_rn(IO::load(x, r * d + i), n);
  }
}

template <class IO, int DK, int DV>
launch_result launch_step_t(const StepArgs& a, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(a.N) * a.H;
  hipLaunchKernelGGL((step_kernel<IO, DK, DV>), dim3(static_cast<unsigned>(blocks)),
                     dim3(StepShape<DK, DV>::NT), 0, stream, a);
  return hipGetLastError();
}

template <class IO, int DK>
launch_result dispatch_dv(const StepArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 16: return launch_step_t<IO, DK, 16>(a, s);
    case 32: return launch_step_t<IO, DK, 32>(a, s);
    case 64: return launch_step_t<IO, DK, 64>(a, s);
    case 128: return launch_step_t<IO, DK, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class IO>
launch_result dispatch_dk(const StepArgs& a, hipStream_t s) {
  switch (a.dk) {
    case 16: return dispatch_dv<IO, 16>(a, s);
    case 32: return dispatch_dv<IO, 32>(a, s);
    case 64: return dispatch_dv<IO, 64>(a, s);
    case 128: return dispatch_dv<IO, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool step_supported(int32_t dk, int32_t dv) {
  auto ok = [](int32_t x) { return x == 16 || x == 32 || x == 64 || x == 128; };
  return ok(dk) && ok(dv);
}

launch_result launch_step(const StepArgs& a, int32_t io_dtype, hipStream_t stream) {
  if (static_cast<int64_t>(a.N) * a.H == 0) return hipSuccess;
  return io_dtype == CKDA_DTYPE_BF16 ? dispatch_dk<io_bf16>(a, stream)
                                     : dispatch_dk<io_f32>(a, stream);
}

launch_result launch_l2norm_debug(const void* x, float* y, int64_t rows, int32_t d,
                                  int32_t dtype, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(rows < 65536 ? rows : 65536);
  if (dtype == CKDA_DTYPE_BF16)
    hipLaunchKernelGGL(l2norm_debug_kernel<io_bf16>, dim3(grid), dim3(64), 0, stream, x, y,
                       rows, d);
  else
    hipLaunchKernelGGL(l2norm_debug_kernel<io_f32>, dim3(grid), dim3(64), 0, stream, x, y,
                       rows, d);
  return hipGetLastError();
}

}  // namespace ckda
