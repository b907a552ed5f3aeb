// Fused single-token recurrent step (decode) and the row-normalisation test
// export.
//
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
// head) against ~7 dk dv flops.  One workgroup owns a slab of up to 32
// columns of one (sequence, head) state; each thread holds one float4 column
// group of two rows (one for the smallest shapes) in registers between the
// read and the write, so every state byte crosses HBM exactly once per
// direction, in 16-byte accesses that cover whole 128-byte row pieces.  Few
// loads per thread matter on gfx950: an in-place read-modify-write streams
// HBM markedly faster with one or two 16-byte loads in flight per thread
// than with sixteen, and this shape moves the step from ~67% to ~73% of the
// 8 TB/s peak.  The column sums over the rows run as butterflies across the
// rows a wave holds, then across the waves in LDS.
#include "ckda_internal.h"

namespace ckda {
namespace {

template <int DK, int DV>
struct StepShape {
  static constexpr int DVS = DV < 32 ? DV : 32;                     // columns per workgroup
  static constexpr int NS = DV / DVS;                               // workgroups per (n, h)
  static constexpr int CG = DVS / 4;                                // float4 column groups
  static constexpr int RW = 64 / CG;                                // rows per wave and pass
  static constexpr int NW = DK / (2 * RW) > 1 ? DK / (2 * RW) : 1;  // waves
  static constexpr int RB = NW * RW;                                // rows per pass of the block
  static constexpr int RPT = DK / RB;                               // rows per thread
  static constexpr int NT = 64 * NW;
  static constexpr int MINW = NW >= 8 ? 6 : 8;                      // waves per SIMD (3 or more workgroups per CU)
  static_assert(DV % DVS == 0 && DVS % 4 == 0 && 64 % CG == 0, "bad decode shape");
  static_assert(RB * RPT == DK && RPT >= 1 && RPT <= 2, "bad decode rows");
  static_assert(NT >= DK, "one thread per key channel loads q, k, alpha");
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <class IO, int DK, int DV>
__global__ __launch_bounds__((StepShape<DK, DV>::NT), (StepShape<DK, DV>::MINW)) void step_kernel(StepArgs a) {
  using SH = StepShape<DK, DV>;
  constexpr int DVS = SH::DVS, NS = SH::NS, CG = SH::CG, RW = SH::RW, NW = SH::NW, RB = SH::RB,
                RPT = SH::RPT;
  using T = typename IO::storage;

  __shared__ float s_q[DK], s_k[DK], s_a[DK];
  __shared__ f32x4 s_pw[NW][CG], s_py[NW][CG], s_d[CG];
  __shared__ float s_scal[3];

  // (sequence, head) and column slab.  Workgroups are dealt to the 8 XCDs in
  // turn, so the NS slabs of one state sit 8 workgroups apart: they run on
  // the same XCD and read q, k, alpha through its L2 once.
  int64_t nh;
  int sp;
  if (NS > 1 && gridDim.x % (8 * NS) == 0) {
    const int64_t slot = blockIdx.x / 8;
    nh = (slot / NS) * 8 + blockIdx.x % 8;
    sp = static_cast<int>(slot % NS);
  } else {
    nh = blockIdx.x / NS;
    sp = static_cast<int>(blockIdx.x % NS);
  }
  const int c0 = sp * DVS;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int cg = lane % CG, r0 = wave * RW + lane / CG;  // rows r0 + RB * i

  const f32x4* S0 = reinterpret_cast<const f32x4*>(a.h0 + nh * DK * DV + c0);
  f32x4* S1 = reinterpret_cast<f32x4*>(a.ht + nh * DK * DV + c0);

  // The token's small inputs are issued first and the state after them, so
  // their latency overlaps the state loads and waiting for them does not
  // wait for the state.
  // query/key head of this value head (grouped value heads share one)
  const int64_t nhk = (nh / a.H) * a.Hk + (nh % a.H) / (a.H / a.Hk);
  const bool ckda = a.gate_range == CKDA_GATE_CKDA;
  f32x4 vt = {0.f, 0.f, 0.f, 0.f};
  if (t < CG) {
    const T* v = static_cast<const T*>(a.v) + nh * DV + c0 + 4 * t;
    vt = f32x4{IO::load(v, 0), IO::load(v, 1), IO::load(v, 2), IO::load(v, 3)};
  }
  float xq = 0.f, xk = 0.f, xa = 0.f;
  if (t < DK) {
    xq = IO::load(static_cast<const T*>(a.q) + nhk * DK, t);
    xk = IO::load(static_cast<const T*>(a.k) + nhk * DK, t);
    xa = load_alpha_rt(a.alpha, nh * DK + t, a.gate_input, ckda);
  }
  const float bt = load_beta_rt(a.beta, nh, a.gate_input, ckda);
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&S0[(r0 + RB * i) * (DV / 4) + cg]);
  if (t < DK) {
    s_q[t] = xq;
    s_k[t] = xk;
    s_a[t] = xa;
  }
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
  const float rq = s_scal[0], rk = s_scal[1];

  // per-thread partial column sums over its rows, then over the wave's rows
  // (lanes that differ above the column-group bits), then over the waves
  f32x4 pw = {0.f, 0.f, 0.f, 0.f}, py = pw;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = r0 + RB * i;
    const float al = s_a[r], kh = s_k[r] * rk, qh = s_q[r] * rq;
    s[i] *= al;
    pw += s[i] * kh;
    py += s[i] * qh;
  }
#pragma unroll
  for (int m = CG; m < 64; m <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pw[c] += __shfl_xor(pw[c], m, 64);
      py[c] += __shfl_xor(py[c], m, 64);
    }
  }
  if (lane < CG) {
    s_pw[wave][cg] = pw;
    s_py[wave][cg] = py;
  }
  __syncthreads();
  if (t < CG) {
    f32x4 w = s_pw[0][t], y = s_py[0][t];
#pragma unroll
    for (int g = 1; g < NW; ++g) {
      w += s_pw[g][t];
      y += s_py[g][t];
    }
    const f32x4 d = vt - w;
    s_d[t] = d;
    const float bkq = bt * s_scal[2];
    T* o = static_cast<T*>(a.o) + nh * DV + c0 + 4 * t;
    IO::store(o, 0, a.scale * (y.x + bkq * d.x));
    IO::store(o, 1, a.scale * (y.y + bkq * d.y));
    IO::store(o, 2, a.scale * (y.z + bkq * d.z));
    IO::store(o, 3, a.scale * (y.w + bkq * d.w));
  }
  __syncthreads();

  const f32x4 d = s_d[cg];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = r0 + RB * i;
    const float bk = bt * (s_k[r] * rk);
    const f32x4 u = s[i] + bk * d;
    __builtin_nontemporal_store(u, &S1[r * (DV / 4) + cg]);
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
    // one reciprocal per row, then a multiply per element: the arithmetic
    // of the row scales in the transform pass and the decode step
    const float rn = __fdiv_rn(1.f, __fsqrt_rn(ss + kL2Eps));
    for (int i = threadIdx.x; i < d; i += 64) y[r * d + i] = IO::load(x, r * d + i) * rn;
  }
}

template <class IO, int DK, int DV>
launch_result launch_step_t(const StepArgs& a, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(a.N) * a.H * StepShape<DK, DV>::NS;
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
