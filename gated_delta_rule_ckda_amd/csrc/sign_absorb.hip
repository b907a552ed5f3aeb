// Global sign absorption: the CKDA forward run as a KDA forward on |alpha|.
//
// Write Diag(alpha_t) = D_t Diag(|alpha_t|) with D_t = Diag(sign alpha_t)
// (sign 0 taken as +1) and Sigma_t = D_t Sigma_{t-1}, Sigma_0 = I, the
// cumulative sign of every key channel since the start of the sequence.  The
// state St_t = Sigma_t S_t then follows the same recurrence with the gate
// |alpha_t| and the key Sigma_t k_t, and o_t = St_t^T (Sigma_t q_t): the
// signs fold into q and k and the recurrence that remains only ever sees
// gates in [0, 1].  S_T = Sigma_T St_T flips the rows of the final state
// whose channel ended negative.  This is the implementation route of the
// compiled-PyTorch variant in the picx.dev summary (section
// "Implementation"); the native kernels carry the signs in their running
// gate products instead, and this path is kept as the comparison.
//
// Three kernels around the unchanged transform and state passes:
//   sign_mask_kernel    per (chunk, head): the chunk's sign parity per
//                       channel (one bit each)
//   sign_absorb_kernel  per (chunk, head): the parity of the sequence's
//                       earlier chunks, then row by row Sigma_t; writes
//                       Sigma q, Sigma k, |alpha| and beta (activated, float32)
//                       for every value head, and the sequence's final
//                       parity from its last chunk
//   sign_fix_kernel     per (sequence, head): negates the rows of ht whose
//                       final parity is odd
// Flipping a sign is exact in every storage type, so the absorbed inputs
// hold exactly the magnitudes of the native ones.
#include <type_traits>

#include "ckda_internal.h"

namespace ckda {
namespace {

constexpr int nwords(int dk) { return (dk + 31) / 32; }

// chunk slot c: sequence n, first token t0, length L, first chunk of the
// sequence, whether c is its last chunk; false for an unused slot
struct Slot {
  int64_t t0;
  int n, L, first;
  bool last;
};
__device__ __forceinline__ bool slot_of(const FwdArgs& a, int c, Slot& s) {
  const int C = a.chunk;
  if (a.cu_seqlens) {
    const int n = a.chunk_seq[c];
    if (n < 0) return false;
    const int f = a.first[n], f1 = a.first[n + 1];
    const int64_t s0 = a.cu_seqlens[n], s1 = a.cu_seqlens[n + 1];
    s.n = n;
    s.first = f;
    s.last = c == f1 - 1;
    s.t0 = s0 + static_cast<int64_t>(c - f) * C;
    s.L = static_cast<int>((s1 - s.t0) < C ? (s1 - s.t0) : C);
  } else {
    const int n = c / a.nc, i = c % a.nc;
    s.n = n;
    s.first = n * a.nc;
    s.last = i == a.nc - 1;
    s.t0 = static_cast<int64_t>(n) * a.T + static_cast<int64_t>(i) * C;
    s.L = (a.T - i * C) < C ? (a.T - i * C) : C;
  }
  return true;
}

// one thread per key channel; (blockIdx.x = c * H + h)
template <class G, int DK>
__global__ __launch_bounds__(DK < 64 ? 64 : DK) void sign_mask_kernel(FwdArgs a) {
  const int H = a.H;
  const int c = static_cast<int>(blockIdx.x / H), h = static_cast<int>(blockIdx.x % H);
  const int ch = threadIdx.x;
  Slot s;
  if (!slot_of(a, c, s)) return;
  const bool ckda = a.gate_range == CKDA_GATE_CKDA;
  bool odd = false;
  if (ch < DK) {
    const int64_t base = (s.t0 * H + h) * DK + ch;
#pragma unroll 8
    for (int r = 0; r < s.L; ++r)
      odd ^= load_alpha<G>(a.alpha, base + static_cast<int64_t>(r) * H * DK, ckda) < 0.f;
  }
  const uint64_t bits = __ballot(odd && ch < DK);
  uint32_t* m = a.cmask + (static_cast<int64_t>(h) * a.maxc + c) * nwords(DK);
  const int w = ch >> 6, lane = ch & 63;
  if (lane == 0) m[2 * w] = static_cast<uint32_t>(bits);
  if (lane == 32 && 2 * w + 1 < nwords(DK)) m[2 * w + 1] = static_cast<uint32_t>(bits >> 32);
}

template <class IO, class G, int DK>
__global__ __launch_bounds__(DK < 64 ? 64 : DK) void sign_absorb_kernel(FwdArgs a) {
  using T = typename IO::storage;
  using U = std::conditional_t<sizeof(T) == 2, uint16_t, uint32_t>;
  constexpr U kSign = static_cast<U>(U(1) << (8 * sizeof(T) - 1));
  const int H = a.H, Hk = a.Hk;
  const int c = static_cast<int>(blockIdx.x / H), h = static_cast<int>(blockIdx.x % H);
  const int hk = h / (H / Hk);
  const int ch = threadIdx.x;
  Slot s;
  if (!slot_of(a, c, s)) return;
  const bool ckda = a.gate_range == CKDA_GATE_CKDA;
  // beta, activated to float32
  for (int r = ch; r < s.L; r += blockDim.x) {
    const int64_t i = (s.t0 + r) * H + h;
    a.sb[i] = load_beta<G>(a.beta, i, ckda);
  }
  bool odd = false;
  if (ch < DK) {
    // parity of the sequence's earlier chunks
    const uint32_t* m = a.cmask + static_cast<int64_t>(h) * a.maxc * nwords(DK) + (ch >> 5);
#pragma unroll 8
    for (int j = s.first; j < c; ++j) odd ^= (m[static_cast<int64_t>(j) * nwords(DK)] >> (ch & 31)) & 1u;
    const U* q = static_cast<const U*>(a.q);
    const U* k = static_cast<const U*>(a.k);
    U* sq = static_cast<U*>(a.sq);
    U* sk = static_cast<U*>(a.sk);
#pragma unroll 4
    for (int r = 0; r < s.L; ++r) {
      const int64_t t = s.t0 + r;
      const int64_t iv = (t * H + h) * DK + ch, iq = (t * Hk + hk) * DK + ch;
      const float al = load_alpha<G>(a.alpha, iv, ckda);
      odd ^= al < 0.f;
      const U flip = odd ? kSign : U(0);
      sq[iv] = static_cast<U>(q[iq] ^ flip);
      sk[iv] = static_cast<U>(k[iq] ^ flip);
      a.sa[iv] = fabsf(al);
    }
  }
  if (s.last) {
    const uint64_t bits = __ballot(odd && ch < DK);
    uint32_t* m = a.tmask + (static_cast<int64_t>(s.n) * H + h) * nwords(DK);
    const int w = ch >> 6, lane = ch & 63;
    if (lane == 0) m[2 * w] = static_cast<uint32_t>(bits);
    if (lane == 32 && 2 * w + 1 < nwords(DK)) m[2 * w + 1] = static_cast<uint32_t>(bits >> 32);
  }
}

// negate row r of ht[n][h] when the sequence is not empty and its final
// parity of channel r is odd; (blockIdx.x = n * H + h)
__global__ __launch_bounds__(256) void sign_fix_kernel(FwdArgs a) {
  const int64_t nh = blockIdx.x;
  const int n = static_cast<int>(nh / a.H);
  const bool empty = a.cu_seqlens ? a.cu_seqlens[n + 1] == a.cu_seqlens[n] : a.T == 0;
  if (empty) return;
  const int dk = a.dk, dv = a.dv, nw = nwords(dk);
  const uint32_t* m = a.tmask + nh * nw;
  float* S = a.ht + nh * dk * dv;
  for (int e = threadIdx.x; e < dk * dv; e += blockDim.x) {
    const int r = e / dv;
    if ((m[r >> 5] >> (r & 31)) & 1u) S[e] = -S[e];
  }
}

template <class IO, class G, int DK>
launch_result launch_dk(const FwdArgs& a, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(a.maxc) * a.H);
  const unsigned threads = DK < 64 ? 64 : DK;
  hipLaunchKernelGGL((sign_mask_kernel<G, DK>), dim3(blocks), dim3(threads), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sign_absorb_kernel<IO, G, DK>), dim3(blocks), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

template <class IO, class G>
launch_result launch_g(const FwdArgs& a, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_dk<IO, G, 16>(a, stream);
    case 32: return launch_dk<IO, G, 32>(a, stream);
    case 64: return launch_dk<IO, G, 64>(a, stream);
    case 128: return launch_dk<IO, G, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <class IO>
launch_result launch_io(const FwdArgs& a, hipStream_t stream) {
  switch (a.gate_input) {
    case CKDA_GATES_F32: return launch_g<IO, gate_f32>(a, stream);
    case CKDA_GATES_LOGITS_F32: return launch_g<IO, gate_logit_f32>(a, stream);
    case CKDA_GATES_LOGITS_BF16: return launch_g<IO, gate_logit_bf16>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int64_t sign_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t num_seqs,
                             int64_t maxc, int32_t io_dtype) {
  const int64_t es = io_dtype == CKDA_DTYPE_BF16 ? 2 : 4;
  const int64_t tok = static_cast<int64_t>(B) * T;
  auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
  return up(4 * H * maxc * nwords(dk)) + up(4 * static_cast<int64_t>(num_seqs) * H * nwords(dk)) +
         2 * up(tok * H * dk * es) + up(tok * H * dk * 4) + up(tok * H * 4);
}

void sign_layout(FwdArgs& a, unsigned char* base, int32_t io_dtype) {
  const int64_t es = io_dtype == CKDA_DTYPE_BF16 ? 2 : 4;
  const int64_t tok = static_cast<int64_t>(a.B) * a.T;
  auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
  a.cmask = reinterpret_cast<uint32_t*>(base);
  base += up(4 * static_cast<int64_t>(a.H) * a.maxc * nwords(a.dk));
  a.tmask = reinterpret_cast<uint32_t*>(base);
  base += up(4 * static_cast<int64_t>(a.num_seqs) * a.H * nwords(a.dk));
  a.sq = base;
  base += up(tok * a.H * a.dk * es);
  a.sk = base;
  base += up(tok * a.H * a.dk * es);
  a.sa = reinterpret_cast<float*>(base);
  base += up(tok * a.H * a.dk * 4);
  a.sb = reinterpret_cast<float*>(base);
}

launch_result launch_sign_absorb(const FwdArgs& a, int32_t io_dtype, hipStream_t stream) {
  if (static_cast<int64_t>(a.maxc) * a.H == 0) return hipSuccess;
  return io_dtype == CKDA_DTYPE_BF16 ? launch_io<io_bf16>(a, stream) : launch_io<io_f32>(a, stream);
}

launch_result launch_sign_fix(const FwdArgs& a, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(a.num_seqs) * a.H;
  if (blocks == 0 || !a.ht) return hipSuccess;
  hipLaunchKernelGGL(sign_fix_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ckda
