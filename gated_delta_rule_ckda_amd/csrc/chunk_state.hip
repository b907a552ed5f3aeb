// State pass of the chunked forward, and the host launcher of both passes.
//
// One workgroup walks one (sequence, head, dv-tile) chain over its chunks in
// order.  Per chunk, from the block the transform pass wrote:
//   U  = X' V - W S                  (the chunk's corrected values)
//   O  = Qt' S + P' U                (outputs, scale and norms folded in)
//   S <- Diag(g) S + Kh'^T U
// (chunked form of the recurrence of the picx.dev summary of the Complex KDA
// paper, section "Background"; the derivation is in the transform pass.)
//
// Waves 0..NSW-1 ("state waves") each own a 16-column slab of the dv-tile:
// the slab of S lives in fp32 accumulators, and U is produced and consumed in
// registers too, so a chunk step needs no barrier among the state waves.  The
// operands that are shared by all columns (X', W, Qt', P', Kh'^T, g) and the
// V tile sit in LDS, read as MFMA row fragments in the permuted K order that
// matches the register fragments (mfma_ops.h).
//
// The last four waves ("loader waves") stream the blocks: a chunk's block and
// V rows are loaded into registers two chunks ahead and written to LDS while
// the state waves wait at a barrier, so HBM latency overlaps the arithmetic.
#include "mfma_ops.h"

namespace ckda {
namespace {

template <class OpT, class IOT, int C_, int DK_, int DV_, int DVT_>
struct StateCfg {
  using Op = OpT;
  using IO = IOT;
  using T = typename Op::T;
  using Frag = typename Op::Frag;
  static constexpr int C = C_, DK = DK_, DV = DV_, DVT = DVT_;
  static constexpr int NSPLIT = DV / DVT;
  static constexpr int NSW = DVT / 16;               // state waves
  static constexpr int NLW = 4;                      // loader waves
  static constexpr int NT = 64 * (NSW + NLW);
  static constexpr int NLT = 64 * NLW;               // loader threads
  static constexpr int NB = C / 16;
  static constexpr int NMC = DK / 16;
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int IOES = static_cast<int>(sizeof(typename IO::storage));
  static constexpr int PAD = 16 / ES;
  static constexpr int LDK = DK + PAD;
  static constexpr int LDC = C + PAD;
  static constexpr int KS = Op::KS;                  // K per register fragment
  static constexpr int NFK = (DK + KS - 1) / KS;     // fragments over dk
  static constexpr int NFC = (C + KS - 1) / KS;      // fragments over the chunk rows

  // the block in global memory (bytes)
  static constexpr int GB_X = 0;
  static constexpr int GB_W = C * C * ES;
  static constexpr int GB_Q = GB_W + C * DK * ES;
  static constexpr int GB_P = GB_Q + C * DK * ES;
  static constexpr int GB_K = GB_P + C * C * ES;
  static constexpr int GB_G = GB_K + DK * C * ES;
  static constexpr int GB_END = GB_G + DK * 4;
  static constexpr int EP = 16 / ES;                 // elements per 16-byte piece
  static constexpr int NPB = GB_END / 16;            // pieces of a block
  static constexpr int VPR = DVT * IOES / 16;        // pieces per V row of the tile
  static constexpr int NPV = C * VPR;                // pieces of the V tile
  static constexpr int NPT = (NPB + NPV + NLT - 1) / NLT;  // pieces per loader thread

  // LDS (bytes)
  static constexpr int O_X = 0;                                  // X'  [C][LDC]
  static constexpr int O_W = align16(O_X + C * LDC * ES);        // -W  [C][LDK]
  static constexpr int O_Q = align16(O_W + C * LDK * ES);        // Qt' [C][LDK]
  static constexpr int O_P = align16(O_Q + C * LDK * ES);        // P'  [C][LDC]
  static constexpr int O_K = align16(O_P + C * LDC * ES);        // Kh'^T [DK][LDC]
  static constexpr int O_VT = align16(O_K + DK * LDC * ES);      // V^T [DVT][LDC]
  static constexpr int O_G = align16(O_VT + DVT * LDC * ES);     // g [DK] fp32
  static constexpr int LDS_BYTES = align16(O_G + DK * 4);

  static_assert(GB_END == blk_g_byte(C, DK, ES) + 4 * DK, "block layout");
  static_assert(GB_X % 16 == 0 && GB_W % 16 == 0 && GB_P % 16 == 0 && GB_K % 16 == 0 &&
                GB_G % 16 == 0, "piece alignment");
  static_assert((C * ES) % 16 == 0 && (DK * ES) % 16 == 0 && (DVT * IOES) % 16 == 0, "rows in pieces");
  static_assert(DV % DVT == 0 && DVT % 16 == 0 && NSW >= 1 && NSW <= 4, "dv tiling");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// One loader thread's pieces of one chunk, in flight.
template <class Cfg>
struct Pieces {
  uint32_t d[Cfg::NPT][4];
};

// Issue the loads of chunk (block base, V rows t0 .. t0+L-1) into pf.
template <class Cfg>
__device__ __forceinline__ void issue_chunk(Pieces<Cfg>& pf, const unsigned char* blk,
                                            const void* v, int64_t t0, int L, int H, int h,
                                            int dv0, int lt) {
  using ST = typename Cfg::IO::storage;
  const rsrc_t rb = make_rsrc(blk, Cfg::GB_END);
  const int vrow = H * Cfg::DV * Cfg::IOES;  // bytes per token in v
  const rsrc_t rv = make_rsrc(static_cast<const ST*>(v) + (t0 * H + h) * static_cast<int64_t>(Cfg::DV) + dv0,
                              L * vrow);
#pragma unroll
  for (int u = 0; u < Cfg::NPT; ++u) {
    const int p = lt + Cfg::NLT * u;
    if (p < Cfg::NPB) {
      ldraw<16>(rb, 16 * p, pf.d[u]);
    } else if (p < Cfg::NPB + Cfg::NPV) {
      const int pv = p - Cfg::NPB;
      const int j = iclamp(pv / Cfg::VPR, L - 1);
      ldraw<16>(rv, j * vrow + 16 * (pv % Cfg::VPR), pf.d[u]);
    }
  }
}

// Write a chunk's pieces into the padded LDS layout (V rows >= L as zeros).
template <class Cfg>
__device__ __forceinline__ void store_chunk(const Pieces<Cfg>& pf, unsigned char* smem, int L,
                                            int lt) {
  using T = typename Cfg::T;
  constexpr int C = Cfg::C, DK = Cfg::DK, ES = Cfg::ES, LDK = Cfg::LDK, LDC = Cfg::LDC;
#pragma unroll
  for (int u = 0; u < Cfg::NPT; ++u) {
    const int p = lt + Cfg::NLT * u;
    const uint4 val = make_uint4(pf.d[u][0], pf.d[u][1], pf.d[u][2], pf.d[u][3]);
    if (p < Cfg::NPB) {
      const int b = 16 * p;
      int dst;
      if (b < Cfg::GB_W) {
        dst = Cfg::O_X + (b / (C * ES)) * LDC * ES + b % (C * ES);
      } else if (b < Cfg::GB_Q) {
        const int o = b - Cfg::GB_W;
        dst = Cfg::O_W + (o / (DK * ES)) * LDK * ES + o % (DK * ES);
      } else if (b < Cfg::GB_P) {
        const int o = b - Cfg::GB_Q;
        dst = Cfg::O_Q + (o / (DK * ES)) * LDK * ES + o % (DK * ES);
      } else if (b < Cfg::GB_K) {
        const int o = b - Cfg::GB_P;
        dst = Cfg::O_P + (o / (C * ES)) * LDC * ES + o % (C * ES);
      } else if (b < Cfg::GB_G) {
        const int o = b - Cfg::GB_K;
        dst = Cfg::O_K + (o / (C * ES)) * LDC * ES + o % (C * ES);
      } else {
        dst = Cfg::O_G + (b - Cfg::GB_G);
      }
      *reinterpret_cast<uint4*>(smem + dst) = val;
    } else if (p < Cfg::NPB + Cfg::NPV) {
      const int pv = p - Cfg::NPB;
      const int j = pv / Cfg::VPR, c0 = (pv % Cfg::VPR) * (16 / Cfg::IOES);
      T* vt = reinterpret_cast<T*>(smem + Cfg::O_VT);
      const bool in = j < L;
      constexpr int NE = 16 / Cfg::IOES;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float x = in ? dec<typename Cfg::IO>(pf.d[u], e) : 0.f;
        vt[(c0 + e) * LDC + j] = Cfg::Op::cvt(x);
      }
    }
  }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT, 1) void state_kernel(FwdArgs a) {
  using Op = typename Cfg::Op;
  using IO = typename Cfg::IO;
  using T = typename Cfg::T;
  using Frag = typename Cfg::Frag;
  using ST = typename IO::storage;
  constexpr int C = Cfg::C, DK = Cfg::DK, DVT = Cfg::DVT, NB = Cfg::NB, NMC = Cfg::NMC;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC;

  extern __shared__ __align__(16) unsigned char smem[];
  const T* sX = reinterpret_cast<const T*>(smem + Cfg::O_X);
  const T* sW = reinterpret_cast<const T*>(smem + Cfg::O_W);
  const T* sQ = reinterpret_cast<const T*>(smem + Cfg::O_Q);
  const T* sP = reinterpret_cast<const T*>(smem + Cfg::O_P);
  const T* sK = reinterpret_cast<const T*>(smem + Cfg::O_K);
  const T* sVT = reinterpret_cast<const T*>(smem + Cfg::O_VT);
  const float* sg = reinterpret_cast<const float*>(smem + Cfg::O_G);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const bool is_state = wave < Cfg::NSW;
  const int lt = tid - 64 * Cfg::NSW;  // loader thread index (loader waves)

  // ---- which chain: the dv-tiles of one (sequence, head) sit 8 workgroups
  // apart so that they land on the same XCD and share its L2 for the blocks.
  const int64_t nblk = gridDim.x;
  const int64_t b = blockIdx.x;
  int64_t pair;
  int split;
  if (Cfg::NSPLIT > 1 && nblk % (8 * Cfg::NSPLIT) == 0) {
    const int64_t xcd = b % 8, slot = b / 8;
    pair = (slot / Cfg::NSPLIT) * 8 + xcd;
    split = static_cast<int>(slot % Cfg::NSPLIT);
  } else {
    pair = b / Cfg::NSPLIT;
    split = static_cast<int>(b % Cfg::NSPLIT);
  }
  const int H = a.H;
  const int n = static_cast<int>(pair / H);
  const int h = static_cast<int>(pair % H);
  int64_t s0;
  int c_begin, nch;
  if (a.cu_seqlens) {
    s0 = uniform64(a.cu_seqlens[n]);
    c_begin = uniform32(a.first[n]);
    nch = uniform32(a.first[n + 1]) - c_begin;
  } else {
    s0 = static_cast<int64_t>(n) * a.T;
    c_begin = n * a.nc;
    nch = a.nc;
  }
  const int64_t s1 = a.cu_seqlens ? uniform64(a.cu_seqlens[n + 1]) : s0 + a.T;
  const int dv0 = split * DVT;
  const unsigned char* blocks = a.blocks + static_cast<int64_t>(h) * a.maxc * a.blk_bytes;

  // ---- state slab: tile mc holds rows 16mc + 4lq + i, column dv0 + 16*wave + l16
  f32x4 sacc[NMC];
  const int64_t st_base = (static_cast<int64_t>(n) * H + h) * DK * a.dv + dv0 + 16 * wave + l16;
  if (is_state) {
#pragma unroll
    for (int mc = 0; mc < NMC; ++mc) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc[mc][i] = a.h0 ? a.h0[st_base + static_cast<int64_t>(16 * mc + 4 * lq + i) * a.dv] : 0.f;
    }
  }

  auto chunk_t0 = [&](int i) { return s0 + static_cast<int64_t>(i) * C; };
  auto chunk_len = [&](int i) {
    const int64_t rem = s1 - chunk_t0(i);
    return static_cast<int>(rem < C ? rem : C);
  };

  // The two roles run separate loops with the same two barriers per chunk,
  // so the loaders' in-flight registers and the state registers never need
  // to be live at the same time.
  if (is_state) {
    ST* go = static_cast<ST*>(a.o);
    for (int i = 0; i < nch; ++i) {
      __syncthreads();  // LDS holds chunk i
      const int L = chunk_len(i);
      const int64_t t0 = chunk_t0(i);
      Frag sf[Cfg::NFK];
      Op::template frags<DK>(sf, sacc);
      // U tiles: X' V - W S
      f32x4 uacc[NB];
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        uacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        Op::template mmaK<C>(uacc[rb], sX + 16 * rb * LDC, LDC, sVT + 16 * wave * LDC, LDC, lane);
        Op::template mma_perm<DK, true>(uacc[rb], sW + (16 * rb + l16) * LDK, sf, lq);
      }
      Frag uf[Cfg::NFC];
      Op::template frags<C>(uf, uacc);
      // O^T tiles: S^T Qt'^T + U^T P'^T
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
        Op::template mma_perm<DK, false>(oacc, sQ + (16 * rb + l16) * LDK, sf, lq);
        Op::template mma_perm<C, false>(oacc, sP + (16 * rb + l16) * LDC, uf, lq);
        const int r = 16 * rb + l16;
        if (r < L)
          IO::store4(go + ((t0 + r) * H + h) * static_cast<int64_t>(a.dv) + dv0 + 16 * wave + 4 * lq,
                     oacc);
      }
      // S <- Diag(g) S + Kh'^T U
#pragma unroll
      for (int mc = 0; mc < NMC; ++mc) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(sg + 16 * mc + 4 * lq);
        sacc[mc] *= gv;
        Op::template mma_perm<C, true>(sacc[mc], sK + (16 * mc + l16) * LDC, uf, lq);
      }
      __syncthreads();  // done with chunk i
    }
  } else {
    // chunks 0 and 1 in flight, chunk 0 into LDS, chunk 2 in flight
    Pieces<Cfg> pa, pb;
    auto issue = [&](Pieces<Cfg>& pf, int i) {
      issue_chunk<Cfg>(pf, blocks + static_cast<int64_t>(c_begin + i) * a.blk_bytes, a.v,
                       chunk_t0(i), chunk_len(i), H, h, dv0, lt);
    };
    if (nch > 0) issue(pa, 0);
    if (nch > 1) issue(pb, 1);
    if (nch > 0) store_chunk<Cfg>(pa, smem, chunk_len(0), lt);
    if (nch > 2) issue(pa, 2);
    // step i: chunk i+1 (in `nxt`) goes to LDS once the state waves are done
    // with chunk i; `nxt` then takes chunk i+3
    auto step = [&](int i, Pieces<Cfg>& nxt) {
      __syncthreads();  // LDS holds chunk i
      __syncthreads();  // the state waves are done with chunk i
      if (i + 1 < nch) {
        store_chunk<Cfg>(nxt, smem, chunk_len(i + 1), lt);
        if (i + 3 < nch) issue(nxt, i + 3);
      }
    };
    int i = 0;
    for (; i + 1 < nch; i += 2) {
      step(i, pb);
      step(i + 1, pa);
    }
    if (i < nch) step(i, pb);
  }

  if (is_state && a.ht) {
#pragma unroll
    for (int mc = 0; mc < NMC; ++mc) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        a.ht[st_base + static_cast<int64_t>(16 * mc + 4 * lq + ii) * a.dv] = sacc[mc][ii];
    }
  }
}

template <class Cfg>
launch_result launch_cfg(const FwdArgs& a, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&state_kernel<Cfg>), hipFuncAttributeMaxDynamicSharedMemorySize,
      Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = static_cast<int64_t>(a.num_seqs) * a.H * Cfg::NSPLIT;
  hipLaunchKernelGGL(state_kernel<Cfg>, dim3(static_cast<unsigned>(blocks)), dim3(Cfg::NT),
                     Cfg::LDS_BYTES, stream, a);
  return hipGetLastError();
}

struct Entry {
  int chunk, dk, dv, dtype;
  launch_result (*fn)(const FwdArgs&, hipStream_t);
};

template <class Op, class IO, int C, int D, int DVT>
constexpr Entry entry(int dtype) {
  return Entry{C, D, D, dtype, &launch_cfg<StateCfg<Op, IO, C, D, D, DVT>>};
}

const Entry kEntries[] = {
    entry<OpBF16, io_bf16, 64, 128, 64>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 32, 128, 64>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 16, 128, 64>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 64, 64, 32>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 32, 64, 32>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 16, 64, 32>(CKDA_DTYPE_BF16),
    entry<OpF32, io_f32, 16, 16, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 16, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 64, 16, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 16, 32, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 32, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 64, 32, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 16, 64, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 64, 32>(CKDA_DTYPE_F32),
};

const Entry* find(int32_t chunk, int32_t dk, int32_t dv, int32_t dtype) {
  for (const Entry& e : kEntries)
    if (e.chunk == chunk && e.dk == dk && e.dv == dv && e.dtype == dtype) return &e;
  return nullptr;
}

int64_t max_chunks(int32_t B, int32_t T, int32_t num_seqs, int32_t chunk, bool packed) {
  const int64_t per = (static_cast<int64_t>(T) + chunk - 1) / chunk;
  return packed ? per + num_seqs : per * B;
}

}  // namespace

bool state_supported(int32_t chunk, int32_t dk, int32_t dv, int32_t io_dtype) {
  return find(chunk, dk, dv, io_dtype) != nullptr;
}

bool fwd_supported(int32_t chunk, int32_t dk, int32_t dv, int32_t io_dtype) {
  return state_supported(chunk, dk, dv, io_dtype) && prep_supported(chunk, dk, io_dtype);
}

size_t fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t num_seqs,
                           int32_t chunk, int32_t io_dtype, bool packed) {
  const int64_t maxc = max_chunks(B, T, num_seqs, chunk, packed);
  const int64_t es = io_dtype == CKDA_DTYPE_BF16 ? 2 : 4;
  const int64_t map = packed ? ((4 * (num_seqs + 1 + maxc) + 255) & ~int64_t(255)) : 0;
  return static_cast<size_t>(map + static_cast<int64_t>(H) * maxc * blk_bytes(chunk, dk, es));
}

launch_result launch_fwd(FwdArgs a, int32_t io_dtype, void* ws, hipStream_t stream) {
  if (static_cast<int64_t>(a.B) * a.T == 0) {
    // no tokens: every chain is empty and only copies h0 to ht (or zeros);
    // run the state pass as a dense batch with no chunks and no workspace
    a.cu_seqlens = nullptr;
    a.T = 0;
    a.B = a.num_seqs;
  }
  const bool packed = a.cu_seqlens != nullptr;
  const int64_t es = io_dtype == CKDA_DTYPE_BF16 ? 2 : 4;
  const int64_t maxc = max_chunks(a.B, a.T, a.num_seqs, a.chunk, packed);
  unsigned char* base = static_cast<unsigned char*>(ws);
  a.maxc = static_cast<int32_t>(maxc);
  a.nc = static_cast<int32_t>((static_cast<int64_t>(a.T) + a.chunk - 1) / a.chunk);
  a.blk_bytes = blk_bytes(a.chunk, a.dk, es);
  a.first = nullptr;
  a.chunk_seq = nullptr;
  if (packed) {
    a.first = reinterpret_cast<int32_t*>(base);
    a.chunk_seq = a.first + a.num_seqs + 1;
    base += (4 * (a.num_seqs + 1 + maxc) + 255) & ~int64_t(255);
  }
  a.blocks = base;
  const Entry* e = find(a.chunk, a.dk, a.dv, io_dtype);
  if (!e) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.num_seqs) * a.H == 0) return hipSuccess;
  if (packed) {
    const launch_result r = launch_chunk_map(a, stream);
    if (r != hipSuccess) return r;
  }
  if (maxc > 0) {
    const launch_result r = launch_prep(a, io_dtype, stream);
    if (r != hipSuccess) return r;
  }
  return e->fn(a, stream);
}

}  // namespace ckda
