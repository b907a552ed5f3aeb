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
// matches the register fragments; the transform pass stores those rows in
// that order already (perm32 in mfma_ops.h), so each fragment is one 16-byte
// read.
//
// The last eight waves ("loader waves") stream the blocks: a chunk's block and
// V rows are loaded into registers two chunks ahead and written to LDS while
// the state waves wait at a barrier, so HBM latency overlaps the arithmetic.
// They also write the outputs: the state waves leave a chunk's O tile in LDS
// and the loaders store it one chunk later as whole rows of the dv tile (16
// bytes per thread, non-temporal) rather than 32-byte pieces from each state
// wave.
#include "mfma_ops.h"

namespace ckda {
namespace {

// 16 bytes of the output, stored with the non-temporal hint: o is not read
// again here, and plain stores would displace the workspace blocks the pass
// still reads from the last-level cache.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class OpT, class IOT, int C_, int DK_, int DV_, int DVT_>
struct StateCfg {
  using Op = OpT;
  using IO = IOT;
  using T = typename Op::T;
  using Frag = typename Op::Frag;
  static constexpr int C = C_, DK = DK_, DV = DV_, DVT = DVT_;
  static constexpr int NSPLIT = DV / DVT;
  static constexpr int NSW = DVT / 16;               // state waves
  static constexpr int NLW = 8;                      // loader waves
  static constexpr int NT = 64 * (NSW + NLW);
  static constexpr int NLT = 64 * NLW;               // loader threads
  static constexpr int NB = C / 16;
  static constexpr int NMC = DK / 16;
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int IOES = static_cast<int>(sizeof(typename IO::storage));
  static constexpr int LDK = frag_stride(DK, ES);
  static constexpr int LDC = frag_stride(C, ES);
  static constexpr int KS = Op::KS;                  // K per register fragment
  static constexpr int NFK = (DK + KS - 1) / KS;     // fragments over dk
  static constexpr int NFC = (C + KS - 1) / KS;      // fragments over the chunk rows
  // X' and P' are lower triangular: K fragment s of row block rb holds a
  // nonzero only if its first column is at or left of the block's last row
  static constexpr bool tri_live(int rb, int s) { return KS * s <= 16 * rb + 15; }

  // the block in global memory (bytes); X' and P' packed when TRI
  static constexpr bool TRI = tri_packed(C, ES);
  static constexpr int TRIB = static_cast<int>(tri_elems(C, ES)) * ES;  // bytes of X' (or P')
  static constexpr int GB_X = 0;
  static constexpr int GB_W = TRIB;
  static constexpr int GB_Q = GB_W + C * DK * ES;
  static constexpr int GB_P = GB_Q + C * DK * ES;
  static constexpr int GB_K = GB_P + TRIB;
  static constexpr int GB_G = GB_K + DK * C * ES;
  static constexpr int GB_END = GB_G + DK * 4;
  static constexpr int VPR = DVT * IOES / 16;        // 16-byte pieces per V row of the tile
  static constexpr int NVU = (C / 2) * VPR;          // V units: one piece of two adjacent rows

  // LDS (bytes)
  static constexpr int O_X = 0;                                  // X'  [C][LDC]
  static constexpr int O_W = align16(O_X + C * LDC * ES);        // -W  [C][LDK]
  static constexpr int O_Q = align16(O_W + C * LDK * ES);        // Qt' [C][LDK]
  static constexpr int O_P = align16(O_Q + C * LDK * ES);        // P'  [C][LDC]
  static constexpr int O_K = align16(O_P + C * LDC * ES);        // Kh'^T [DK][LDC]
  static constexpr int O_VT = align16(O_K + DK * LDC * ES);      // V^T [DVT][LDC]
  static constexpr int O_G = align16(O_VT + DVT * LDC * ES);     // g [DK] fp32
  static constexpr int LDO = DVT * IOES + 16;                    // O tile row stride (bytes)
  static constexpr int O_O = align16(O_G + DK * 4);              // O tile [C][DVT] (io type)
  // the state entering a chunk [DK][DVT] (io type; only when the backward's
  // records are kept), staged for whole-row stores by the loader waves
  static constexpr int LDH = DVT * IOES + 16;
  static constexpr int O_HC = align16(O_O + C * LDO);
  static constexpr int LDS_BYTES = align16(O_HC + DK * LDH);

  static_assert(GB_END == blk_g_byte(C, DK, ES) + 4 * DK, "block layout");
  static_assert(GB_X % 16 == 0 && GB_W % 16 == 0 && GB_P % 16 == 0 && GB_K % 16 == 0 &&
                GB_G % 16 == 0, "piece alignment");
  static_assert((C * ES) % 16 == 0 && (DK * ES) % 16 == 0 && (DVT * IOES) % 16 == 0, "rows in pieces");
  static_assert(DV % DVT == 0 && DVT % 16 == 0 && NSW >= 1 && NSW <= 4, "dv tiling");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Sections of a block as the loaders copy them: global byte offset and row
// length, LDS byte offset and row stride, and 16-byte pieces.  Every section's
// rows are whole pieces, so a piece never straddles a row.  tri: X' or P',
// whose first C/2 rows hold half a row each when the block is packed.
struct Sec {
  int g0, grow, l0, lrow, n;
  bool tri;
};
template <class Cfg>
struct Secs {
  static constexpr int C = Cfg::C, DK = Cfg::DK, ES = Cfg::ES;
  static constexpr Sec s[6] = {
      {Cfg::GB_X, C * ES, Cfg::O_X, Cfg::LDC * ES, Cfg::TRIB / 16, true},
      {Cfg::GB_W, DK * ES, Cfg::O_W, Cfg::LDK * ES, C * DK * ES / 16, false},
      {Cfg::GB_Q, DK * ES, Cfg::O_Q, Cfg::LDK * ES, C * DK * ES / 16, false},
      {Cfg::GB_P, C * ES, Cfg::O_P, Cfg::LDC * ES, Cfg::TRIB / 16, true},
      {Cfg::GB_K, C * ES, Cfg::O_K, Cfg::LDC * ES, DK * C * ES / 16, false},
      {Cfg::GB_G, DK * 4, Cfg::O_G, DK * 4, DK * 4 / 16, false},
  };
  // LDS byte offset of piece p of section k (the packed rows of X' and P'
  // first: C/2 rows of C/2 elements, then C/2 rows of C)
  static __device__ __forceinline__ int lds_of(int k, int p) {
    int row, col;
    if (Cfg::TRI && s[k].tri) {
      constexpr int HP = C / 2 * ES / 16;  // pieces of a half row
      constexpr int NH = C / 2 * HP;       // pieces of the packed rows
      row = p < NH ? p / HP : C / 2 + (p - NH) / (2 * HP);
      col = 16 * (p < NH ? p % HP : (p - NH) % (2 * HP));
    } else {
      row = 16 * p / s[k].grow;
      col = 16 * p % s[k].grow;
    }
    return s[k].l0 + row * s[k].lrow + col;
  }
  // loads per loader thread for section k
  static constexpr int per(int k) { return (s[k].n + Cfg::NLT - 1) / Cfg::NLT; }
  static constexpr int NV = (Cfg::NVU + Cfg::NLT - 1) / Cfg::NLT;  // V units per thread
};

// The loaders move a block in two groups, by when the state waves read them:
// group A (X', -W and the V tile) feeds U, group B (Qt', P', Kh'^T, g) feeds
// the outputs and the state update.  Group B of chunk i is written while the
// state waves compute U(i), group A of chunk i+1 while they compute O(i) and
// S(i); two groups of each kind are in flight.
//
// One loader thread's pieces of sections [K0, K1) (plus the V tile if WITH_V)
// of one chunk.  Every load is issued unconditionally (indices clamped into
// range; duplicates are discarded at the store), so the number of loads per
// group is fixed and each wait can leave the newer groups outstanding.
template <class Cfg, int K0, int K1, bool WITH_V>
struct Group {
  using S = Secs<Cfg>;
  static constexpr int first(int k) { return k <= K0 ? 0 : first(k - 1) + S::per(k - 1); }
  static constexpr int NBL = first(K1);
  static constexpr int NV = WITH_V ? S::NV : 0;
  uint32_t d[NBL + 2 * NV][4];

  __device__ __forceinline__ void issue(const unsigned char* blk, const void* v, int64_t t0, int L,
                                        int H, int h, int dv0, int lt) {
    using ST = typename Cfg::IO::storage;
    const rsrc_t rb = make_rsrc(blk, Cfg::GB_END);
#pragma unroll
    for (int k = K0; k < K1; ++k) {
#pragma unroll
      for (int u = 0; u < S::per(k); ++u) {
        const int p = iclamp(lt + Cfg::NLT * u, S::s[k].n - 1);
        ldraw<16>(rb, S::s[k].g0 + 16 * p, d[first(k) + u]);
      }
    }
    if constexpr (WITH_V) {
      const int vrow = H * Cfg::DV * Cfg::IOES;  // bytes per token in v
      const rsrc_t rv = make_rsrc(
          static_cast<const ST*>(v) + (t0 * H + h) * static_cast<int64_t>(Cfg::DV) + dv0, L * vrow);
      // unit -> (row pair jp, piece cp) with jp fastest, so that the
      // transposed LDS writes of 32 lanes land in 32 different banks
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int uv = iclamp(lt + Cfg::NLT * u, Cfg::NVU - 1);
        const int jp = uv % (Cfg::C / 2), cp = uv / (Cfg::C / 2);
        ldraw<16>(rv, iclamp(2 * jp, L - 1) * vrow + 16 * cp, d[NBL + 2 * u]);
        ldraw<16>(rv, iclamp(2 * jp + 1, L - 1) * vrow + 16 * cp, d[NBL + 2 * u + 1]);
      }
    }
  }

  // Write the pieces into the padded LDS layout (V rows >= L as zeros).
  __device__ __forceinline__ void store(unsigned char* smem, int L, int lt) const {
    using T = typename Cfg::T;
#pragma unroll
    for (int k = K0; k < K1; ++k) {
#pragma unroll
      for (int u = 0; u < S::per(k); ++u) {
        const int p = lt + Cfg::NLT * u;
        if (S::s[k].n % Cfg::NLT == 0 || p < S::s[k].n) {
          const int dst = S::lds_of(k, p);
          const uint32_t* q = d[first(k) + u];
          *reinterpret_cast<uint4*>(smem + dst) = make_uint4(q[0], q[1], q[2], q[3]);
        }
      }
    }
    if constexpr (WITH_V) {
      T* vt = reinterpret_cast<T*>(smem + Cfg::O_VT);
      constexpr int NE = 16 / Cfg::IOES;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int uv = lt + Cfg::NLT * u;
        if (Cfg::NVU % Cfg::NLT == 0 || uv < Cfg::NVU) {
          const int jp = uv % (Cfg::C / 2), c0 = (uv / (Cfg::C / 2)) * NE;
          const bool in0 = 2 * jp < L, in1 = 2 * jp + 1 < L;
          // rows 2jp and 2jp+1 are adjacent in the storage order too
          const int q = Cfg::Op::template pos<Cfg::C>(2 * jp);
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const float x0 = in0 ? dec<typename Cfg::IO>(d[NBL + 2 * u], e) : 0.f;
            const float x1 = in1 ? dec<typename Cfg::IO>(d[NBL + 2 * u + 1], e) : 0.f;
            Cfg::Op::store2(vt + (c0 + e) * Cfg::LDC + q, x0, x1);
          }
        }
      }
    }
  }
};

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
  // packed sequences go out longest first, so the chains that decide when
  // the pass ends start first and the short ones fill in behind them
  const int n = a.cu_seqlens ? uniform32(a.seq_order[pair / H]) : static_cast<int>(pair / H);
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
    for (int i = 0; i < nch; ++i) {
      if (a.hc) {  // the state entering chunk i, for the backward: staged,
                   // the loaders store it as whole rows
        ST* hs = reinterpret_cast<ST*>(smem + Cfg::O_HC) + 16 * wave + l16;
#pragma unroll
        for (int mc = 0; mc < NMC; ++mc)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            IO::store(hs, (16 * mc + 4 * lq + ii) * (Cfg::LDH / Cfg::IOES), sacc[mc][ii]);
      }
      __syncthreads();  // group A of chunk i is in LDS
      Frag sf[Cfg::NFK];
      Op::template frags<DK>(sf, sacc);
      // U tiles: X' V - W S.  All LDS fragments of the phase are read first
      // (one exposure of LDS latency), then the MFMAs run.
      f32x4 uacc[NB];
      {
        Frag xf[NB][Cfg::NFC], wf[NB][Cfg::NFK], vf[Cfg::NFC];
        const T* vrow = sVT + (16 * wave + l16) * LDC;
#pragma unroll
        for (int s = 0; s < Cfg::NFC; ++s) vf[s] = Op::template row_frag<C>(vrow, s, lq);
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
          for (int s = 0; s < Cfg::NFC; ++s)
            if (Cfg::tri_live(rb, s)) xf[rb][s] = Op::template row_frag<C>(sX + (16 * rb + l16) * LDC, s, lq);
#pragma unroll
          for (int s = 0; s < Cfg::NFK; ++s)
            wf[rb][s] = Op::template row_frag<DK>(sW + (16 * rb + l16) * LDK, s, lq);
        }
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
          uacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < Cfg::NFC; ++s)
            if (Cfg::tri_live(rb, s)) Op::mma(uacc[rb], xf[rb][s], vf[s]);
#pragma unroll
          for (int s = 0; s < Cfg::NFK; ++s) Op::mma(uacc[rb], wf[rb][s], sf[s]);
        }
      }
      Frag uf[Cfg::NFC];
      Op::template frags<C>(uf, uacc);
      __syncthreads();  // group B of chunk i is in LDS
      // O^T tiles: S^T Qt'^T + U^T P'^T
      {
        Frag qf[NB][Cfg::NFK], pf[NB][Cfg::NFC];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
          for (int s = 0; s < Cfg::NFK; ++s)
            qf[rb][s] = Op::template row_frag<DK>(sQ + (16 * rb + l16) * LDK, s, lq);
#pragma unroll
          for (int s = 0; s < Cfg::NFC; ++s)
            if (Cfg::tri_live(rb, s)) pf[rb][s] = Op::template row_frag<C>(sP + (16 * rb + l16) * LDC, s, lq);
        }
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
          f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < Cfg::NFK; ++s) Op::mma(oacc, sf[s], qf[rb][s]);
#pragma unroll
          for (int s = 0; s < Cfg::NFC; ++s)
            if (Cfg::tri_live(rb, s)) Op::mma(oacc, uf[s], pf[rb][s]);
          // to the O tile; rows >= L are dropped when the tile is written out
          IO::store4(reinterpret_cast<ST*>(smem + Cfg::O_O + (16 * rb + l16) * Cfg::LDO) +
                         16 * wave + 4 * lq,
                     oacc);
        }
      }
      // S <- Diag(g) S + Kh'^T U
      {
        Frag kf[NMC][Cfg::NFC];
        f32x4 gv[NMC];
#pragma unroll
        for (int mc = 0; mc < NMC; ++mc) {
          gv[mc] = *reinterpret_cast<const f32x4*>(sg + 16 * mc + 4 * lq);
#pragma unroll
          for (int s = 0; s < Cfg::NFC; ++s)
            kf[mc][s] = Op::template row_frag<C>(sK + (16 * mc + l16) * LDC, s, lq);
        }
#pragma unroll
        for (int mc = 0; mc < NMC; ++mc) {
          sacc[mc] *= gv[mc];
#pragma unroll
          for (int s = 0; s < Cfg::NFC; ++s) Op::mma(sacc[mc], kf[mc][s], uf[s]);
        }
      }
    }
  } else {
    using GA = Group<Cfg, 0, 2, true>;
    // the O tile of chunk i to o: rows < L, 16 bytes per thread
    auto write_o = [&](int i) {
      constexpr int PR = DVT * Cfg::IOES / 16, NOP = C * PR;
      const int L = chunk_len(i);
      const int64_t t0 = chunk_t0(i);
#pragma unroll
      for (int u = 0; u < (NOP + Cfg::NLT - 1) / Cfg::NLT; ++u) {
        const int p = lt + Cfg::NLT * u;
        const int r = p / PR, cp = p % PR;
        if ((NOP % Cfg::NLT == 0 || p < NOP) && r < L) {
          const u32x4 val = *reinterpret_cast<const u32x4*>(smem + Cfg::O_O + r * Cfg::LDO + 16 * cp);
          __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(
                                               static_cast<unsigned char*>(a.o) +
                                               (((t0 + r) * H + h) * static_cast<int64_t>(a.dv) + dv0) * Cfg::IOES +
                                               16 * cp));
        }
      }
    };
    using GB = Group<Cfg, 2, 6, false>;
    // Loads are issued for every step (the chunk index clamped to the last
    // chunk), so each wait counts the same number of newer loads on every path.
    auto blk = [&](int i) {
      const int ic = i < nch - 1 ? i : nch - 1;
      return blocks + static_cast<int64_t>(c_begin + ic) * a.blk_bytes;
    };
    auto clampi = [&](int i) { return i < nch - 1 ? i : nch - 1; };
    auto issueA = [&](GA& g, int i) {
      const int ic = clampi(i);
      g.issue(blk(ic), a.v, chunk_t0(ic), chunk_len(ic), H, h, dv0, lt);
    };
    auto issueB = [&](GB& g, int i) { g.issue(blk(clampi(i)), nullptr, 0, 1, H, h, dv0, lt); };
    GA sa0, sa1;
    GB sb0, sb1;
    if (nch > 0) {
      issueA(sa0, 0);
      issueB(sb0, 0);
      issueA(sa1, 1);
      issueB(sb1, 1);
      sa0.store(smem, chunk_len(0), lt);
      issueA(sa0, 2);
    }
    // step i: B(i) (in gb) goes to LDS while U(i) runs, then A(i+1) (in ga)
    // while O(i) and S(i) run; gb then takes B(i+2) and ga takes A(i+3)
    auto step = [&](int i, GB& gb, GA& ga) {
      __syncthreads();  // U(i) may start; the state waves are done with B(i-1) and O(i-1)
      gb.store(smem, 0, lt);
      issueB(gb, i + 2);
      if (i > 0 && a.o) write_o(i - 1);
      if (a.hc)  // staged before this barrier; the next one is staged after the next
        flush_rows<DK, DVT * Cfg::IOES, Cfg::LDH, Cfg::NLT>(
            smem + Cfg::O_HC,
            static_cast<unsigned char*>(a.hc) +
                ((static_cast<int64_t>(h) * a.maxc + c_begin + i) * DK * a.dv + dv0) * Cfg::IOES,
            static_cast<int64_t>(a.dv) * Cfg::IOES, DK, lt);
      __syncthreads();  // O(i), S(i) may start; the state waves are done with A(i)
      // unconditional (past the last chunk it rewrites the last chunk's group
      // A, which nothing reads any more): a skipped store would leave these
      // registers' loads pending when the next issue overwrites them
      ga.store(smem, chunk_len(clampi(i + 1)), lt);
      issueA(ga, i + 3);
    };
    int i = 0;
    for (; i + 1 < nch; i += 2) {
      step(i, sb0, sa1);
      step(i + 1, sb1, sa0);
    }
    if (i < nch) step(i, sb0, sa1);
  }
  __syncthreads();  // the last O tile is in LDS
  if (!is_state && nch > 0 && a.o) {
    constexpr int PR = DVT * Cfg::IOES / 16, NOP = C * PR;
    const int il = nch - 1, L = chunk_len(il);
    const int64_t t0 = chunk_t0(il);
    for (int p = lt; p < NOP; p += Cfg::NLT) {
      const int r = p / PR, cp = p % PR;
      if (r < L)
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x4*>(smem + Cfg::O_O + r * Cfg::LDO + 16 * cp),
            reinterpret_cast<u32x4*>(static_cast<unsigned char*>(a.o) +
                                     (((t0 + r) * H + h) * static_cast<int64_t>(a.dv) + dv0) * Cfg::IOES +
                                     16 * cp));
    }
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
                           int32_t chunk, int32_t io_dtype, bool packed, bool sign_absorb) {
  const int64_t maxc = max_chunks(B, T, num_seqs, chunk, packed);
  const int64_t es = io_dtype == CKDA_DTYPE_BF16 ? 2 : 4;
  const int64_t map = packed ? ((8 * maxc + 4 * (2 * int64_t(num_seqs) + 1 + maxc) + 255) & ~int64_t(255)) : 0;
  const int64_t flags = (4 * static_cast<int64_t>(H) * maxc + 255) & ~int64_t(255);
  const int64_t sign = sign_absorb ? sign_workspace_bytes(B, T, H, dk, num_seqs, maxc, io_dtype) : 0;
  return static_cast<size_t>(map + flags + static_cast<int64_t>(H) * maxc * blk_bytes(chunk, dk, es) +
                             sign);
}

namespace {
// Chunk bookkeeping and the workspace's map, flags and blocks; returns the
// first byte after them.
unsigned char* fwd_layout(FwdArgs& a, int32_t io_dtype, void* ws) {
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
  a.seq_order = nullptr;
  a.chunk_geo = nullptr;
  if (packed) {
    a.chunk_geo = reinterpret_cast<int2*>(base);
    a.first = reinterpret_cast<int32_t*>(base + 8 * maxc);
    a.chunk_seq = a.first + a.num_seqs + 1;
    a.seq_order = a.chunk_seq + maxc;
    base += (8 * maxc + 4 * (2 * int64_t(a.num_seqs) + 1 + maxc) + 255) & ~int64_t(255);
  }
  a.irregular = reinterpret_cast<int32_t*>(base);
  base += (4 * static_cast<int64_t>(a.H) * maxc + 255) & ~int64_t(255);
  a.blocks = base;
  base += static_cast<int64_t>(a.H) * maxc * a.blk_bytes;
  return base;
}
}  // namespace

launch_result launch_fwd(FwdArgs a, int32_t io_dtype, void* ws, hipStream_t stream,
                         bool prepare, bool finish) {
  unsigned char* base = fwd_layout(a, io_dtype, ws);
  const bool packed = a.cu_seqlens != nullptr;
  const int64_t maxc = a.maxc;
  const Entry* e = find(a.chunk, a.dk, a.dv, io_dtype);
  if (!e) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.num_seqs) * a.H == 0) return hipSuccess;
  // sign absorption: a chain with no tokens has nothing to absorb
  const bool absorb = a.sign_absorb != 0 && static_cast<int64_t>(a.B) * a.T > 0;
  FwdArgs run = a;
  if (absorb) {
    sign_layout(run, base, io_dtype);
    a = run;  // the sign passes read the caller's tensors through `a`
    run.q = run.sq;
    run.k = run.sk;
    run.alpha = run.sa;
    run.beta = run.sb;
    run.Hk = run.H;
    run.gate_input = CKDA_GATES_F32;
  }
  if (prepare && packed) {
    const launch_result r = launch_chunk_map(a, stream);
    if (r != hipSuccess) return r;
  }
  if (prepare && absorb) {
    const launch_result r = launch_sign_absorb(a, io_dtype, stream);
    if (r != hipSuccess) return r;
  }
  if (prepare && maxc > 0) {
    const launch_result r = launch_prep(run, io_dtype, stream);
    if (r != hipSuccess) return r;
  }
  if (!finish) return hipSuccess;
  const launch_result r = e->fn(run, stream);
  if (r != hipSuccess || !absorb) return r;
  return launch_sign_fix(run, stream);
}

size_t bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                           int32_t num_seqs, int32_t chunk, int32_t io_dtype, bool packed) {
  const int64_t maxc = max_chunks(B, T, num_seqs, chunk, packed);
  return fwd_workspace_bytes(B, T, H, dk, num_seqs, chunk, io_dtype, packed, false) +
         static_cast<size_t>(bwd_extra_bytes(H, maxc, chunk, dk, dv, io_dtype));
}

launch_result launch_bwd(BwdArgs b, int32_t io_dtype, void* ws, hipStream_t stream) {
  FwdArgs& a = b.f;
  a.sign_absorb = 0;
  unsigned char* base = fwd_layout(a, io_dtype, ws);
  const Entry* e = find(a.chunk, a.dk, a.dv, io_dtype);
  if (!e) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.num_seqs) * a.H == 0) return hipSuccess;
  bwd_layout(b, base, io_dtype);
  // the forward again, keeping X and the chunk entry states, writing no output
  a.o = nullptr;
  a.ht = nullptr;
  if (a.cu_seqlens) {
    const launch_result r = launch_chunk_map(a, stream);
    if (r != hipSuccess) return r;
  }
  if (a.maxc > 0) {
    const launch_result r = launch_prep(a, io_dtype, stream);
    if (r != hipSuccess) return r;
  }
  const launch_result r = e->fn(a, stream);
  if (r != hipSuccess) return r;
  return launch_bwd_passes(b, io_dtype, stream);
}

launch_result launch_fwd_save(FwdArgs fa, int32_t io_dtype, void* ws, hipStream_t stream) {
  BwdArgs b{};
  b.f = fa;
  FwdArgs& a = b.f;
  a.sign_absorb = 0;
  unsigned char* base = fwd_layout(a, io_dtype, ws);
  const Entry* e = find(a.chunk, a.dk, a.dv, io_dtype);
  if (!e) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.num_seqs) * a.H == 0) return hipSuccess;
  // the records go where launch_bwd would put them; o and ht are written too
  bwd_layout(b, base, io_dtype);
  if (a.cu_seqlens) {
    const launch_result r = launch_chunk_map(a, stream);
    if (r != hipSuccess) return r;
  }
  if (a.maxc > 0) {
    const launch_result r = launch_prep(a, io_dtype, stream);
    if (r != hipSuccess) return r;
  }
  return e->fn(a, stream);
}

launch_result launch_bwd_saved(BwdArgs b, int32_t io_dtype, void* ws, hipStream_t stream) {
  FwdArgs& a = b.f;
  a.sign_absorb = 0;
  unsigned char* base = fwd_layout(a, io_dtype, ws);
  const Entry* e = find(a.chunk, a.dk, a.dv, io_dtype);
  if (!e) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.num_seqs) * a.H == 0) return hipSuccess;
  bwd_layout(b, base, io_dtype);
  a.o = nullptr;
  a.ht = nullptr;
  return launch_bwd_passes(b, io_dtype, stream);
}

}  // namespace ckda
