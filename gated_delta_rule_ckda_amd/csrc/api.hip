// Host side of the C ABI declared in include/ckda.h: argument validation,
// shape dispatch and error reporting.  Validation never touches the GPU, so a
// non-OK status means nothing was enqueued; only a launch can return
// CKDA_ERR_HIP.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "ckda_internal.h"

namespace {

thread_local std::string g_last_error;

ckda_status_t fail(ckda_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ckda_status_t fail(ckda_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ckda_status_t ok() {
  g_last_error.clear();
  return CKDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range& a, const Range& b) {
  return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

int64_t elem_bytes(int32_t dtype) { return dtype == CKDA_DTYPE_BF16 ? 2 : 4; }

static_assert(CKDA_GATES_F32 == 0 && CKDA_GATES_LOGITS_F32 == 1 && CKDA_GATES_LOGITS_BF16 == 2,
              "the kernels index their variants by ckda_gate_input_t");
// q/k heads: 0 means as many as value heads
int32_t qk_heads_of(int32_t H, int32_t qk_heads) { return qk_heads == 0 ? H : qk_heads; }
bool valid_qk_heads(int32_t H, int32_t qk_heads) {
  const int32_t hk = qk_heads_of(H, qk_heads);
  return hk > 0 && H > 0 && H % hk == 0;
}

bool valid_gate_input(int32_t g) { return g >= CKDA_GATES_F32 && g <= CKDA_GATES_LOGITS_BF16; }
int64_t gate_bytes(int32_t g) { return g == CKDA_GATES_LOGITS_BF16 ? 2 : 4; }

ckda_status_t from_hip(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(CKDA_ERR_HIP, "HIP launch error %d: %s", static_cast<int>(e), hipGetErrorString(e));
}

// ---- static scratch of ckda_chunk_fwd_noalloc
// Device memory the allocation-free forward uses as its workspace: every GPU
// the library runs on holds its own copy for the life of the process.  In
// host code `scratch` names a host-side stand-in, never a device address:
// its device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is handed to kernels.
__device__ __align__(256) unsigned char scratch[CKDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // per device; nullptr until looked up

// The device address of the scratch copy on the device that `stream` belongs
// to (the current device for the null stream).
hipError_t scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t ckda_abi_version(void) { return CKDA_ABI_VERSION; }

const char* ckda_last_error(void) { return g_last_error.c_str(); }

const char* ckda_status_string(int32_t s) {
  switch (s) {
    case CKDA_OK: return "ok";
    case CKDA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CKDA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case CKDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case CKDA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t ckda_fwd_supported(const ckda_fwd_desc_t* d) {
  if (!d) return 0;
  return ckda::fwd_supported(d->chunk_size, d->dk, d->dv, d->io_dtype) ? 1 : 0;
}

size_t ckda_chunk_fwd_workspace_size(const ckda_fwd_desc_t* d, int32_t packed) {
  if (!d || d->B <= 0 || d->T < 0 || d->H <= 0 || d->dk <= 0 || d->num_seqs < 0) return 0;
  if (d->io_dtype != CKDA_DTYPE_BF16 && d->io_dtype != CKDA_DTYPE_F32) return 0;
  if (d->chunk_size != 16 && d->chunk_size != 32 && d->chunk_size != 64) return 0;
  if (static_cast<int64_t>(d->B) * d->T == 0 || d->num_seqs == 0) return 0;
  return ckda::fwd_workspace_bytes(d->B, d->T, d->H, d->dk, d->num_seqs, d->chunk_size,
                                   d->io_dtype, packed != 0, d->sign_absorb == 1);
}

size_t ckda_chunk_bwd_workspace_size(const ckda_fwd_desc_t* d, int32_t packed) {
  if (!d || d->B <= 0 || d->T < 0 || d->H <= 0 || d->dk <= 0 || d->dv <= 0 || d->num_seqs < 0)
    return 0;
  if (d->io_dtype != CKDA_DTYPE_BF16 && d->io_dtype != CKDA_DTYPE_F32) return 0;
  if (d->chunk_size != 16 && d->chunk_size != 32 && d->chunk_size != 64) return 0;
  if (static_cast<int64_t>(d->B) * d->T == 0 || d->num_seqs == 0) return 0;
  if (!valid_gate_input(d->gate_input) || !valid_qk_heads(d->H, d->qk_heads)) return 0;
  const size_t core = ckda::bwd_workspace_bytes(d->B, d->T, d->H, d->dk, d->dv, d->num_seqs,
                                                d->chunk_size, d->io_dtype, packed != 0);
  const size_t extra = ckda::bwd_gates_extra_bytes(d->B, d->T, d->H, qk_heads_of(d->H, d->qk_heads),
                                                   d->dk, d->io_dtype, d->gate_input != CKDA_GATES_F32);
  return extra == 0 ? core : ((core + 255) & ~size_t(255)) + extra;
}

}  // extern "C"

namespace {

constexpr int kPrepare = 1, kFinish = 2;

// Host validation shared by the chunked-forward entry points.  `passes` says
// which tensors the call uses: kPrepare needs q, k, alpha, beta; kFinish
// needs v and o (and reads h0, writes ht).  Pointers a pass does not use must
// be NULL.
ckda_status_t validate_fwd(const ckda_fwd_desc_t* d, const void* q, const void* k,
                           const void* v, const void* alpha, const void* beta,
                           const int32_t* cu_seqlens, const float* h0, const void* o,
                           const float* ht, const void* workspace, size_t workspace_bytes,
                           int passes, bool check_workspace = true) {
  if (!d) return fail(CKDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->B <= 0 || d->T < 0 || d->H <= 0 || d->dk <= 0 || d->dv <= 0 || d->num_seqs < 0)
    return fail(CKDA_ERR_INVALID_ARGUMENT,
                "non-positive size: B=%d T=%d H=%d dk=%d dv=%d num_seqs=%d", d->B, d->T, d->H,
                d->dk, d->dv, d->num_seqs);
  if (d->io_dtype != CKDA_DTYPE_BF16 && d->io_dtype != CKDA_DTYPE_F32)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "io_dtype %d is not a ckda_dtype_t", d->io_dtype);
  if (d->gate_range != CKDA_GATE_KDA && d->gate_range != CKDA_GATE_CKDA)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "gate_range %d is not a ckda_gate_t", d->gate_range);
  if (!valid_gate_input(d->gate_input))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "gate_input %d is not a ckda_gate_input_t",
                d->gate_input);
  if (!valid_qk_heads(d->H, d->qk_heads))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "qk_heads %d does not divide H=%d", d->qk_heads, d->H);
  if (d->sign_absorb != 0 && d->sign_absorb != 1)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "sign_absorb must be 0 or 1");
  if (d->use_qk_l2norm != 0 && d->use_qk_l2norm != 1)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "use_qk_l2norm must be 0 or 1");
  if (d->chunk_size != 16 && d->chunk_size != 32 && d->chunk_size != 64)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "chunk_size %d is not 16, 32 or 64", d->chunk_size);
  if (cu_seqlens) {
    if (d->B != 1)
      return fail(CKDA_ERR_INVALID_ARGUMENT, "cu_seqlens given with B=%d (must be 1)", d->B);
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
      return fail(CKDA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
  } else if (d->num_seqs != d->B) {
    return fail(CKDA_ERR_INVALID_ARGUMENT, "num_seqs=%d must equal B=%d without cu_seqlens",
                d->num_seqs, d->B);
  }
  const int64_t tokens = static_cast<int64_t>(d->B) * d->T;
  if (tokens > 0 && (passes & kPrepare) && (!q || !k || !alpha || !beta))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "q, k, alpha and beta must not be NULL");
  if (tokens > 0 && (passes & kFinish) && (!v || !o))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "v and o must not be NULL");
  const void* ptrs[] = {q, k, v, alpha, beta, h0, o, ht};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "h0", "o", "ht"};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(CKDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);

  const int64_t eb = elem_bytes(d->io_dtype);
  const int64_t gb = gate_bytes(d->gate_input);
  const int64_t hk = qk_heads_of(d->H, d->qk_heads);
  const int64_t state_bytes = static_cast<int64_t>(d->num_seqs) * d->H * d->dk * d->dv * 4;
  const Range ro = range("o", o, o ? tokens * d->H * d->dv * eb : 0);
  const Range ins[] = {range("q", q, q ? tokens * hk * d->dk * eb : 0),
                       range("k", k, k ? tokens * hk * d->dk * eb : 0),
                       range("v", v, v ? tokens * d->H * d->dv * eb : 0),
                       range("alpha", alpha, alpha ? tokens * d->H * d->dk * gb : 0),
                       range("beta", beta, beta ? tokens * d->H * gb : 0),
                       range("h0", h0, h0 ? state_bytes : 0),
                       range("ht", ht, ht ? state_bytes : 0),
                       range("cu_seqlens", cu_seqlens,
                             cu_seqlens ? 4 * (static_cast<int64_t>(d->num_seqs) + 1) : 0)};
  for (const Range& r : ins)
    if (overlap(ro, r)) return fail(CKDA_ERR_INVALID_ARGUMENT, "o overlaps %s", r.name);
  if (ht) {
    const Range rh = range("ht", ht, state_bytes);
    for (int i = 0; i < 5; ++i)
      if (overlap(rh, ins[i])) return fail(CKDA_ERR_INVALID_ARGUMENT, "ht overlaps %s", ins[i].name);
    if (h0 && h0 != ht && overlap(rh, ins[5]))
      return fail(CKDA_ERR_INVALID_ARGUMENT, "ht partially overlaps h0");
  }
  const size_t need = check_workspace ? ckda_chunk_fwd_workspace_size(d, cu_seqlens ? 1 : 0) : 0;
  if (need > 0) {
    if (!workspace)
      return fail(CKDA_ERR_INVALID_ARGUMENT, "workspace is NULL (%zu bytes needed)", need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(CKDA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(CKDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed",
                  workspace_bytes, need);
    const Range rw = range("workspace", workspace, static_cast<int64_t>(need));
    if (overlap(rw, ro)) return fail(CKDA_ERR_INVALID_ARGUMENT, "workspace overlaps o");
    for (const Range& r : ins)
      if (overlap(rw, r)) return fail(CKDA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
  }
  if (!ckda::fwd_supported(d->chunk_size, d->dk, d->dv, d->io_dtype))
    return fail(CKDA_ERR_UNSUPPORTED, "no chunked kernel for chunk_size=%d dk=%d dv=%d io_dtype=%d",
                d->chunk_size, d->dk, d->dv, d->io_dtype);
  return ok();
}

ckda_status_t run_fwd(const ckda_fwd_desc_t* d, const void* q, const void* k, const void* v,
                      const void* alpha, const void* beta, const int32_t* cu_seqlens,
                      const float* h0, void* o, float* ht, void* workspace, size_t workspace_bytes,
                      void* stream, int passes) {
  const ckda_status_t st = validate_fwd(d, q, k, v, alpha, beta, cu_seqlens, h0, o, ht,
                                        workspace, workspace_bytes, passes);
  if (st != CKDA_OK) return st;
  if (d->num_seqs == 0) return ok();
  ckda::FwdArgs a{d->B, d->T, d->H, d->dk, d->dv, d->num_seqs, d->chunk_size,
                  qk_heads_of(d->H, d->qk_heads), d->use_qk_l2norm, d->gate_range, d->gate_input,
                  d->sign_absorb, d->scale, q, k, v, alpha, beta,
                  cu_seqlens, h0, o, ht, nullptr, nullptr, nullptr, nullptr, 0, 0, 0};
  return from_hip(ckda::launch_fwd(a, d->io_dtype, workspace, static_cast<hipStream_t>(stream),
                                   (passes & kPrepare) != 0, (passes & kFinish) != 0));
}

// The backward takes the forward's inputs plus dout (in the place of o) and
// dht, and writes fp32 gradients.
ckda_status_t run_bwd(const ckda_fwd_desc_t* d, const void* q, const void* k, const void* v,
                      const void* alpha, const void* beta, const int32_t* cu_seqlens,
                      const float* h0, const void* dout, const float* dht, float* dq, float* dk,
                      float* dv, float* dalpha, float* dbeta, float* dh0, void* workspace,
                      size_t workspace_bytes, void* stream, bool recompute) {
  ckda_status_t st = validate_fwd(d, q, k, v, alpha, beta, cu_seqlens, h0, dout, nullptr, nullptr,
                                  0, kPrepare | kFinish, false);
  if (st != CKDA_OK) return st;
  if (d->sign_absorb != 0)
    return fail(CKDA_ERR_UNSUPPORTED, "the backward has no sign-absorption path");
  const int64_t tokens = static_cast<int64_t>(d->B) * d->T;
  if (tokens > 0 && (!dq || !dk || !dv || !dalpha || !dbeta))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "dq, dk, dv, dalpha and dbeta must not be NULL");
  const void* outp[] = {dq, dk, dv, dalpha, dbeta, dh0};
  const char* onames[] = {"dq", "dk", "dv", "dalpha", "dbeta", "dh0"};
  for (int i = 0; i < 6; ++i)
    if (outp[i] && !aligned16(outp[i]))
      return fail(CKDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", onames[i]);
  if (dht && !aligned16(dht)) return fail(CKDA_ERR_INVALID_ARGUMENT, "dht is not 16-byte aligned");
  const int64_t eb = elem_bytes(d->io_dtype), gb = gate_bytes(d->gate_input);
  const int32_t Hk = qk_heads_of(d->H, d->qk_heads);
  const int64_t state_bytes = static_cast<int64_t>(d->num_seqs) * d->H * d->dk * d->dv * 4;
  // q, k, dq, dk on the q/k heads; alpha, dalpha, beta, dbeta on the value heads
  const int64_t nqk = tokens * Hk * d->dk, na = tokens * d->H * d->dk, nv = tokens * d->H * d->dv;
  const Range outs[] = {range("dq", dq, dq ? 4 * nqk : 0), range("dk", dk, dk ? 4 * nqk : 0),
                        range("dv", dv, dv ? 4 * nv : 0), range("dalpha", dalpha, dalpha ? 4 * na : 0),
                        range("dbeta", dbeta, dbeta ? 4 * tokens * d->H : 0),
                        range("dh0", dh0, dh0 ? state_bytes : 0)};
  const Range ins[] = {range("q", q, q ? nqk * eb : 0), range("k", k, k ? nqk * eb : 0),
                       range("v", v, v ? nv * eb : 0), range("alpha", alpha, alpha ? gb * na : 0),
                       range("beta", beta, beta ? gb * tokens * d->H : 0),
                       range("h0", h0, h0 ? state_bytes : 0), range("dout", dout, dout ? nv * eb : 0),
                       range("dht", dht, dht ? state_bytes : 0),
                       range("cu_seqlens", cu_seqlens,
                             cu_seqlens ? 4 * (static_cast<int64_t>(d->num_seqs) + 1) : 0)};
  for (int i = 0; i < 6; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(CKDA_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, r.name);
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(CKDA_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  const size_t need = ckda_chunk_bwd_workspace_size(d, cu_seqlens ? 1 : 0);
  if (need > 0) {
    if (!workspace)
      return fail(CKDA_ERR_INVALID_ARGUMENT, "workspace is NULL (%zu bytes needed)", need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(CKDA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(CKDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed",
                  workspace_bytes, need);
    const Range rw = range("workspace", workspace, static_cast<int64_t>(need));
    for (const Range& r : ins)
      if (overlap(rw, r)) return fail(CKDA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
    for (const Range& r : outs)
      if (overlap(rw, r)) return fail(CKDA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
  }
  if (d->num_seqs == 0) return ok();
  ckda::BwdArgs b{};
  b.f = ckda::FwdArgs{d->B, d->T, d->H, d->dk, d->dv, d->num_seqs, d->chunk_size, Hk,
                      d->use_qk_l2norm, d->gate_range, d->gate_input, 0, d->scale, q, k, v,
                      alpha, beta, cu_seqlens, h0, nullptr, nullptr};
  b.dout = dout;
  b.dht = dht;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.dalpha = dalpha;
  b.dbeta = dbeta;
  b.dh0 = dh0;
  const size_t core = ckda::bwd_workspace_bytes(d->B, d->T, d->H, d->dk, d->dv, d->num_seqs,
                                                d->chunk_size, d->io_dtype, cu_seqlens != nullptr);
  return from_hip(ckda::launch_bwd_full(b, d->io_dtype, workspace, core,
                                        static_cast<hipStream_t>(stream), recompute));
}

// The forward that also keeps the backward's records in `saved` (laid out as
// the backward's workspace), for ckda_chunk_bwd_saved.
ckda_status_t run_fwd_save(const ckda_fwd_desc_t* d, const void* q, const void* k, const void* v,
                           const void* alpha, const void* beta, const int32_t* cu_seqlens,
                           const float* h0, void* o, float* ht, void* saved, size_t saved_bytes,
                           void* stream) {
  ckda_status_t st = validate_fwd(d, q, k, v, alpha, beta, cu_seqlens, h0, o, ht, nullptr, 0,
                                  kPrepare | kFinish, false);
  if (st != CKDA_OK) return st;
  if (d->sign_absorb != 0)
    return fail(CKDA_ERR_UNSUPPORTED, "the backward's records have no sign-absorption path");
  const int64_t tokens = static_cast<int64_t>(d->B) * d->T;
  const int64_t eb = elem_bytes(d->io_dtype), gb = gate_bytes(d->gate_input);
  const int32_t Hk = qk_heads_of(d->H, d->qk_heads);
  const int64_t state_bytes = static_cast<int64_t>(d->num_seqs) * d->H * d->dk * d->dv * 4;
  const int64_t nqk = tokens * Hk * d->dk, na = tokens * d->H * d->dk, nv = tokens * d->H * d->dv;
  const Range others[] = {range("q", q, q ? nqk * eb : 0), range("k", k, k ? nqk * eb : 0),
                          range("v", v, v ? nv * eb : 0), range("alpha", alpha, alpha ? gb * na : 0),
                          range("beta", beta, beta ? gb * tokens * d->H : 0),
                          range("h0", h0, h0 ? state_bytes : 0), range("o", o, o ? nv * eb : 0),
                          range("ht", ht, ht ? state_bytes : 0),
                          range("cu_seqlens", cu_seqlens,
                                cu_seqlens ? 4 * (static_cast<int64_t>(d->num_seqs) + 1) : 0)};
  const size_t need = ckda_chunk_bwd_workspace_size(d, cu_seqlens ? 1 : 0);
  if (need > 0) {
    if (!saved) return fail(CKDA_ERR_INVALID_ARGUMENT, "saved is NULL (%zu bytes needed)", need);
    if ((reinterpret_cast<uintptr_t>(saved) & 255u) != 0)
      return fail(CKDA_ERR_INVALID_ARGUMENT, "saved is not 256-byte aligned");
    if (saved_bytes < need)
      return fail(CKDA_ERR_WORKSPACE_TOO_SMALL, "saved has %zu bytes, %zu needed", saved_bytes, need);
    const Range rs = range("saved", saved, static_cast<int64_t>(need));
    for (const Range& r : others)
      if (overlap(rs, r)) return fail(CKDA_ERR_INVALID_ARGUMENT, "saved overlaps %s", r.name);
  }
  if (d->num_seqs == 0) return ok();
  ckda::FwdArgs a{d->B, d->T, d->H, d->dk, d->dv, d->num_seqs, d->chunk_size, Hk,
                  d->use_qk_l2norm, d->gate_range, d->gate_input, 0, d->scale, q, k, v, alpha,
                  beta, cu_seqlens, h0, o, ht, nullptr, nullptr, nullptr, nullptr, 0, 0, 0};
  return from_hip(ckda::launch_fwd_save(a, d->io_dtype, saved, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

ckda_status_t ckda_chunk_bwd(const ckda_fwd_desc_t* d, const void* q, const void* k,
                             const void* v, const void* alpha, const void* beta,
                             const int32_t* cu_seqlens, const float* h0, const void* dout,
                             const float* dht, float* dq, float* dk, float* dv, float* dalpha,
                             float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return run_bwd(d, q, k, v, alpha, beta, cu_seqlens, h0, dout, dht, dq, dk, dv, dalpha, dbeta,
                 dh0, workspace, workspace_bytes, stream, true);
}

ckda_status_t ckda_chunk_fwd_save(const ckda_fwd_desc_t* d, const void* q, const void* k,
                                  const void* v, const void* alpha, const void* beta,
                                  const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
                                  void* saved, size_t saved_bytes, void* stream) {
  return run_fwd_save(d, q, k, v, alpha, beta, cu_seqlens, h0, o, ht, saved, saved_bytes, stream);
}

ckda_status_t ckda_chunk_bwd_saved(const ckda_fwd_desc_t* d, const void* q, const void* k,
                                   const void* v, const void* alpha, const void* beta,
                                   const int32_t* cu_seqlens, const float* h0, const void* dout,
                                   const float* dht, float* dq, float* dk, float* dv,
                                   float* dalpha, float* dbeta, float* dh0, void* saved,
                                   size_t saved_bytes, void* stream) {
  return run_bwd(d, q, k, v, alpha, beta, cu_seqlens, h0, dout, dht, dq, dk, dv, dalpha, dbeta,
                 dh0, saved, saved_bytes, stream, false);
}

ckda_status_t ckda_chunk_fwd(const ckda_fwd_desc_t* d, const void* q, const void* k,
                             const void* v, const void* alpha, const void* beta,
                             const int32_t* cu_seqlens, const float* h0, void* o,
                             float* ht, void* workspace, size_t workspace_bytes, void* stream) {
  return run_fwd(d, q, k, v, alpha, beta, cu_seqlens, h0, o, ht, workspace, workspace_bytes,
                 stream, kPrepare | kFinish);
}

ckda_status_t ckda_chunk_fwd_noalloc(const ckda_fwd_desc_t* d, const void* q, const void* k,
                                     const void* v, const void* alpha, const void* beta,
                                     const int32_t* cu_seqlens, const float* h0, void* o,
                                     float* ht, void* stream) {
  if (!d) return fail(CKDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  // sizes first, on the host: a call whose workspace would not fit the
  // static scratch is refused before anything touches the GPU
  const size_t need = ckda_chunk_fwd_workspace_size(d, cu_seqlens ? 1 : 0);
  if (need > CKDA_NOALLOC_SCRATCH_BYTES)
    return fail(CKDA_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of scratch; the static scratch of "
                "ckda_chunk_fwd_noalloc holds %zu (use ckda_chunk_fwd with a workspace)",
                need, static_cast<size_t>(CKDA_NOALLOC_SCRATCH_BYTES));
  const ckda_status_t st = validate_fwd(d, q, k, v, alpha, beta, cu_seqlens, h0, o, ht, nullptr,
                                        0, kPrepare | kFinish, false);
  if (st != CKDA_OK) return st;
  if (d->num_seqs == 0 || need == 0) return ok();
  void* ws = nullptr;
  const hipError_t e = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess)
    return fail(CKDA_ERR_HIP, "looking up the static scratch failed: HIP error %d: %s",
                static_cast<int>(e), hipGetErrorString(e));
  return run_fwd(d, q, k, v, alpha, beta, cu_seqlens, h0, o, ht, ws, CKDA_NOALLOC_SCRATCH_BYTES,
                 stream, kPrepare | kFinish);
}

ckda_status_t ckda_chunk_fwd_prepare(const ckda_fwd_desc_t* d, const void* q, const void* k,
                                     const void* alpha, const void* beta,
                                     const int32_t* cu_seqlens, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return run_fwd(d, q, k, nullptr, alpha, beta, cu_seqlens, nullptr, nullptr, nullptr, workspace,
                 workspace_bytes, stream, kPrepare);
}

ckda_status_t ckda_chunk_fwd_finish(const ckda_fwd_desc_t* d, const void* v,
                                    const int32_t* cu_seqlens, const float* h0, void* o,
                                    float* ht, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return run_fwd(d, nullptr, nullptr, v, nullptr, nullptr, cu_seqlens, h0, o, ht, workspace,
                 workspace_bytes, stream, kFinish);
}

ckda_status_t ckda_recurrent_step(int32_t N, int32_t H, int32_t qk_heads, int32_t dk,
                                  int32_t dv, int32_t io_dtype, int32_t gate_range, int32_t gate_input,
                                  int32_t use_qk_l2norm, float scale, const void* q,
                                  const void* k, const void* v, const void* alpha,
                                  const void* beta, const float* h0,
                                  float* ht, void* o, void* stream) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "bad size: N=%d H=%d dk=%d dv=%d", N, H, dk, dv);
  if (io_dtype != CKDA_DTYPE_BF16 && io_dtype != CKDA_DTYPE_F32)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "io_dtype %d is not a ckda_dtype_t", io_dtype);
  if (gate_range != CKDA_GATE_KDA && gate_range != CKDA_GATE_CKDA)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "gate_range %d is not a ckda_gate_t", gate_range);
  if (!valid_gate_input(gate_input))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "gate_input %d is not a ckda_gate_input_t", gate_input);
  if (!valid_qk_heads(H, qk_heads))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "qk_heads %d does not divide H=%d", qk_heads, H);
  if (use_qk_l2norm != 0 && use_qk_l2norm != 1)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "use_qk_l2norm must be 0 or 1");
  if (N > 0 && (!q || !k || !v || !alpha || !beta || !h0 || !ht || !o))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "no pointer argument may be NULL");
  const void* ptrs[] = {q, k, v, alpha, beta, h0, ht, o};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "h0", "ht", "o"};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(CKDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  const int64_t nh = static_cast<int64_t>(N) * H;
  if (nh > (int64_t(1) << 21))  // one launch of up to 2048 work-items per (sequence, head)
    return fail(CKDA_ERR_UNSUPPORTED, "N*H = %lld exceeds 2^21 for one decode launch",
                static_cast<long long>(nh));
  const int64_t nhk = static_cast<int64_t>(N) * qk_heads_of(H, qk_heads);
  const int64_t eb = elem_bytes(io_dtype);
  const int64_t gb = gate_bytes(gate_input);
  const int64_t sb = nh * dk * dv * 4;
  const Range ro = range("o", o, nh * dv * eb);
  const Range rht = range("ht", ht, sb);
  const Range ins[] = {range("q", q, nhk * dk * eb), range("k", k, nhk * dk * eb),
                       range("v", v, nh * dv * eb), range("alpha", alpha, nh * dk * gb),
                       range("beta", beta, nh * gb), range("h0", h0, sb)};
  for (const Range& r : ins)
    if (overlap(ro, r)) return fail(CKDA_ERR_INVALID_ARGUMENT, "o overlaps %s", r.name);
  if (overlap(ro, rht)) return fail(CKDA_ERR_INVALID_ARGUMENT, "o overlaps ht");
  for (int i = 0; i < 5; ++i)
    if (overlap(rht, ins[i])) return fail(CKDA_ERR_INVALID_ARGUMENT, "ht overlaps %s", ins[i].name);
  if (h0 != ht && overlap(rht, ins[5]))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "ht partially overlaps h0");
  if (!ckda::step_supported(dk, dv))
    return fail(CKDA_ERR_UNSUPPORTED, "no decode kernel for dk=%d dv=%d", dk, dv);
  if (nh == 0) return ok();
  ckda::StepArgs a{N, H, dk, dv, qk_heads_of(H, qk_heads), use_qk_l2norm, gate_range, gate_input, scale, q, k, v,
                   alpha, beta, h0, ht, o};
  return from_hip(ckda::launch_step(a, io_dtype, static_cast<hipStream_t>(stream)));
}

ckda_status_t ckda_l2norm_debug(const void* x, float* y, int64_t rows, int32_t d,
                                int32_t dtype, void* stream) {
  if (rows < 0 || d <= 0 || d > 1024)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "bad size: rows=%lld d=%d",
                static_cast<long long>(rows), d);
  if (dtype != CKDA_DTYPE_BF16 && dtype != CKDA_DTYPE_F32)
    return fail(CKDA_ERR_INVALID_ARGUMENT, "dtype %d is not a ckda_dtype_t", dtype);
  if (rows > 0 && (!x || !y)) return fail(CKDA_ERR_INVALID_ARGUMENT, "x and y must not be NULL");
  if ((x && !aligned16(x)) || (y && !aligned16(y)))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned");
  if (overlap(range("x", x, rows * d * elem_bytes(dtype)), range("y", y, rows * d * 4)))
    return fail(CKDA_ERR_INVALID_ARGUMENT, "y overlaps x");
  if (rows == 0) return ok();
  return from_hip(ckda::launch_l2norm_debug(x, y, rows, d, dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
