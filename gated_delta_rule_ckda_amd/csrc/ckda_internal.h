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
  int32_t use_l2norm;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* h0;
  float* ht;
  void* o;
};
bool step_supported(int32_t dk, int32_t dv);
launch_result launch_step(const StepArgs& a, int32_t io_dtype, hipStream_t stream);

// Row normalisation test export.
launch_result launch_l2norm_debug(const void* x, float* y, int64_t rows,
                                  int32_t d, int32_t dtype, hipStream_t stream);

// Chunked forward.
struct FwdArgs {
  int32_t B, T, H, dk, dv, num_seqs, chunk;
  int32_t use_l2norm;
  int32_t gate_range;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const int32_t* cu_seqlens;
  const float* h0;
  void* o;
  float* ht;
};
bool fwd_supported(int32_t chunk, int32_t dk, int32_t dv, int32_t io_dtype);
launch_result launch_fwd(const FwdArgs& a, int32_t io_dtype, hipStream_t stream);

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

}  // namespace ckda
