// Internal declarations shared by the HIP translation units of libhwa.
// gfx950 (CDNA4) only: wave64, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hwa.h"

namespace hwa {

typedef uint16_t bf16_t;  // bfloat16 storage

// Problem geometry shared by every kernel of one call.
struct Geom {
  int B, H, d, F, S, chunk, radius, nch;
  long long N;  // F * S
};

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(bf16_t, h);
}

template <typename T>
__device__ __forceinline__ float ld_io(const T* p, long long i);
template <>
__device__ __forceinline__ float ld_io<float>(const float* p, long long i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld_io<bf16_t>(const bf16_t* p, long long i) {
  return bf16_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void st_io(T* p, long long i, float x);
template <>
__device__ __forceinline__ void st_io<float>(float* p, long long i, float x) {
  p[i] = x;
}
template <>
__device__ __forceinline__ void st_io<bf16_t>(bf16_t* p, long long i, float x) {
  p[i] = f32_to_bf16(x);
}

__device__ __forceinline__ float silu_f(float x) {
  return x / (1.0f + __expf(-x));
}

__device__ __forceinline__ float sigmoid_f(float x) {
  return 1.0f / (1.0f + __expf(-x));
}

// Window of query frame t (article: chunk-aligned, radius chunks each side).
__device__ __forceinline__ void window_of(int t, int F, int chunk, int radius,
                                          int& lo, int& hi) {
  int c = t / chunk;
  int l = (c - radius) * chunk;
  int h = (c + radius + 1) * chunk - 1;
  lo = l < 0 ? 0 : l;
  hi = h > F - 1 ? F - 1 : h;
}

// ---------------------------------------------------------------- launchers
// Each returns hipGetLastError() after its launch(es).
hipError_t launch_window_table(const Geom& g, int32_t* lohi, hipStream_t st);

hipError_t launch_softmax(const Geom& g, int dtype, const void* q,
                          const void* k, const void* v, const bf16_t* v_t,
                          const int32_t* lohi, void* out, hipStream_t st);

hipError_t launch_vtranspose(const Geom& g, const bf16_t* v, bf16_t* v_t,
                             hipStream_t st);

// A_f, B_f of every (b, h, f). conv == false: text mode (no conv on k, raw v).
hipError_t launch_stats(const Geom& g, int dtype, const void* k,
                        const void* v, const float* beta, const float* conv_k,
                        const float* conv_v, bool conv, float* A, float* Bm,
                        hipStream_t st);

// G_f, C_f of the affine update S -> S G_f + C_f for every (b, h, f).
// alpha == NULL means alpha = 1. G may be NULL (not written).
hipError_t launch_factor(const Geom& g, int rule, float c, const float* A,
                         const float* Bm, const float* alpha, float* G,
                         float* C, hipStream_t st);

hipError_t launch_scan(const Geom& g, const float* G, const float* C,
                       const float* text_state, float text_scale,
                       float* bank_p, float* bank_q, int32_t* bank_e,
                       hipStream_t st);

hipError_t launch_readout(const Geom& g, int dtype, const void* q,
                          const void* gate, const float* alpha,
                          const int32_t* lohi, const float* bank_p,
                          const float* bank_q, const int32_t* bank_e,
                          const float* rms_weight, float rms_eps,
                          bool accumulate, void* out, hipStream_t st);

}  // namespace hwa
