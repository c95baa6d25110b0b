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

// Hardware reciprocal / reciprocal square root / exp2 (about 1 ulp each);
// the IEEE-exact division and sqrt sequences are not needed anywhere here.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// x * sigmoid(x) = x / (1 + e^-x)
__device__ __forceinline__ float silu_f(float x) {
  return x * fast_rcp(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

__device__ __forceinline__ float sigmoid_f(float x) {
  return fast_rcp(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// 1 / max(||x||, 1e-12) from the squared norm
__device__ __forceinline__ float inv_l2(float ss) {
  return fast_rsq(fmaxf(ss, 1e-24f));
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

// Work-queue counters of the bf16 softmax kernel (one per XCD), kept in the
// workspace and zeroed by the window-table kernel, which runs first.
constexpr int HWA_SCHED_WORDS = 8;

// ---------------------------------------------------------------- launchers
// Each returns hipGetLastError() after its launch(es).
// The window table; also zeroes sched[0 .. HWA_SCHED_WORDS) when sched is not null.
hipError_t launch_window_table(const Geom& g, int32_t* lohi, hipStream_t st,
                               unsigned* sched = nullptr);

// Per-call inputs of the bf16 linear-branch readout (device pointers)
struct ReadoutArgs {
  const bf16_t* gate;
  const _Float16* st;    // [B*H, F, d, d] S_t of every frame, scaled (launch_state)
  const float* st_eps;   // [B*H, F] RMSNorm eps at that scale
  const float* rms_w;    // [d] or null (ones)
  int F;
  const bf16_t* q_raw;   // raw q when the softmax branch runs on a rotated q, else null
};

// S_t = P_{lo-1} diag(a_t) + Q_{hi+1} diag(b_t) of every (b, h, t) for the
// bf16 readouts: fp16, scaled by the power of two that puts its largest entry
// in [2^14, 2^15), and st_eps = eps at the same scale (bank_e holds the
// power-of-two exponents of the prefix bank rows, then the suffix's).
hipError_t launch_state(const Geom& g, const float* decay, const float* bank_p,
                        const float* bank_q, const int32_t* bank_e, float eps,
                        _Float16* st, float* st_eps, hipStream_t st_stream);

// fuse != null (bf16 only): the softmax kernel also adds the linear-branch
// readout y = RMSNorm(S_t q^) * sigmoid(gate) of its queries before it writes
// out (q^ from the softmax's own q, or from fuse->q_raw when that is set: the
// softmax then runs on a rotated q). sched (bf16 only): HWA_SCHED_WORDS
// counters, zero at launch (the kernel leaves them non-zero). lse (or null):
// [B*H, N] fp32 log-sum-exp of each query's scaled scores; sm_out (or null):
// o_sm alone, in the I/O dtype.
// Kept 128-key blocks of every (b, h, chunk, 256-query tile) for the routed
// softmax: count [B*H, nch, tiles], list [B*H, nch, tiles, nkb_max] (block
// indices relative to the window's first block, increasing).
struct RouteArgs {
  const int* count;
  const uint16_t* list;
  int nkb_max;
};

// route (bf16 only) != null: the block-sparse variant, on route's lists.
hipError_t launch_softmax(const Geom& g, int dtype, const void* q,
                          const void* k, const void* v, const bf16_t* v_t,
                          const int32_t* lohi, void* out, hipStream_t st,
                          const ReadoutArgs* fuse, unsigned* sched, float* lse,
                          void* sm_out, const RouteArgs* route = nullptr);

// Block means and kept-block lists of the routed softmax (route.hip), from
// the softmax branch's q, k (bf16); qmean [B*H, nch, tiles, d] and ksum
// [B*H, nch, pieces, d] fp32 are scratch.
hipError_t launch_route(const Geom& g, const bf16_t* q, const bf16_t* k, const int32_t* lohi,
                        float tau, float* qmean, float* ksum, int* sel_count,
                        uint16_t* sel_list, int nkb_max, hipStream_t st);
int route_tiles(const Geom& g);    // 256-query tiles per chunk
int route_pieces(const Geom& g);   // 128-key pieces per chunk
int route_blocks_max(const Geom& g);  // key blocks of a window, at most

hipError_t launch_vtranspose(const Geom& g, const bf16_t* v, bf16_t* v_t,
                             hipStream_t st);

// A_f, B_f of every (b, h, f). conv == false: text mode (no conv on k, raw v).
// v_t (bf16 calls with S % 4 == 0 only, else null): also writes the raw v
// transposed, [B*H][d][round_up64(N)] with zeros past N, as launch_vtranspose
// does.
hipError_t launch_stats(const Geom& g, int dtype, const void* k,
                        const void* v, const float* beta, const float* conv_k,
                        const float* conv_v, bool conv, float* A, float* Bm,
                        hipStream_t st, bf16_t* v_t = nullptr);

// M_f = (I + c2 A_f)^-1 for every (b, h, f) (Gauss-Jordan sweep, fp32).
hipError_t launch_inverse(const Geom& g, float c2, const float* A, float* M,
                          hipStream_t st);

// fp32 update matrices M_f: (I + c2 A_f)^-1 (invert), else I - c2 A_f
hipError_t launch_update_f32(const Geom& g, bool invert, float c2, const float* A, float* M,
                             hipStream_t st);

// bf16 calls: M_f = (I + c2 A_f)^-1 (invert) or M_f = I - c2 A_f (not invert),
// as hi and lo bf16 matrices in the bf16 scan's operand order, [B*H*F][2][d*d]
// (d = 64 or 128).
hipError_t launch_update_packed(const Geom& g, bool invert, float c2, const float* A,
                                bf16_t* packed, hipStream_t st);

// C = B M for every (b, h, f).
hipError_t launch_matmul_bm(const Geom& g, const float* Bm, const float* M,
                            float* C, hipStream_t st);

// Prefix/suffix scans; writes the chunk-boundary state banks.
hipError_t launch_scan(const Geom& g, int dtype, int rule, float c,
                       const float* A, const float* Bm, const float* M,
                       const float* alpha, const float* text_state,
                       float text_scale, float* bank_p, float* bank_q,
                       int32_t* bank_e, hipStream_t st);

// Per-frame forget gate alpha [B*H, F, d] = exp(-exp(a_log) softplus(mean_f(k) W + bias))
// (W: [H, d, d], input channel x output channel; bias, a_log: [H, d]).
hipError_t launch_frame_alpha(const Geom& g, int dtype, const void* k, const float* w,
                              const float* bias, const float* a_log, float* alpha,
                              hipStream_t st);

// The forward's bf16 scan on packed update matrices (launch_update_packed).
hipError_t launch_scan_packed(const Geom& g, int rule, float c, const bf16_t* Mp,
                              const float* Bm, const float* alpha, const float* text_state,
                              float text_scale, float* bank_p, float* bank_q,
                              int32_t* bank_e, hipStream_t st);

// The attention block's projections (bf16 MFMA). QKV: x [M = B*T, H*d] times
// W_qkv [3*H*d, H*d]^T into q, k, v [B, H, T, d] and the 3D-rotated qr, kr
// (S tokens per frame, grid_w latent columns, base theta). Output: the
// attention output att [B, H, T, d] read as [M, H*d], times W_o [H*d, H*d]^T
// into y [M, H*d]. M * H * d * 2 < 2^31.
hipError_t launch_gemm_qkv(const bf16_t* x, const bf16_t* w_qkv, int M, int T, int H, int d,
                           int S, int grid_w, float theta, bf16_t* q, bf16_t* k, bf16_t* v,
                           bf16_t* qr, bf16_t* kr, hipStream_t st);
hipError_t launch_gemm_out(const bf16_t* att, const bf16_t* w_o, int M, int T, int H, int d,
                           bf16_t* y, hipStream_t st);

// Bridge decays of every (b, h, t): prod_{j=lo..t} alpha_j, prod_{j=t..hi}.
hipError_t launch_decay(const Geom& g, const float* alpha, const int32_t* lohi,
                        float* decay, hipStream_t st);

// fp32: forms S_t itself from the banks; bf16: reads it from st / st_eps
// (launch_state) and ignores decay, banks and rms_eps.
hipError_t launch_readout(const Geom& g, int dtype, const void* q,
                          const void* gate, const float* decay,
                          const int32_t* lohi, const float* bank_p,
                          const float* bank_q, const int32_t* bank_e,
                          const _Float16* st16, const float* st_eps,
                          const float* rms_weight, float rms_eps,
                          bool accumulate, void* out, hipStream_t st);

// Backward of the softmax branch. delta = g . o_sm and lse2 = lse * log2(e)
// per query, [B*H, Np] (Np = N rounded up to 64, zeros past N).
hipError_t launch_bwd_prep(const Geom& g, int dtype, const void* o, const void* go,
                           const float* lse, float* delta, float* lse2, hipStream_t st);

// part 0: dq; part 1: dk and dv; from q, k, v, the upstream gradient go and
// the prep arrays.
hipError_t launch_softmax_bwd(const Geom& g, int dtype, int part, const void* q, const void* k,
                              const void* v, const void* go, const float* lse2,
                              const float* delta, const int32_t* lohi, void* dq, void* dk,
                              void* dv, hipStream_t st);

}  // namespace hwa

namespace hwa {

// ---------------------------------------------------------------- MFMA helpers
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// x ~= hi + lo with hi = bf16(x) and lo = bf16(x - hi): the split-bf16
// ("bf16x3") products hi*hi + hi*lo + lo*hi keep ~16 mantissa bits.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b,
                                           f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// C += A*B with both operands given as (hi, lo) pairs: three MFMAs.
__device__ __forceinline__ f32x16_t mfma32x3(bf16x8_t ah, bf16x8_t al,
                                             bf16x8_t bh, bf16x8_t bl,
                                             f32x16_t c) {
  c = mfma32(al, bh, c);
  c = mfma32(ah, bl, c);
  return mfma32(ah, bh, c);
}

}  // namespace hwa
