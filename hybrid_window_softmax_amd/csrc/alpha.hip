// Per-frame forget gate of the linear branch (VDN-H3 article, "Step 3":
// D = diag(alpha), a per-channel gate in (0, 1) that the article's
// FrameKDAAlpha layer produces; the article gives no formula, so the gate is
// the stated form)
//   m_f = mean_{n in f} k_n,  z_f = m_f W + b,  alpha_f = exp(-exp(a) softplus(z_f))
// One workgroup per (b, h, frame): the frame's raw k rows are summed with
// 16-byte loads (a thread owns 16 / sizeof(T) channels of every RS-th row),
// the RS partial sums meet in LDS, then one thread per output channel forms
// z (W read column-wise across the threads: consecutive addresses), the
// softplus and the gate. HBM: k read once, alpha written once.

#include "hwa_internal.h"

namespace hwa {

template <typename T, int D>
__global__ __launch_bounds__(256) void frame_alpha_kernel(
    const T* __restrict__ k, const float* __restrict__ w, const float* __restrict__ bias,
    const float* __restrict__ a_log, float* __restrict__ alpha, int F, int S, int H,
    long long N) {
  constexpr int VEC = 16 / sizeof(T);  // channels per 16-byte load
  constexpr int TPR = D / VEC;         // threads per row
  constexpr int RS = 256 / TPR;        // rows summed in parallel
  static_assert(D % VEC == 0 && 256 % TPR == 0, "row split");
  __shared__ float part[RS][D + 1];
  __shared__ float m[D];

  const int tid = threadIdx.x;
  const int f = blockIdx.x;
  const int bh = blockIdx.y;
  const int h = bh % H;
  const int c0 = (tid % TPR) * VEC;
  const int r0 = tid / TPR;
  const T* kp = k + ((long long)bh * N + (long long)f * S) * D;

  float acc[VEC];
#pragma unroll
  for (int u = 0; u < VEC; ++u) acc[u] = 0.0f;
  for (int s = r0; s < S; s += RS) {
    const uint4 raw = *(const uint4*)(kp + (long long)s * D + c0);
    if constexpr (sizeof(T) == 2) {
      const uint32_t x[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[2 * u] += __uint_as_float(x[u] << 16);
        acc[2 * u + 1] += __uint_as_float(x[u] & 0xffff0000u);
      }
    } else {
      acc[0] += __uint_as_float(raw.x);
      acc[1] += __uint_as_float(raw.y);
      acc[2] += __uint_as_float(raw.z);
      acc[3] += __uint_as_float(raw.w);
    }
  }
#pragma unroll
  for (int u = 0; u < VEC; ++u) part[r0][c0 + u] = acc[u];
  __syncthreads();
  if (tid < D) {
    float t = 0.0f;
#pragma unroll 8
    for (int j = 0; j < RS; ++j) t += part[j][tid];
    m[tid] = t / (float)S;
  }
  __syncthreads();
  if (tid < D) {
    const float* wh = w + (long long)h * D * D;
    float z = bias[(long long)h * D + tid];
#pragma unroll 8
    for (int i = 0; i < D; ++i) z = fmaf(m[i], wh[(long long)i * D + tid], z);
    const float sp = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));  // softplus, no overflow
    alpha[((long long)bh * F + f) * D + tid] = expf(-expf(a_log[(long long)h * D + tid]) * sp);
  }
}

hipError_t launch_frame_alpha(const Geom& g, int dtype, const void* k, const float* w,
                              const float* bias, const float* a_log, float* alpha,
                              hipStream_t st) {
  dim3 grid(g.F, g.B * g.H);
#define FA_LAUNCH(TT, DD)                                                                \
  hipLaunchKernelGGL((frame_alpha_kernel<TT, DD>), grid, dim3(256), 0, st, (const TT*)k, w, \
                     bias, a_log, alpha, g.F, g.S, g.H, g.N)
#define FA_D(TT)                         \
  switch (g.d) {                         \
    case 16: FA_LAUNCH(TT, 16); break;   \
    case 32: FA_LAUNCH(TT, 32); break;   \
    case 64: FA_LAUNCH(TT, 64); break;   \
    default: FA_LAUNCH(TT, 128); break;  \
  }
  if (dtype == HWA_BF16) {
    FA_D(bf16_t)
  } else {
    FA_D(float)
  }
#undef FA_D
#undef FA_LAUNCH
  return hipGetLastError();
}

}  // namespace hwa
