// Per-frame affine form of the delta-rule update (VDN-H3 article, "Step 3:
// delta-rule state update" and its rules table). Every rule maps the state
// as S -> S G_f + C_f:
//   vdn_solve    G = D M,          C = B M,    M = (I + A)^-1
//   vdn_scaled   G = D M,          C = c B M,  M = (I + c^2 A)^-1
//   sana_scaled  G = D (I - c^2 A), C = c B
// with D = diag(alpha_f) (alpha scales the state's key columns: S D). G and
// C do not depend on the state, so all frames are handled in parallel here
// and the sequential scan only multiplies by G_f and adds C_f.
//
// The exact inverse of the SPD matrix I + c~^2 A is formed in fp32 in LDS:
// Cholesky L L^T = I + c~^2 A, W = L^-1 by forward elimination, M = W^T W.
// One workgroup (256 threads) per (b, h, frame).

#include "hwa_internal.h"

namespace hwa {

template <int D>
__global__ __launch_bounds__(256) void factor_kernel(
    const float* __restrict__ A, const float* __restrict__ Bm,
    const float* __restrict__ alpha, float* __restrict__ G,
    float* __restrict__ C, int rule, float c, int F) {
  constexpr int LD = D + 1;
  constexpr int BS = D / 16;
  __shared__ float X[D * LD];
  __shared__ float Y[D * LD];

  const int tid = threadIdx.x;
  const long long mi = (long long)blockIdx.y * F + blockIdx.x;  // (bh, f)
  const float* Am = A + mi * D * D;
  const float* Bmm = Bm + mi * D * D;
  const float* al = alpha ? alpha + mi * D : nullptr;

  if (rule == HWA_RULE_SANA_SCALED) {
    const float c2 = c * c;
    for (int e = tid; e < D * D; e += 256) {
      int i = e / D, j = e % D;
      float ai = al ? al[i] : 1.0f;
      if (G) G[mi * D * D + e] = ai * ((i == j ? 1.0f : 0.0f) - c2 * Am[e]);
      C[mi * D * D + e] = c * Bmm[e];
    }
    return;
  }
  const float cc = rule == HWA_RULE_VDN_SCALED ? c : 1.0f;  // c~
  const float cb = rule == HWA_RULE_VDN_SCALED ? c : 1.0f;  // scale of B
  const float c2 = cc * cc;

  // X = I + c~^2 A ; Y = I
  for (int e = tid; e < D * D; e += 256) {
    int i = e / D, j = e % D;
    X[i * LD + j] = (i == j ? 1.0f : 0.0f) + c2 * Am[e];
    Y[i * LD + j] = (i == j ? 1.0f : 0.0f);
  }
  __syncthreads();

  // ---- Cholesky, right-looking, lower triangle of X
  for (int j = 0; j < D; ++j) {
    const float djj = sqrtf(X[j * LD + j]);
    for (int i = j + 1 + tid; i < D; i += 256) X[i * LD + j] = X[i * LD + j] / djj;
    __syncthreads();
    const int n = D - j - 1;
    for (int e = tid; e < n * n; e += 256) {
      int i = j + 1 + e / n, kk = j + 1 + e % n;
      if (kk <= i) X[i * LD + kk] -= X[i * LD + j] * X[kk * LD + j];
    }
    if (tid == 0) X[j * LD + j] = djj;
    __syncthreads();
  }

  // ---- W = L^-1 into Y (lower): forward elimination on [L | I]
  for (int j = 0; j < D; ++j) {
    const float ljj = X[j * LD + j];
    for (int kk = tid; kk <= j; kk += 256) Y[j * LD + kk] = Y[j * LD + kk] / ljj;
    __syncthreads();
    const int n = D - j - 1;
    for (int e = tid; e < n * (j + 1); e += 256) {
      int i = j + 1 + e / (j + 1), kk = e % (j + 1);
      Y[i * LD + kk] -= X[i * LD + j] * Y[j * LD + kk];
    }
    __syncthreads();
  }

  // ---- M = W^T W into X (Y's upper triangle is zero)
  const int ib = tid / 16, jb = tid % 16;
  {
    float acc[BS][BS];
#pragma unroll
    for (int a = 0; a < BS; ++a)
#pragma unroll
      for (int b = 0; b < BS; ++b) acc[a][b] = 0.0f;
    for (int kk = 0; kk < D; ++kk) {
      float wa[BS], wb[BS];
#pragma unroll
      for (int a = 0; a < BS; ++a) {
        wa[a] = Y[kk * LD + ib * BS + a];
        wb[a] = Y[kk * LD + jb * BS + a];
      }
#pragma unroll
      for (int a = 0; a < BS; ++a)
#pragma unroll
        for (int b = 0; b < BS; ++b) acc[a][b] = fmaf(wa[a], wb[b], acc[a][b]);
    }
    __syncthreads();  // every thread is done reading Y (W) and X (L)
#pragma unroll
    for (int a = 0; a < BS; ++a)
#pragma unroll
      for (int b = 0; b < BS; ++b) X[(ib * BS + a) * LD + jb * BS + b] = acc[a][b];
  }
  // B into Y
  for (int e = tid; e < D * D; e += 256) Y[(e / D) * LD + e % D] = Bmm[e];
  __syncthreads();

  // ---- G = D M, C = cb B M
  {
    float acc[BS][BS];
#pragma unroll
    for (int a = 0; a < BS; ++a)
#pragma unroll
      for (int b = 0; b < BS; ++b) acc[a][b] = 0.0f;
    for (int kk = 0; kk < D; ++kk) {
      float ba[BS], mb[BS];
#pragma unroll
      for (int a = 0; a < BS; ++a) {
        ba[a] = Y[(ib * BS + a) * LD + kk];
        mb[a] = X[kk * LD + jb * BS + a];
      }
#pragma unroll
      for (int a = 0; a < BS; ++a)
#pragma unroll
        for (int b = 0; b < BS; ++b) acc[a][b] = fmaf(ba[a], mb[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < BS; ++a) {
      const int i = ib * BS + a;
      const float ai = al ? al[i] : 1.0f;
#pragma unroll
      for (int b = 0; b < BS; ++b) {
        const int j = jb * BS + b;
        C[mi * D * D + (long long)i * D + j] = cb * acc[a][b];
        if (G) G[mi * D * D + (long long)i * D + j] = ai * X[i * LD + j];
      }
    }
  }
}

hipError_t launch_factor(const Geom& g, int rule, float c, const float* A,
                         const float* Bm, const float* alpha, float* G,
                         float* C, hipStream_t st) {
  dim3 grid(g.F, g.B * g.H);
#define FACTOR_LAUNCH(DD)                                                    \
  hipLaunchKernelGGL(factor_kernel<DD>, grid, dim3(256), 0, st, A, Bm, alpha, \
                     G, C, rule, c, g.F)
  switch (g.d) {
    case 16: FACTOR_LAUNCH(16); break;
    case 32: FACTOR_LAUNCH(32); break;
    case 64: FACTOR_LAUNCH(64); break;
    default: FACTOR_LAUNCH(128); break;
  }
#undef FACTOR_LAUNCH
  return hipGetLastError();
}

}  // namespace hwa
