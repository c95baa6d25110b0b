// Per-frame statistics of the linear branch with the NoPE features fused in
// (VDN-H3 article, "Step 1: NoPE features" and "Step 2: per-frame
// statistics A, B"):
//   k^ = L2(SiLU(conv_k(k))), v^ = conv_v(v)   (conv: depthwise, causal,
//        width 4, along the frame's token order, zero before the frame start)
//   A_f = sum_{n in f} beta_n k^_n k^_n^T,  B_f = sum_{n in f} beta_n v^_n k^_n^T
// One workgroup per (b, h, frame). Tokens stream through LDS 32 at a time;
// every thread owns a (d/16) x (d/16) block of A and of B in registers.
// Text mode (conv == false) forms k^ = L2(SiLU(k)) and v^ = v.

#include "hwa_internal.h"

namespace hwa {

constexpr int ST_TT = 32;  // tokens per LDS tile

template <typename T, int D>
__global__ __launch_bounds__(256) void stats_kernel(
    const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ conv_k,
    const float* __restrict__ conv_v, int conv, float* __restrict__ A,
    float* __restrict__ Bm, int F, int S, int H, long long N) {
  constexpr int TPT = 256 / ST_TT;  // threads per token (8)
  constexpr int CPT = D / TPT;      // channels per thread
  constexpr int BS = D / 16;        // accumulator block edge
  __shared__ float kh_lds[ST_TT][D + 4];
  __shared__ float kb_lds[ST_TT][D + 4];
  __shared__ float vb_lds[ST_TT][D + 4];

  const int tid = threadIdx.x;
  const int f = blockIdx.x;
  const int bh = blockIdx.y;
  const int h = bh % H;
  const T* kp = k + (long long)bh * N * D;
  const T* vp = v + (long long)bh * N * D;
  const float* bp = beta + (long long)bh * N;
  const long long n0 = (long long)f * S;

  // conv taps of this thread's channels
  const int tt = tid / TPT;
  const int ch0 = (tid % TPT) * CPT;
  float wk[CPT][4], wv[CPT][4];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wk[i][j] = conv ? conv_k[((long long)h * D + ch0 + i) * 4 + j] : (j == 0 ? 1.0f : 0.0f);
      wv[i][j] = conv ? conv_v[((long long)h * D + ch0 + i) * 4 + j] : (j == 0 ? 1.0f : 0.0f);
    }

  const int ib = tid / 16, jb = tid % 16;  // accumulator block (rows, cols)
  float accA[BS][BS], accB[BS][BS];
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) accA[a][b] = accB[a][b] = 0.0f;

  for (int s0 = 0; s0 < S; s0 += ST_TT) {
    const int s = s0 + tt;
    float kc[CPT], vc[CPT];
    float ss = 0.0f;
    float bt = 0.0f;
    if (s < S) {
      bt = bp[n0 + s];
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        float ak = 0.0f, av = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (s - j >= 0) {
            long long idx = (n0 + s - j) * D + ch0 + i;
            ak = fmaf(wk[i][j], ld_io<T>(kp, idx), ak);
            av = fmaf(wv[i][j], ld_io<T>(vp, idx), av);
          }
        }
        kc[i] = silu_f(ak);
        vc[i] = av;
        ss = fmaf(kc[i], kc[i], ss);
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) kc[i] = vc[i] = 0.0f;
    }
    // L2 norm over the token's d channels: TPT consecutive lanes
#pragma unroll
    for (int off = 1; off < TPT; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      float kh = kc[i] * inv;
      kh_lds[tt][ch0 + i] = kh;
      kb_lds[tt][ch0 + i] = bt * kh;
      vb_lds[tt][ch0 + i] = bt * vc[i];
    }
    __syncthreads();
#pragma unroll 4
    for (int t = 0; t < ST_TT; ++t) {
      float kr[BS], kbr[BS], vbr[BS];
#pragma unroll
      for (int a = 0; a < BS; ++a) {
        kbr[a] = kb_lds[t][ib * BS + a];
        vbr[a] = vb_lds[t][ib * BS + a];
        kr[a] = kh_lds[t][jb * BS + a];
      }
#pragma unroll
      for (int a = 0; a < BS; ++a)
#pragma unroll
        for (int b = 0; b < BS; ++b) {
          accA[a][b] = fmaf(kbr[a], kr[b], accA[a][b]);
          accB[a][b] = fmaf(vbr[a], kr[b], accB[a][b]);
        }
    }
    __syncthreads();
  }

  const long long mo = ((long long)bh * F + f) * D * D;
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) {
      long long e = mo + (long long)(ib * BS + a) * D + jb * BS + b;
      A[e] = accA[a][b];
      Bm[e] = accB[a][b];
    }
}

hipError_t launch_stats(const Geom& g, int dtype, const void* k,
                        const void* v, const float* beta, const float* conv_k,
                        const float* conv_v, bool conv, float* A, float* Bm,
                        hipStream_t st) {
  dim3 grid(g.F, g.B * g.H);
#define STATS_LAUNCH(TT, DD)                                                  \
  hipLaunchKernelGGL((stats_kernel<TT, DD>), grid, dim3(256), 0, st,          \
                     (const TT*)k, (const TT*)v, beta, conv_k, conv_v,        \
                     (int)conv, A, Bm, g.F, g.S, g.H, g.N)
#define STATS_D(TT)                        \
  switch (g.d) {                           \
    case 16: STATS_LAUNCH(TT, 16); break;  \
    case 32: STATS_LAUNCH(TT, 32); break;  \
    case 64: STATS_LAUNCH(TT, 64); break;  \
    default: STATS_LAUNCH(TT, 128); break; \
  }
  if (dtype == HWA_BF16) {
    STATS_D(bf16_t)
  } else {
    STATS_D(float)
  }
#undef STATS_D
#undef STATS_LAUNCH
  return hipGetLastError();
}

}  // namespace hwa
