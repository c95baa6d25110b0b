// Bidirectional frame scan of the linear branch (VDN-H3 article, "Step 4:
// bidirectional scan + boundary gather" and "Text state"):
//   prefix  P_{-1} = s0,  P_f = P_{f-1} G_f + C_f   for f = 0 .. F-1
//   suffix  Q_F    = s0,  Q_f = Q_{f+1} G_f + C_f   for f = F-1 .. 0
// with s0 = text_scale * S_text (zero without a text state) and (G_f, C_f)
// the affine form of the update rule. Only the states a window can gather
// are kept: bank slot m holds P_{min(F, m*chunk)-1} and Q_{min(F, m*chunk)}.
//
// The update right-multiplies the state, so its rows evolve independently:
// a workgroup owns 8 rows of one (b, h, direction) chain for the whole scan
// and never exchanges data with the other row blocks. G_f is staged in LDS
// once per step and shared by the workgroup's rows.
//
// Every state row carries a power-of-two exponent e (row = stored * 2^e).
// When a row's max |value| passes 2^64 it is rescaled by an exact power of
// two; C_f is scaled by 2^-e before it is added. This keeps a diverging
// sana_scaled scan finite in fp32 and is a no-op for the contracting rules.

#include "hwa_internal.h"

namespace hwa {

constexpr int SC_R = 8;  // state rows per workgroup

template <int D>
__global__ __launch_bounds__(256) void scan_kernel(
    const float* __restrict__ G, const float* __restrict__ C,
    const float* __restrict__ text_state, float text_scale,
    float* __restrict__ bank_p, float* __restrict__ bank_q,
    int32_t* __restrict__ bank_e, int F, int chunk, int nch, int BH) {
  constexpr int TPR = D / 4;  // threads per state row (4 columns each)
  __shared__ __attribute__((aligned(16))) float g_lds[D * D];
  __shared__ float s_lds[SC_R][D];

  const int tid = threadIdx.x;
  const int rb = blockIdx.x;   // row block
  const int dir = blockIdx.y;  // 0 prefix, 1 suffix
  const int bh = blockIdx.z;
  const int r = tid / TPR;
  const int j0 = (tid % TPR) * 4;
  const bool active = r < SC_R;
  const int row = rb * SC_R + r;

  float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int e = 0;
  if (active && text_state) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      s[q] = text_scale * text_state[((long long)bh * D + row) * D + j0 + q];
  }
  float* bank = dir == 0 ? bank_p : bank_q;
  int32_t* be = bank_e + (long long)dir * BH * (nch + 1) * D;

  auto store = [&](int slot) {
    if (!active) return;
    float* dst = bank + (((long long)bh * (nch + 1) + slot) * D + row) * D + j0;
    *(float4*)dst = make_float4(s[0], s[1], s[2], s[3]);
    if (j0 == 0) be[((long long)bh * (nch + 1) + slot) * D + row] = e;
  };
  store(dir == 0 ? 0 : nch);

  for (int i = 0; i < F; ++i) {
    const int f = dir == 0 ? i : F - 1 - i;
    const long long mo = ((long long)bh * F + f) * D * D;
    for (int x = tid; x < D * D / 4; x += 256)
      *(float4*)&g_lds[x * 4] = *(const float4*)&G[mo + (long long)x * 4];
    if (active) {
#pragma unroll
      for (int q = 0; q < 4; ++q) s_lds[r][j0 + q] = s[q];
    }
    __syncthreads();
    if (active) {
      float4 cv = *(const float4*)&C[mo + (long long)row * D + j0];
      float acc[4] = {ldexpf(cv.x, -e), ldexpf(cv.y, -e), ldexpf(cv.z, -e),
                      ldexpf(cv.w, -e)};
#pragma unroll 8
      for (int kk = 0; kk < D; ++kk) {
        const float sv = s_lds[r][kk];
        const float4 gv = *(const float4*)&g_lds[kk * D + j0];
        acc[0] = fmaf(sv, gv.x, acc[0]);
        acc[1] = fmaf(sv, gv.y, acc[1]);
        acc[2] = fmaf(sv, gv.z, acc[2]);
        acc[3] = fmaf(sv, gv.w, acc[3]);
      }
      float mx = fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])),
                       fmaxf(fabsf(acc[2]), fabsf(acc[3])));
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      if (mx > 0x1p64f) {
        int ex;
        frexpf(mx, &ex);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = ldexpf(acc[q], -ex);
        e += ex;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] = acc[q];
    }
    if (dir == 0) {
      if ((f + 1) % chunk == 0 || f + 1 == F) store((f + chunk) / chunk);
    } else {
      if (f % chunk == 0) store(f / chunk);
    }
    __syncthreads();
  }
}

hipError_t launch_scan(const Geom& g, const float* G, const float* C,
                       const float* text_state, float text_scale,
                       float* bank_p, float* bank_q, int32_t* bank_e,
                       hipStream_t st) {
  dim3 grid(g.d / SC_R, 2, g.B * g.H);
#define SCAN_LAUNCH(DD)                                                      \
  hipLaunchKernelGGL(scan_kernel<DD>, grid, dim3(256), 0, st, G, C,          \
                     text_state, text_scale, bank_p, bank_q, bank_e, g.F,    \
                     g.chunk, g.nch, g.B * g.H)
  switch (g.d) {
    case 16: SCAN_LAUNCH(16); break;
    case 32: SCAN_LAUNCH(32); break;
    case 64: SCAN_LAUNCH(64); break;
    default: SCAN_LAUNCH(128); break;
  }
#undef SCAN_LAUNCH
  return hipGetLastError();
}

}  // namespace hwa
