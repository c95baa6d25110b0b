// Gather, readout, RMSNorm and output gate of the linear branch, added to
// the softmax output (VDN-H3 article, "Step 4" bridge mechanism and "Step 5:
// readout and gating"):
//   S_t = P_{lo-1} diag(a_t) + Q_{hi+1} diag(b_t),
//         a_t = prod_{j=lo..t} alpha_j,  b_t = prod_{j=t..hi} alpha_j
//   o_n = S_t q^_n,  q^_n = L2(SiLU(q_n))
//   y_n = o_n / sqrt(mean(o_n^2) + eps) * w * sigmoid(g_n)
//   out_n = (accumulate ? out_n : 0) + y_n
// A workgroup takes up to 256 tokens of one frame: it forms S_t once in LDS
// (with the bank rows' power-of-two exponents brought to one common scale E,
// and eps scaled by 2^-2E), then streams its tokens 16 at a time.

#include "hwa_internal.h"

namespace hwa {

constexpr int RO_TOK = 256;  // tokens per workgroup
constexpr int RO_TT = 16;    // tokens per inner tile

template <typename T, int D>
__global__ __launch_bounds__(256) void readout_kernel(
    const T* __restrict__ q, const T* __restrict__ gate,
    const float* __restrict__ alpha, const int32_t* __restrict__ lohi,
    const float* __restrict__ bank_p, const float* __restrict__ bank_q,
    const int32_t* __restrict__ bank_e, const float* __restrict__ rms_w,
    float eps, int accumulate, T* __restrict__ out, int F, int S, int chunk,
    int radius, int nch, int BH, long long N) {
  constexpr int LD = D + 1;
  constexpr int TPT = 256 / RO_TT;  // threads per token (16)
  constexpr int RPT = D / TPT;      // output rows per thread
  __shared__ float st_lds[D * LD];
  __shared__ float dec[2][D];
  __shared__ int rowexp[2][D];
  __shared__ float qh_lds[RO_TT][D + 1];
  __shared__ int emax_s;

  const int tid = threadIdx.x;
  const int t = blockIdx.y;   // frame
  const int bh = blockIdx.z;
  const int tok0 = blockIdx.x * RO_TOK;
  if (tok0 >= S) return;
  const int lo = lohi[t], hi = lohi[F + t];
  const int c = t / chunk;
  const int slot_p = max(0, c - radius);
  const int slot_q = min(nch, c + radius + 1);

  // decays a_t, b_t and row exponents
  const float* al = alpha + (long long)bh * F * D;
  const int32_t* ep = bank_e + ((long long)bh * (nch + 1) + slot_p) * D;
  const int32_t* eq = bank_e + (long long)BH * (nch + 1) * D +
                      ((long long)bh * (nch + 1) + slot_q) * D;
  for (int j = tid; j < D; j += 256) {
    float a = 1.0f, b = 1.0f;
    for (int x = lo; x <= t; ++x) a *= al[(long long)x * D + j];
    for (int x = t; x <= hi; ++x) b *= al[(long long)x * D + j];
    dec[0][j] = a;
    dec[1][j] = b;
    rowexp[0][j] = ep[j];
    rowexp[1][j] = eq[j];
  }
  if (tid == 0) emax_s = INT32_MIN;
  __syncthreads();
  if (tid < D) atomicMax(&emax_s, max(rowexp[0][tid], rowexp[1][tid]));
  __syncthreads();
  const int E = emax_s;
  const float* Pm = bank_p + ((long long)bh * (nch + 1) + slot_p) * D * D;
  const float* Qm = bank_q + ((long long)bh * (nch + 1) + slot_q) * D * D;
  for (int x = tid; x < D * D; x += 256) {
    int i = x / D, j = x % D;
    float pv = ldexpf(Pm[x], rowexp[0][i] - E) * dec[0][j];
    float qv = ldexpf(Qm[x], rowexp[1][i] - E) * dec[1][j];
    st_lds[i * LD + j] = pv + qv;
  }
  const float eps_s = ldexpf(eps, -2 * E);
  __syncthreads();

  const T* qb = q + (long long)bh * N * D;
  const T* gb = gate + (long long)bh * N * D;
  T* ob = out + (long long)bh * N * D;
  const int tt = tid / TPT;
  const int i0 = (tid % TPT) * RPT;
  const int tok_end = min(S, tok0 + RO_TOK);
  for (int s0 = tok0; s0 < tok_end; s0 += RO_TT) {
    const int s = s0 + tt;
    const bool valid = s < tok_end;
    const long long n = (long long)t * S + s;
    // q^ = L2(SiLU(q)) of this token; the thread loads RPT channels
    float qv[RPT];
    float ss = 0.0f;
#pragma unroll
    for (int a = 0; a < RPT; ++a) {
      qv[a] = valid ? silu_f(ld_io<T>(qb, n * D + i0 + a)) : 0.0f;
      ss = fmaf(qv[a], qv[a], ss);
    }
#pragma unroll
    for (int off = 1; off < TPT; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int a = 0; a < RPT; ++a) qh_lds[tt][i0 + a] = qv[a] * inv;
    __syncthreads();
    float o[RPT];
#pragma unroll
    for (int a = 0; a < RPT; ++a) o[a] = 0.0f;
    for (int j = 0; j < D; ++j) {
      const float x = qh_lds[tt][j];
#pragma unroll
      for (int a = 0; a < RPT; ++a) o[a] = fmaf(st_lds[(i0 + a) * LD + j], x, o[a]);
    }
    float sq = 0.0f;
#pragma unroll
    for (int a = 0; a < RPT; ++a) sq = fmaf(o[a], o[a], sq);
#pragma unroll
    for (int off = 1; off < TPT; off <<= 1) sq += __shfl_xor(sq, off);
    const float rn = 1.0f / sqrtf(sq / (float)D + eps_s);
    if (valid) {
#pragma unroll
      for (int a = 0; a < RPT; ++a) {
        const long long idx = n * D + i0 + a;
        const float w = rms_w ? rms_w[i0 + a] : 1.0f;
        float y = o[a] * rn * w * sigmoid_f(ld_io<T>(gb, idx));
        if (accumulate) y += ld_io<T>(ob, idx);
        st_io<T>(ob, idx, y);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_readout(const Geom& g, int dtype, const void* q,
                          const void* gate, const float* alpha,
                          const int32_t* lohi, const float* bank_p,
                          const float* bank_q, const int32_t* bank_e,
                          const float* rms_weight, float rms_eps,
                          bool accumulate, void* out, hipStream_t st) {
  dim3 grid((g.S + RO_TOK - 1) / RO_TOK, g.F, g.B * g.H);
#define RO_LAUNCH(TT, DD)                                                     \
  hipLaunchKernelGGL((readout_kernel<TT, DD>), grid, dim3(256), 0, st,        \
                     (const TT*)q, (const TT*)gate, alpha, lohi, bank_p,      \
                     bank_q, bank_e, rms_weight, rms_eps, (int)accumulate,    \
                     (TT*)out, g.F, g.S, g.chunk, g.radius, g.nch, g.B * g.H, \
                     g.N)
#define RO_D(TT)                        \
  switch (g.d) {                        \
    case 16: RO_LAUNCH(TT, 16); break;  \
    case 32: RO_LAUNCH(TT, 32); break;  \
    case 64: RO_LAUNCH(TT, 64); break;  \
    default: RO_LAUNCH(TT, 128); break; \
  }
  if (dtype == HWA_BF16) {
    RO_D(bf16_t)
  } else {
    RO_D(float)
  }
#undef RO_D
#undef RO_LAUNCH
  return hipGetLastError();
}

}  // namespace hwa
