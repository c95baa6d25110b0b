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
#include "readout_core.h"

namespace hwa {

constexpr int RO_TOK = 256;  // tokens per workgroup
constexpr int RO_TT = 16;    // tokens per inner tile

template <typename T, int D>
__global__ __launch_bounds__(256) void readout_kernel(
    const T* __restrict__ q, const T* __restrict__ gate,
    const float* __restrict__ decay, const int32_t* __restrict__ lohi,
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
  const int c = t / chunk;
  const int slot_p = max(0, c - radius);
  const int slot_q = min(nch, c + radius + 1);

  // decays a_t, b_t and row exponents
  const float* dct = decay + ((long long)bh * F + t) * 2 * D;
  const int32_t* ep = bank_e + ((long long)bh * (nch + 1) + slot_p) * D;
  const int32_t* eq = bank_e + (long long)BH * (nch + 1) * D +
                      ((long long)bh * (nch + 1) + slot_q) * D;
  for (int j = tid; j < D; j += 256) {
    dec[0][j] = dct[j];
    dec[1][j] = dct[D + j];
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
    const float inv = inv_l2(ss);
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
    const float rn = fast_rsq(sq / (float)D + eps_s);
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

// ---------------------------------------------------------------- bf16 S_t
// One workgroup per (b, h, t): the two gathered states' rows are brought to
// one power-of-two scale 2^E (the bank rows carry exponents), the bridge
// decays applied, then the whole matrix is scaled by 2^-k so that its largest
// entry lies in [2^14, 2^15): fp16 then keeps every entry down to 2^-28 of
// the largest with 11 significant bits, and the RMSNorm is unchanged when
// eps is scaled by 2^-2(E+k) as well (the scale-up is capped at 2^40 so that
// the scaled eps stays finite; an all-zero S_t keeps k = 0).
template <int D>
__global__ __launch_bounds__(256) void state_kernel(
    const float* __restrict__ decay, const float* __restrict__ bank_p,
    const float* __restrict__ bank_q, const int32_t* __restrict__ bank_e, float eps,
    _Float16* __restrict__ st, float* __restrict__ st_eps, int F, int chunk, int radius,
    int nch, int BH) {
  constexpr int NT = 256;
  constexpr int NX = D * D / (NT * 8);  // groups of eight columns per thread
  static_assert(D * D % (NT * 8) == 0, "whole groups");
  __shared__ float dec[2][D];
  __shared__ int rowexp[2][D];
  __shared__ int emax;
  __shared__ unsigned vmax;  // bits of the largest |entry| (a non-negative float)
  const int tid = threadIdx.x;
  const int t = blockIdx.x, bh = blockIdx.y;
  const int c = t / chunk;
  const int slot_p = max(0, c - radius);
  const int slot_q = min(nch, c + radius + 1);
  const float* dct = decay + ((long long)bh * F + t) * 2 * D;
  const int32_t* ep = bank_e + ((long long)bh * (nch + 1) + slot_p) * D;
  const int32_t* eq = bank_e + (long long)BH * (nch + 1) * D +
                      ((long long)bh * (nch + 1) + slot_q) * D;
  for (int j = tid; j < D; j += NT) {
    dec[0][j] = dct[j];
    dec[1][j] = dct[D + j];
    rowexp[0][j] = ep[j];
    rowexp[1][j] = eq[j];
  }
  if (tid == 0) {
    emax = INT32_MIN;
    vmax = 0u;
  }
  __syncthreads();
  if (tid < D) atomicMax(&emax, max(rowexp[0][tid], rowexp[1][tid]));
  __syncthreads();
  const int E = emax;
  const float* Pm = bank_p + ((long long)bh * (nch + 1) + slot_p) * D * D;
  const float* Qm = bank_q + ((long long)bh * (nch + 1) + slot_q) * D * D;
  float v[NX][8];
  float vm = 0.0f;
#pragma unroll
  for (int s = 0; s < NX; ++s) {
    const int x = (tid + s * NT) * 8;
    const int i = x / D, j = x % D;
    const float4 p0 = *(const float4*)&Pm[x], p1 = *(const float4*)&Pm[x + 4];
    const float4 q0 = *(const float4*)&Qm[x], q1 = *(const float4*)&Qm[x + 4];
    const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const int sp = rowexp[0][i] - E, sq = rowexp[1][i] - E;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[s][u] = ldexpf(pv[u], sp) * dec[0][j + u] + ldexpf(qv[u], sq) * dec[1][j + u];
      vm = fmaxf(vm, fabsf(v[s][u]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) vm = fmaxf(vm, __shfl_xor(vm, off));
  if ((tid & 63) == 0) atomicMax(&vmax, __float_as_uint(vm));
  __syncthreads();
  const float m = __uint_as_float(vmax);
  int k = 0;
  if (m > 0.0f) {
    int ex;
    frexpf(m, &ex);
    k = max(ex - 15, -40);
  }
  _Float16* dst = st + ((long long)bh * F + t) * D * D;
#pragma unroll
  for (int s = 0; s < NX; ++s) {
    const int x = (tid + s * NT) * 8;
    f16x8_t h8;
#pragma unroll
    for (int u = 0; u < 8; ++u) h8[u] = (_Float16)ldexpf(v[s][u], -k);
    *(f16x8_t*)&dst[x] = h8;
  }
  if (tid == 0) st_eps[(long long)bh * F + t] = ldexpf(eps, -2 * (E + k));
}

hipError_t launch_state(const Geom& g, const float* decay, const float* bank_p,
                        const float* bank_q, const int32_t* bank_e, float eps,
                        _Float16* st, float* st_eps, hipStream_t s) {
  dim3 grid(g.F, g.B * g.H);
#define ST_LAUNCH(DD)                                                             \
  hipLaunchKernelGGL(state_kernel<DD>, grid, dim3(256), 0, s, decay, bank_p, bank_q, \
                     bank_e, eps, st, st_eps, g.F, g.chunk, g.radius, g.nch, g.B * g.H)
  if (g.d == 128) ST_LAUNCH(128);
  else ST_LAUNCH(64);
#undef ST_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------- bf16 MFMA
// A workgroup takes up to 1024 tokens of one frame: it brings S_t into LDS,
// then each wave streams 32 tokens at a time, q of its next tokens loaded
// while the current ones go through the MFMAs (readout_core.h).
template <int D>
__global__ __launch_bounds__(256, 2) void readout_mfma_kernel(
    const bf16_t* __restrict__ q, ReadoutArgs a, int accumulate, bf16_t* __restrict__ out,
    int S, long long N, int tok_per_wg) {
  __shared__ ReadoutLds<D> L;
  const int tid = threadIdx.x;
  const int t = blockIdx.y;
  const int bh = blockIdx.z;
  const int tok0 = blockIdx.x * tok_per_wg;
  {
    StateChunks<D, 256> stc;
    stc.load(a.st + ((long long)bh * a.F + t) * D * D, tid);
    load_weight<D, 256>(L, a.rms_w, tid);
    stc.store(L, tid);
  }
  const float eps_s = a.st_eps[(long long)bh * a.F + t];
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int tok_end = min(S, tok0 + tok_per_wg);
  const bf16_t* qb = q + (long long)bh * N * D;
  const bf16_t* gb = a.gate + (long long)bh * N * D;
  bf16_t* ob = out + (long long)bh * N * D;
  struct KOff {
    static constexpr int at(int kk) { return kk * 16; }
  };
  const int qlane = half * 8;  // chunk kk of the lane half: channels 16 kk + 8 half + 0..7
  // q of this lane's token (channels 16*kk + 8*half + 0..7), one tile ahead
  u32x4_t qraw[D / 16];
  auto load_q = [&](int s0) {
    const int s = s0 + col;
    const long long n = (long long)t * S + s;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qraw[kk] = u32x4_t{0u, 0u, 0u, 0u};
      if (s < tok_end) qraw[kk] = *(const u32x4_t*)(qb + n * D + qlane + KOff::at(kk));
    }
  };
  load_q(tok0 + wave * 32);
  for (int s0 = tok0 + wave * 32; s0 < tok_end; s0 += 128) {
    const int s = s0 + col;
    const long long n = (long long)t * S + s;
    bf16_t* orow = ob + n * D;
    const bf16_t* grow = gb + n * D;
    readout_token<D, KOff>(
        L, eps_s, qraw, qlane, s < tok_end, orow,
        [&]() {
          if (s0 + 128 < tok_end) load_q(s0 + 128);
        },
        [&](int ib, int g4) { return *(const uint2*)(grow + ib * 32 + g4 * 8 + half * 4); },
        [&](int ib, int g4) {
          return accumulate ? *(const uint2*)(orow + ib * 32 + g4 * 8 + half * 4)
                            : make_uint2(0u, 0u);
        });
  }
}

// ---------------------------------------------------------------- decays
// a_t = prod_{j=lo_t..t} alpha_j and b_t = prod_{j=t..hi_t} alpha_j for every
// (b, h, t) and channel, in parallel (the readout then reads 2*d floats).
__global__ void decay_kernel(const float* __restrict__ alpha,
                             const int32_t* __restrict__ lohi,
                             float* __restrict__ decay, int F, int D) {
  const int t = blockIdx.x, bh = blockIdx.y;
  const int lo = lohi[t], hi = lohi[F + t];
  const float* al = alpha + (long long)bh * F * D;
  float* dst = decay + ((long long)bh * F + t) * 2 * D;
  for (int j = threadIdx.x; j < D; j += blockDim.x) {
    float a = 1.0f, b = 1.0f;
    for (int x = lo; x <= t; ++x) a *= al[(long long)x * D + j];
    for (int x = t; x <= hi; ++x) b *= al[(long long)x * D + j];
    dst[j] = a;
    dst[D + j] = b;
  }
}

hipError_t launch_decay(const Geom& g, const float* alpha, const int32_t* lohi,
                        float* decay, hipStream_t st) {
  hipLaunchKernelGGL(decay_kernel, dim3(g.F, g.B * g.H), dim3(g.d), 0, st,
                     alpha, lohi, decay, g.F, g.d);
  return hipGetLastError();
}

hipError_t launch_readout(const Geom& g, int dtype, const void* q,
                          const void* gate, const float* decay,
                          const int32_t* lohi, const float* bank_p,
                          const float* bank_q, const int32_t* bank_e,
                          const _Float16* st16, const float* st_eps,
                          const float* rms_weight, float rms_eps,
                          bool accumulate, void* out, hipStream_t st) {
  if (dtype == HWA_BF16) {
    // split each frame evenly into <= 1024-token pieces of whole 128-token tiles
    const int pieces = (g.S + 1023) / 1024;
    const int per = ((g.S + pieces - 1) / pieces + 127) / 128 * 128;
    dim3 grid((g.S + per - 1) / per, g.F, g.B * g.H);
    const ReadoutArgs ra{(const bf16_t*)gate, st16, st_eps, rms_weight, g.F};
#define RM_LAUNCH(DD)                                                        \
  hipLaunchKernelGGL(readout_mfma_kernel<DD>, grid, dim3(256), 0, st,        \
                     (const bf16_t*)q, ra, (int)accumulate, (bf16_t*)out, g.S, \
                     g.N, per)
    if (g.d == 128) RM_LAUNCH(128);
    else RM_LAUNCH(64);
#undef RM_LAUNCH
    return hipGetLastError();
  }
  dim3 grid((g.S + RO_TOK - 1) / RO_TOK, g.F, g.B * g.H);
#define RO_LAUNCH(TT, DD)                                                     \
  hipLaunchKernelGGL((readout_kernel<TT, DD>), grid, dim3(256), 0, st,        \
                     (const TT*)q, (const TT*)gate, decay, lohi, bank_p,      \
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
  RO_D(float)
#undef RO_D
#undef RO_LAUNCH
  return hipGetLastError();
}

}  // namespace hwa
