// Device code shared by the bf16 readouts of the linear branch: the
// standalone readout kernel and the epilogue of the softmax kernel (VDN-H3
// article, "Step 4" bridge mechanism and "Step 5: readout and gating"):
//   S_t = P_{lo-1} diag(a_t) + Q_{hi+1} diag(b_t)
//   o_n = S_t q^_n,  q^_n = L2(SiLU(q_n))
//   y_n = o_n / sqrt(mean(o_n^2) + eps) * w * sigmoid(g_n),  out_n = addend_n + y_n
// o = S_t q^ runs as one fp16 MFMA product per step (v_mfma_f32_32x32x16_f16,
// fp32 accumulation). S_t sits in LDS as the A operand (rows = output
// channels), scaled by an exact power of two 2^-k that puts its largest entry
// in [2^14, 2^15): fp16 then holds every entry down to 2^-28 of the largest
// with 11 significant bits, and the RMSNorm is unchanged when eps is scaled
// by 2^-2k as well. Each lane forms q^ of one token in registers as the B
// operand (|q^| <= 1, so fp16 needs no scaling). The output block holds one
// token per lane, so the RMSNorm needs one exchange between the lane halves.

#pragma once

#include "hwa_internal.h"

namespace hwa {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// LDS working set of one S_t
template <int D>
struct ReadoutLds {
  static constexpr int SP = D + 8;  // padded row (fp16): 16-byte aligned rows
  _Float16 st[D * SP];
  float dec[2][D];
  int rowexp[2][D];
  float w[D];
  int emax;
  unsigned vmax;  // bits of the largest |entry| (a non-negative float)
};

// Forms S_t of frame t of head bh in L (every thread of the NT-thread
// workgroup calls it; it synchronises the workgroup). The two gathered
// states' rows are brought to one power-of-two scale 2^E, then the whole
// matrix to 2^-k; returns eps scaled by 2^-2(E+k) to match.
template <int D, int NT>
__device__ __forceinline__ float build_st(ReadoutLds<D>& L, const ReadoutArgs& a, int bh,
                                          int t, int tid) {
  constexpr int SP = ReadoutLds<D>::SP;
  constexpr int NX = D * D / (NT * 8);  // groups of eight columns per thread
  static_assert(D * D % (NT * 8) == 0, "whole groups");
  const int c = t / a.chunk;
  const int slot_p = max(0, c - a.radius);
  const int slot_q = min(a.nch, c + a.radius + 1);
  const float* dct = a.decay + ((long long)bh * a.F + t) * 2 * D;
  const int32_t* ep = a.bank_e + ((long long)bh * (a.nch + 1) + slot_p) * D;
  const int32_t* eq = a.bank_e + (long long)a.BH * (a.nch + 1) * D +
                      ((long long)bh * (a.nch + 1) + slot_q) * D;
  for (int j = tid; j < D; j += NT) {
    L.dec[0][j] = dct[j];
    L.dec[1][j] = dct[D + j];
    L.rowexp[0][j] = ep[j];
    L.rowexp[1][j] = eq[j];
    L.w[j] = a.rms_w ? a.rms_w[j] : 1.0f;
  }
  if (tid == 0) {
    L.emax = INT32_MIN;
    L.vmax = 0u;
  }
  __syncthreads();
  if (tid < D) atomicMax(&L.emax, max(L.rowexp[0][tid], L.rowexp[1][tid]));
  __syncthreads();
  const int E = L.emax;
  const float* Pm = a.bank_p + ((long long)bh * (a.nch + 1) + slot_p) * D * D;
  const float* Qm = a.bank_q + ((long long)bh * (a.nch + 1) + slot_q) * D * D;
  // entries in registers (eight consecutive columns per group) and their max
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
    const int sp = L.rowexp[0][i] - E, sq = L.rowexp[1][i] - E;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[s][u] = ldexpf(pv[u], sp) * L.dec[0][j + u] + ldexpf(qv[u], sq) * L.dec[1][j + u];
      vm = fmaxf(vm, fabsf(v[s][u]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) vm = fmaxf(vm, __shfl_xor(vm, off));
  if ((tid & 63) == 0) atomicMax(&L.vmax, __float_as_uint(vm));
  __syncthreads();
  // largest entry -> [2^14, 2^15); the scale-up is capped at 2^40 so that the
  // scaled eps stays finite (an all-zero S_t keeps k = 0)
  const float m = __uint_as_float(L.vmax);
  int k = 0;
  if (m > 0.0f) {
    int ex;
    frexpf(m, &ex);
    k = max(ex - 15, -40);
  }
#pragma unroll
  for (int s = 0; s < NX; ++s) {
    const int x = (tid + s * NT) * 8;
    f16x8_t h8;
#pragma unroll
    for (int u = 0; u < 8; ++u) h8[u] = (_Float16)ldexpf(v[s][u], -k);
    *(f16x8_t*)&L.st[(x / D) * SP + x % D] = h8;
  }
  __syncthreads();
  return ldexpf(a.eps, -2 * (E + k));
}

// y of this lane's token (lane % 32 of the calling wave; the wave must be
// converged): qraw[kk] holds raw q channels qlane + KOff::at(kk) + 0..7 (any
// permutation of the channels, applied to S_t's columns alike; qlane is the
// lane-dependent part, KOff::at a compile-time one). after_features() runs
// once qraw has been read for the last time (the caller may then overwrite
// it, e.g. with the next token's q). When `valid`, writes
// out[i] = addend(ib, g4) + y[i] for the lane's channels i = 32 ib + 8 g4 +
// 4 half + 0..3, with the gate pre-activations gate_at(ib, g4) and addend as
// four packed bf16 each.
template <int D, typename KOff, typename AfterF, typename GateAt, typename Addend>
__device__ __forceinline__ void readout_token(const ReadoutLds<D>& L, float eps_s,
                                              const u32x4_t (&qraw)[D / 16], int qlane,
                                              bool valid, bf16_t* orow, AfterF after_features,
                                              GateAt gate_at, Addend addend) {
  constexpr int SP = ReadoutLds<D>::SP;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  // q^ = L2(SiLU(q)): SiLU once into fp32 registers, the norm, then fp16 per
  // MFMA step
  float fq[D / 16][8];
  float ss = 0.0f;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w = qraw[kk][u];
      fq[kk][2 * u] = silu_f(__uint_as_float(w << 16));
      fq[kk][2 * u + 1] = silu_f(__uint_as_float(w & 0xffff0000u));
      ss = fmaf(fq[kk][2 * u], fq[kk][2 * u], fmaf(fq[kk][2 * u + 1], fq[kk][2 * u + 1], ss));
    }
  after_features();
  ss += __shfl_xor(ss, 32);
  const float inv = inv_l2(ss);
  f32x16_t acc[D / 32];
#pragma unroll
  for (int ib = 0; ib < D / 32; ++ib)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ib][r] = 0.0f;
  // S_t does not change across tokens: keep its operands in LDS (one lane
  // base, immediate offsets) rather than letting the compiler hoist them
  int ro_base = col * SP + qlane;
  asm volatile("" : "+v"(ro_base));
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    f16x8_t qh;
#pragma unroll
    for (int u = 0; u < 8; ++u) qh[u] = (_Float16)(fq[kk][u] * inv);
#pragma unroll
    for (int ib = 0; ib < D / 32; ++ib) {
      const f16x8_t as = *(const f16x8_t*)&L.st[ro_base + ib * 32 * SP + KOff::at(kk)];
      acc[ib] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as, qh, acc[ib], 0, 0, 0);
    }
  }
  float sq = 0.0f;
#pragma unroll
  for (int ib = 0; ib < D / 32; ++ib)
#pragma unroll
    for (int r = 0; r < 16; ++r) sq = fmaf(acc[ib][r], acc[ib][r], sq);
  sq += __shfl_xor(sq, 32);
  const float rn = fast_rsq(sq / (float)D + eps_s);
  if (!valid) return;
#pragma unroll
  for (int ib = 0; ib < D / 32; ++ib)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int i0 = ib * 32 + g4 * 8 + half * 4;
      const uint2 graw = gate_at(ib, g4);
      const uint2 oraw = addend(ib, g4);
      const uint32_t gw[2] = {graw.x, graw.y};
      const uint32_t ow[2] = {oraw.x, oraw.y};
      uint32_t res[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float y2[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int r = g4 * 4 + u * 2 + e2;
          const float gv = __uint_as_float(e2 ? (gw[u] & 0xffff0000u) : (gw[u] << 16));
          const float ov = __uint_as_float(e2 ? (ow[u] & 0xffff0000u) : (ow[u] << 16));
          y2[e2] = acc[ib][r] * rn * L.w[i0 + u * 2 + e2] * sigmoid_f(gv) + ov;
        }
        res[u] = (uint32_t)f32_to_bf16(y2[0]) | ((uint32_t)f32_to_bf16(y2[1]) << 16);
      }
      *(uint2*)(orow + i0) = make_uint2(res[0], res[1]);
    }
}

}  // namespace hwa
