// Device code shared by the bf16 readouts of the linear branch: the
// standalone readout kernel and the epilogue of the softmax kernel (VDN-H3
// article, "Step 5: readout and gating"):
//   o_n = S_t q^_n,  q^_n = L2(SiLU(q_n))
//   y_n = o_n / sqrt(mean(o_n^2) + eps) * w * sigmoid(g_n),  out_n = addend_n + y_n
// S_t comes ready from state_kernel (fp16, scaled by a power of two, with eps
// scaled to match). o = S_t q^ runs as one fp16 MFMA product per step
// (v_mfma_f32_32x32x16_f16, fp32 accumulation): S_t sits in LDS as the A
// operand (rows = output channels); each lane forms q^ of one token in
// registers as the B operand (|q^| <= 1, so fp16 needs no scaling). The
// output block holds one token per lane, so the RMSNorm needs one exchange
// between the lane halves.

#pragma once

#include "hwa_internal.h"

namespace hwa {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// LDS working set of one S_t
template <int D>
struct ReadoutLds {
  static constexpr int SP = D + 8;  // padded row (fp16): 16-byte aligned rows
  _Float16 st[D * SP];
  float w[D];
};

// S_t of one frame (fp16, row-major d x d as state_kernel writes it) on its
// way from global memory to LDS: each of the NT threads of the workgroup
// holds NCH 16-byte chunks, loaded with one 1 KB run per wave instruction.
template <int D, int NT>
struct StateChunks {
  static constexpr int NCH = D * D / 8 / NT;
  static_assert(D * D / 8 % NT == 0, "whole chunks per thread");
  u32x4_t c[NCH];
  __device__ __forceinline__ void load(const _Float16* src, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) c[i] = *(const u32x4_t*)(src + (i * NT + tid) * 8);
  }
  __device__ __forceinline__ void store(ReadoutLds<D>& L, int tid) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int x = (i * NT + tid) * 8;
      *(u32x4_t*)&L.st[(x / D) * ReadoutLds<D>::SP + x % D] = c[i];
    }
  }
};

// RMSNorm weight into L (every thread of the NT-thread workgroup calls it)
template <int D, int NT>
__device__ __forceinline__ void load_weight(ReadoutLds<D>& L, const float* rms_w, int tid) {
  for (int j = tid; j < D; j += NT) L.w[j] = rms_w ? rms_w[j] : 1.0f;
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
