// Bidirectional frame scan of the linear branch (VDN-H3 article, "Step 4:
// bidirectional scan + boundary gather" and "Text state"):
//   prefix  P_{-1} = s0,  P_f = R_f(P_{f-1})   for f = 0 .. F-1
//   suffix  Q_F    = s0,  Q_f = R_f(Q_{f+1})   for f = F-1 .. 0
// with s0 = text_scale * S_text (zero without a text state). Every update
// rule of the rules table is one step
//   X = S diag(alpha_f) + c1 B_f,   R_f(S) = X M_f + c2 B_f
//   vdn_solve    c1 = 1, c2 = 0, M_f = (I + A_f)^-1
//   vdn_scaled   c1 = c, c2 = 0, M_f = (I + c^2 A_f)^-1
//   sana_scaled  c1 = 0, c2 = c, M_f = I - c^2 A_f (formed here from A_f)
// Only the states a window can gather are kept: bank slot m holds
// P_{min(F, m*chunk)-1} and Q_{min(F, m*chunk)}.
//
// The update right-multiplies the state, so its rows evolve independently:
// a workgroup owns 8 rows of one (b, h, direction) chain for the whole scan
// and never exchanges data with the other row blocks. M_f is staged in LDS
// once per step and shared by the workgroup's rows (fp32 throughout).
//
// Every state row carries a power-of-two exponent e (row = stored * 2^e).
// When a row's max |value| passes 2^64 it is rescaled by an exact power of
// two, and B_f enters scaled by 2^-e. This keeps a diverging sana_scaled scan
// finite in fp32 and is a no-op for the contracting rules.

#include "hwa_internal.h"

namespace hwa {

constexpr int SC_R = 8;  // state rows per workgroup

template <int D>
__global__ __launch_bounds__(256) void scan_kernel(
    const float* __restrict__ Am, const float* __restrict__ Bm,
    const float* __restrict__ Mi, const float* __restrict__ alpha, int rule,
    float c, const float* __restrict__ text_state, float text_scale,
    float* __restrict__ bank_p, float* __restrict__ bank_q,
    int32_t* __restrict__ bank_e, int F, int chunk, int nch, int BH) {
  constexpr int TPR = D / 4;  // threads per state row (4 columns each)
  __shared__ __attribute__((aligned(16))) float g_lds[D * D];
  __shared__ float x_lds[SC_R][D];

  const int tid = threadIdx.x;
  const int rb = blockIdx.x;   // row block
  const int dir = blockIdx.y;  // 0 prefix, 1 suffix
  const int bh = blockIdx.z;
  const int r = tid / TPR;
  const int j0 = (tid % TPR) * 4;
  const bool active = r < SC_R;
  const int row = rb * SC_R + r;
  const bool sana = rule == HWA_RULE_SANA_SCALED;
  const float c1 = sana ? 0.0f : (rule == HWA_RULE_VDN_SCALED ? c : 1.0f);
  const float c2 = sana ? c : 0.0f;
  const float cs = c * c;

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
    if (sana) {
      for (int x = tid; x < D * D / 4; x += 256) {
        const float4 a4 = *(const float4*)&Am[mo + (long long)x * 4];
        const int kk = (x * 4) / D, jj = (x * 4) % D;
        float4 g4 = make_float4(-cs * a4.x, -cs * a4.y, -cs * a4.z, -cs * a4.w);
        if (kk >= jj && kk < jj + 4) (&g4.x)[kk - jj] += 1.0f;
        *(float4*)&g_lds[x * 4] = g4;
      }
    } else {
      for (int x = tid; x < D * D / 4; x += 256)
        *(float4*)&g_lds[x * 4] = *(const float4*)&Mi[mo + (long long)x * 4];
    }
    float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (active) {
      const float4 b4 = *(const float4*)&Bm[mo + (long long)row * D + j0];
      const float4 a4 = *(const float4*)&alpha[((long long)bh * F + f) * D + j0];
      bv[0] = ldexpf(b4.x, -e);
      bv[1] = ldexpf(b4.y, -e);
      bv[2] = ldexpf(b4.z, -e);
      bv[3] = ldexpf(b4.w, -e);
      x_lds[r][j0 + 0] = fmaf(c1, bv[0], s[0] * a4.x);
      x_lds[r][j0 + 1] = fmaf(c1, bv[1], s[1] * a4.y);
      x_lds[r][j0 + 2] = fmaf(c1, bv[2], s[2] * a4.z);
      x_lds[r][j0 + 3] = fmaf(c1, bv[3], s[3] * a4.w);
    }
    __syncthreads();
    if (active) {
      float acc[4] = {c2 * bv[0], c2 * bv[1], c2 * bv[2], c2 * bv[3]};
#pragma unroll 8
      for (int kk = 0; kk < D; ++kk) {
        const float xv = x_lds[r][kk];
        const float4 gv = *(const float4*)&g_lds[kk * D + j0];
        acc[0] = fmaf(xv, gv.x, acc[0]);
        acc[1] = fmaf(xv, gv.y, acc[1]);
        acc[2] = fmaf(xv, gv.z, acc[2]);
        acc[3] = fmaf(xv, gv.w, acc[3]);
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

// ---------------------------------------------------------------- bf16 path
// Same recurrence on MFMA (v_mfma_f32_32x32x16_bf16, split-bf16 operands:
// hi*hi + hi*lo + lo*hi, about 16 mantissa bits per product; the state stays
// fp32). A workgroup owns 32 state rows of one (b, h, direction) chain for
// the whole scan; wave w owns the 32 x 32 output block of columns 32w..32w+31
// and holds it in the MFMA accumulator layout (lane: column lane % 32, rows
// 8*(r/4) + 4*(lane/32) + r%4). Per frame:
//   X = S diag(alpha) + c1 2^-e B  -> split to bf16 (hi, lo) in LDS (double
//   buffered);
//   M_f -> split to bf16 (hi, lo) in LDS: every thread splits the part it
//   read, one frame ahead, with loads where each instruction covers 1 KB of
//   consecutive memory (a per-lane row read touched 64 cache lines per
//   instruction and left the step waiting on the vector memory pipeline);
//   S = X M (+ c2 2^-e B): A operand = rows of X, B operand = rows of M (M is
//   symmetric, so row n is the needed column n), both from LDS; the three
//   partial products accumulate separately so the MFMAs do not wait on each
//   other.
// Two barriers per frame: X and M visible; everyone done reading M.
// Row exponents (diverging sana_scaled only, SANA = true): the row max over
// all d columns is combined across waves through LDS.
template <int D, bool SANA>
__global__ __launch_bounds__(2 * D) void scan_mfma_kernel(
    const float* __restrict__ Msrc, const float* __restrict__ Bm,
    const float* __restrict__ alpha, float c1, float c2, float cs,
    const float* __restrict__ text_state, float text_scale,
    float* __restrict__ bank_p, float* __restrict__ bank_q,
    int32_t* __restrict__ bank_e, int F, int chunk, int nch, int BH) {
  constexpr int NT = 2 * D;    // threads
  constexpr int XP = D + 8;    // padded X / M row (bf16)
  constexpr int MV = D * D / 4 / NT;  // float4 of M per thread and frame
  __shared__ __attribute__((aligned(16))) bf16_t x_hi[2][32 * XP];
  __shared__ __attribute__((aligned(16))) bf16_t x_lo[2][32 * XP];
  __shared__ __attribute__((aligned(16))) bf16_t m_hi[D * XP];
  __shared__ __attribute__((aligned(16))) bf16_t m_lo[D * XP];
  __shared__ unsigned rmax[2][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int rb = blockIdx.x;   // 32-row block
  const int dir = blockIdx.y;  // 0 prefix, 1 suffix
  const int bh = blockIdx.z;
  const int n = wave * 32 + col;  // this lane's state column
  // rows of accumulator register r: 8*(r/4) + 4*half + r%4 (within the block)
  auto rowof = [&](int r) { return 8 * (r / 4) + 4 * half + (r % 4); };

  float sv[16];
  int e[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = rb * 32 + rowof(r);
    sv[r] = text_state ? text_scale * text_state[((long long)bh * D + row) * D + n] : 0.0f;
    e[r] = 0;
  }
  if (tid < 32) rmax[0][tid] = rmax[1][tid] = 0u;  // published by the first barrier
  float* bank = dir == 0 ? bank_p : bank_q;
  int32_t* be = bank_e + (long long)dir * BH * (nch + 1) * D;
  auto store = [&](int slot) {
    float* dst = bank + ((long long)bh * (nch + 1) + slot) * D * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(long long)(rb * 32 + rowof(r)) * D + n] = sv[r];
    if (wave == 0 && col == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        be[((long long)bh * (nch + 1) + slot) * D + rb * 32 + rowof(r)] = e[r];
    }
  };
  store(dir == 0 ? 0 : nch);

  // the next frame, read ahead: M_f in consecutive float4 (element 4*(j*NT +
  // tid) .. +3 in mraw[j]), this block's B rows, alpha
  float4 mraw[MV];
  float braw[16], anext;
  auto fetch = [&](int f) {
    const long long mo = ((long long)bh * F + f) * D * D;
    const float4* m4 = (const float4*)(Msrc + mo);
#pragma unroll
    for (int j = 0; j < MV; ++j) mraw[j] = m4[j * NT + tid];
#pragma unroll
    for (int r = 0; r < 16; ++r) braw[r] = Bm[mo + (long long)(rb * 32 + rowof(r)) * D + n];
    anext = alpha[((long long)bh * F + f) * D + n];
  };
  // this thread's part of the M operand (hi, lo) -> LDS
  auto put_m = [&]() {
#pragma unroll
    for (int j = 0; j < MV; ++j) {
      const int el = 4 * (j * NT + tid);
      const int r = el / D, c = el % D;
      const float mv[4] = {mraw[j].x, mraw[j].y, mraw[j].z, mraw[j].w};
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t h4, l4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float m = SANA ? ((r == c + u ? 1.0f : 0.0f) - cs * mv[u]) : mv[u];
        __bf16 h, l;
        split_bf16(m, h, l);
        h4[u] = h;
        l4[u] = l;
      }
      *(bf16x4_t*)&m_hi[r * XP + c] = h4;
      *(bf16x4_t*)&m_lo[r * XP + c] = l4;
    }
  };
  fetch(dir == 0 ? 0 : F - 1);

  for (int i = 0; i < F; ++i) {
    const int f = dir == 0 ? i : F - 1 - i;
    const int buf = i & 1;
    // ---- X = S diag(alpha) + c1 2^-e B (own block) -> LDS (hi, lo)
    float bcur[16];
    const float acur = anext;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      bcur[r] = ldexpf(braw[r], -e[r]);
      const float x = fmaf(c1, bcur[r], sv[r] * acur);
      __bf16 h, l;
      split_bf16(x, h, l);
      x_hi[buf][rowof(r) * XP + n] = __builtin_bit_cast(bf16_t, h);
      x_lo[buf][rowof(r) * XP + n] = __builtin_bit_cast(bf16_t, l);
    }
    // ---- this frame's M operand -> LDS (the previous frame's readers are
    // done: barrier at the end of the last step); then fetch the next frame
    put_m();
    if (i + 1 < F) fetch(dir == 0 ? f + 1 : f - 1);
    __syncthreads();
    // ---- S = X M (+ c2 2^-e B), the three split products on their own
    // accumulators
    f32x16_t acc, acc1, acc2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[r] = c2 * bcur[r];
      acc1[r] = 0.0f;
      acc2[r] = 0.0f;
    }
    const bf16_t* xh = &x_hi[buf][col * XP + half * 8];
    const bf16_t* xl = &x_lo[buf][col * XP + half * 8];
    const bf16_t* mh = &m_hi[n * XP + half * 8];
    const bf16_t* ml = &m_lo[n * XP + half * 8];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8_t ah = *(const bf16x8_t*)(xh + kk * 16);
      const bf16x8_t al = *(const bf16x8_t*)(xl + kk * 16);
      const bf16x8_t bh = *(const bf16x8_t*)(mh + kk * 16);
      const bf16x8_t bl = *(const bf16x8_t*)(ml + kk * 16);
      acc = mfma32(ah, bh, acc);
      acc1 = mfma32(ah, bl, acc1);
      acc2 = mfma32(al, bh, acc2);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = acc[r] + (acc1[r] + acc2[r]);
    __syncthreads();  // M and this X buffer are read: free for the next frame
    if (SANA) {
      // rows are renormalised only when some entry passed 2^64 (every dozen
      // frames or so at 1,560 tokens per frame): the row maxima are gathered
      // only then
      bool big = false;
#pragma unroll
      for (int r = 0; r < 16; ++r) big |= fabsf(sv[r]) > 0x1p64f;
      if (__syncthreads_or(big)) {
        // row max |S| over all columns: 32 lanes of a half, then the waves
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float m = fabsf(sv[r]);
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
          if (col == 0) atomicMax(&rmax[buf][rowof(r)], __float_as_uint(m));
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float m = __uint_as_float(rmax[buf][rowof(r)]);
          if (m > 0x1p64f) {
            int ex;
            frexpf(m, &ex);
            sv[r] = ldexpf(sv[r], -ex);
            e[r] += ex;
          }
        }
      }
      if (tid < 32) rmax[buf ^ 1][tid] = 0u;  // cleared for the next frame
    }
    if (dir == 0) {
      if ((f + 1) % chunk == 0 || f + 1 == F) store((f + chunk) / chunk);
    } else {
      if (f % chunk == 0) store(f / chunk);
    }
  }
}

// ---------------------------------------------------------------- bf16 path,
// update matrices packed by launch_update_packed
// The forward's bf16 scan. M_f (or I - c^2 A_f for sana_scaled) arrives as
// hi and lo bf16 matrices already in MFMA operand order: wave w's B operand
// of step kk is one contiguous 1 KB block per part, which every lane loads
// straight into registers (16 bytes each), one frame ahead. Only X goes
// through LDS. Per frame:
//   X = S diag(alpha) + c1 2^-e B (own 32 x 32 block) -> split to bf16 (hi,
//   lo) -> LDS (double buffered); one barrier;
//   S = X M (+ c2 2^-e B): A operand = rows of X from LDS, B operand = the
//   registers; the three split products (hi*hi, hi*lo, lo*hi) on separate
//   accumulators.
// A write of X buffer b in frame i + 2 cannot overtake a read of it in frame
// i: every wave passes frame i + 1's barrier after its frame-i reads.
// Row exponents (SANA, the diverging rule): as in scan_mfma_kernel.
template <int D, bool SANA>
__global__ __launch_bounds__(2 * D) void scan_packed_kernel(
    const bf16_t* __restrict__ Mp, const float* __restrict__ Bm,
    const float* __restrict__ alpha, float c1, float c2,
    const float* __restrict__ text_state, float text_scale,
    float* __restrict__ bank_p, float* __restrict__ bank_q,
    int32_t* __restrict__ bank_e, int F, int chunk, int nch, int BH) {
  constexpr int XP = D + 8;    // padded X row (bf16)
  constexpr int KK = D / 16;   // MFMA steps over the contraction
  __shared__ __attribute__((aligned(16))) bf16_t x_hi[2][32 * XP];
  __shared__ __attribute__((aligned(16))) bf16_t x_lo[2][32 * XP];
  __shared__ unsigned rmax[2][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int rb = blockIdx.x;   // 32-row block
  const int dir = blockIdx.y;  // 0 prefix, 1 suffix
  const int bh = blockIdx.z;
  const int n = wave * 32 + col;  // this lane's state column
  auto rowof = [&](int r) { return 8 * (r / 4) + 4 * half + (r % 4); };

  float sv[16];
  int e[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = rb * 32 + rowof(r);
    sv[r] = text_state ? text_scale * text_state[((long long)bh * D + row) * D + n] : 0.0f;
    e[r] = 0;
  }
  if (SANA && tid < 32) rmax[0][tid] = rmax[1][tid] = 0u;  // published by the first barrier
  float* bank = dir == 0 ? bank_p : bank_q;
  int32_t* be = bank_e + (long long)dir * BH * (nch + 1) * D;
  auto store = [&](int slot) {
    float* dst = bank + ((long long)bh * (nch + 1) + slot) * D * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(long long)(rb * 32 + rowof(r)) * D + n] = sv[r];
    if (wave == 0 && col == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        be[((long long)bh * (nch + 1) + slot) * D + rb * 32 + rowof(r)] = e[r];
    }
  };
  store(dir == 0 ? 0 : nch);

  // the next frame, read ahead: this wave's B operands (hi, lo), this
  // block's B rows, alpha of this column
  u32x4_t mnext[2][KK];
  float braw[16], anext;
  auto fetch = [&](int f) {
    const u32x4_t* m4 = (const u32x4_t*)(Mp + ((long long)bh * F + f) * 2 * D * D);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      mnext[0][kk] = m4[(wave * KK + kk) * 64 + lane];
      mnext[1][kk] = m4[D * D / 8 + (wave * KK + kk) * 64 + lane];
    }
    const long long mo = ((long long)bh * F + f) * D * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) braw[r] = Bm[mo + (long long)(rb * 32 + rowof(r)) * D + n];
    anext = alpha[((long long)bh * F + f) * D + n];
  };
  fetch(dir == 0 ? 0 : F - 1);

  for (int i = 0; i < F; ++i) {
    const int f = dir == 0 ? i : F - 1 - i;
    const int buf = i & 1;
    // ---- X = S diag(alpha) + c1 2^-e B (own block) -> LDS (hi, lo)
    float bcur[16];
    const float acur = anext;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      bcur[r] = ldexpf(braw[r], -e[r]);
      const float x = fmaf(c1, bcur[r], sv[r] * acur);
      __bf16 h, l;
      split_bf16(x, h, l);
      x_hi[buf][rowof(r) * XP + n] = __builtin_bit_cast(bf16_t, h);
      x_lo[buf][rowof(r) * XP + n] = __builtin_bit_cast(bf16_t, l);
    }
    u32x4_t mcur[2][KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      mcur[0][kk] = mnext[0][kk];
      mcur[1][kk] = mnext[1][kk];
    }
    if (i + 1 < F) fetch(dir == 0 ? f + 1 : f - 1);
    __syncthreads();
    // ---- S = X M (+ c2 2^-e B)
    f32x16_t acc, acc1, acc2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[r] = c2 * bcur[r];
      acc1[r] = 0.0f;
      acc2[r] = 0.0f;
    }
    const bf16_t* xh = &x_hi[buf][col * XP + half * 8];
    const bf16_t* xl = &x_lo[buf][col * XP + half * 8];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8_t ah = *(const bf16x8_t*)(xh + kk * 16);
      const bf16x8_t al = *(const bf16x8_t*)(xl + kk * 16);
      const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, mcur[0][kk]);
      const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, mcur[1][kk]);
      acc = mfma32(ah, bh, acc);
      acc1 = mfma32(ah, bl, acc1);
      acc2 = mfma32(al, bh, acc2);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = acc[r] + (acc1[r] + acc2[r]);
    if (SANA) {
      // rows are renormalised only when some entry passed 2^64 (every dozen
      // frames or so at 1,560 tokens per frame): the row maxima are gathered
      // only then
      bool big = false;
#pragma unroll
      for (int r = 0; r < 16; ++r) big |= fabsf(sv[r]) > 0x1p64f;
      if (__syncthreads_or(big)) {
        // row max |S| over all columns: 32 lanes of a half, then the waves
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float m = fabsf(sv[r]);
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
          if (col == 0) atomicMax(&rmax[buf][rowof(r)], __float_as_uint(m));
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float m = __uint_as_float(rmax[buf][rowof(r)]);
          if (m > 0x1p64f) {
            int ex;
            frexpf(m, &ex);
            sv[r] = ldexpf(sv[r], -ex);
            e[r] += ex;
          }
        }
      }
      if (tid < 32) rmax[buf ^ 1][tid] = 0u;  // cleared for the next frame
    }
    if (dir == 0) {
      if ((f + 1) % chunk == 0 || f + 1 == F) store((f + chunk) / chunk);
    } else {
      if (f % chunk == 0) store(f / chunk);
    }
  }
}

hipError_t launch_scan_packed(const Geom& g, int rule, float c, const bf16_t* Mp,
                              const float* Bm, const float* alpha, const float* text_state,
                              float text_scale, float* bank_p, float* bank_q,
                              int32_t* bank_e, hipStream_t st) {
  const bool sana = rule == HWA_RULE_SANA_SCALED;
  const float c1 = sana ? 0.0f : (rule == HWA_RULE_VDN_SCALED ? c : 1.0f);
  const float c2 = sana ? c : 0.0f;
  dim3 grid(g.d / 32, 2, g.B * g.H);
#define SP_SCAN(DD, SN)                                                                 \
  hipLaunchKernelGGL((scan_packed_kernel<DD, SN>), grid, dim3(2 * DD), 0, st, Mp, Bm, alpha, \
                     c1, c2, text_state, text_scale, bank_p, bank_q, bank_e, g.F, g.chunk,   \
                     g.nch, g.B * g.H)
  if (g.d == 128) {
    if (sana) SP_SCAN(128, true); else SP_SCAN(128, false);
  } else {
    if (sana) SP_SCAN(64, true); else SP_SCAN(64, false);
  }
#undef SP_SCAN
  return hipGetLastError();
}

hipError_t launch_scan(const Geom& g, int dtype, int rule, float c,
                       const float* A, const float* Bm, const float* M,
                       const float* alpha, const float* text_state,
                       float text_scale, float* bank_p, float* bank_q,
                       int32_t* bank_e, hipStream_t st) {
  if (dtype == HWA_BF16) {
    const bool sana = rule == HWA_RULE_SANA_SCALED;
    const float c1 = sana ? 0.0f : (rule == HWA_RULE_VDN_SCALED ? c : 1.0f);
    const float c2 = sana ? c : 0.0f;
    const float* msrc = sana ? A : M;
    dim3 grid(g.d / 32, 2, g.B * g.H);
#define SM_SCAN(DD, SN)                                                         \
  hipLaunchKernelGGL((scan_mfma_kernel<DD, SN>), grid, dim3(2 * DD), 0, st,    \
                     msrc, Bm, alpha, c1, c2, c * c, text_state, text_scale,   \
                     bank_p, bank_q, bank_e, g.F, g.chunk, g.nch, g.B * g.H)
    if (g.d == 128) {
      if (sana) SM_SCAN(128, true); else SM_SCAN(128, false);
    } else {
      if (sana) SM_SCAN(64, true); else SM_SCAN(64, false);
    }
#undef SM_SCAN
    return hipGetLastError();
  }
  dim3 grid(g.d / SC_R, 2, g.B * g.H);
#define SCAN_LAUNCH(DD)                                                       \
  hipLaunchKernelGGL(scan_kernel<DD>, grid, dim3(256), 0, st, A, Bm, M, alpha, \
                     rule, c, text_state, text_scale, bank_p, bank_q, bank_e, \
                     g.F, g.chunk, g.nch, g.B * g.H)
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
