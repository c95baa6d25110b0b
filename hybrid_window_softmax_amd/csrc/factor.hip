// Exact inverse of the SPD matrices of the delta-rule update (VDN-H3
// article, "Step 3: delta-rule state update" and its rules table):
//   vdn_solve    S -> (S D + B)(I + A)^-1
//   vdn_scaled   S -> (S D + c B)(I + c^2 A)^-1
// M_f = (I + c~^2 A_f)^-1 (c~ = 1 or c) does not depend on the state, so all
// frames are inverted in parallel here and the sequential scan only
// multiplies by M_f. (sana_scaled, S -> (S D)(I - c^2 A) + c B, needs no
// inverse.)
//
// bf16 calls take M in the operand order of the bf16 scan, split into hi and
// lo bf16 parts (launch_update_packed; for sana_scaled the same kernel writes
// I - c^2 A without inverting).
//
// Inversion is the in-place Gauss-Jordan sweep without pivoting. It is
// stable here because I + c~^2 A >= I: every pivot is a Schur complement of
// an SPD matrix >= I, hence >= 1. A workgroup of 256 threads inverts one
// d x d matrix with the matrix held in registers (each thread owns a
// (d/16) x (d/16) block); step k needs the pre-step row k and column k, which
// their owners publish through a double-buffered LDS line, so every pivot
// costs one barrier.

#include "hwa_internal.h"

namespace hwa {

// Element (r, c) of a d x d matrix in the bf16 scan's operand order: the
// B operand of wave w = r / 32 (output columns 32w .. 32w+31) at step
// kk = c / 16 is one contiguous 1 KB block, lane (c % 16) / 8 * 32 + r % 32
// holding the 8 consecutive elements c - c % 8 .. (the scan multiplies by M
// from the right and M is symmetric, so row r of M is column r).
__host__ __device__ constexpr long long packed_index(int D, int r, int c) {
  return ((((long long)(r / 32) * (D / 16) + c / 16) * 64) + ((c % 16) / 8) * 32 + r % 32) * 8 +
         c % 8;
}

// PACK: write M as two bf16 matrices, hi = bf16(M) then lo = bf16(M - hi), in
// the order of packed_index (2 * d * d elements per matrix), for the bf16
// scan. INVERT == false: M = I - c2 A itself (sana_scaled's update matrix).
template <int D, bool PACK, bool INVERT>
__global__ __launch_bounds__(256) void inverse_kernel(
    const float* __restrict__ A, void* __restrict__ Mout, float c2) {
  constexpr int BS = D / 16;
  __shared__ float rowbuf[2][D];
  __shared__ float colbuf[2][D];

  const int tid = threadIdx.x;
  const int ib = tid / 16, jb = tid % 16;
  const long long mo = (long long)blockIdx.x * D * D;
  float m[BS][BS];
  const float sgn = INVERT ? 1.0f : -1.0f;
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) {
      const int i = ib * BS + a, j = jb * BS + b;
      m[a][b] = (i == j ? 1.0f : 0.0f) + sgn * c2 * A[mo + (long long)i * D + j];
    }

  // pivot k = kb * BS + kr; kr is unrolled so register indices are static
  for (int kb = 0; kb < (INVERT ? 16 : 0); ++kb) {
#pragma unroll
    for (int kr = 0; kr < BS; ++kr) {
      const int k = kb * BS + kr;
      const int buf = k & 1;
      if (ib == kb) {
#pragma unroll
        for (int b = 0; b < BS; ++b) rowbuf[buf][jb * BS + b] = m[kr][b];
      }
      if (jb == kb) {
#pragma unroll
        for (int a = 0; a < BS; ++a) colbuf[buf][ib * BS + a] = m[a][kr];
      }
      __syncthreads();
      const float rp = 1.0f / rowbuf[buf][k];
      float row[BS], colv[BS];
#pragma unroll
      for (int b = 0; b < BS; ++b) row[b] = rowbuf[buf][jb * BS + b];
#pragma unroll
      for (int a = 0; a < BS; ++a) colv[a] = colbuf[buf][ib * BS + a] * rp;
      // every element: m[i][j] -= m[i][k] m[k][j] / p
#pragma unroll
      for (int a = 0; a < BS; ++a)
#pragma unroll
        for (int b = 0; b < BS; ++b) m[a][b] = fmaf(-colv[a], row[b], m[a][b]);
      // pivot row m[k][j] = m[k][j] / p, column m[i][k] = -m[i][k] / p,
      // pivot 1 / p
      if (ib == kb) {
#pragma unroll
        for (int b = 0; b < BS; ++b) m[kr][b] = row[b] * rp;
      }
      if (jb == kb) {
#pragma unroll
        for (int a = 0; a < BS; ++a) m[a][kr] = -colv[a];
        if (ib == kb) m[kr][kr] = rp;
      }
    }
  }
  if constexpr (PACK) {
    // Each part (hi, then lo) is assembled in LDS in the packed order and
    // then copied out with consecutive lanes on consecutive 16-byte pieces:
    // written straight from the registers, every store instruction touched
    // 64 lines 16 bytes at a time, and the memory counters showed three
    // times the matrix's bytes written.
    __shared__ __attribute__((aligned(16))) uint4 pk[D * D / 8];
    bf16_t* P = (bf16_t*)Mout + (long long)blockIdx.x * 2 * D * D;
    bf16_t* pkb = (bf16_t*)pk;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
#pragma unroll
      for (int a = 0; a < BS; ++a) {
        const int r = ib * BS + a;
        uint32_t w[BS / 2];
#pragma unroll
        for (int b = 0; b < BS; b += 2) {
          __bf16 h0, l0, h1, l1;
          split_bf16(m[a][b], h0, l0);
          split_bf16(m[a][b + 1], h1, l1);
          w[b / 2] = part == 0 ? ((uint32_t)__builtin_bit_cast(bf16_t, h0) |
                                  ((uint32_t)__builtin_bit_cast(bf16_t, h1) << 16))
                               : ((uint32_t)__builtin_bit_cast(bf16_t, l0) |
                                  ((uint32_t)__builtin_bit_cast(bf16_t, l1) << 16));
        }
        const int o = (int)packed_index(D, r, jb * BS);
        if constexpr (BS == 8) {
          *(uint4*)(pkb + o) = make_uint4(w[0], w[1], w[2], w[3]);
        } else if constexpr (BS == 4) {
          *(uint2*)(pkb + o) = make_uint2(w[0], w[1]);
        }
      }
      __syncthreads();
      uint4* dst = (uint4*)(P + part * D * D);
#pragma unroll
      for (int i = tid; i < D * D / 8; i += 256) dst[i] = pk[i];
      __syncthreads();
    }
  } else {
    float* M = (float*)Mout;
#pragma unroll
    for (int a = 0; a < BS; ++a)
#pragma unroll
      for (int b = 0; b < BS; ++b)
        M[mo + (long long)(ib * BS + a) * D + jb * BS + b] = m[a][b];
  }
}

// C = B M for every matrix (text state: S_text = B (I + A)^-1).
template <int D>
__global__ __launch_bounds__(256) void matmul_bm_kernel(
    const float* __restrict__ Bm, const float* __restrict__ M,
    float* __restrict__ C) {
  constexpr int BS = D / 16;
  __shared__ float ms[D][D + 1];
  const int tid = threadIdx.x;
  const long long mo = (long long)blockIdx.x * D * D;
  for (int e = tid; e < D * D; e += 256) ms[e / D][e % D] = M[mo + e];
  __syncthreads();
  const int ib = tid / 16, jb = tid % 16;
  float acc[BS][BS];
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) acc[a][b] = 0.0f;
  for (int kk = 0; kk < D; ++kk) {
    float bv[BS], mv[BS];
#pragma unroll
    for (int a = 0; a < BS; ++a) bv[a] = Bm[mo + (long long)(ib * BS + a) * D + kk];
#pragma unroll
    for (int b = 0; b < BS; ++b) mv[b] = ms[kk][jb * BS + b];
#pragma unroll
    for (int a = 0; a < BS; ++a)
#pragma unroll
      for (int b = 0; b < BS; ++b) acc[a][b] = fmaf(bv[a], mv[b], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b)
      C[mo + (long long)(ib * BS + a) * D + jb * BS + b] = acc[a][b];
}

hipError_t launch_inverse(const Geom& g, float c2, const float* A, float* M,
                          hipStream_t st) {
  dim3 grid((unsigned)((long long)g.B * g.H * g.F));
#define INV_LAUNCH(DD) \
  hipLaunchKernelGGL((inverse_kernel<DD, false, true>), grid, dim3(256), 0, st, A, M, c2)
  switch (g.d) {
    case 16: INV_LAUNCH(16); break;
    case 32: INV_LAUNCH(32); break;
    case 64: INV_LAUNCH(64); break;
    default: INV_LAUNCH(128); break;
  }
#undef INV_LAUNCH
  return hipGetLastError();
}

hipError_t launch_update_f32(const Geom& g, bool invert, float c2, const float* A, float* M,
                             hipStream_t st) {
  if (invert) return launch_inverse(g, c2, A, M, st);
  dim3 grid((unsigned)((long long)g.B * g.H * g.F));
#define UF_LAUNCH(DD) \
  hipLaunchKernelGGL((inverse_kernel<DD, false, false>), grid, dim3(256), 0, st, A, (void*)M, c2)
  switch (g.d) {
    case 16: UF_LAUNCH(16); break;
    case 32: UF_LAUNCH(32); break;
    case 64: UF_LAUNCH(64); break;
    default: UF_LAUNCH(128); break;
  }
#undef UF_LAUNCH
  return hipGetLastError();
}

hipError_t launch_update_packed(const Geom& g, bool invert, float c2, const float* A,
                                bf16_t* packed, hipStream_t st) {
  dim3 grid((unsigned)((long long)g.B * g.H * g.F));
  if (g.d == 128) {
    if (invert)
      hipLaunchKernelGGL((inverse_kernel<128, true, true>), grid, dim3(256), 0, st, A,
                         (void*)packed, c2);
    else
      hipLaunchKernelGGL((inverse_kernel<128, true, false>), grid, dim3(256), 0, st, A,
                         (void*)packed, c2);
  } else {
    if (invert)
      hipLaunchKernelGGL((inverse_kernel<64, true, true>), grid, dim3(256), 0, st, A,
                         (void*)packed, c2);
    else
      hipLaunchKernelGGL((inverse_kernel<64, true, false>), grid, dim3(256), 0, st, A,
                         (void*)packed, c2);
  }
  return hipGetLastError();
}

hipError_t launch_matmul_bm(const Geom& g, const float* Bm, const float* M,
                            float* C, hipStream_t st) {
  dim3 grid((unsigned)((long long)g.B * g.H * g.F));
#define BM_LAUNCH(DD) \
  hipLaunchKernelGGL(matmul_bm_kernel<DD>, grid, dim3(256), 0, st, Bm, M, C)
  switch (g.d) {
    case 16: BM_LAUNCH(16); break;
    case 32: BM_LAUNCH(32); break;
    case 64: BM_LAUNCH(64); break;
    default: BM_LAUNCH(128); break;
  }
#undef BM_LAUNCH
  return hipGetLastError();
}

}  // namespace hwa
