// Block-sparse routing of the windowed softmax (H3 acceleration report,
// section 9.7.3 "Sol-Attn Ampere" and 9.8: 128-token blocks, block means of
// Q and K, trial scores q_mean . k_mean^T, keep the blocks above mean + tau *
// std, exact attention on the kept blocks only). Reading of the pages, per
// (b, h) and chunk c with key window [kb, ke) = [lo_c S, (hi_c + 1) S):
//   query tiles t: 256 queries from the chunk's first one (the softmax
//   kernel's workgroup tile); key blocks j: the global 128-token blocks
//   [128 j, 128 j + 128) cut to the window; q_mean_t, k_mean_j: plain means;
//   s_tj = q_mean_t . k_mean_j / sqrt(d); keep j when s_tj >= mu_t + tau
//   sigma_t (mean and population standard deviation over the window's
//   blocks), and always the first block of largest s_tj.
// Two kernels:
//   route_sums_kernel, one workgroup per (b, h, chunk): reads the chunk's q
//   and k once; writes the mean of q over every query tile and the sum of k
//   over every piece (a global 128-block cut to the chunk; a key block of a
//   window is the union of its pieces in the window's chunks);
//   route_select_kernel, one workgroup per (b, h, chunk), one thread per
//   query tile: three passes over the window's key blocks (staged 32 at a
//   time in LDS from the piece sums): the mean of s, then the spread about
//   it and the first maximum, then the kept list -- block indices relative to
//   the window's first block, in increasing order, for the softmax kernel.

#include "hwa_internal.h"

namespace hwa {

constexpr int RT_QT = 256;  // query tile
constexpr int RT_KB = 128;  // key block
constexpr int RT_STAGE = 32;

__host__ __device__ inline int route_pieces_per_chunk(int chunk, int S) {
  return (chunk * S + RT_KB - 1) / RT_KB + 1;
}
__host__ __device__ inline int route_tiles_per_chunk(int chunk, int S) {
  return (chunk * S + RT_QT - 1) / RT_QT;
}

// 16-byte loads of 8 bf16 channels; a thread owns 8 channels of every RS-th row
template <int D>
__global__ __launch_bounds__(256) void route_sums_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, float* __restrict__ qmean,
    float* __restrict__ ksum, int F, int S, int chunk, long long N) {
  constexpr int TPR = D / 8, RS = 256 / TPR;
  __shared__ float part[RS][D + 1];
  const int tid = threadIdx.x;
  const int c = blockIdx.x, bh = blockIdx.y, nch = gridDim.x;
  const int c0 = (tid % TPR) * 8, r0 = tid / TPR;
  const long long a = (long long)c * chunk * S;
  const long long e = (long long)min(F, (c + 1) * chunk) * S;
  const int ntq = route_tiles_per_chunk(chunk, S), npc = route_pieces_per_chunk(chunk, S);
  // sum of rows [x0, x1) of src, written (times scale) to dst[0 .. D)
  auto seg_sum = [&](const bf16_t* src, long long x0, long long x1, float scale, float* dst) {
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.0f;
    for (long long x = x0 + r0; x < x1; x += RS) {
      const uint4 raw = *(const uint4*)(src + x * D + c0);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[2 * u] += __uint_as_float(w[u] << 16);
        acc[2 * u + 1] += __uint_as_float(w[u] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) part[r0][c0 + u] = acc[u];
    __syncthreads();
    if (tid < D) {
      float t = 0.0f;
      for (int j = 0; j < RS; ++j) t += part[j][tid];
      dst[tid] = t * scale;
    }
    __syncthreads();
  };
  const bf16_t* qb = q + (long long)bh * N * D;
  const bf16_t* kb = k + (long long)bh * N * D;
  for (int t = 0; t < ntq; ++t) {
    const long long x0 = a + (long long)t * RT_QT;
    const long long x1 = min(e, x0 + RT_QT);
    float* dst = qmean + (((long long)bh * nch + c) * ntq + t) * D;
    if (x0 < e) seg_sum(qb, x0, x1, 1.0f / (float)(x1 - x0), dst);
  }
  const long long j0 = a / RT_KB;
  for (int p = 0; p < npc; ++p) {
    const long long jb = j0 + p;
    const long long x0 = max(a, jb * RT_KB), x1 = min(e, (jb + 1) * RT_KB);
    float* dst = ksum + (((long long)bh * nch + c) * npc + p) * D;
    if (x0 < x1) seg_sum(kb, x0, x1, 1.0f, dst);
  }
}

template <int D>
__global__ __launch_bounds__(256) void route_select_kernel(
    const float* __restrict__ qmean, const float* __restrict__ ksum,
    const int32_t* __restrict__ lohi, float tau, int F, int S, int chunk, int nkb_max,
    int* __restrict__ sel_count, uint16_t* __restrict__ sel_list) {
  __shared__ float kmean[RT_STAGE][D];
  const int tid = threadIdx.x;
  const int c = blockIdx.x, bh = blockIdx.y, nch = gridDim.x;
  const int ntq = route_tiles_per_chunk(chunk, S), npc = route_pieces_per_chunk(chunk, S);
  // query tiles of this chunk (the last chunk may hold fewer frames)
  const long long qa = (long long)c * chunk * S, qe = (long long)min(F, (c + 1) * chunk) * S;
  const int ntq_c = (int)((qe - qa + RT_QT - 1) / RT_QT);
  const long long kb = (long long)lohi[c * chunk] * S;
  const long long ke = (long long)(lohi[F + c * chunk] + 1) * S;
  const long long jfirst = kb / RT_KB;
  const int nkb = (int)((ke - 1) / RT_KB - jfirst + 1);
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float* qm = qmean + ((long long)bh * nch + c) * ntq * D;
  // key block j of the window: the pieces of block jfirst + j in the chunks
  // of the window, over the block's tokens inside the window
  auto stage = [&](int j0) {
    for (int x = tid; x < RT_STAGE * D; x += 256) {
      const int jj = x / D, ch = x % D;
      const long long jb = jfirst + j0 + jj;
      float v = 0.0f;
      if (j0 + jj < nkb) {
        const long long x0 = max(kb, jb * RT_KB), x1 = min(ke, (jb + 1) * RT_KB);
        const int cf = (int)(x0 / ((long long)chunk * S)), cl = (int)((x1 - 1) / ((long long)chunk * S));
        for (int cc = cf; cc <= cl; ++cc) {
          const long long pa = (long long)cc * chunk * S;
          const int p = (int)(jb - pa / RT_KB);
          v += ksum[(((long long)bh * nch + cc) * npc + p) * D + ch];
        }
        v /= (float)(x1 - x0);
      }
      kmean[jj][ch] = v;
    }
    __syncthreads();
  };
  for (int t0 = 0; t0 < ntq; t0 += 256) {
    const int t = t0 + tid;
    const bool act = t < ntq_c;
    float qv[D];
#pragma unroll
    for (int ch = 0; ch < D; ++ch) qv[ch] = act ? qm[(long long)t * D + ch] : 0.0f;
    auto score = [&](int jj) {
      float s = 0.0f;
#pragma unroll
      for (int ch = 0; ch < D; ++ch) s = fmaf(qv[ch], kmean[jj][ch], s);
      return s * inv_sqrt_d;
    };
    // pass 1: mean
    float sum = 0.0f;
    for (int j0 = 0; j0 < nkb; j0 += RT_STAGE) {
      stage(j0);
      for (int jj = 0; jj < RT_STAGE && j0 + jj < nkb; ++jj) sum += score(jj);
      __syncthreads();
    }
    const float mu = sum / (float)nkb;
    // pass 2: spread about the mean, first maximum
    float ss = 0.0f, best = -INFINITY;
    int arg = 0;
    for (int j0 = 0; j0 < nkb; j0 += RT_STAGE) {
      stage(j0);
      for (int jj = 0; jj < RT_STAGE && j0 + jj < nkb; ++jj) {
        const float s = score(jj);
        ss = fmaf(s - mu, s - mu, ss);
        if (s > best) {
          best = s;
          arg = j0 + jj;
        }
      }
      __syncthreads();
    }
    const float thr = mu + tau * sqrtf(ss / (float)nkb);
    // pass 3: the kept blocks, in increasing order
    int n = 0;
    uint16_t* list = sel_list + (((long long)bh * nch + c) * ntq + t) * nkb_max;
    for (int j0 = 0; j0 < nkb; j0 += RT_STAGE) {
      stage(j0);
      for (int jj = 0; jj < RT_STAGE && j0 + jj < nkb; ++jj) {
        const int j = j0 + jj;
        if (act && (score(jj) >= thr || j == arg)) list[n++] = (uint16_t)j;
      }
      __syncthreads();
    }
    if (act) sel_count[((long long)bh * nch + c) * ntq + t] = n;
  }
}

int route_tiles(const Geom& g) { return route_tiles_per_chunk(g.chunk, g.S); }
int route_pieces(const Geom& g) { return route_pieces_per_chunk(g.chunk, g.S); }
int route_blocks_max(const Geom& g) { return (int)((g.N + RT_KB - 1) / RT_KB) + 1; }

hipError_t launch_route(const Geom& g, const bf16_t* q, const bf16_t* k, const int32_t* lohi,
                        float tau, float* qmean, float* ksum, int* sel_count,
                        uint16_t* sel_list, int nkb_max, hipStream_t st) {
  dim3 grid(g.nch, g.B * g.H);
  if (g.d == 128) {
    hipLaunchKernelGGL(route_sums_kernel<128>, grid, dim3(256), 0, st, q, k, qmean, ksum, g.F,
                       g.S, g.chunk, g.N);
    hipLaunchKernelGGL(route_select_kernel<128>, grid, dim3(256), 0, st, qmean, ksum, lohi, tau,
                       g.F, g.S, g.chunk, nkb_max, sel_count, sel_list);
  } else {
    hipLaunchKernelGGL(route_sums_kernel<64>, grid, dim3(256), 0, st, q, k, qmean, ksum, g.F,
                       g.S, g.chunk, g.N);
    hipLaunchKernelGGL(route_select_kernel<64>, grid, dim3(256), 0, st, qmean, ksum, lohi, tau,
                       g.F, g.S, g.chunk, nkb_max, sel_count, sel_list);
  }
  return hipGetLastError();
}

}  // namespace hwa
