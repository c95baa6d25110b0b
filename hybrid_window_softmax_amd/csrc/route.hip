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
//   route_sums_kernel, one workgroup per (b, h, chunk, segment): q and k are
//   read once; it writes the mean of q over every query tile and the sum of
//   k over every piece (a global 128-block cut to the chunk; a key block of a
//   window is the union of its pieces in the window's chunks);
//   route_select_kernel, one wave per (b, h, chunk, query tile): the scores
//   of the window's key blocks, their mean, then the spread about it and the
//   first maximum, then the kept list -- block indices relative to the
//   window's first block, in increasing order, for the softmax kernel.
// (A first version ran both on one workgroup per (b, h, chunk), one thread
// per query tile in the selection: 1.24 ms at 132,600 tokens, 24 heads.)

#include "hwa_internal.h"

namespace hwa {

constexpr int RT_QT = 256;  // query tile
constexpr int RT_KB = 128;  // key block
// key blocks of a window, at most: the routed call allows windows of up to
// 4092 64-key tiles, i.e. 2046 blocks plus one partial block at each end
constexpr int RT_MAXB = 2048;

__host__ __device__ inline int route_pieces_per_chunk(int chunk, int S) {
  return (chunk * S + RT_KB - 1) / RT_KB + 1;
}
__host__ __device__ inline int route_tiles_per_chunk(int chunk, int S) {
  return (chunk * S + RT_QT - 1) / RT_QT;
}

// One workgroup per segment of a chunk: segment x < ntq is query tile x
// (the mean of its queries), segment ntq + p is piece p (the sum of its
// keys). 16-byte loads of 8 bf16 channels: a thread owns 8 channels of every
// RS-th row of the segment.
template <int D>
__global__ __launch_bounds__(256) void route_sums_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, float* __restrict__ qmean,
    float* __restrict__ ksum, int F, int S, int chunk, long long N) {
  constexpr int TPR = D / 8, RS = 256 / TPR;
  __shared__ float part[RS][D + 1];
  const int tid = threadIdx.x;
  const int seg = blockIdx.x, c = blockIdx.y, bh = blockIdx.z, nch = gridDim.y;
  const int c0 = (tid % TPR) * 8, r0 = tid / TPR;
  const long long a = (long long)c * chunk * S;
  const long long e = (long long)min(F, (c + 1) * chunk) * S;
  const int ntq = route_tiles_per_chunk(chunk, S), npc = route_pieces_per_chunk(chunk, S);
  long long x0, x1;
  const bf16_t* src;
  float* dst;
  float scale = 1.0f;
  if (seg < ntq) {
    x0 = a + (long long)seg * RT_QT;
    x1 = min(e, x0 + RT_QT);
    src = q + (long long)bh * N * D;
    dst = qmean + (((long long)bh * nch + c) * ntq + seg) * D;
  } else {
    const int p = seg - ntq;
    const long long jb = a / RT_KB + p;
    x0 = max(a, jb * RT_KB);
    x1 = min(e, (jb + 1) * RT_KB);
    src = k + (long long)bh * N * D;
    dst = ksum + (((long long)bh * nch + c) * npc + p) * D;
  }
  if (x0 >= x1) return;  // a tile or piece past the chunk's end (uniform)
  if (seg < ntq) scale = 1.0f / (float)(x1 - x0);
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
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// One wave per query tile of a chunk: the scores of every key block of the
// window (lane j, j + 64, ...; the block mean from its pieces) into LDS, the
// mean and spread by wave sums, the first maximum, then the kept list in
// increasing order by ballots.
template <int D>
__global__ __launch_bounds__(64) void route_select_kernel(
    const float* __restrict__ qmean, const float* __restrict__ ksum,
    const int32_t* __restrict__ lohi, float tau, int F, int S, int chunk, int nkb_max,
    int* __restrict__ sel_count, uint16_t* __restrict__ sel_list) {
  __shared__ __attribute__((aligned(16))) float qs[D];
  __shared__ float sc[RT_MAXB];
  const int lane = threadIdx.x;
  const int t = blockIdx.x, c = blockIdx.y, bh = blockIdx.z, nch = gridDim.y;
  const int ntq = route_tiles_per_chunk(chunk, S), npc = route_pieces_per_chunk(chunk, S);
  // query tiles of this chunk (the last chunk may hold fewer frames)
  const long long qa = (long long)c * chunk * S, qe = (long long)min(F, (c + 1) * chunk) * S;
  const int ntq_c = (int)((qe - qa + RT_QT - 1) / RT_QT);
  if (t >= ntq_c) return;
  const long long cs = (long long)chunk * S;
  const long long kb = (long long)lohi[c * chunk] * S;
  const long long ke = (long long)(lohi[F + c * chunk] + 1) * S;
  const long long jfirst = kb / RT_KB;
  const int nkb = (int)((ke - 1) / RT_KB - jfirst + 1);
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float* qm = qmean + (((long long)bh * nch + c) * ntq + t) * D;
  for (int ch = lane; ch < D; ch += 64) qs[ch] = qm[ch];
  __syncthreads();
  // pass 1: scores and their mean
  float sum = 0.0f;
  for (int j = lane; j < nkb; j += 64) {
    const long long jb = jfirst + j;
    const long long x0 = max(kb, jb * RT_KB), x1 = min(ke, (jb + 1) * RT_KB);
    const int cf = (int)(x0 / cs), cl = (int)((x1 - 1) / cs);
    float dot = 0.0f;
    for (int cc = cf; cc <= cl; ++cc) {
      const int p = (int)(jb - (long long)cc * cs / RT_KB);
      const float4* kr = (const float4*)(ksum + (((long long)bh * nch + cc) * npc + p) * D);
#pragma unroll 8
      for (int u = 0; u < D / 4; ++u) {
        const float4 kv = kr[u];
        const float4 qv = *(const float4*)&qs[4 * u];
        dot = fmaf(kv.x, qv.x, dot);
        dot = fmaf(kv.y, qv.y, dot);
        dot = fmaf(kv.z, qv.z, dot);
        dot = fmaf(kv.w, qv.w, dot);
      }
    }
    const float s = dot / (float)(x1 - x0) * inv_sqrt_d;
    sc[j] = s;
    sum += s;
  }
  const float mu = wave_sum(sum) / (float)nkb;
  // pass 2: spread about the mean, the first maximum
  float ss = 0.0f, best = -INFINITY;
  int arg = 0x7fffffff;
  for (int j = lane; j < nkb; j += 64) {
    const float s = sc[j];
    ss = fmaf(s - mu, s - mu, ss);
    if (s > best) {
      best = s;
      arg = j;
    }
  }
  ss = wave_sum(ss);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oa = __shfl_xor(arg, o);
    if (ob > best || (ob == best && oa < arg)) {
      best = ob;
      arg = oa;
    }
  }
  // tau = -inf keeps every block (mu + tau * 0 would be NaN)
  const float thr = (isinf(tau) && tau < 0.0f) ? -INFINITY : mu + tau * sqrtf(ss / (float)nkb);
  // pass 3: the kept blocks, in increasing order
  uint16_t* list = sel_list + (((long long)bh * nch + c) * ntq + t) * nkb_max;
  int n = 0;
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const int j = j0 + lane;
    const bool keep = j < nkb && (sc[j] >= thr || j == arg);
    const unsigned long long m = __ballot(keep);
    if (keep) list[n + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)j;
    n += __popcll(m);
  }
  if (lane == 0) sel_count[((long long)bh * nch + c) * ntq + t] = n;
}

int route_tiles(const Geom& g) { return route_tiles_per_chunk(g.chunk, g.S); }
int route_pieces(const Geom& g) { return route_pieces_per_chunk(g.chunk, g.S); }
int route_blocks_max(const Geom& g) { return (int)((g.N + RT_KB - 1) / RT_KB) + 1; }

hipError_t launch_route(const Geom& g, const bf16_t* q, const bf16_t* k, const int32_t* lohi,
                        float tau, float* qmean, float* ksum, int* sel_count,
                        uint16_t* sel_list, int nkb_max, hipStream_t st) {
  // the longest window: (2 radius + 1) chunks of keys
  const long long wkeys = (2LL * g.radius + 1) * g.chunk * (long long)g.S;
  if (wkeys / RT_KB + 2 > RT_MAXB) return hipErrorInvalidValue;
  const int ntq = route_tiles_per_chunk(g.chunk, g.S), npc = route_pieces_per_chunk(g.chunk, g.S);
  const dim3 gs(ntq + npc, g.nch, g.B * g.H), gq(ntq, g.nch, g.B * g.H);
  if (g.d == 128) {
    hipLaunchKernelGGL(route_sums_kernel<128>, gs, dim3(256), 0, st, q, k, qmean, ksum, g.F,
                       g.S, g.chunk, g.N);
    hipLaunchKernelGGL(route_select_kernel<128>, gq, dim3(64), 0, st, qmean, ksum, lohi, tau,
                       g.F, g.S, g.chunk, nkb_max, sel_count, sel_list);
  } else {
    hipLaunchKernelGGL(route_sums_kernel<64>, gs, dim3(256), 0, st, q, k, qmean, ksum, g.F,
                       g.S, g.chunk, g.N);
    hipLaunchKernelGGL(route_select_kernel<64>, gq, dim3(64), 0, st, qmean, ksum, lohi, tau,
                       g.F, g.S, g.chunk, nkb_max, sel_count, sel_list);
  }
  return hipGetLastError();
}

}  // namespace hwa
