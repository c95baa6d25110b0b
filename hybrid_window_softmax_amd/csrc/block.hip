// The attention block around the hybrid attention (VDN-H3 article, "Why
// video models are stuck on attention": one QKV projection feeds both
// branches; "Step 1: NoPE features": the softmax branch takes RoPE'd q and
// k, the linear branch the unrotated ones). Two bf16 GEMMs on MFMA with
// fused epilogues:
//   QKV:  [q | k | v] = x W_qkv^T, written head-major [B, H, N, d], with the
//         3D-rotated q and k (the block's stated RoPE) written alongside;
//   O:    y = concat_h(out_h) W_o^T, reading the attention output in its
//         head-major layout (a 64-wide K step never crosses a head).
// Both are "NT" products C[m][n] = sum_k A[m][k] W[n][k]: both operands are
// read along k, so their tiles are rows of 128 bytes (64 bf16 of k) copied
// global -> LDS by the gfx950 direct load, chunks XOR-swizzled by row as in
// the attention kernels.
//
// W rows past N_out (a width that is not a multiple of 128) read zeros through
// the load descriptor and their columns are not written.
// Tile: 128 x 128 outputs per workgroup of 4 waves (2 x 2, 64 x 64 each: 2 x 2
// blocks of v_mfma_f32_32x32x16_bf16), k in steps of 64 through two LDS
// stages (64 KB: two workgroups per CU). Each XCD (workgroup p runs on XCD
// p % 8) takes a contiguous range of tiles in grouped order (8 row tiles,
// then the next column tile): row-tile-major order made every row tile
// re-read all of W from beyond the L2 (62.6 GB fetched for 0.87 GB of
// operands in the QKV projection of 132,600 tokens).

#include "attn_tile.h"

namespace hwa {

constexpr int GT = 128;   // tile edge (rows of A and of W)
constexpr int GK = 64;    // k per LDS stage
constexpr int GM = 8;     // row tiles per group of the tile order
constexpr int SROW = 68;  // floats per row of a wave's epilogue staging (64 + 4 pad)
static_assert(4 * 32 * SROW * 4 <= 4 * GT * GK * 2, "epilogue staging fits the operand stages");

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// A operand source: row-major [M][K], or the attention output [B][H][T][d]
// read as [B*T][H*d].
enum { GA_ROWMAJOR = 0, GA_HEADMAJOR = 1 };
// epilogue: C row-major [M][N] bf16, or the QKV split (+ RoPE of q and k)
enum { GE_ROWMAJOR = 0, GE_QKV = 1 };

struct GemmArgs {
  const bf16_t* A;
  const bf16_t* W;
  int M, Nout, K;
  int T, H, d;            // tokens per batch element, heads, head_dim
  bf16_t* C;              // GE_ROWMAJOR
  bf16_t *q, *k, *v, *qr, *kr;  // GE_QKV, [B, H, T, d]
  int S, grid_w;          // RoPE: tokens per frame, latent grid columns
  int pt, ph;             // RoPE: time and row pairs (the rest are column pairs)
  float log2_theta;
  int tiles_n, tiles;
};

template <int AMODE, int EMODE>
__global__ __launch_bounds__(256, 2) void gemm_nt_kernel(GemmArgs g) {
  // operand stages: A stage st at st * GT * GK, W stage st at (2 + st) * GT * GK
  __shared__ __attribute__((aligned(16))) bf16_t smem[4 * GT * GK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  // XCD-contiguous tile ranges
  const int per_x = (g.tiles + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per_x + (int)(blockIdx.x / 8);
  if (t >= g.tiles) return;
  // grouped order: GM row tiles at a time, column tile by column tile, so
  // the workgroups an XCD runs together (about 64) cover GM x 8 tiles and
  // share both operands' rows in its L2
  const int tiles_m = g.tiles / g.tiles_n;
  const int grp = t / (GM * g.tiles_n);
  const int first_m = grp * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int r_in = t - grp * GM * g.tiles_n;
  const int m0 = (first_m + r_in % gm) * GT;
  const int n0 = (r_in / gm) * GT;
  const int wm = wave >> 1, wn = wave & 1;

  // per-lane byte offsets of the 4 direct-load slots of each tile: slot
  // s = (wave + 4 j) * 64 + lane lands at LDS byte 16 s = row 128 + chunk 16
  // and holds logical chunk pc ^ swz(row)
  int w_off[4];
  long long a_row_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = (wave + 4 * j) * 64 + lane;
    const int row = s >> 3, pc = s & 7;
    const int lc = pc ^ swz(row);
    w_off[j] = ((n0 + row) * g.K + lc * 8) * 2;
    const int m = m0 + row;
    if constexpr (AMODE == GA_ROWMAJOR) {
      a_row_base[j] = (long long)m * g.K + lc * 8;
    } else {
      const int b = m / g.T, tok = m % g.T;
      a_row_base[j] = ((long long)b * g.H * g.T + tok) * g.d + lc * 8;  // + h T d + c0
    }
  }
  const long long a_elems = (long long)(AMODE == GA_ROWMAJOR ? (long long)g.M * g.K
                                                             : (long long)g.M * g.H * g.d);
  auto rsrc = [&](const bf16_t* base, long long elems) __attribute__((always_inline)) {
    const unsigned long long p = (unsigned long long)base;
    hwa_i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)(p & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(p >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)(unsigned)(elems * 2));
    r[3] = 0x00020000;
    return r;
  };
  const hwa_i32x4 ra = rsrc(g.A, a_elems);
  const hwa_i32x4 rw = rsrc(g.W, (long long)g.Nout * g.K);
  auto load_tile = [&](int k0, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      long long ae;
      if constexpr (AMODE == GA_ROWMAJOR) {
        ae = a_row_base[j] + k0;
      } else {
        const int h = k0 / g.d, c0 = k0 % g.d;
        ae = a_row_base[j] + (long long)h * g.T * g.d + c0;
      }
      // rows past M: offsets past the descriptor's end read zeros
      const int aoff = ae * 2 < a_elems * 2 ? (int)(ae * 2) : (int)(a_elems * 2);
      hwa_raw_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)&smem[st * GT * GK + (wave + 4 * j) * 512],
                              16, aoff, 0, 0, 0);
      hwa_raw_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)&smem[(2 + st) * GT * GK + (wave + 4 * j) * 512],
                              16, w_off[j] + k0 * 2, 0, 0, 0);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.0f;

  const int nk = g.K / GK;
  load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * GK, st ^ 1);
    const bf16_t* as = &smem[st * GT * GK];
    const bf16_t* ws = &smem[(2 + st) * GT * GK];
#pragma unroll
    for (int j = 0; j < GK / 16; ++j) {
      const int ch = op_chunk(j, half);
      bf16x8_t ao[2], bo[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra_ = wm * 64 + i * 32 + col;
        ao[i] = *(const bf16x8_t*)(as + ra_ * 64 + ((ch ^ swz(ra_)) << 3));
        const int rw_ = wn * 64 + i * 32 + col;
        bo[i] = *(const bf16x8_t*)(ws + rw_ * 64 + ((ch ^ swz(rw_)) << 3));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) acc[i][jn] = mfma32(ao[i], bo[jn], acc[i][jn]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue. A lane holds rows 8 (r / 4) + 4 half + r % 4 of each
  // 32 x 32 output block, column col. Each wave turns its 64 x 64 results
  // around through LDS, 32 rows at a time, so that a lane then holds 8
  // consecutive columns of one row: 16-byte stores, and each RoPE pair
  // (2i, 2i + 1) in one lane. The last k step ended with a barrier, so the
  // operand stages are free.
  float* stage = (float*)smem + wave * (32 * SROW);
  const int cq = lane & 7;        // 8-column group read back
  const int rq = lane >> 3;       // row within 8 of a pass
  const int n = n0 + wn * 64 + 8 * cq;
  // per-lane column facts (the QKV split and the pairs' axis and frequency)
  int which = 0, hh = 0, c = 0;
  int axis[4];
  float fr[4];
  if constexpr (EMODE == GE_QKV) {
    const int D = g.H * g.d;
    which = n / D;
    hh = (n - which * D) / g.d;
    c = n - which * D - hh * g.d;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pi = (c >> 1) + e;
      int u, P;
      if (pi < g.pt) {
        axis[e] = 0; u = pi; P = g.pt;
      } else if (pi < g.pt + g.ph) {
        axis[e] = 1; u = pi - g.pt; P = g.ph;
      } else {
        axis[e] = 2; u = pi - g.pt - g.ph; P = g.d / 2 - g.pt - g.ph;
      }
      // theta^(-u / P) radians per position step, in turns (the hardware
      // sine and cosine take turns)
      fr[e] = exp2f(-(float)u / (float)P * g.log2_theta) * 0.15915494309189535f;
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stage[(8 * (r / 4) + 4 * half + (r % 4)) * SROW + jn * 32 + col] = acc[i][jn][r];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's own rows
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int rr = pass * 8 + rq;
      const float4 lo4 = *(const float4*)(stage + rr * SROW + 8 * cq);
      const float4 hi4 = *(const float4*)(stage + rr * SROW + 8 * cq + 4);
      const float v8[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
      const int m = m0 + wm * 64 + i * 32 + rr;
      if (m >= g.M || n >= g.Nout) continue;
      uint4 raw;
      raw.x = pack_bf16x2(v8[0], v8[1]);
      raw.y = pack_bf16x2(v8[2], v8[3]);
      raw.z = pack_bf16x2(v8[4], v8[5]);
      raw.w = pack_bf16x2(v8[6], v8[7]);
      if constexpr (EMODE == GE_ROWMAJOR) {
        *(uint4*)(g.C + (long long)m * g.Nout + n) = raw;
      } else {
        const int b = m / g.T, tok = m - b * g.T;
        const long long o = (((long long)b * g.H + hh) * g.T + tok) * g.d + c;
        *(uint4*)((which == 0 ? g.q : (which == 1 ? g.k : g.v)) + o) = raw;
        if (which < 2) {
          const int ft = tok / g.S, sp = tok - ft * g.S;
          const int gy = sp / g.grid_w, gx = sp - gy * g.grid_w;
          float rot[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pos = axis[e] == 0 ? ft : (axis[e] == 1 ? gy : gx);
            float turns = (float)pos * fr[e];
            turns -= floorf(turns);
            const float sn = __builtin_amdgcn_sinf(turns), cs = __builtin_amdgcn_cosf(turns);
            const float a = v8[2 * e], bb = v8[2 * e + 1];
            rot[2 * e] = fmaf(-bb, sn, a * cs);
            rot[2 * e + 1] = fmaf(a, sn, bb * cs);
          }
          uint4 rv;
          rv.x = pack_bf16x2(rot[0], rot[1]);
          rv.y = pack_bf16x2(rot[2], rot[3]);
          rv.z = pack_bf16x2(rot[4], rot[5]);
          rv.w = pack_bf16x2(rot[6], rot[7]);
          *(uint4*)((which == 0 ? g.qr : g.kr) + o) = rv;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_gemm_qkv(const bf16_t* x, const bf16_t* w_qkv, int M, int T, int H, int d,
                           int S, int grid_w, float theta, bf16_t* q, bf16_t* k, bf16_t* v,
                           bf16_t* qr, bf16_t* kr, hipStream_t st) {
  GemmArgs g{};
  g.A = x;
  g.W = w_qkv;
  g.M = M;
  g.K = H * d;
  g.Nout = 3 * H * d;
  g.T = T;
  g.H = H;
  g.d = d;
  g.q = q; g.k = k; g.v = v; g.qr = qr; g.kr = kr;
  g.S = S;
  g.grid_w = grid_w;
  g.ph = (d / 2) / 3;
  g.pt = d / 2 - 2 * g.ph;
  g.log2_theta = log2f(theta);
  g.tiles_n = (g.Nout + GT - 1) / GT;
  g.tiles = ((M + GT - 1) / GT) * g.tiles_n;
  const int per_x = (g.tiles + 7) / 8;
  hipLaunchKernelGGL((gemm_nt_kernel<GA_ROWMAJOR, GE_QKV>), dim3(per_x * 8), dim3(256), 0, st,
                     g);
  return hipGetLastError();
}

hipError_t launch_gemm_out(const bf16_t* att, const bf16_t* w_o, int M, int T, int H, int d,
                           bf16_t* y, hipStream_t st) {
  GemmArgs g{};
  g.A = att;
  g.W = w_o;
  g.M = M;
  g.K = H * d;
  g.Nout = H * d;
  g.T = T;
  g.H = H;
  g.d = d;
  g.C = y;
  g.tiles_n = (g.Nout + GT - 1) / GT;
  g.tiles = ((M + GT - 1) / GT) * g.tiles_n;
  const int per_x = (g.tiles + 7) / 8;
  hipLaunchKernelGGL((gemm_nt_kernel<GA_HEADMAJOR, GE_ROWMAJOR>), dim3(per_x * 8), dim3(256), 0,
                     st, g);
  return hipGetLastError();
}

}  // namespace hwa
