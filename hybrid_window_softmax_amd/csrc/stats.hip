// Per-frame statistics of the linear branch with the NoPE features fused in
// (VDN-H3 article, "Step 1: NoPE features" and "Step 2: per-frame
// statistics A, B"):
//   k^ = L2(SiLU(conv_k(k))), v^ = conv_v(v)   (conv: depthwise, causal,
//        width 4, along the frame's token order, zero before the frame start)
//   A_f = sum_{n in f} beta_n k^_n k^_n^T,  B_f = sum_{n in f} beta_n v^_n k^_n^T
// One workgroup per (b, h, frame). Tokens stream through LDS 32 at a time;
// every thread owns a (d/16) x (d/16) block of A and of B in registers.
// Text mode (conv == false) forms k^ = L2(SiLU(k)) and v^ = v.
// fp32 calls use the VALU kernel (fp32 arithmetic throughout). bf16 calls use
// the MFMA kernel below, whose operands carry sqrt(beta); it is exact only
// for beta >= 0, so after it the VALU kernel recomputes, in fp32, the frames
// that hold a negative beta (the others exit after reading their betas).

#include "hwa_internal.h"

namespace hwa {

constexpr int ST_TT = 32;  // tokens per LDS tile

template <typename T, int D>
__global__ __launch_bounds__(256) void stats_kernel(
    const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ conv_k,
    const float* __restrict__ conv_v, int conv, float* __restrict__ A,
    float* __restrict__ Bm, int F, int S, int H, long long N, int neg_only) {
  constexpr int TPT = 256 / ST_TT;  // threads per token (8)
  constexpr int CPT = D / TPT;      // channels per thread
  constexpr int BS = D / 16;        // accumulator block edge
  __shared__ float kh_lds[ST_TT][D + 4];
  __shared__ float kb_lds[ST_TT][D + 4];
  __shared__ float vb_lds[ST_TT][D + 4];

  const int tid = threadIdx.x;
  const int f = blockIdx.x;
  const int bh = blockIdx.y;
  const int h = bh % H;
  const T* kp = k + (long long)bh * N * D;
  const T* vp = v + (long long)bh * N * D;
  const float* bp = beta + (long long)bh * N;
  const long long n0 = (long long)f * S;
  if (neg_only) {  // only frames that hold a negative beta
    int cnt = 0;
    for (int s = tid; s < S; s += 256) cnt += bp[n0 + s] < 0.0f ? 1 : 0;
    if (__syncthreads_or(cnt) == 0) return;
  }

  // conv taps of this thread's channels
  const int tt = tid / TPT;
  const int ch0 = (tid % TPT) * CPT;
  float wk[CPT][4], wv[CPT][4];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wk[i][j] = conv ? conv_k[((long long)h * D + ch0 + i) * 4 + j] : (j == 0 ? 1.0f : 0.0f);
      wv[i][j] = conv ? conv_v[((long long)h * D + ch0 + i) * 4 + j] : (j == 0 ? 1.0f : 0.0f);
    }

  const int ib = tid / 16, jb = tid % 16;  // accumulator block (rows, cols)
  float accA[BS][BS], accB[BS][BS];
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) accA[a][b] = accB[a][b] = 0.0f;

  for (int s0 = 0; s0 < S; s0 += ST_TT) {
    const int s = s0 + tt;
    float kc[CPT], vc[CPT];
    float ss = 0.0f;
    float bt = 0.0f;
    if (s < S) {
      bt = bp[n0 + s];
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        float ak = 0.0f, av = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (s - j >= 0) {
            long long idx = (n0 + s - j) * D + ch0 + i;
            ak = fmaf(wk[i][j], ld_io<T>(kp, idx), ak);
            av = fmaf(wv[i][j], ld_io<T>(vp, idx), av);
          }
        }
        kc[i] = silu_f(ak);
        vc[i] = av;
        ss = fmaf(kc[i], kc[i], ss);
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) kc[i] = vc[i] = 0.0f;
    }
    // L2 norm over the token's d channels: TPT consecutive lanes
#pragma unroll
    for (int off = 1; off < TPT; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv = inv_l2(ss);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      float kh = kc[i] * inv;
      kh_lds[tt][ch0 + i] = kh;
      kb_lds[tt][ch0 + i] = bt * kh;
      vb_lds[tt][ch0 + i] = bt * vc[i];
    }
    __syncthreads();
#pragma unroll 4
    for (int t = 0; t < ST_TT; ++t) {
      float kr[BS], kbr[BS], vbr[BS];
#pragma unroll
      for (int a = 0; a < BS; ++a) {
        kbr[a] = kb_lds[t][ib * BS + a];
        vbr[a] = vb_lds[t][ib * BS + a];
        kr[a] = kh_lds[t][jb * BS + a];
      }
#pragma unroll
      for (int a = 0; a < BS; ++a)
#pragma unroll
        for (int b = 0; b < BS; ++b) {
          accA[a][b] = fmaf(kbr[a], kr[b], accA[a][b]);
          accB[a][b] = fmaf(vbr[a], kr[b], accB[a][b]);
        }
    }
    __syncthreads();
  }

  const long long mo = ((long long)bh * F + f) * D * D;
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) {
      long long e = mo + (long long)(ib * BS + a) * D + jb * BS + b;
      A[e] = accA[a][b];
      Bm[e] = accB[a][b];
    }
}

// ---------------------------------------------------------------- bf16 MFMA
// bf16 I/O: the two contractions over a frame's tokens run on MFMA
// (v_mfma_f32_32x32x16_bf16) as split-bf16 products. With
// k' = sqrt(beta) k^ and v' = sqrt(beta) v^:  A = K'^T K',  B = V'^T K'
// (for beta >= 0; a frame with a negative beta is overwritten afterwards by
// the fp32 kernel above).
// Waves in two roles per (b, h, frame), so that the feature VALU work and
// the MFMAs overlap:
//  - SX_PW(d) producer waves turn 64-token tiles into features (thread = 4
//    consecutive tokens x 4 channels; the conv reads raw rows held in
//    registers, fetched one tile ahead; the L2 norm is reduced with DPP over
//    the d/4 lanes that share the tokens) and store them channel-major
//    (hi, lo) to one of two LDS buffers;
//  - four consumer waves run the MFMAs of the previous tile from the other
//    buffer; each owns a quarter of the 32 x 32 output blocks (A, then B).
// One barrier per tile; both roles pass the same number of barriers.
// With vt set, the producers also write the raw v rows they hold transposed
// into vt ([d][Np] per (b, h), the softmax's V^T operand), which spares a
// separate transpose pass over v; this needs S % 4 == 0, so that every thread's
// 4 tokens lie inside the frame or outside it and its 8-byte stores are
// aligned.
constexpr int SX_TT = 64;  // tokens per tile
typedef unsigned v2u32_t __attribute__((ext_vector_type(2)));
// producer waves: d / 16 (4 channels x 4 tokens per thread over a 64-token tile)
__host__ __device__ constexpr int sx_pw(int d) { return d / 16; }

// sum over the 32 (W = 32) or 16 (W = 16) consecutive lanes of a row group,
// in every lane of it: DPP quad / half-mirror / mirror within each 16-lane
// row, then one exchange between the two rows of a 32-lane group
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, false));
}
template <int W>
__device__ __forceinline__ float row_group_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  if constexpr (W == 32) x += __shfl_xor(x, 16);
  return x;
}

template <int D>
__global__ __launch_bounds__(64 * (sx_pw(D) + 4)) void stats_mfma_kernel(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ conv_k,
    const float* __restrict__ conv_v, int conv, float* __restrict__ A,
    float* __restrict__ Bm, int F, int S, int H, long long N, bf16_t* __restrict__ vt,
    long long Np) {
  constexpr int NPW = sx_pw(D);      // producer waves
  constexpr int NP = 64 * NPW;       // producer threads
  constexpr int CG = D / 4;          // channel groups of 4
  constexpr int TG = NP / CG;        // token groups
  constexpr int TPG = SX_TT / TG;    // tokens per producer thread (8 or 4)
  constexpr int TP = SX_TT + 8;      // padded LDS row (tokens)
  constexpr int NB = D / 32;         // 32-wide blocks per dimension
  constexpr int BPW = 2 * NB * NB / 4;  // output blocks per consumer wave
  static_assert(TPG == 4, "token group");
  static_assert(CG == 32 || CG == 16, "channel groups span a 32- or 16-lane group");
  typedef __bf16 bf16xT_t __attribute__((ext_vector_type(TPG)));
  // [stage][k hi, k lo, v hi, v lo][channel][token]
  __shared__ __attribute__((aligned(16))) bf16_t buf[2][4][D * TP];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int f = blockIdx.x;
  const int bh = blockIdx.y;
  const int h = bh % H;
  const long long n0 = (long long)f * S;
  const int ntiles = (S + SX_TT - 1) / SX_TT;

  if (wave < NPW) {
    // ------------------------------------------------ producers: features
    const bf16_t* kp = k + (long long)bh * N * D;
    const bf16_t* vp = v + (long long)bh * N * D;
    const float* bp = beta + (long long)bh * N;
    const int tg = tid / CG, cg = tid % CG;
    const int c0 = cg * 4;
    float wk[4][4], wv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wk[i][j] = conv ? conv_k[((long long)h * D + c0 + i) * 4 + j] : (j == 0 ? 1.0f : 0.0f);
        wv[i][j] = conv ? conv_v[((long long)h * D + c0 + i) * 4 + j] : (j == 0 ? 1.0f : 0.0f);
      }
    // raw rows sb-3 .. sb+TPG-1 (4 channels each) of k and v, and beta of
    // rows sb .. sb+TPG-1, for one tile, fetched one tile ahead so the loads
    // overlap the feature work
    uint2 kraw[TPG + 3], vraw[TPG + 3];
    float braw[TPG];
    // the frame's rows through buffer descriptors sized to the frame: a row
    // before its start (a negative offset, past num_records as unsigned) or
    // past its end reads zeros, with no branch per row
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kp + n0 * D), 0, S * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vp + n0 * D), 0, S * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t brs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(bp + n0), 0, S * 4, 0x00020000);
    // this (b, h)'s transposed v, [d][Np] (fewer than 2^31 bytes, as the
    // softmax requires of it); unused without vt
    const __amdgpu_buffer_rsrc_t vts = __builtin_amdgcn_make_buffer_rsrc(
        vt ? (void*)(vt + (long long)bh * D * Np) : nullptr, 0, vt ? (int)(D * Np * 2) : 0,
        0x00020000);
    auto fetch = [&](int s0) {
      const int sb = s0 + tg * TPG;
#pragma unroll
      for (int u = 0; u < TPG; ++u) {
        int off = (sb + u) * 4;
        asm volatile("" : "+v"(off));  // the whole offset stays in the range check
        braw[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(brs, off, 0, 0));
      }
#pragma unroll
      for (int x = 0; x < TPG + 3; ++x) {
        int off = ((sb - 3 + x) * D + c0) * 2;
        asm volatile("" : "+v"(off));
        kraw[x] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(krs, off, 0, 0));
        vraw[x] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, 0));
      }
    };
    // causal width-4 conv of TPG tokens x 4 channels
    auto conv4 = [&](const uint2 (&raw)[TPG + 3], const float (&w)[4][4], float (&o)[TPG][4]) {
      float r[TPG + 3][4];
#pragma unroll
      for (int x = 0; x < TPG + 3; ++x) {
        r[x][0] = __uint_as_float(raw[x].x << 16);
        r[x][1] = __uint_as_float(raw[x].x & 0xffff0000u);
        r[x][2] = __uint_as_float(raw[x].y << 16);
        r[x][3] = __uint_as_float(raw[x].y & 0xffff0000u);
      }
#pragma unroll
      for (int u = 0; u < TPG; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) a = fmaf(w[i][j], r[u + 3 - j][i], a);
          o[u][i] = a;
        }
    };
    auto store = [&](int st, int arr, int i, const float (&x)[TPG]) {
      bf16xT_t hv, lv;
#pragma unroll
      for (int u = 0; u < TPG; ++u) {
        __bf16 hb, lb;
        split_bf16(x[u], hb, lb);
        hv[u] = hb;
        lv[u] = lb;
      }
      const int o = (c0 + i) * TP + tg * TPG;
      *(bf16xT_t*)&buf[st][arr][o] = hv;
      *(bf16xT_t*)&buf[st][arr + 1][o] = lv;
    };
    // features of the tile at token s0 -> LDS stage st; prefetches the next
    auto make = [&](int s0, int st) {
      float sqb[TPG];
#pragma unroll
      for (int u = 0; u < TPG; ++u) sqb[u] = __builtin_amdgcn_sqrtf(braw[u]);  // 0 past S
      float kf[TPG][4], vf[TPG][4];
      conv4(kraw, wk, kf);
      conv4(vraw, wv, vf);
      if (vt) {
        // raw v of this thread's tokens, channel by channel: rows 3..6 of
        // vraw hold tokens sb..sb+3, channels c0..c0+3 as two bf16 pairs;
        // a thread whose tokens lie past the frame stores out of range
        // (dropped)
        const int sb = s0 + tg * TPG;
        int off = sb < S ? (c0 * (int)Np + (int)n0 + sb) * 2 : (int)0x80000000;
        const int step = sb < S ? (int)Np * 2 : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t w0 = i < 2 ? vraw[3].x : vraw[3].y, w1 = i < 2 ? vraw[4].x : vraw[4].y;
          const uint32_t w2 = i < 2 ? vraw[5].x : vraw[5].y, w3 = i < 2 ? vraw[6].x : vraw[6].y;
          const uint2 val = make_uint2(__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w3, w2, sel));
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32_t, val), vts, off, 0, 0);
          off += step;
        }
      }
      // the next tile's rows (rows past the frame read zeros, so the last
      // tile fetches too)
      fetch(s0 + SX_TT);
      // k' = sqrt(beta) L2(SiLU(conv_k(k)))
      float ss[TPG];
#pragma unroll
      for (int u = 0; u < TPG; ++u) {
        ss[u] = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kf[u][i] = silu_f(kf[u][i]);
          ss[u] = fmaf(kf[u][i], kf[u][i], ss[u]);
        }
        ss[u] = sqb[u] * inv_l2(row_group_sum<CG>(ss[u]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[TPG], y[TPG];
#pragma unroll
        for (int u = 0; u < TPG; ++u) {
          x[u] = kf[u][i] * ss[u];
          y[u] = vf[u][i] * sqb[u];  // v' = sqrt(beta) conv_v(v)
        }
        store(st, 0, i, x);
        store(st, 2, i, y);
      }
    };
    if (vt && f == F - 1) {  // keys past N of the transposed v read as zeros
      const int pad = (int)(Np - N);
      for (int x = tid; x < D * pad; x += NP)
        vt[((long long)bh * D + x / pad) * Np + N + x % pad] = (bf16_t)0;
    }
    fetch(0);
    make(0, 0);
    __syncthreads();  // tile 0 is in stage 0
    for (int i = 0; i < ntiles; ++i) {
      if (i + 1 < ntiles) make((i + 1) * SX_TT, (i + 1) & 1);
      __syncthreads();
    }
  } else {
    // ------------------------------------------------ consumers: MFMAs
    const int cw = wave - NPW;
    const int half = lane >> 5, col = lane & 31;
    f32x16_t acc[BPW];
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;
    __syncthreads();  // tile 0 is in stage 0
    for (int i = 0; i < ntiles; ++i) {
      const int st = i & 1;
#pragma unroll
      for (int kk = 0; kk < SX_TT / 16; ++kk) {
        const int to = kk * 16 + half * 8;
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
          const int blk = cw * BPW + b;
          const int isB = blk / (NB * NB);
          const int ib = (blk / NB) % NB, jb = blk % NB;
          const int ra = (ib * 32 + col) * TP + to;
          const int rb = (jb * 32 + col) * TP + to;
          const bf16x8_t ah = *(const bf16x8_t*)&buf[st][isB ? 2 : 0][ra];
          const bf16x8_t al = *(const bf16x8_t*)&buf[st][isB ? 3 : 1][ra];
          const bf16x8_t bh8 = *(const bf16x8_t*)&buf[st][0][rb];
          const bf16x8_t bl8 = *(const bf16x8_t*)&buf[st][1][rb];
          acc[b] = mfma32x3(ah, al, bh8, bl8, acc[b]);
        }
      }
      __syncthreads();
    }
    // write: lane holds rows 8*(r/4) + 4*half + r%4, column col
    const long long mo = ((long long)bh * F + f) * D * D;
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      const int blk = cw * BPW + b;
      const int isB = blk / (NB * NB);
      const int ib = (blk / NB) % NB, jb = blk % NB;
      float* dst = (isB ? Bm : A) + mo;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = ib * 32 + (r / 4) * 8 + half * 4 + (r % 4);
        dst[(long long)i * D + jb * 32 + col] = acc[b][r];
      }
    }
  }
}

hipError_t launch_stats(const Geom& g, int dtype, const void* k,
                        const void* v, const float* beta, const float* conv_k,
                        const float* conv_v, bool conv, float* A, float* Bm,
                        hipStream_t st, bf16_t* v_t) {
  dim3 grid(g.F, g.B * g.H);
#define STATS_LAUNCH(TT, DD)                                                  \
  hipLaunchKernelGGL((stats_kernel<TT, DD>), grid, dim3(256), 0, st,          \
                     (const TT*)k, (const TT*)v, beta, conv_k, conv_v,        \
                     (int)conv, A, Bm, g.F, g.S, g.H, g.N, NEG_ONLY)
#define STATS_D(TT)                        \
  switch (g.d) {                           \
    case 16: STATS_LAUNCH(TT, 16); break;  \
    case 32: STATS_LAUNCH(TT, 32); break;  \
    case 64: STATS_LAUNCH(TT, 64); break;  \
    default: STATS_LAUNCH(TT, 128); break; \
  }
  if (dtype == HWA_BF16) {
    if (v_t && g.S % 4 != 0) return hipErrorInvalidValue;
    const long long Np = (g.N + 63) / 64 * 64;
#define SX_LAUNCH(DD)                                                        \
  hipLaunchKernelGGL(stats_mfma_kernel<DD>, grid, dim3(64 * (sx_pw(DD) + 4)), 0, st, \
                     (const bf16_t*)k, (const bf16_t*)v, beta, conv_k,       \
                     conv_v, (int)conv, A, Bm, g.F, g.S, g.H, g.N, v_t, Np)
    if (g.d == 128) SX_LAUNCH(128);
    else SX_LAUNCH(64);
#undef SX_LAUNCH
    // frames with a negative beta again, exactly
#define NEG_ONLY 1
    STATS_D(bf16_t)
#undef NEG_ONLY
  } else {
#define NEG_ONLY 0
    STATS_D(float)
#undef NEG_ONLY
  }
#undef STATS_D
#undef STATS_LAUNCH
  return hipGetLastError();
}

}  // namespace hwa
