// Windowed softmax branch (VDN-H3 article, "What the far field outside the
// window is"): query frame t attends to all tokens of key frames
// [lo_t, hi_t] with scale 1/sqrt(d), no mask inside the window.
//
// Because windows are chunk-aligned, every query of chunk c shares one key
// range [lo_c * S, (hi_c + 1) * S). A bf16 workgroup takes 256 consecutive
// queries of one chunk (the fp32 one 128; a tile may span frames of the
// chunk, never two chunks) and streams the chunk's key range through LDS in
// tiles of 64 keys (fp32: 32).
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16), per wave of 32 queries:
//   S^T[key][query] = K . Q^T  with K rows from LDS as the A operand and the
//                    wave's Q held in registers as the B operand;
//   O^T[d][query] += V^T . P^T  with V^T rows from LDS as the A operand and P
//                    (bf16) as the B operand straight from the S registers.
// Both products leave one query per lane (column n = lane % 32), so the
// online-softmax statistics and the O rescale are lane-local; the two lane
// halves hold different keys of the same query and meet once per tile for
// the running max and once at the end for the sum.
// K rows are loaded into the S MFMA in a permuted order so that each lane
// half ends up with 16 consecutive keys per 32-key block: the P registers are
// then directly the PV B operand and each V^T read is one 16-byte LDS load.
// V is read from a transposed copy V^T [B, H, d, Np] (Np = N rounded up to
// 64, zero padded) made by vtranspose_kernel.

#include <type_traits>

#include "hwa_internal.h"
#include "readout_core.h"
#include "attn_tile.h"

namespace hwa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int SM_NW = 8;                // waves per workgroup
constexpr int SM_QT = 32 * SM_NW;       // queries per workgroup
constexpr int SM_KT = 64;   // keys per LDS tile
constexpr int SM_THREADS = 64 * SM_NW;
// workgroups per XCD beyond its share of the tiles (four rounds of its 32
// CUs; measured at 132,600 tokens: 16 spare 1.3 % slower than 64, 128 and
// 256 within 0.3 % of it)
constexpr int SM_SPARE = 128;
#ifndef SM_PREFETCH
#define SM_PREFETCH 2
#endif
constexpr int SM_RB = 128;             // key block of the routed variant
constexpr int SM_ROUTE_TILES = 4096;   // kept tiles per window, at most

// ---------------------------------------------------------------- window table
__global__ void window_table_kernel(int F, int chunk, int radius,
                                    int32_t* lohi, unsigned* zero, int nzero) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (zero && t < nzero) zero[t] = 0u;  // work-queue counters of the softmax kernel
  if (t >= F) return;
  int lo, hi;
  window_of(t, F, chunk, radius, lo, hi);
  lohi[t] = lo;
  lohi[F + t] = hi;
}

hipError_t launch_window_table(const Geom& g, int32_t* lohi, hipStream_t st,
                               unsigned* sched) {
  int threads = 256;
  int blocks = (g.F + threads - 1) / threads;
  hipLaunchKernelGGL(window_table_kernel, dim3(blocks), dim3(threads), 0, st,
                     g.F, g.chunk, g.radius, lohi, sched, HWA_SCHED_WORDS);
  return hipGetLastError();
}

// ---------------------------------------------------------------- V transpose
// v [B,H,N,d] bf16 -> v_t [B,H,d,Np] bf16, keys >= N zero.
template <int D>
__global__ __launch_bounds__(256) void vtranspose_kernel(
    const bf16_t* __restrict__ v, bf16_t* __restrict__ vt, long long N,
    long long Np) {
  __shared__ bf16_t tile[64][D + 8];
  const int bh = blockIdx.y;
  const long long n0 = (long long)blockIdx.x * 64;
  const bf16_t* src = v + (long long)bh * N * D;
  bf16_t* dst = vt + (long long)bh * D * Np;
  constexpr int CH = 64 * D / 8;  // 16-byte chunks per tile
  for (int c = threadIdx.x; c < CH; c += 256) {
    int row = c / (D / 8), c8 = c % (D / 8);
    long long n = n0 + row;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (n < N) val = *(const u32x4*)(src + n * D + c8 * 8);
    *(u32x4*)(&tile[row][c8 * 8]) = val;
  }
  __syncthreads();
  constexpr int OCH = D * 8;  // output chunks: D rows x 8 chunks of 8 keys
  for (int c = threadIdx.x; c < OCH; c += 256) {
    int dr = c / 8, k8 = c % 8;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)tile[k8 * 8 + 2 * i][dr] |
             ((uint32_t)tile[k8 * 8 + 2 * i + 1][dr] << 16);
    u32x4 out = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(dst + (long long)dr * Np + n0 + k8 * 8) = out;
  }
}

hipError_t launch_vtranspose(const Geom& g, const bf16_t* v, bf16_t* v_t,
                             hipStream_t st) {
  long long Np = round_up64(g.N);
  dim3 grid((unsigned)(Np / 64), g.B * g.H);
  if (g.d == 128)
    hipLaunchKernelGGL(vtranspose_kernel<128>, grid, dim3(256), 0, st, v, v_t,
                       g.N, Np);
  else
    hipLaunchKernelGGL(vtranspose_kernel<64>, grid, dim3(256), 0, st, v, v_t,
                       g.N, Np);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bf16 MFMA
// LDS tiles are unpadded rows of 128 bytes (8 chunks of 16 bytes): V^T as
// [d][64 keys], K as [d / 64][64 rows][64 d] where LDS row m of the key tile
// holds key 32 * (m / 32) + perm32(m % 32). Row m keeps logical chunk c at
// chunk c ^ swz(m). For an MFMA operand read, lane (col, half) of step j takes
// row 32 * blk + col, chunk op_chunk(j, half); with this swizzle a wave's
// ds_read_b128 completes in the minimum four LDS cycles on gfx950 (measured:
// a 1 KB contiguous wave read, or the 256-byte-row layout, takes eight). The
// contraction index d is read in the same permuted chunk order for K and Q.
// Tiles are copied global -> LDS by the gfx950 direct load
// (buffer_load_dwordx4 ... lds: lane l of a wave writes its 16 bytes at
// dst + 16 * l); each lane fetches the global chunk that belongs in its slot.
//
// Software pipeline, per key tile i (K runs two tiles ahead of V): one
// stream of D/4 MFMA groups, S(i+1) = K(i+1) Q^T then O += V(i-1)^T P(i-1)^T,
// carrying the exp2 work of S(i), the lane max of S(i+1) and the direct loads
// K(i+2), V(i); then the running-max update, wait for the loads, barrier.
// Two K and two V stages (64 KB at d = 128); the loop is unrolled by two so
// that stage indices are compile-time. Eight waves (256 queries) share every
// tile; one workgroup per CU (two waves per SIMD).

// ROUTED: the block-sparse variant -- the workgroup streams only the 64-key
// tiles of the 128-key blocks its query tile kept (route.hip's lists), in
// increasing order; with every block kept it visits exactly the dense tiles.
template <int D, bool ROUTED>
__global__ __launch_bounds__(SM_THREADS, 1) void softmax_bf16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ vt, const int32_t* __restrict__ lohi,
    bf16_t* __restrict__ out, int F, int S, int chunk, int nch, long long N,
    long long Np, int tiles_per_chunk, float scale_log2, ReadoutArgs ra, int fuse,
    unsigned* __restrict__ sched, int ntiles_total, float* __restrict__ lse_out,
    bf16_t* __restrict__ sm_out, RouteArgs rt) {
  // the body uses device-only lambdas; the host pass needs only the stub
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KC = D / 8;          // 16-byte chunks per key
  constexpr int VC = SM_KT / 8;      // 16-byte chunks per V^T row
  constexpr int KINS = SM_KT * KC / 64;  // DMA instructions per K tile
  constexpr int VINS = D * VC / 64;      // DMA instructions per V^T tile
  constexpr int KPW = KINS / SM_NW;      // per wave
  constexpr int VPW = VINS / SM_NW;
  constexpr int NST = 2;                 // pipeline stages
  static_assert(KINS % SM_NW == 0 && VINS % SM_NW == 0, "uniform DMA per wave");
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[NST][SM_KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[NST][D * SM_KT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5;
  const int col = lane & 31;
  // Work queues. The logical tiles (head-major, then chunk, then query tile)
  // form 8 contiguous ranges, one per XCD (workgroup p runs on XCD p % 8), so
  // that the query tiles of one (head, chunk), which all stream the same key
  // range, share that XCD's L2. A workgroup takes the next tile of its XCD's
  // range from an atomic counter (sched[x], zero at launch) and, once that
  // range is empty, of the other ranges. The grid holds a few more workgroups
  // per XCD than its range has tiles: an XCD that runs faster than the others
  // then takes over their last tiles instead of idling at the end, and the
  // workgroups that find every range empty exit at once.
  __shared__ int next_tile;
  if (tid == 0) {
    const int xq = ntiles_total / 8, xr = ntiles_total % 8;
    const int home = blockIdx.x % 8;
    int lt = -1;
    for (int pr = 0; pr < 8; ++pr) {
      const int x = (home + pr) % 8;
      const unsigned i = atomicAdd(&sched[x], 1u);
      if (i < (unsigned)(xq + (x < xr ? 1 : 0))) {
        lt = x * xq + min(x, xr) + (int)i;
        break;
      }
    }
    next_tile = lt;
  }
  __syncthreads();
  const int L = __builtin_amdgcn_readfirstlane(next_tile);
  if (L < 0) return;
  const int per_bh = tiles_per_chunk * nch;
  const int bh = L / per_bh;
  const int c = (L % per_bh) / tiles_per_chunk;
  const int tile = L % tiles_per_chunk;

  const long long q_begin = (long long)c * chunk * S;
  const int f_end = min(F, (c + 1) * chunk);
  const long long q_end = (long long)f_end * S;
  const long long q_tile0 = q_begin + (long long)tile * SM_QT;
  if (q_tile0 >= q_end) return;  // partial last chunk: fewer tiles

  const int lo = lohi[c * chunk];
  const int hi = lohi[F + c * chunk];
  const long long k_begin = (long long)lo * S;
  const long long k_end = (long long)(hi + 1) * S;

  const bf16_t* qb = q + (long long)bh * N * D;
  const bf16_t* kb = k + (long long)bh * N * D;
  const bf16_t* vb = vt + (long long)bh * D * Np;

  // Q fragment: B operand of S^T = K Q^T, query = col; step kk takes the d
  // chunk 8 * (kk / 4) + op_chunk(kk % 4, half), as the K operand does
  const long long my_q = q_tile0 + wave * 32 + col;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 t = {0u, 0u, 0u, 0u};
    const int dc = 8 * (kk / 4) + op_chunk(kk % 4, half);
    if (my_q < N) t = *(const u32x4*)(qb + my_q * D + dc * 8);
    qreg[kk] = __builtin_bit_cast(bf16x8, t);
  }

  // per-lane DMA sources inside a tile (fixed for the whole kernel):
  // instruction wave + SM_NW*j fills slots 64*(wave + SM_NW*j) + lane
  // per-lane byte offsets inside a tile (fixed for the kernel): slot
  // (wave + SM_NW * j) * 64 + lane holds K row k_row, column k_col, resp. the
  // V^T element at row r, column chunk c of the tile
  int k_off[KPW], v_off[VPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int slot = (wave + SM_NW * j) * 64 + lane;
    const int sub = slot / 512, m = (slot / 8) % 64, pc = slot % 8;
    const int k_row = 32 * (m / 32) + perm32(m % 32);
    const int k_col = (8 * sub + (pc ^ swz(m))) * 8;
    k_off[j] = (k_row * D + k_col) * 2;
  }
#pragma unroll
  for (int j = 0; j < VPW; ++j) {
    const int slot = (wave + SM_NW * j) * 64 + lane;
    const int r = slot / VC, pc = slot % VC;
    v_off[j] = (r * (int)Np + (pc ^ swz(r)) * 8) * 2;
  }
  // buffer descriptor of a tile: base at the tile's first byte, num_records =
  // bytes left in this head (clamped to 32 bits), so K rows past N read zeros
  // (they are masked or never read); all fields wave-uniform
  // (a head holds fewer than 2^31 bytes on this path, which the ABI enforces,
  // so byte offsets fit in 32 unsigned bits even a few tiles past its end)
  auto tile_rsrc = [&] __device__(const bf16_t* head, long long head_elems, long long first)
                       __attribute__((always_inline)) {
    const unsigned long long base = (unsigned long long)(head + first);
    const unsigned hb = (unsigned)(head_elems * 2), fb = (unsigned)(first * 2);
    hwa_i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)(base & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(base >> 32));  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)(fb < hb ? hb - fb : 0u));
    r[3] = 0x00020000;  // raw buffer, 32-bit data format
    return r;
  };
  // direct loads of the K (resp. V^T) tile at key kt0 into stage st
  auto dma_k = [&] __device__(long long kt0, int st) __attribute__((always_inline)) {
    const hwa_i32x4 rs = tile_rsrc(kb, N * D, kt0 * D);
#pragma unroll
    for (int j = 0; j < KPW; ++j)
      hwa_raw_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)&k_lds[st][(wave + SM_NW * j) * 512],
                              16, k_off[j], 0, 0, 0);
  };
  auto dma_v = [&] __device__(long long kt0, int st) __attribute__((always_inline)) {
    const hwa_i32x4 rs = tile_rsrc(vb, (long long)D * Np, kt0);
#pragma unroll
    for (int j = 0; j < VPW; ++j)
      hwa_raw_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)&v_lds[st][(wave + SM_NW * j) * 512],
                              16, v_off[j], 0, 0, 0);
  };

  f32x16 acc_o[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[j][r] = 0.0f;
  // m_run may lag the true running max by up to 2^8 in exp2 units: p <= 256
  // stays exact in fp32/bf16 and the O rescale is only paid when it grows
  const float lag = 8.0f / scale_log2;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // LDS operand offsets (elements): step j of lane (col, half) reads row col,
  // chunk op_chunk(j, half) ^ swz(col) of a 32-row block of 128-byte rows;
  // K block blk, part kk / 4 and V^T block dblk add constant offsets, so each
  // operand read is one ds_read_b128 with a per-lane address and an immediate
  // offset (stage bases are compile-time: the loop is unrolled over stages)
  int voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) voff[j] = col * 64 + ((op_chunk(j, half) ^ swz(col)) * 8);
  auto k_op = [&] __device__(const bf16_t* ks, int blk, int kk) __attribute__((always_inline)) {
    return *(const bf16x8*)(ks + (kk / 4) * (SM_KT * 64) + blk * (32 * 64) + voff[kk % 4]);
  };
  auto v_op = [&] __device__(const bf16_t* vs, int dblk, int j) __attribute__((always_inline)) {
    return *(const bf16x8*)(vs + dblk * (32 * SM_KT) + voff[j]);
  };
  auto qk_full = [&] __device__(const bf16_t* ks, f32x16 (&sv)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[blk][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        sv[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            k_op(ks, blk, kk), qreg[kk], sv[blk], 0, 0, 0);
    }
  };

  const long long kt_first = k_begin / SM_KT * SM_KT;
  int ntiles = (int)((k_end - kt_first + SM_KT - 1) / SM_KT);
  // routed: the kept tiles (offsets from kt_first in tiles); the halves of a
  // kept block that lie outside the window are left out
  __shared__ uint16_t tlist[ROUTED ? SM_ROUTE_TILES : 1];
  __shared__ int tlist_n;
  if constexpr (ROUTED) {
    if (tid == 0) {
      const long long slot = ((long long)bh * nch + c) * tiles_per_chunk + tile;
      const int cnt = rt.count[slot];
      const uint16_t* lst = rt.list + slot * rt.nkb_max;
      const long long jfirst = k_begin / SM_RB;
      int n = 0;
      for (int i = 0; i < cnt; ++i) {
        const long long key0 = (jfirst + lst[i]) * SM_RB;
        for (int h = 0; h < SM_RB / SM_KT; ++h) {
          const long long tk = key0 + (long long)h * SM_KT;
          if (tk + SM_KT > k_begin && tk < k_end && n < SM_ROUTE_TILES)
            tlist[n++] = (uint16_t)((tk - kt_first) / SM_KT);
        }
      }
      tlist_n = n;
    }
    __syncthreads();
    ntiles = __builtin_amdgcn_readfirstlane(tlist_n);
  }
  // first key of tile `it` of this workgroup's sequence
  auto tile_key = [&] __device__(int it) __attribute__((always_inline)) -> long long {
    if constexpr (ROUTED) return kt_first + (long long)tlist[it] * SM_KT;
    else return kt_first + (long long)it * SM_KT;
  };

  // keys of tile `it` outside [k_begin, k_end) score -inf (first and last
  // tile only); returns whether the tile needed it
  auto mask = [&] __device__(int it, f32x16 (&sv)[2]) __attribute__((always_inline)) {
    const long long kt = tile_key(it);
    const int lo_rel = (int)(k_begin - kt);  // keys before lo_rel and
    const int hi_rel = (int)(k_end - kt);    // from hi_rel on are out
    if (lo_rel <= 0 && hi_rel >= SM_KT) return false;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = blk * 32 + half * 16 + r;
        if (key < lo_rel || key >= hi_rel) sv[blk][r] = -INFINITY;
      }
    return true;
  };
  auto lane_max = [&] __device__(const f32x16 (&sv)[2]) __attribute__((always_inline)) {
    float mx = fmaxf(sv[0][0], sv[0][1]);
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(fmaxf(mx, sv[e / 8][(2 * e) % 16]), sv[e / 8][(2 * e) % 16 + 1]);
    return mx;
  };
  // running max from a lane's partial max over its 32 scores of a tile (the
  // lane pair l, l ^ 32 shares the query): m_run moves only when the tile max
  // passes it by more than the lag; corr rescales l_run now and O after the
  // next PV, when `moved`
  float corr = 1.0f;
  bool moved = false;
  auto update_max = [&] __device__(float mx) __attribute__((always_inline)) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float m_new = mx > m_run + lag ? fmaxf(m_run, mx) : m_run;
    corr = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
    moved = m_new != m_run;
    m_run = m_new;
    l_run *= corr;
  };

  // One pipeline step i (stage indices are compile-time: SI = i % 2), one
  // stream of D/4 MFMA groups: S(i+1) = K(i+1) Q^T (D/8 groups), then
  // O += V(i-1)^T P(i-1)^T (D/8 groups, consecutive ones on different
  // accumulators). Riding on the groups: the 16 probability pairs of S(i)
  // (exp2, bf16 P(i), row sums), the direct loads K(i+2) -> K[i%2] and
  // V(i) -> V[i%2] (needed in step i+1), and the lane max of S(i+1) once its
  // MFMAs are done. Then: the pending O rescale (after PV(i-1)), the running
  // max update for S(i+1), wait for this step's loads, barrier.
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  constexpr int NQK = D / 8, NG = D / 4, EVERY = NG / 16;
  static_assert(NG % 16 == 0, "16 probability pairs over the MFMA groups");
  constexpr int G_MAX = NQK + 2;  // first group that reads the finished S(i+1)
  constexpr int PF = SM_PREFETCH;
  auto step = [&] __device__(auto si_tag, int it, f32x16 (&sc)[2], f32x16 (&sn)[2],
                             bf16x8 (&pp)[4], bf16x8 (&pc)[4])
                   __attribute__((always_inline)) {
    constexpr int SI = decltype(si_tag)::value;
    constexpr int SO = SI ^ 1;  // K(i+1) and V(i-1)
    // K(i+2) (past the last tile: the last one again, which nothing reads)
    // and V(i)
    const long long kt0 = tile_key(it);
    const long long kt2 = ROUTED ? tile_key(min(it + 2, ntiles - 1)) : kt0 + 2 * SM_KT;
    const bf16_t* ks = &k_lds[SO][0];
    const bf16_t* vs = &v_lds[SO][0];
    const float mb = m_run * scale_log2;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[blk][r] = 0.0f;
    float mx = -INFINITY;
    // operands are read PF groups ahead of their MFMA
    bf16x8 opa[PF + 1];
    auto op_read = [&] __device__(int gn) __attribute__((always_inline)) {
      if (gn < NQK) return k_op(ks, gn % 2, gn / 2);
      return v_op(vs, (gn - NQK) % (D / 32), (gn - NQK) / (D / 32));
    };
#pragma unroll
    for (int g = 0; g < PF; ++g) opa[g] = op_read(g);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      // operand read for group g + PF (QK groups 0..NQK-1, PV groups after)
      if (g + PF < NG) opa[(g + PF) % (PF + 1)] = op_read(g + PF);
      // this step's direct loads: waves 0..3 issue theirs with group 0, waves
      // 4..7 at mid-step, so the eight waves' loads do not queue up at once
      // (K(i+2) past the last tile loads rows that nothing reads)
      if (g == 0 || g == NG / 2) {
        if ((wave < SM_NW / 2) == (g == 0)) {
          dma_k(kt2, SI);
          dma_v(kt0, SI);
        }
      }
      if (g < NQK) {
        sn[g % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[g % (PF + 1)], qreg[g / 2],
                                                            sn[g % 2], 0, 0, 0);
      } else {  // PV(i-1); in step 0 it multiplies P = 0 by a zeroed stage
        const int dblk = (g - NQK) % (D / 32), j = (g - NQK) / (D / 32);
        acc_o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[g % (PF + 1)], pp[j],
                                                              acc_o[dblk], 0, 0, 0);
      }
      if (g % EVERY == EVERY - 1) {
        const int e = g / EVERY, blk = e / 8, r = (e % 8) * 2;
        // the empty volatile asm statements pin this pair between the MFMAs of
        // its group: instruction selection may otherwise move pure arithmetic
        // across the (memory-ordered) scheduling barriers
        f32x2 s01 = {sc[blk][r], sc[blk][r + 1]};
        asm volatile("" : "+v"(s01));
        const f32x2 e2 = {__builtin_amdgcn_exp2f(fmaf(s01[0], scale_log2, -mb)),
                          __builtin_amdgcn_exp2f(fmaf(s01[1], scale_log2, -mb))};
        bf16x2_t p2 = __builtin_convertvector(e2, bf16x2_t);
        asm volatile("" : "+v"(p2));
        pc[blk * 2 + r / 8][r % 8] = p2[0];
        pc[blk * 2 + r / 8][r % 8 + 1] = p2[1];
        l_run = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_run, false);
      }
      if (g >= G_MAX) {  // lane max of S(i+1): 16 pairs over groups G_MAX..NG-1
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (G_MAX + (e * (NG - G_MAX)) / 16 == g)
            mx = fmaxf(fmaxf(mx, sn[e / 8][(2 * e) % 16]), sn[e / 8][(2 * e) % 16 + 1]);
        asm volatile("" : "+v"(mx));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- rare: rescale O (which now includes PV(i-1)) when the max moved
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[j][r] *= corr;
    }
    if (it + 1 < ntiles) {
      if (mask(it + 1, sn)) mx = lane_max(sn);  // first or last tile only
      update_max(mx);
    }
    // this step's loads are needed by the next step
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // prologue: K(0), K(1) land; S(0) and its max
  f32x16 sa[2], sb[2];
  bf16x8 pa[4], pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int u = 0; u < 8; ++u) pb[j][u] = (__bf16)0.0f;  // P(-1)
  // V stage 1 is read (times P = 0) by step 0's PV: make it finite
  for (int x = tid; x < D * SM_KT / 8; x += SM_THREADS)
    *(u32x4*)&v_lds[1][x * 8] = u32x4{0u, 0u, 0u, 0u};
  // fused readout: S_t of the tile's first frame goes into LDS now, while the
  // first key tiles load (the main loop leaves that LDS alone)
  __shared__ ReadoutLds<D> rl;
  const int t_first = (int)(q_tile0 / S);
  StateChunks<D, SM_THREADS> stc;  // S_t of a frame, global -> registers -> LDS
  if (fuse) stc.load(ra.st + ((long long)bh * ra.F + t_first) * D * D, tid);
  dma_k(tile_key(0), 0);
  if (ntiles > 1) dma_k(tile_key(1), 1);
  if (fuse) {
    load_weight<D, SM_THREADS>(rl, ra.rms_w, tid);
    stc.store(rl, tid);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // A wave whose 32 queries all lie past the chunk's end (the last, partial
  // tile of a chunk) only loads its share of every tile and keeps the
  // barriers: the other wave on its SIMD then has the matrix core alone.
  const bool wave_active = q_tile0 + wave * 32 < q_end;  // wave-uniform
  if (wave_active) {
  qk_full(&k_lds[0][0], sa);
  __syncthreads();  // K stage 0 is refilled in step 0
  mask(0, sa);
  update_max(lane_max(sa));
  typedef std::integral_constant<int, 0> S0;
  typedef std::integral_constant<int, 1> S1;
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(S0{}, it, sa, sb, pb, pa);
    step(S1{}, it + 1, sb, sa, pa, pb);
  }
  if (it < ntiles) step(S0{}, it, sa, sb, pb, pa);
  // drain: O += V(last)^T P(last)^T (P of even tiles is in pa, odd in pb)
  {
    const int last = ntiles - 1;
    const bf16_t* vs = &v_lds[last % NST][0];
    auto drain = [&] __device__(const bf16x8(&pl)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc_o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_op(vs, dblk, j), pl[j],
                                                                acc_o[dblk], 0, 0, 0);
    };
    if (last % 2 == 0) drain(pa);
    else drain(pb);
  }
  } else {
    // the same loads and barriers as a step of the active waves
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const long long kt0 = tile_key(it);
      dma_k(ROUTED ? tile_key(min(it + 2, ntiles - 1)) : kt0 + 2 * SM_KT, it & 1);
      dma_v(kt0, it & 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- normalise: lane holds d = 32*dblk + 8*(r/4) + 4*half + r%4, as bf16
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  // log sum_m exp(s_m / sqrt(d)) = (m_run * scale_log2 + log2(l_tot)) * ln 2
  if (lse_out && half == 0 && my_q < q_end)
    lse_out[(long long)bh * N + my_q] =
        (m_run * scale_log2 + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f;
  uint2 osm[D / 32][4];
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x2 a2 = {acc_o[dblk][g4 * 4 + 0] * inv, acc_o[dblk][g4 * 4 + 1] * inv};
      const f32x2 b2 = {acc_o[dblk][g4 * 4 + 2] * inv, acc_o[dblk][g4 * 4 + 3] * inv};
      osm[dblk][g4] = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(a2, bf16x2)),
                                 __builtin_bit_cast(uint32_t, __builtin_convertvector(b2, bf16x2)));
    }
  bf16_t* orow = out + (long long)bh * N * D + my_q * D;
  if (sm_out && my_q < q_end) {
    bf16_t* srow = sm_out + (long long)bh * N * D + my_q * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(uint2*)(srow + dblk * 32 + g4 * 8 + half * 4) = osm[dblk][g4];
  }
  if (!fuse) {
    if (my_q < q_end) {
#pragma unroll
      for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(uint2*)(orow + dblk * 32 + g4 * 8 + half * 4) = osm[dblk][g4];
    }
    return;
  }

  // ---- fused linear-branch readout: out = o_sm + y, frame by frame (a tile
  // of SM_QT queries spans at most two frames when S >= SM_QT; in general
  // every frame from the first query's to the last's). q^ comes from the raw
  // q in the chunk order of the QK operand: qreg itself, or, when the softmax
  // ran on a rotated q, the raw rows loaded here in that order; S_t's columns
  // are read in the same order.
  // chunk kk of the lane half: channels 8 * (8 * (kk / 4) + op_chunk(kk % 4, half)),
  // a lane part 16 * half plus a compile-time part
  struct KOff {
    static constexpr int at(int kk) { return 64 * (kk / 4) + 32 * ((kk % 4) / 2) + 8 * (kk % 2); }
  };
  const int qlane = 16 * half;
  u32x4 qraw[D / 16];
  if (ra.q_raw) {
    const bf16_t* qrow = ra.q_raw + (long long)bh * N * D + my_q * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int dc = 8 * (kk / 4) + op_chunk(kk % 4, half);
      qraw[kk] = my_q < N ? *(const u32x4*)(qrow + dc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qraw[kk] = __builtin_bit_cast(u32x4, qreg[kk]);
  }
  const long long q_last = min(q_tile0 + SM_QT, q_end) - 1;
  const int t_last = (int)(q_last / S);
  const int my_t = my_q < q_end ? (int)(my_q / S) : -1;
  // the gate rows of the tile's queries go to the K/V stage LDS (free after
  // the drain) by direct loads, alongside S_t of the first frame:
  // 16-byte chunk c of row r sits at slot r*CH + (c ^ (r % CH)); rows past
  // the head's end read zeros (never used)
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int KSLOTS = NST * SM_KT * D / 8;   // 16-byte slots in k_lds
  constexpr int GPW = SM_QT * CH / 64 / SM_NW;  // load instructions per wave
  static_assert(SM_QT * CH == 2 * KSLOTS, "the gate tile fills the K and V stages");
  __syncthreads();  // every wave is done reading the K/V stages
  {
    const hwa_i32x4 rs = tile_rsrc(ra.gate + (long long)bh * N * D, N * D, q_tile0 * D);
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      const int s0 = (wave + SM_NW * j) * 64;  // first slot of this instruction
      const int slot = s0 + lane;
      const int r = slot / CH, c = (slot % CH) ^ (r % CH);
      bf16_t* dst = s0 < KSLOTS ? &k_lds[0][0] + s0 * 8 : &v_lds[0][0] + (s0 - KSLOTS) * 8;
      hwa_raw_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16,
                              (r * D + c * 8) * 2, 0, 0, 0);
    }
  }
  auto gate_at = [&] __device__(int ib, int g4) __attribute__((always_inline)) {
    const int r = wave * 32 + col, c = ib * 4 + g4;
    const int slot = r * CH + (c ^ (r % CH));
    const bf16_t* src = slot < KSLOTS ? &k_lds[0][0] + slot * 8 : &v_lds[0][0] + (slot - KSLOTS) * 8;
    return *(const uint2*)(src + half * 4);
  };
  for (int t = t_first; t <= t_last; ++t) {
    // S_t of the first frame is in LDS since the prologue
    if (t > t_first) {
      stc.load(ra.st + ((long long)bh * ra.F + t) * D * D, tid);
      stc.store(rl, tid);
    }
    const float eps_s = ra.st_eps[(long long)bh * ra.F + t];
    // S_t and, the first time, every wave's gate rows have landed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool mine = my_t == t;
    if (__builtin_amdgcn_ballot_w64(mine) != 0)
      readout_token<D, KOff>(rl, eps_s, qraw, qlane, mine, orow, [&]() {}, gate_at,
                       [&](int ib, int g4) { return osm[ib][g4]; });
    __syncthreads();  // S_t of the next frame overwrites rl
  }
#endif
}

// ---------------------------------------------------------------- fp32 VALU
// One thread per query, keys staged in LDS 32 at a time. Used for the fp32
// dtype (small exactness workloads); full fp32 products and accumulation.
template <int D>
__global__ __launch_bounds__(128) void softmax_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const int32_t* __restrict__ lohi,
    float* __restrict__ out, int F, int S, int chunk, long long N,
    int tiles_per_chunk, float scale_log2, float* __restrict__ lse_out,
    float* __restrict__ sm_out) {
  constexpr int QT = 128, KT = 32;
  __shared__ float k_lds[KT][D];
  __shared__ float v_lds[KT][D];
  const int tid = threadIdx.x;
  const int c = blockIdx.x / tiles_per_chunk;
  const int tile = blockIdx.x % tiles_per_chunk;
  const int bh = blockIdx.y;
  const long long q_begin = (long long)c * chunk * S;
  const long long q_end = (long long)min(F, (c + 1) * chunk) * S;
  const long long q0 = q_begin + (long long)tile * QT;
  if (q0 >= q_end) return;
  const long long k_begin = (long long)lohi[c * chunk] * S;
  const long long k_end = (long long)(lohi[F + c * chunk] + 1) * S;
  const float* qb = q + (long long)bh * N * D;
  const float* kb = k + (long long)bh * N * D;
  const float* vb = v + (long long)bh * N * D;
  const long long my_q = q0 + tid;
  const bool valid = my_q < q_end;

  float qr[D], o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qr[i] = valid ? qb[my_q * D + i] : 0.0f;
    o[i] = 0.0f;
  }
  float m_run = -INFINITY, l_run = 0.0f;
  for (long long kt0 = k_begin; kt0 < k_end; kt0 += KT) {
    for (int e = tid; e < KT * D; e += QT) {
      int r = e / D, cc = e % D;
      long long n = kt0 + r;
      bool in = n < k_end;
      k_lds[r][cc] = in ? kb[n * D + cc] : 0.0f;
      v_lds[r][cc] = in ? vb[n * D + cc] : 0.0f;
    }
    __syncthreads();
    const int nk = (int)min((long long)KT, k_end - kt0);
    float s[KT];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) acc = fmaf(qr[i], k_lds[j][i], acc);
      s[j] = j < nk ? acc : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
    m_run = m_new;
    l_run *= corr;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] *= corr;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float p = __builtin_amdgcn_exp2f((s[j] - m_new) * scale_log2);
      l_run += p;
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] = fmaf(p, v_lds[j][i], o[i]);
    }
    __syncthreads();
  }
  if (valid) {
    float inv = 1.0f / l_run;
    float* orow = out + (long long)bh * N * D + my_q * D;
#pragma unroll
    for (int i = 0; i < D; ++i) orow[i] = o[i] * inv;
    if (sm_out) {
      float* srow = sm_out + (long long)bh * N * D + my_q * D;
#pragma unroll
      for (int i = 0; i < D; ++i) srow[i] = o[i] * inv;
    }
    // log sum_m exp(s_m / sqrt(d)); m_run is a raw score q.k
    if (lse_out)
      lse_out[(long long)bh * N + my_q] = m_run * (scale_log2 * 0.6931471805599453f) + logf(l_run);
  }
}

hipError_t launch_softmax(const Geom& g, int dtype, const void* q,
                          const void* k, const void* v, const bf16_t* v_t,
                          const int32_t* lohi, void* out, hipStream_t st,
                          const ReadoutArgs* fuse, unsigned* sched, float* lse,
                          void* sm_out, const RouteArgs* route) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)g.d);
  const int qpc = g.chunk * g.S;  // queries of a full chunk
  if (dtype == HWA_BF16) {
    const int tpc = (qpc + SM_QT - 1) / SM_QT;
    const int ntiles = tpc * g.nch * g.B * g.H;
    // SM_SPARE extra workgroups per XCD take over tiles from slower XCDs
    dim3 grid(ntiles + 8 * SM_SPARE);
    const long long Np = round_up64(g.N);
    const ReadoutArgs ra = fuse ? *fuse : ReadoutArgs{};
    const RouteArgs rt = route ? *route : RouteArgs{};
#define SM_LAUNCH(DD, RR)                                                        \
  hipLaunchKernelGGL((softmax_bf16_kernel<DD, RR>), grid, dim3(SM_THREADS), 0, st, \
                     (const bf16_t*)q, (const bf16_t*)k, v_t, lohi,              \
                     (bf16_t*)out, g.F, g.S, g.chunk, g.nch, g.N, Np, tpc,       \
                     scale_log2, ra, fuse ? 1 : 0, sched, ntiles, lse,           \
                     (bf16_t*)sm_out, rt)
    if (g.d == 128) {
      if (route) SM_LAUNCH(128, true); else SM_LAUNCH(128, false);
    } else {
      if (route) SM_LAUNCH(64, true); else SM_LAUNCH(64, false);
    }
#undef SM_LAUNCH
  } else {
    const int tpc = (qpc + 127) / 128;
    dim3 grid(tpc * g.nch, g.B * g.H);
#define SF_LAUNCH(DD)                                                          \
  hipLaunchKernelGGL(softmax_f32_kernel<DD>, grid, dim3(128), 0, st,           \
                     (const float*)q, (const float*)k, (const float*)v, lohi,  \
                     (float*)out, g.F, g.S, g.chunk, g.N, tpc, scale_log2,     \
                     lse, (float*)sm_out)
    switch (g.d) {
      case 16: SF_LAUNCH(16); break;
      case 32: SF_LAUNCH(32); break;
      case 64: SF_LAUNCH(64); break;
      default: SF_LAUNCH(128); break;
    }
#undef SF_LAUNCH
  }
  return hipGetLastError();
}

}  // namespace hwa
