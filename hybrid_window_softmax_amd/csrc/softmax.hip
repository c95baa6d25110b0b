// Windowed softmax branch (VDN-H3 article, "What the far field outside the
// window is"): query frame t attends to all tokens of key frames
// [lo_t, hi_t] with scale 1/sqrt(d), no mask inside the window.
//
// Because windows are chunk-aligned, every query of chunk c shares one key
// range [lo_c * S, (hi_c + 1) * S). A workgroup takes 128 consecutive queries
// of one chunk (a tile may span frames of the chunk, never two chunks) and
// streams the chunk's key range through LDS in tiles of 64 keys.
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

#include "hwa_internal.h"

namespace hwa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int SM_NW = 8;                // waves per workgroup
constexpr int SM_QT = 32 * SM_NW;       // queries per workgroup
constexpr int SM_KT = 64;   // keys per LDS tile
constexpr int SM_THREADS = 64 * SM_NW;

__host__ __device__ inline long long round_up64(long long n) {
  return (n + 63) / 64 * 64;
}

// ---------------------------------------------------------------- window table
__global__ void window_table_kernel(int F, int chunk, int radius,
                                    int32_t* lohi) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= F) return;
  int lo, hi;
  window_of(t, F, chunk, radius, lo, hi);
  lohi[t] = lo;
  lohi[F + t] = hi;
}

hipError_t launch_window_table(const Geom& g, int32_t* lohi, hipStream_t st) {
  int threads = 256;
  int blocks = (g.F + threads - 1) / threads;
  hipLaunchKernelGGL(window_table_kernel, dim3(blocks), dim3(threads), 0, st,
                     g.F, g.chunk, g.radius, lohi);
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
// Row of the 32-row MFMA block that lands on "16 consecutive keys per lane
// half": MFMA output row m is held by lane half (m / 4) % 2 in register
// 4 * (m / 8) + m % 4; loading tile key perm32(m) into row m makes register r
// of half h hold key 16 * h + r.
__device__ __forceinline__ int perm32(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// LDS tiles are unpadded and XOR-swizzled by 16-byte chunk: K row r keeps
// logical chunk c at chunk c ^ swz_k(r), V^T row r at c ^ swz_v(r). The
// swizzles make the 16 lanes of every LDS pass of an MFMA operand read hit 16
// distinct bank groups. Tiles are copied global -> LDS by the gfx950 direct
// load (global_load_lds_dwordx4: lane l of a wave writes its 16 bytes at
// dst + 16 * l); each lane fetches the global chunk that belongs in its slot.
//
// Software pipeline, per wave and key tile i (K runs one tile ahead of V):
//   issue DMA K(i+3), V(i+2);  S(i+1) = K(i+1) Q^T (MFMA) interleaved with
//   the exp2 work of S(i);  O += V(i)^T P(i)^T;  wait for the DMA issued one
//   step earlier; barrier.
// Three K and three V stages (96 KB at d = 128): loads have a whole step to
// land. Eight waves (256 queries) share every tile; one workgroup per CU.
__device__ __forceinline__ int swz_k(int r, int chunks) {
  return chunks == 16 ? ((r + 8 * (r >> 4)) & 15) : (((r >> 1) + 4 * (r >> 4)) & 7);
}
__device__ __forceinline__ int swz_v(int r) { return (r >> 1) & 7; }

// s_waitcnt vmcnt(n) for a small run-time n (the immediate must be constant)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
  }
}

template <int D>
__global__ __launch_bounds__(SM_THREADS, 1) void softmax_bf16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ vt, const int32_t* __restrict__ lohi,
    bf16_t* __restrict__ out, int F, int S, int chunk, int nch, long long N,
    long long Np, int tiles_per_chunk, float scale_log2) {
  // the body uses device-only lambdas; the host pass needs only the stub
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KC = D / 8;          // 16-byte chunks per K row
  constexpr int VC = SM_KT / 8;      // 16-byte chunks per V^T row
  constexpr int KINS = SM_KT * KC / 64;  // DMA instructions per K tile
  constexpr int VINS = D * VC / 64;      // DMA instructions per V^T tile
  constexpr int KPW = KINS / SM_NW;      // per wave
  constexpr int VPW = VINS / SM_NW;
  constexpr int NST = 3;                 // pipeline stages
  static_assert(KINS % SM_NW == 0 && VINS % SM_NW == 0, "uniform DMA per wave");
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[NST][SM_KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[NST][D * SM_KT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  // XCD-aware order: workgroup p is dispatched to XCD p % 8; give each XCD a
  // contiguous run of logical tiles so that the query tiles of one (head,
  // chunk), which all stream the same key range, share that XCD's L2
  const int G = gridDim.x;
  const int p = blockIdx.x;
  const int xq = G / 8, xr = G % 8, xcd = p % 8;
  const int L = xcd * xq + min(xcd, xr) + p / 8;
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

  // Q fragment: B operand of S^T = K Q^T, query = col, d = 16*kk + 8*half + i
  const long long my_q = q_tile0 + wave * 32 + col;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 t = {0u, 0u, 0u, 0u};
    if (my_q < N) t = *(const u32x4*)(qb + my_q * D + kk * 16 + half * 8);
    qreg[kk] = __builtin_bit_cast(bf16x8, t);
  }

  // per-lane DMA sources inside a tile (fixed for the whole kernel):
  // instruction wave + SM_NW*j fills slots 64*(wave + SM_NW*j) + lane
  int k_row[KPW], k_col[KPW], v_off[VPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int slot = (wave + SM_NW * j) * 64 + lane;
    const int r = slot / KC, pc = slot % KC;
    k_row[j] = r;
    k_col[j] = (pc ^ swz_k(r, KC)) * 8;
  }
#pragma unroll
  for (int j = 0; j < VPW; ++j) {
    const int slot = (wave + SM_NW * j) * 64 + lane;
    const int r = slot / VC, pc = slot % VC;
    v_off[j] = r * (int)Np + (pc ^ swz_v(r)) * 8;
  }
  auto dma_k = [&] __device__(long long kt0, int st) {
    const bool whole = kt0 + SM_KT <= N;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      long long n = kt0 + k_row[j];
      if (!whole) n = n < N ? n : N - 1;  // rows past N: any valid row, masked
      __builtin_amdgcn_global_load_lds(kb + n * D + k_col[j],
                                       &k_lds[st][(wave + SM_NW * j) * 512], 16, 0, 0);
    }
  };
  auto dma_v = [&] __device__(long long kt0, int st) {
#pragma unroll
    for (int j = 0; j < VPW; ++j)
      __builtin_amdgcn_global_load_lds(vb + kt0 + v_off[j],
                                       &v_lds[st][(wave + SM_NW * j) * 512], 16, 0, 0);
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

  // LDS operand reads: K row (blk*32 + perm32(col)), logical chunk 2*kk + half;
  // V^T row (dblk*32 + col), logical chunk 2*half + 4*(j/2) + (j%2)
  const int kr0 = perm32(col), kr1 = 32 + perm32(col);
  const int ksw0 = swz_k(kr0, KC), ksw1 = swz_k(kr1, KC);
  auto kop = [&] __device__(int st, int blk, int kk) {
    const int r = blk ? kr1 : kr0, sw = blk ? ksw1 : ksw0;
    return *(const bf16x8*)&k_lds[st][r * D + (((2 * kk + half) ^ sw) * 8)];
  };
  auto vop = [&] __device__(int st, int dblk, int j) {
    const int r = dblk * 32 + col;
    const int lc = 2 * half + 4 * (j / 2) + (j % 2);
    return *(const bf16x8*)&v_lds[st][r * SM_KT + ((lc ^ swz_v(r)) * 8)];
  };
  auto qk = [&] __device__(int st, f32x16 (&sv)[2]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[blk][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        sv[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop(st, blk, kk), qreg[kk],
                                                          sv[blk], 0, 0, 0);
    }
  };

  const long long kt_first = k_begin / SM_KT * SM_KT;
  const int ntiles = (int)((k_end - kt_first + SM_KT - 1) / SM_KT);

  // one pipeline step: consumes scores sc of tile it, produces sn of tile it+1
  auto step = [&] __device__(int it, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    const int sv = it % NST;            // V(it)
    const int sk = (it + 1) % NST;      // K(it+1)
    const long long kt0 = kt_first + (long long)it * SM_KT;
    int issued = 0;
    if (it + 3 < ntiles) { dma_k(kt0 + 3 * SM_KT, it % NST); issued += KPW; }
    if (it + 2 < ntiles) { dma_v(kt0 + 2 * SM_KT, (it + 2) % NST); issued += VPW; }
    // ---- mask keys outside [k_begin, k_end) (first and last tile only)
    if (kt0 < k_begin || kt0 + SM_KT > k_end) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const long long key = kt0 + blk * 32 + half * 16 + r;
          if (key < k_begin || key >= k_end) sc[blk][r] = -INFINITY;
        }
    }
    // ---- running max of S(i); m_run may lag the true one by up to 2^8 in
    // exp2 units (p <= 256 stays exact) and moves only past that lag, so
    // the O rescale below is rare
    float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, sc[0][r]), sc[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = mx > m_run + lag ? fmaxf(m_run, mx) : m_run;
    const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
    if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[j][r] *= corr;
    }
    m_run = m_new;
    l_run *= corr;
    const float mb = m_run * scale_log2;

    // ---- the MFMAs of S(i+1) (on the last tile they read a stale stage and
    // are discarded) interleaved by hand with exp2 of S(i): group g issues
    // the LDS read of the K operand of group g + 2, the MFMA of group g and
    // one pair of probabilities (2 exp2, bf16 pack, row-sum dot2); the
    // sched_barrier fences keep the compiler from regrouping them, so the
    // VALU work fills the MFMA pipeline's issue gaps.
    constexpr int NG = 2 * (D / 16);  // QK MFMAs per tile (16 at d = 128)
    bf16x8 ka[3];
    ka[0] = kop(sk, 0, 0);
    ka[1] = kop(sk, 1, 0);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[blk][r] = 0.0f;
    bf16x8 pb[4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {  // g: blk = g % 2, kk = g / 2
      if (g + 2 < NG) ka[(g + 2) % 3] = kop(sk, (g + 2) % 2, (g + 2) / 2);
      sn[g % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[g % 3], qreg[g / 2],
                                                          sn[g % 2], 0, 0, 0);
#pragma unroll
      for (int e = g * 16 / NG; e < (g + 1) * 16 / NG; ++e) {
        const int blk = e / 8, r = (e % 8) * 2;
        const f32x2 e2 = {
            __builtin_amdgcn_exp2f(fmaf(sc[blk][r], scale_log2, -mb)),
            __builtin_amdgcn_exp2f(fmaf(sc[blk][r + 1], scale_log2, -mb))};
        const bf16x2 p2 = __builtin_convertvector(e2, bf16x2);
        pb[blk * 2 + r / 8][r % 8] = p2[0];
        pb[blk * 2 + r / 8][r % 8 + 1] = p2[1];
        l_run = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_run, false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- O^T += V^T P^T: P block j holds keys 32*(j/2) + 16*half + 8*(j%2) + i
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc_o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            vop(sv, dblk, j), pb[j], acc_o[dblk], 0, 0, 0);
    // the loads issued one step earlier are needed by the next step
    wait_vmcnt(issued);
    __syncthreads();
  };

  // prologue: K(0), V(0), K(1) land first; K(2), V(1) stay in flight
  f32x16 sa[2], sb[2];
  dma_k(kt_first, 0);
  dma_v(kt_first, 0);
  if (ntiles > 1) dma_k(kt_first + SM_KT, 1);
  int pend = 0;
  if (ntiles > 2) { dma_k(kt_first + 2 * SM_KT, 2); pend += KPW; }
  if (ntiles > 1) { dma_v(kt_first + SM_KT, 1); pend += VPW; }
  wait_vmcnt(pend);
  __syncthreads();
  qk(0, sa);
  __syncthreads();  // K stage 0 is refilled in step 0
  for (int it = 0; it < ntiles; it += 2) {
    step(it, sa, sb);
    if (it + 1 >= ntiles) break;
    step(it + 1, sb, sa);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- normalise and store: lane holds d = 32*dblk + 8*(r/4) + 4*half + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (my_q < q_end) {
    bf16_t* orow = out + (long long)bh * N * D + my_q * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dblk * 32 + g4 * 8 + half * 4;
        const f32x2 a2 = {acc_o[dblk][g4 * 4 + 0] * inv, acc_o[dblk][g4 * 4 + 1] * inv};
        const f32x2 b2 = {acc_o[dblk][g4 * 4 + 2] * inv, acc_o[dblk][g4 * 4 + 3] * inv};
        const bf16x2 pa = __builtin_convertvector(a2, bf16x2);
        const bf16x2 pb2 = __builtin_convertvector(b2, bf16x2);
        *(uint2*)(orow + d0) = make_uint2(__builtin_bit_cast(uint32_t, pa),
                                          __builtin_bit_cast(uint32_t, pb2));
      }
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
    int tiles_per_chunk, float scale_log2) {
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
  }
}

hipError_t launch_softmax(const Geom& g, int dtype, const void* q,
                          const void* k, const void* v, const bf16_t* v_t,
                          const int32_t* lohi, void* out, hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)g.d);
  const int qpc = g.chunk * g.S;  // queries of a full chunk
  if (dtype == HWA_BF16) {
    const int tpc = (qpc + SM_QT - 1) / SM_QT;
    dim3 grid(tpc * g.nch * g.B * g.H);
    const long long Np = round_up64(g.N);
#define SM_LAUNCH(DD)                                                        \
  hipLaunchKernelGGL(softmax_bf16_kernel<DD>, grid, dim3(SM_THREADS), 0, st, \
                     (const bf16_t*)q, (const bf16_t*)k, v_t, lohi,          \
                     (bf16_t*)out, g.F, g.S, g.chunk, g.nch, g.N, Np, tpc,   \
                     scale_log2)
    if (g.d == 128) SM_LAUNCH(128);
    else SM_LAUNCH(64);
#undef SM_LAUNCH
  } else {
    const int tpc = (qpc + 127) / 128;
    dim3 grid(tpc * g.nch, g.B * g.H);
#define SF_LAUNCH(DD)                                                          \
  hipLaunchKernelGGL(softmax_f32_kernel<DD>, grid, dim3(128), 0, st,           \
                     (const float*)q, (const float*)k, (const float*)v, lohi,  \
                     (float*)out, g.F, g.S, g.chunk, g.N, tpc, scale_log2)
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
