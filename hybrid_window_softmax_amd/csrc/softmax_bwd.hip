// Backward pass of the windowed softmax branch (VDN-H3 article, "What the
// far field outside the window is", trained as its "Training" section
// describes). With s_nm = q_n.k_m / sqrt(d), p_nm the row softmax over query
// n's window, g_n = dL/do_n, lse_n = log sum_m exp(s_nm) and
// delta_n = g_n . o_n (= sum_m p_nm g_n . v_m):
//   dv_m = sum_n p_nm g_n
//   ds_nm = p_nm (g_n . v_m - delta_n)
//   dq_n = sum_m ds_nm k_m / sqrt(d),  dk_m = sum_n ds_nm q_n / sqrt(d).
// Windows are chunk-aligned and symmetric: the queries that see the keys of
// chunk c are those of the frames lo_c .. hi_c, the chunk's own window.
//
// bf16 path (v_mfma_f32_32x32x16_bf16, fp32 accumulation), two kernels that
// each recompute p from lse:
//  * dq: a workgroup takes 256 queries of one chunk (8 waves x 32) and
//    streams the chunk's key window in tiles of 64 keys, as the forward does:
//    S^T = K Q^T and dP^T = V G^T leave one query per lane, so lse and delta
//    are lane scalars; dQ^T += K^T dS^T takes dS straight from the S^T
//    registers (the key rows are permuted as in the forward).
//  * dk/dv: a workgroup takes 128 keys of one chunk (4 waves x 32) and
//    streams the queries of the chunk's window in tiles of 64: S = Q K^T and
//    dP = G V^T leave one key per lane (query rows permuted), and
//    dV^T += G^T P, dK^T += Q^T dS take P and dS straight from registers.
// The contractions over queries (keys) read their other operand from the
// same row tiles with the gfx950 LDS transpose read (tr_op).

#include <type_traits>

#include "attn_tile.h"

namespace hwa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BT = 64;  // rows (keys or queries) per streamed LDS tile

// Logical tile of workgroup `bid` in a grid of n = 8 * per workgroups: XCD x
// (workgroup p runs on XCD p % 8) takes the contiguous range x * per ..,
// so the tiles that stream one window share that XCD's L2.
__device__ __forceinline__ int xcd_tile(int bid, int n) {
  return (bid % 8) * (n / 8) + bid / 8;
}

// Buffer descriptor of a tile: base at element `first` of a head of
// `head_elems` elements of `es` bytes; bytes past the head read zeros.
__device__ __forceinline__ hwa_i32x4 tile_desc(const void* head, long long head_elems,
                                              long long first, int es) {
  const unsigned long long base = (unsigned long long)((const char*)head + first * es);
  const long long left = (head_elems - first) * es;
  hwa_i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)(base & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(base >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)(left > 0 ? (unsigned)left : 0u));
  r[3] = 0x00020000;
  return r;
}

// Per-lane byte offsets of the direct loads of one 64-row tile whose LDS rows
// hold rows 32 * (m / 32) + perm32(m % 32) of a row-major [*, D] source,
// stored as [D / 64][64 rows][64] with the row swizzle; instruction i of the
// workgroup (i = wave + NW * j) fills 16-byte slots 64 i .. 64 i + 63.
template <int D>
__device__ __forceinline__ int rowtile_off(int slot) {
  const int sub = slot / 512, m = (slot / 8) % 64, pc = slot % 8;
  const int row = 32 * (m / 32) + perm32(m % 32);
  const int colm = (8 * sub + (pc ^ swz(m))) * 8;
  return (row * D + colm) * 2;
}

// The same for a [D][64] tile of a transposed source [D, Np] (row r = one of
// the D channels, 64 consecutive columns).
__device__ __forceinline__ int coltile_off(int slot, long long Np) {
  const int r = slot / 8, pc = slot % 8;
  return (r * (int)Np + (pc ^ swz(r)) * 8) * 2;
}

// A-operand read, step j (k index) of 32-row block blk, from a row tile:
// lane (col, half) reads row 32 * blk + col, chunk op_chunk(j % 4) of the
// 64-wide part j / 4.
template <int D>
__device__ __forceinline__ bf16x8 row_op(const bf16_t* t, int blk, int kk, const int (&off)[4]) {
  return *(const bf16x8*)(t + (kk / 4) * (BT * 64) + blk * (32 * 64) + off[kk % 4]);
}
// From a [D][64] tile: rows 32 * dblk + col, step j of the 64 columns.
__device__ __forceinline__ bf16x8 col_op(const bf16_t* t, int dblk, int j, const int (&off)[4]) {
  return *(const bf16x8*)(t + dblk * (32 * BT) + off[j]);
}

// B operand of a row held in registers: row `row` of a row-major [*, D]
// source, chunk 8 * (kk / 4) + op_chunk(kk % 4, half) in step kk (zeros when
// !valid), matching row_op's order of the contraction index.
template <int D>
__device__ __forceinline__ void load_row_operand(const bf16_t* src, long long row, bool valid,
                                                 int half, bf16x8 (&r)[D / 16]) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 t = {0u, 0u, 0u, 0u};
    const int dc = 8 * (kk / 4) + op_chunk(kk % 4, half);
    if (valid) t = *(const u32x4*)(src + row * D + dc * 8);
    r[kk] = __builtin_bit_cast(bf16x8, t);
  }
}

// Store of a D x 32 accumulator block set (rows = channels, column = this
// lane's row of dst): lane (col, half) holds channels
// 32 * dblk + 8 * (r / 4) + 4 * half + r % 4 in register r of acc[dblk].
template <int D>
__device__ __forceinline__ void store_rows(bf16_t* dst_row, const f32x16 (&acc)[D / 32],
                                           float mul, int half) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x2 a2 = {acc[dblk][g4 * 4 + 0] * mul, acc[dblk][g4 * 4 + 1] * mul};
      const f32x2 b2 = {acc[dblk][g4 * 4 + 2] * mul, acc[dblk][g4 * 4 + 3] * mul};
      *(uint2*)(dst_row + dblk * 32 + g4 * 8 + half * 4) =
          make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(a2, bf16x2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(b2, bf16x2)));
    }
}

}  // namespace

// Direct load of 16 bytes per lane into LDS (lane l writes lds + 16 l; lanes
// whose offset lies past the descriptor's num_records write zeros), written
// out so that the compiler's wait-count tracking does not treat it as an LDS
// write that every later LDS read must wait for (with the intrinsic, the dk/dv
// kernel's operand reads each waited for all loads in flight). The kernel
// orders it itself: s_waitcnt vmcnt(0) before the barrier that publishes a
// stage. It has no register result, and the compiler's own vmcnt waits stay
// sufficient (loads complete in issue order, so extra loads issued after a
// tracked one only make its wait stricter). The nop is the wait state between
// the M0 write and its use.
__device__ __forceinline__ void dma16(hwa_i32x4 rsrc, __attribute__((address_space(3))) void* lds,
                                      int voffset) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)lds);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(rsrc), "{m0}"(base) : "memory");
}

// ---------------------------------------------------------------- prep
// delta_n = g_n . o_n (fp32 from the I/O dtype) and lse2_n = lse_n * log2(e)
// for every query, [B*H, Np] with zeros past N. LPQ lanes share a query, each
// reading 16 bytes of both rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const T* __restrict__ o,
                                                       const T* __restrict__ g,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ delta,
                                                       float* __restrict__ lse2, long long N,
                                                       long long Np) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane
  constexpr int LPQ = D / EPL;              // lanes per query (power of two <= 64)
  const int bh = blockIdx.y;
  const long long n = (long long)blockIdx.x * (256 / LPQ) + threadIdx.x / LPQ;
  const int part = threadIdx.x % LPQ;
  float acc = 0.0f;
  if (n < N) {
    const long long base = ((long long)bh * N + n) * D + part * EPL;
    const u32x4 ov = *(const u32x4*)(o + base);
    const u32x4 gv = *(const u32x4*)(g + base);
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(ov[i]), __uint_as_float(gv[i]), acc);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(__uint_as_float(ov[i] << 16), __uint_as_float(gv[i] << 16), acc);
        acc = fmaf(__uint_as_float(ov[i] & 0xffff0000u), __uint_as_float(gv[i] & 0xffff0000u), acc);
      }
    }
  }
#pragma unroll
  for (int w = LPQ / 2; w >= 1; w /= 2) acc += __shfl_xor(acc, w);
  if (part == 0 && n < Np) {
    const long long i = (long long)bh * Np + n;
    delta[i] = n < N ? acc : 0.0f;
    lse2[i] = n < N ? lse[(long long)bh * N + n] * 1.4426950408889634f : 0.0f;
  }
}

// ---------------------------------------------------------------- bf16 dq
constexpr int DQ_NW = 8;
constexpr int DQ_QT = 32 * DQ_NW;

template <int D>
__global__ __launch_bounds__(64 * DQ_NW, 1) void softmax_bwd_dq_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ g, const float* __restrict__ lse2,
    const float* __restrict__ delta, const int32_t* __restrict__ lohi, bf16_t* __restrict__ dq, int F, int S, int chunk,
    int nch, long long N, long long Np, int tiles_per_chunk, int ntiles, float scale_log2,
    float scale) {
  constexpr int NT = 64 * DQ_NW;
  constexpr int RPW = BT * D / 8 / 64 / DQ_NW;  // direct-load instructions per wave per tile
  static_assert(BT * D / 8 % (64 * DQ_NW) == 0, "uniform loads per wave");
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[2][BT * D];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[2][BT * D];

  const int L = xcd_tile(blockIdx.x, gridDim.x);
  if (L >= ntiles) return;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_bh = tiles_per_chunk * nch;
  const int bh = L / per_bh;
  const int c = (L % per_bh) / tiles_per_chunk;
  const int tile = L % tiles_per_chunk;
  const long long q_end = (long long)min(F, (c + 1) * chunk) * S;
  const long long q_tile0 = (long long)c * chunk * S + (long long)tile * DQ_QT;
  if (q_tile0 >= q_end) return;
  const long long k_begin = (long long)lohi[c * chunk] * S;
  const long long k_end = (long long)(lohi[F + c * chunk] + 1) * S;
  const long long kt_first = k_begin / BT * BT;
  const int ntl = (int)((k_end - kt_first + BT - 1) / BT);

  const long long hoff = (long long)bh * N * D;
  const long long my_q = q_tile0 + wave * 32 + col;
  const bool q_ok = my_q < N;
  bf16x8 qreg[D / 16], greg[D / 16];
  load_row_operand<D>(q + hoff, my_q, q_ok, half, qreg);
  load_row_operand<D>(g + hoff, my_q, q_ok, half, greg);
  const float l2q = q_ok ? lse2[(long long)bh * Np + my_q] : 0.0f;
  const float dlq = q_ok ? delta[(long long)bh * Np + my_q] : 0.0f;

  int r_off[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) r_off[j] = rowtile_off<D>((wave + DQ_NW * j) * 64 + lane);
  auto load_tile = [&](long long kt0, int st) __attribute__((always_inline)) {
    const hwa_i32x4 rk = tile_desc(k + hoff, N * D, kt0 * D, 2);
    const hwa_i32x4 rv = tile_desc(v + hoff, N * D, kt0 * D, 2);
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int s0 = (wave + DQ_NW * j) * 512;
      hwa_raw_buffer_load_lds(rk, (lds_void*)&k_lds[st][s0], 16, r_off[j], 0, 0, 0);
      hwa_raw_buffer_load_lds(rv, (lds_void*)&v_lds[st][s0], 16, r_off[j], 0, 0, 0);
    }
  };
  int off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) off[j] = col * 64 + ((op_chunk(j, half) ^ swz(col)) * 8);

  f32x16 acc[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  load_tile(kt_first, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = 0; it < ntl; ++it) {
    const int st = it & 1;
    const long long kt0 = kt_first + (long long)it * BT;
    if (it + 1 < ntl) load_tile(kt0 + BT, st ^ 1);
    const bf16_t* ks = &k_lds[st][0];
    const bf16_t* vs = &v_lds[st][0];
    f32x16 sT[2], pT[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sT[blk][r] = 0.0f;
        pT[blk][r] = 0.0f;
      }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sT[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op<D>(ks, blk, kk, off), qreg[kk],
                                                          sT[blk], 0, 0, 0);
        pT[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op<D>(vs, blk, kk, off), greg[kk],
                                                          pT[blk], 0, 0, 0);
      }
    }
    // register r of half h in block blk holds key kt0 + 32 blk + 16 h + r;
    // keys outside the window occur in the first and last tiles only
    const int lo_rel = (int)(k_begin - kt0), hi_rel = (int)(k_end - kt0);
    float pr[2][16];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[blk][r] = __builtin_amdgcn_exp2f(fmaf(sT[blk][r], scale_log2, -l2q));
    if (lo_rel > 0 || hi_rel < BT) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = blk * 32 + half * 16 + r;
          if (key < lo_rel || key >= hi_rel) pr[blk][r] = 0.0f;
        }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) dsb[blk * 2 + r / 8][r % 8] = (__bf16)(pr[blk][r] * (pT[blk][r] - dlq));
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_op<D>(ks, dblk, j, lane), dsb[j],
                                                            acc[dblk], 0, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (my_q < q_end) store_rows<D>(dq + hoff + my_q * D, acc, scale, half);
}

// ---------------------------------------------------------------- bf16 dk, dv
// Per wave: 32 keys (K and V rows as B operands in registers; dK^T and dV^T,
// d x 32, accumulate in registers). The queries of the window stream through
// LDS in tiles of 64 = two blocks of 32. Per block b: A(b) = the products
// S(b) = Q_b K^T and dP(b) = G_b V^T; VALU(b) = p and ds of its 16 x 32
// entries per lane (bf16 B operands); B(b) = dV^T += G_b^T P(b) and
// dK^T += Q_b^T dS(b). One stream of MFMAs per step (one block): B(b - 1)
// then A(b + 1), with VALU(b) spread over it, so that the exp work of one
// block runs under the products of its neighbours (one wave per SIMD).
// B reads its operands G^T and Q^T from the same row tiles as A, with the
// LDS transpose read (tr_op). A tile serves A one block before B, so the
// query tiles (Q, G, lse2, delta) rotate through three stages; per tile `it`:
//   step X: B(it-1, 1) | A(it, 1) | VALU(it, 0); barrier
//   step Y: loads of tile it+2 (into the stage of tile it-1) with the first
//           MFMA; B(it, 0) | A(it+1, 0) | VALU(it, 1); wait for the loads;
//           barrier
// so every stage is refilled only after the barrier that follows its last
// reader, and lands before the barrier that precedes its first reader.
constexpr int DK_NW = 4;
constexpr int DK_KT = 32 * DK_NW;

template <int D>
__global__ __launch_bounds__(64 * DK_NW, 1) void softmax_bwd_dkdv_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ g, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ lohi, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int F,
    int S, int chunk, int nch, long long N, long long Np, int tiles_per_chunk, int ntiles,
    float scale_log2, float scale) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RPW = BT * D / 8 / 64 / DK_NW;
  static_assert(BT * D / 8 % (64 * DK_NW) == 0, "uniform loads per wave");
  constexpr int NA = D / 8, NB = D / 8, NG = NA + NB;  // MFMAs of A(b), B(b), a step
#ifndef DK_PF
#define DK_PF 3
#endif
  constexpr int PF = DK_PF;                            // operand reads ahead of their MFMA
  // three stages of a query tile: Q, G (row-major, permuted rows, swizzled)
  // and [lse2, delta] (64 values, then the padding that the rest of the
  // wave's 16-byte direct load writes)
  __shared__ __attribute__((aligned(16))) bf16_t q_lds[3][BT * D];
  __shared__ __attribute__((aligned(16))) bf16_t g_lds[3][BT * D];
  __shared__ __attribute__((aligned(16))) float ls_lds[3][2][4 * 64];

  const int L = xcd_tile(blockIdx.x, gridDim.x);
  if (L >= ntiles) return;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_bh = tiles_per_chunk * nch;
  const int bh = L / per_bh;
  const int c = (L % per_bh) / tiles_per_chunk;
  const int tile = L % tiles_per_chunk;
  const long long key_end = (long long)min(F, (c + 1) * chunk) * S;
  const long long k_tile0 = (long long)c * chunk * S + (long long)tile * DK_KT;
  if (k_tile0 >= key_end) return;
  // the queries that see this chunk's keys: the frames of the chunk's window
  const long long qw_begin = (long long)lohi[c * chunk] * S;
  const long long qw_end = (long long)(lohi[F + c * chunk] + 1) * S;
  const long long qt_first = qw_begin / BT * BT;
  const int ntl = (int)((qw_end - qt_first + BT - 1) / BT);

  const long long hoff = (long long)bh * N * D;
  const long long my_k = k_tile0 + wave * 32 + col;
  const bool k_ok = my_k < key_end;
  bf16x8 kreg[D / 16], vreg[D / 16];
  load_row_operand<D>(k + hoff, my_k, k_ok, half, kreg);
  load_row_operand<D>(v + hoff, my_k, k_ok, half, vreg);

  int r_off[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) r_off[j] = rowtile_off<D>((wave + DK_NW * j) * 64 + lane);
  // Direct loads of query tile `u` (< 0: none) into stage SU (compile-time:
  // the tile loop is unrolled over the three stages), one instruction per
  // call: Q, then G, then lse2 / delta on waves 0 and 1.
  constexpr int NLD = 2 * RPW + 1;  // instructions per step (at most)
  struct Loads {
    hwa_i32x4 rq, rg, rls;
    int u;
  };
  auto make_loads = [&](int u) __attribute__((always_inline)) {
    Loads l;
    l.u = u;
    const long long qt0 = qt_first + (long long)(u < 0 ? 0 : u) * BT;
    l.rq = tile_desc(q + hoff, N * D, qt0 * D, 2);
    l.rg = tile_desc(g + hoff, N * D, qt0 * D, 2);
    l.rls = tile_desc((wave == 0 ? lse2 : delta) + (long long)bh * Np, Np, qt0, 4);
    return l;
  };
  auto issue = [&](auto su_tag, const Loads& l, int j) __attribute__((always_inline)) {
    constexpr int SU = decltype(su_tag)::value;
    if (l.u < 0) return;
    if (j < 2 * RPW) {
      const int jj = j % RPW, s0 = (wave + DK_NW * jj) * 512;
      dma16(j < RPW ? l.rq : l.rg, (lds_void*)(j < RPW ? &q_lds[SU][s0] : &g_lds[SU][s0]),
            r_off[jj]);
    } else if (j == 2 * RPW && wave < 2) {
      // lse2 and delta of the tile's 64 queries: lanes 0..15, 16 bytes each;
      // the other lanes fill the padding
      dma16(l.rls, (lds_void*)&ls_lds[SU][wave][0], lane * 16);
    }
  };
  auto load_all = [&](auto su_tag, const Loads& l) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) issue(su_tag, l, j);
  };
  // Rows of tile `u` outside the window [qw_begin, qw_end) get lse2 = +inf,
  // so that p = exp2(s * scale_log2 - lse2) = 0 and ds = 0 there. Called by
  // wave 0, which loaded lse2, after its loads landed and before the barrier
  // that publishes the tile.
  auto mask_rows = [&](auto su_tag, int u) __attribute__((always_inline)) {
    constexpr int SU = decltype(su_tag)::value;
    const long long qn = qt_first + (long long)u * BT + lane;
    if (qn < qw_begin || qn >= qw_end) ls_lds[SU][0][lane] = __builtin_inff();
  };
  int off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) off[j] = col * 64 + ((op_chunk(j, half) ^ swz(col)) * 8);

  f32x16 acc_k[D / 32], acc_v[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc_k[j][r] = 0.0f;
      acc_v[j][r] = 0.0f;
    }
  // S and dP of the two blocks of a tile; bf16 P and dS of the two blocks
  // (zero until first written: the prologue's VALU runs on block 1)
  f32x16 s_b[2], p_b[2];
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s_b[b2][r] = 0.0f;
      p_b[b2][r] = 0.0f;
    }
  bf16x8 pb[2][2], dsb[2][2];

  // A operand of MFMA a of A(blk): S = Q K^T and dP = G V^T alternate
  auto a_op = [&](int st, int blk, int a) __attribute__((always_inline)) {
    return row_op<D>(a % 2 ? &g_lds[st][0] : &q_lds[st][0], blk, a / 2, off);
  };
  // B operand order, MFMA j of B(blk): G^T (dV) and Q^T (dK) alternate over
  // the channel blocks, then the two 16-query steps; read transposed from the
  // row tiles
  auto b_op = [&](int st, int blk, int j) __attribute__((always_inline)) {
    const int which = j % 2, dblk = (j / 2) % (D / 32), s2 = j / (D / 16);
    return tr_op<D>(which ? &q_lds[st][0] : &g_lds[st][0], dblk, 2 * blk + s2, lane);
  };
  // one probability / ds register r of block blk (query row 32 blk + 16 half + r
  // of the tile; l2v, dlv: lse2 and delta of the lane's 16 rows; lse2 = +inf
  // outside the window)
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  // registers r, r + 1 (r even) of block blk, as one pinned pair
  auto valu_pair = [&](int blk, int r, const f32x4 (&l2v)[4], const f32x4 (&dlv)[4])
                       __attribute__((always_inline)) {
    f32x2v s2 = {s_b[blk][r], s_b[blk][r + 1]};
    asm volatile("" : "+v"(s2));
    const f32x2v e2 = {__builtin_amdgcn_exp2f(fmaf(s2[0], scale_log2, -l2v[r / 4][r % 4])),
                       __builtin_amdgcn_exp2f(fmaf(s2[1], scale_log2, -l2v[r / 4][r % 4 + 1]))};
    const f32x2v d2 = {e2[0] * (p_b[blk][r] - dlv[r / 4][r % 4]),
                       e2[1] * (p_b[blk][r + 1] - dlv[r / 4][r % 4 + 1])};
    bf16x2v p2 = __builtin_convertvector(e2, bf16x2v);
    bf16x2v q2 = __builtin_convertvector(d2, bf16x2v);
    asm volatile("" : "+v"(p2), "+v"(q2));
    pb[blk][r / 8][r % 8] = p2[0];
    pb[blk][r / 8][r % 8 + 1] = p2[1];
    dsb[blk][r / 8][r % 8] = q2[0];
    dsb[blk][r / 8][r % 8 + 1] = q2[1];
  };

  // One step: B(b_blk) from column stage b_st (if DO_B), then A(a_blk) from
  // row stage a_st (if DO_A), with VALU(v_blk) of column stage v_st spread
  // over the MFMAs (if DO_V). Block indices and flags are compile-time (the
  // first and last tiles are peeled), stages wave-uniform.
  auto step = [&](auto b_tag, auto a_tag, auto v_tag, auto flags, auto bst_tag, auto ast_tag,
                  auto vst_tag, auto&& loader) __attribute__((always_inline)) {
    constexpr int BB = decltype(b_tag)::value, AB = decltype(a_tag)::value,
                  VB = decltype(v_tag)::value;
    constexpr int b_st = decltype(bst_tag)::value, a_st = decltype(ast_tag)::value,
                  v_st = decltype(vst_tag)::value;
    constexpr int FL = decltype(flags)::value;
    constexpr bool do_b = FL & 1, do_a = FL & 2, do_v = FL & 4;
    f32x4 l2v[4], dlv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l2v[i] = *(const f32x4*)&ls_lds[v_st][0][32 * VB + 16 * half + 4 * i];
      dlv[i] = *(const f32x4*)&ls_lds[v_st][1][32 * VB + 16 * half + 4 * i];
    }
    if (do_a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s_b[AB][r] = 0.0f;
        p_b[AB][r] = 0.0f;
      }
    }
    bf16x8 opa[PF + 1];
    auto op_read = [&](int gi) __attribute__((always_inline)) {
      if (gi < NB) return b_op(b_st, BB, gi);
      return a_op(a_st, AB, gi - NB);
    };
    constexpr int g_first = do_b ? 0 : NB, g_last = do_a ? NG : NB;
#pragma unroll
    for (int gi = 0; gi < PF; ++gi)
      if (gi >= g_first && gi < g_last) opa[gi] = op_read(gi);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (gi + PF < NG && gi + PF >= g_first && gi + PF < g_last)
        opa[(gi + PF) % (PF + 1)] = op_read(gi + PF);
      if (gi >= g_first && gi < g_last) {
        if (gi < NB) {
          const int which = gi % 2, dblk = (gi / 2) % (D / 32), s2 = gi / (D / 16);
          if (which == 0)
            acc_v[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[gi % (PF + 1)],
                                                                  pb[BB][s2], acc_v[dblk], 0, 0, 0);
          else
            acc_k[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[gi % (PF + 1)],
                                                                  dsb[BB][s2], acc_k[dblk], 0, 0, 0);
        } else {
          const int a = gi - NB;
          if (a % 2 == 0)
            s_b[AB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[gi % (PF + 1)], kreg[a / 2],
                                                              s_b[AB], 0, 0, 0);
          else
            p_b[AB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[gi % (PF + 1)], vreg[a / 2],
                                                              p_b[AB], 0, 0, 0);
        }
      }
      // VALU(v_blk): 16 registers spread over the NG MFMA slots
      if (do_v) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e * NG) / 8 == gi) valu_pair(VB, 2 * e, l2v, dlv);
      }
      // this step's direct loads, all with the first MFMA (measured at
      // 132,600 tokens: 1.5 % faster than half with the first and half at
      // mid-step; one after every other MFMA was 15 times slower)
      if (gi == 0) {
#pragma unroll
        for (int j = 0; j < NLD; ++j) loader(j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  // step flags: 1 = B, 2 = A, 4 = VALU
  typedef std::integral_constant<int, 2> F_A;
  typedef std::integral_constant<int, 6> F_AV;
  typedef std::integral_constant<int, 7> F_BAV;
  typedef std::integral_constant<int, 5> F_BV;
  typedef std::integral_constant<int, 1> F_B;

  typedef std::integral_constant<int, 2> B2;
  auto no_loads = [](int) {};
  // prologue: tiles 0 and 1 into stages 0 and 1; A(0, 0)
  load_all(B0{}, make_loads(0));
  load_all(B1{}, make_loads(ntl > 1 ? 1 : -1));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (wave == 0) {
    mask_rows(B0{}, 0);
    if (ntl > 1) mask_rows(B1{}, 1);
  }
  __syncthreads();
  step(B1{}, B0{}, B1{}, F_A{}, B0{}, B0{}, B0{}, no_loads);
  // Tile `it` lives in stage R = it % 3 (compile-time: the loop runs over
  // three tiles at a time) from Y(it-1) to X(it+1):
  //   X(it): B(it-1, 1) | A(it, 1) | VALU(it, 0)
  //   Y(it): loads of tile it+2 into the stage of tile it-1 with the first
  //          MFMA; B(it, 0) | A(it+1, 0) | VALU(it, 1)
  auto tile_x = [&](auto fl, auto r_tag, int it) __attribute__((always_inline)) {
    constexpr int R = decltype(r_tag)::value;
    typedef std::integral_constant<int, (R + 2) % 3> RP;
    step(B1{}, B1{}, B0{}, fl, RP{}, r_tag, r_tag, no_loads);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto tile_y = [&](auto fl, auto r_tag, int it) __attribute__((always_inline)) {
    constexpr int R = decltype(r_tag)::value;
    typedef std::integral_constant<int, (R + 1) % 3> RN;
    typedef std::integral_constant<int, (R + 2) % 3> RP;
    const Loads l = make_loads(it + 2 < ntl ? it + 2 : -1);
    step(B0{}, B0{}, B1{}, fl, r_tag, RN{}, r_tag, [&](int j) { issue(RP{}, l, j); });
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (wave == 0 && it + 2 < ntl) mask_rows(RP{}, it + 2);
    __syncthreads();
  };
  // drain: B(last, 1)
  auto drain = [&](auto r_tag) __attribute__((always_inline)) {
    step(B1{}, B0{}, B0{}, F_B{}, r_tag, B0{}, B0{}, no_loads);
  };
  auto full = [&](auto r_tag, int it) __attribute__((always_inline)) {
    tile_x(F_BAV{}, r_tag, it);
    tile_y(F_BAV{}, r_tag, it);
  };
  auto last = [&](auto r_tag, int it) __attribute__((always_inline)) {
    tile_x(F_BAV{}, r_tag, it);
    tile_y(F_BV{}, r_tag, it);
    drain(r_tag);
  };
  // first tile: nothing pending for B in X; last tile: no A(ntl, 0) in Y
  tile_x(F_AV{}, B0{}, 0);
  if (ntl == 1) {
    tile_y(F_BV{}, B0{}, 0);
    drain(B0{});
  } else {
    tile_y(F_BAV{}, B0{}, 0);
    int it = 1;
    for (; it + 2 <= ntl - 2; it += 3) {  // middle tiles 1 .. ntl-2
      full(B1{}, it);
      full(B2{}, it + 1);
      full(B0{}, it + 2);
    }
    if (it <= ntl - 2) full(B1{}, it++);
    if (it <= ntl - 2) full(B2{}, it++);
    const int rl = it % 3;  // it == ntl - 1
    if (rl == 0) last(B0{}, it);
    else if (rl == 1) last(B1{}, it);
    else last(B2{}, it);
  }
  if (k_ok) {
    store_rows<D>(dk + hoff + my_k * D, acc_k, scale, half);
    store_rows<D>(dv + hoff + my_k * D, acc_v, 1.0f, half);
  }
#endif
}

// ---------------------------------------------------------------- fp32 VALU
// One thread per query (dq) or per key (dk, dv), the other side staged in LDS
// 32 rows at a time; fp32 products and accumulation. Used for the fp32 dtype
// (small exactness workloads).
template <int D>
__global__ __launch_bounds__(128) void softmax_bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ lohi, float* __restrict__ dq, int F, int S, int chunk,
    long long N, long long Np, int tiles_per_chunk, float scale_log2, float scale) {
  constexpr int QT = 128, KT = 32;
  __shared__ float k_lds[KT][D];
  __shared__ float v_lds[KT][D];
  const int tid = threadIdx.x;
  const int c = blockIdx.x / tiles_per_chunk, tile = blockIdx.x % tiles_per_chunk;
  const int bh = blockIdx.y;
  const long long q_end = (long long)min(F, (c + 1) * chunk) * S;
  const long long q0 = (long long)c * chunk * S + (long long)tile * QT;
  if (q0 >= q_end) return;
  const long long k_begin = (long long)lohi[c * chunk] * S;
  const long long k_end = (long long)(lohi[F + c * chunk] + 1) * S;
  const long long hoff = (long long)bh * N * D;
  const long long my_q = q0 + tid;
  const bool valid = my_q < q_end;
  float qr[D], gr[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qr[i] = valid ? q[hoff + my_q * D + i] : 0.0f;
    gr[i] = valid ? g[hoff + my_q * D + i] : 0.0f;
    acc[i] = 0.0f;
  }
  const float l2 = valid ? lse2[(long long)bh * Np + my_q] : 0.0f;
  const float dl = valid ? delta[(long long)bh * Np + my_q] : 0.0f;
  for (long long kt0 = k_begin; kt0 < k_end; kt0 += KT) {
    for (int e = tid; e < KT * D; e += QT) {
      const int r = e / D, cc = e % D;
      const long long n = kt0 + r;
      const bool in = n < k_end;
      k_lds[r][cc] = in ? k[hoff + n * D + cc] : 0.0f;
      v_lds[r][cc] = in ? v[hoff + n * D + cc] : 0.0f;
    }
    __syncthreads();
    const int nk = (int)min((long long)KT, k_end - kt0);
    for (int j = 0; j < nk; ++j) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        s = fmaf(qr[i], k_lds[j][i], s);
        dp = fmaf(gr[i], v_lds[j][i], dp);
      }
      const float p = exp2f(fmaf(s, scale_log2, -l2));
      const float ds = p * (dp - dl);
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(ds, k_lds[j][i], acc[i]);
    }
    __syncthreads();
  }
  if (valid)
#pragma unroll
    for (int i = 0; i < D; ++i) dq[hoff + my_q * D + i] = acc[i] * scale;
}

template <int D>
__global__ __launch_bounds__(128) void softmax_bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ lohi, float* __restrict__ dk, float* __restrict__ dv, int F,
    int S, int chunk, long long N, long long Np, int tiles_per_chunk, float scale_log2,
    float scale) {
  constexpr int KT = 128, QT = 32;
  __shared__ float q_lds[QT][D];
  __shared__ float g_lds[QT][D];
  __shared__ float l2_lds[QT], dl_lds[QT];
  const int tid = threadIdx.x;
  const int c = blockIdx.x / tiles_per_chunk, tile = blockIdx.x % tiles_per_chunk;
  const int bh = blockIdx.y;
  const long long key_end = (long long)min(F, (c + 1) * chunk) * S;
  const long long k0 = (long long)c * chunk * S + (long long)tile * KT;
  if (k0 >= key_end) return;
  const long long qw_begin = (long long)lohi[c * chunk] * S;
  const long long qw_end = (long long)(lohi[F + c * chunk] + 1) * S;
  const long long hoff = (long long)bh * N * D;
  const long long my_k = k0 + tid;
  const bool valid = my_k < key_end;
  float kr[D], vr[D], ak[D], av[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    kr[i] = valid ? k[hoff + my_k * D + i] : 0.0f;
    vr[i] = valid ? v[hoff + my_k * D + i] : 0.0f;
    ak[i] = 0.0f;
    av[i] = 0.0f;
  }
  for (long long qt0 = qw_begin; qt0 < qw_end; qt0 += QT) {
    for (int e = tid; e < QT * D; e += KT) {
      const int r = e / D, cc = e % D;
      const long long n = qt0 + r;
      const bool in = n < qw_end;
      q_lds[r][cc] = in ? q[hoff + n * D + cc] : 0.0f;
      g_lds[r][cc] = in ? g[hoff + n * D + cc] : 0.0f;
    }
    if (tid < QT) {
      const long long n = qt0 + tid;
      const bool in = n < qw_end;
      l2_lds[tid] = in ? lse2[(long long)bh * Np + n] : 0.0f;
      dl_lds[tid] = in ? delta[(long long)bh * Np + n] : 0.0f;
    }
    __syncthreads();
    const int nq = (int)min((long long)QT, qw_end - qt0);
    for (int j = 0; j < nq; ++j) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        s = fmaf(q_lds[j][i], kr[i], s);
        dp = fmaf(g_lds[j][i], vr[i], dp);
      }
      const float p = exp2f(fmaf(s, scale_log2, -l2_lds[j]));
      const float ds = p * (dp - dl_lds[j]);
#pragma unroll
      for (int i = 0; i < D; ++i) {
        ak[i] = fmaf(ds, q_lds[j][i], ak[i]);
        av[i] = fmaf(p, g_lds[j][i], av[i]);
      }
    }
    __syncthreads();
  }
  if (valid)
#pragma unroll
    for (int i = 0; i < D; ++i) {
      dk[hoff + my_k * D + i] = ak[i] * scale;
      dv[hoff + my_k * D + i] = av[i];
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_bwd_prep(const Geom& g, int dtype, const void* o, const void* go,
                           const float* lse, float* delta, float* lse2, hipStream_t st) {
  const long long Np = round_up64(g.N);
  const int EPL = dtype == HWA_BF16 ? 8 : 4;
  const int qpb = 256 / (g.d / EPL);  // queries per block
  dim3 grid((unsigned)((Np + qpb - 1) / qpb), g.B * g.H);
#define PREP(T, DD)                                                                       \
  hipLaunchKernelGGL((bwd_prep_kernel<T, DD>), grid, dim3(256), 0, st, (const T*)o,       \
                     (const T*)go, lse, delta, lse2, g.N, Np)
  if (dtype == HWA_BF16) {
    if (g.d == 128) PREP(bf16_t, 128);
    else PREP(bf16_t, 64);
  } else {
    switch (g.d) {
      case 16: PREP(float, 16); break;
      case 32: PREP(float, 32); break;
      case 64: PREP(float, 64); break;
      default: PREP(float, 128); break;
    }
  }
#undef PREP
  return hipGetLastError();
}

hipError_t launch_softmax_bwd(const Geom& g, int dtype, int part, const void* q, const void* k,
                              const void* v, const void* go, const float* lse2,
                              const float* delta, const int32_t* lohi, void* dq, void* dk,
                              void* dv, hipStream_t st) {
  const float scale = 1.0f / sqrtf((float)g.d);
  const float scale_log2 = 1.4426950408889634f * scale;
  const long long Np = round_up64(g.N);
  const int qpc = g.chunk * g.S;
  const int bh = g.B * g.H;
  if (dtype == HWA_BF16) {
    const int tq = (qpc + DQ_QT - 1) / DQ_QT, nq = tq * g.nch * bh;
    const int tk = (qpc + DK_KT - 1) / DK_KT, nk = tk * g.nch * bh;
    const dim3 gq((unsigned)((nq + 7) / 8 * 8)), gk((unsigned)((nk + 7) / 8 * 8));
#define BWD(DD)                                                                             \
  do {                                                                                      \
    if (part == 0)                                                                          \
      hipLaunchKernelGGL(softmax_bwd_dq_kernel<DD>, gq, dim3(64 * DQ_NW), 0, st,            \
                         (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,              \
                         (const bf16_t*)go, lse2, delta, lohi, (bf16_t*)dq, g.F, g.S,       \
                         g.chunk, g.nch, g.N, Np, tq, nq, scale_log2, scale);               \
    else                                                                                    \
      hipLaunchKernelGGL(softmax_bwd_dkdv_kernel<DD>, gk, dim3(64 * DK_NW), 0, st,          \
                         (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,              \
                         (const bf16_t*)go, lse2, delta, lohi, (bf16_t*)dk,                 \
                         (bf16_t*)dv, g.F, g.S, g.chunk, g.nch, g.N, Np, tk, nk,            \
                         scale_log2, scale);                                                \
  } while (0)
    if (g.d == 128) BWD(128);
    else BWD(64);
#undef BWD
  } else {
    const int tq = (qpc + 127) / 128, tk = (qpc + 127) / 128;
#define BWD32(DD)                                                                           \
  do {                                                                                      \
    if (part == 0)                                                                          \
      hipLaunchKernelGGL(softmax_bwd_dq_f32_kernel<DD>, dim3(tq * g.nch, bh), dim3(128), 0, \
                         st, (const float*)q, (const float*)k, (const float*)v,             \
                         (const float*)go, lse2, delta, lohi, (float*)dq, g.F, g.S,         \
                         g.chunk, g.N, Np, tq, scale_log2, scale);                          \
    else                                                                                    \
      hipLaunchKernelGGL(softmax_bwd_dkdv_f32_kernel<DD>, dim3(tk * g.nch, bh), dim3(128),  \
                         0, st, (const float*)q, (const float*)k, (const float*)v,          \
                         (const float*)go, lse2, delta, lohi, (float*)dk, (float*)dv, g.F,  \
                         g.S, g.chunk, g.N, Np, tk, scale_log2, scale);                     \
  } while (0)
    switch (g.d) {
      case 16: BWD32(16); break;
      case 32: BWD32(32); break;
      case 64: BWD32(64); break;
      default: BWD32(128); break;
    }
#undef BWD32
  }
  return hipGetLastError();
}

}  // namespace hwa
