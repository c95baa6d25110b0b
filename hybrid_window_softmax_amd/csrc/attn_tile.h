// Tile machinery shared by the bf16 MFMA kernels of the windowed softmax
// (forward and backward): the gfx950 direct load global -> LDS, the row
// permutation that turns an MFMA output block into an operand of the next
// product, and the swizzled 128-byte LDS rows. gfx950 (CDNA4) only.
#pragma once

#include "hwa_internal.h"

// MUBUF direct load global -> LDS (buffer_load_dword* ... lds): lane l of a
// wave writes its bytes at the LDS address in M0 + 16 * l (dwordx4); lanes
// whose offset lies past the descriptor's num_records read zeros. Unlike the
// FLAT-encoded global_load_lds, it is not counted as an LDS access by the
// compiler's wait-count tracking, so waits for ds_read results stay counted.
typedef int hwa_i32x4 __attribute__((ext_vector_type(4)));
extern "C" __device__ void hwa_raw_buffer_load_lds(hwa_i32x4 rsrc,
                                                   __attribute__((address_space(3))) void* lds,
                                                   int size, int voffset, int soffset, int offset,
                                                   int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace hwa {

__host__ __device__ inline long long round_up64(long long n) {
  return (n + 63) / 64 * 64;
}

// Row of the 32-row MFMA block that lands on "16 consecutive keys per lane
// half": MFMA output row m is held by lane half (m / 4) % 2 in register
// 4 * (m / 8) + m % 4; loading tile key perm32(m) into row m makes register r
// of half h hold key 16 * h + r.
__device__ __forceinline__ int perm32(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// Swizzle of a 128-byte LDS row (8 chunks of 16 bytes): row m keeps logical
// chunk c at chunk c ^ swz(m). op_chunk(j, half) is the chunk that lane half
// `half` reads in step j of a 64-wide contraction (4 steps of 16): over the
// four steps each half covers its 16-element quarter of every 32-element
// half, as the permuted rows of an output block hold them.
__device__ __forceinline__ int swz(int m) { return (m >> 1) & 7; }
__device__ __forceinline__ int op_chunk(int j, int half) {
  return 2 * half + 4 * (j / 2) + (j % 2);
}

// Tiles of 64 rows x D channels are stored as [D / 64][64 rows][64]: LDS row
// m holds tile row 32 (m / 32) + perm32(m % 32), logical 16-byte chunk c at
// chunk c ^ swz(m).
//
// A operand with the contraction over the rows of a row tile, read with the
// gfx950 LDS transpose read (ds_read_b64_tr_b16): in each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte chunks that lanes i / 4 + 4 e
// (e = 0..3) address. So if lane j of a group addresses row r0 + j / 4,
// channels c0 + 4 (j % 4) .. + 3, lane i receives channel c0 + i of rows
// r0 .. r0 + 3. For step j of a 64-row contraction (as op_chunk orders it)
// and channel block dblk, lane (col, half) gets channel 32 dblk + col of the
// logical rows 32 (j / 2) + 16 half + 8 (j % 2) + 0..7, two reads of four:
// the rows that register block j holds in a permuted S / P block. Logical
// row q sits in LDS row 32 (q / 32) + perm32^-1(q % 32) of the tile.
__device__ __forceinline__ int inv_perm32(int x) {
  return 8 * ((x >> 2) & 3) + 4 * (x >> 4) + (x & 3);
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
template <int D>
__device__ __forceinline__ bf16x8_t tr_op(const bf16_t* t, int dblk, int j, int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int r0 = 32 * (j / 2) + 16 * (grp >> 1) + 8 * (j % 2) + (i >> 2);
  const int ch = 32 * dblk + 16 * (grp & 1) + 4 * (i & 3);
  i16x4 part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = r0 + 4 * h;
    const int m = 32 * (q >> 5) + inv_perm32(q & 31);
    const int c = (ch & 63) >> 3;
    const int off = (ch >> 6) * (64 * 64) + m * 64 + ((c ^ swz(m)) << 3) + (ch & 7);
    part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(t + off));
  }
  const i16x4 a = part[0], b = part[1];
  const i16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, ab);
}

}  // namespace hwa
