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

}  // namespace hwa
