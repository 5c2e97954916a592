// Repacking of a paged KV cache held one row per slot, [num_blocks, H_kv,
// block_size, D] (the plain layout gllm #116 "What changes — Interface"
// passes to PagedAttention), into the tiled layouts the partition kernels
// read.  A pure permutation of bytes: the result is bit-identical to the
// input values.
//
//   K: slots in groups of 16, each group two halves (slots 0-3, 8-11 and
//      4-7, 12-15), each half a [D/E][8][E] tile, E = 8 elements (16 for
//      one-byte elements); a column of one slot is E contiguous elements of
//      its row, so K moves in 16-byte pieces.  Head dims that are not a
//      multiple of E keep one row per slot (a plain copy).
//   V: slots in groups of EV (8, or 16 for one-byte elements), each group a
//      [D][EV] tile: EV consecutive slots of one dim are contiguous.
#pragma once

#include "pa_common.h"
#include "pa_valu.h"  // kValuMaxD

namespace pa {

struct PackArgs {
  const uint8_t* k_rows;  // [num_blocks, H_kv, bs, D] elements of `es` bytes
  const uint8_t* v_rows;
  uint8_t* k_cache;       // tiled layouts (see pa_decode.h)
  uint8_t* v_cache;
  const int32_t* block_ids;  // blocks to repack, or null: block = blockIdx.y
  int num_blocks;
  int num_kv_heads;
  int log2_bs;
  int head_dim;
  int es;                 // bytes per element: 1, 2 or 4
};

// [EV][D] -> [D][EV] for each group of EV slots of a slab (256 threads).
template <typename T, int EV>
__device__ inline void transpose_groups(const uint8_t* src, uint8_t* dst, int bs, int D) {
  __shared__ T tile[EV * kValuMaxD];
  const T* s = (const T*)src;
  T* d = (T*)dst;
  const int n = EV * D;
  for (int g = 0; g < bs / EV; ++g) {
    for (int i = threadIdx.x; i < n; i += 256) tile[i] = s[(size_t)g * n + i];
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) {
      const int dd = i / EV, r = i - dd * EV;
      d[(size_t)g * n + i] = tile[r * D + dd];
    }
    __syncthreads();
  }
}

// Grid: x = block (or entry of block_ids), y = KV head.  256 threads.
__global__ __launch_bounds__(256) void pack_kv(PackArgs a) {
  const int h = blockIdx.y;
  int blk = blockIdx.x;
  if (a.block_ids) {
    blk = a.block_ids[blockIdx.x];
    if (blk < 0 || blk >= a.num_blocks) return;  // not a block of this cache
  }
  const int bs = 1 << a.log2_bs, D = a.head_dim, es = a.es;
  const size_t slab = ((size_t)bs * D) * es;  // bytes per (block, head)
  const size_t off = ((size_t)blk * a.num_kv_heads + h) * slab;
  const uint8_t* kr = a.k_rows + off;
  const uint8_t* vr = a.v_rows + off;
  uint8_t* kc = a.k_cache + off;
  uint8_t* vc = a.v_cache + off;
  const int row_bytes = D * es;

  // K: columns of E elements (E = 8, or 16 for one-byte elements), moved in
  // 16-byte pieces (a column is one piece, two for four-byte elements)
  const int E = es == 1 ? 16 : 8;
  if (D % E == 0) {
    const int cb = E * es;                 // bytes per column
    const int cols = D / E;
    const int pieces = cb / 16;            // 16-byte pieces per column
    for (int c = threadIdx.x; c < bs * cols * pieces; c += 256) {
      const int s = c / (cols * pieces);
      const int rest = c - s * cols * pieces;
      const int col = rest / pieces, k = rest - col * pieces;
      const int u = s & 15;
      const int half = (u >> 2) & 1, place = (u & 3) | ((u >> 3) << 2);
      const size_t dst = ((size_t)((s >> 4) * 2 + half) * cols + col) * 8 * cb + place * cb + k * 16;
      *(u32x4*)(kc + dst) = *(const u32x4*)(kr + (size_t)s * row_bytes + col * cb + k * 16);
    }
  } else {
    for (size_t i = threadIdx.x; i < slab; i += 256) kc[i] = kr[i];
  }

  // V: each group of EV slots is the same byte range in both layouts, read
  // as [EV][D] (rows) and written as [D][EV]: a transpose through shared
  // memory, both sides coalesced
  if (es == 1) transpose_groups<uint8_t, 16>(vr, vc, bs, D);
  else if (es == 2) transpose_groups<uint16_t, 8>(vr, vc, bs, D);
  else transpose_groups<uint32_t, 8>(vr, vc, bs, D);
}

}  // namespace pa
