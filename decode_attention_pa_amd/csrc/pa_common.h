// Shared device/host helpers of the paged-attention decode kernels (gfx950).
//
// Index arithmetic lives here once so that the partition kernels, the LSE
// reduce and the index-dump kernel agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cross-lane combines that stay in the vector ALUs (no trip through the LDS
// crossbar, and no wait that also covers outstanding scalar loads, as a
// ds_bpermute's would).  32-bit values (float or int); `op` must be
// commutative: a lane may see its own value and its partner's in either
// order, and both lanes of a pair get the same bits.  All lanes active.
template <typename T>
__device__ __forceinline__ uint32_t lane_bits(T x) {
  return __builtin_bit_cast(uint32_t, x);
}
template <typename T>
__device__ __forceinline__ T from_lane_bits(uint32_t x) {
  return __builtin_bit_cast(T, x);
}
// op(x, x of lane ^ 16) and op(x, x of lane ^ 32): gfx950's row swaps
// (v_permlane16_swap / v_permlane32_swap) of x with itself hand every lane
// both values of its pair.
template <typename T, typename F>
__device__ __forceinline__ T xor16_op(T x, F op) {
  const auto r = __builtin_amdgcn_permlane16_swap(lane_bits(x), lane_bits(x), false, false);
  return op(from_lane_bits<T>(r[0]), from_lane_bits<T>(r[1]));
}
template <typename T, typename F>
__device__ __forceinline__ T xor32_op(T x, F op) {
  const auto r = __builtin_amdgcn_permlane32_swap(lane_bits(x), lane_bits(x), false, false);
  return op(from_lane_bits<T>(r[0]), from_lane_bits<T>(r[1]));
}
// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), [2,3,0,1] (lane ^ 2),
// row_ror:8 (lane ^ 8 inside a 16-lane row), half-row and row mirrors.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppXor8 = 0x128;
constexpr int kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL, typename T>
__device__ __forceinline__ T dpp(T x) {
  return from_lane_bits<T>(__builtin_amdgcn_update_dpp(0, (int)lane_bits(x), CTRL, 0xF, 0xF, false));
}
// op over each 16-lane row, every lane receiving the result: lane ^ 1 and
// lane ^ 2 leave every lane of a quad with the quad's value, the half-row
// mirror meets each quad with the other quad of its half, the row mirror
// each half with the other.  Associative, commutative ops (sums: one fixed
// order, the same bits on every lane).
template <typename T, typename F>
__device__ __forceinline__ T row16_op(T x, F op) {
  x = op(x, dpp<kDppXor1>(x));
  x = op(x, dpp<kDppXor2>(x));
  x = op(x, dpp<kDppHalfMirror>(x));
  return op(x, dpp<kDppMirror>(x));
}
// op over the whole wave.
template <typename T, typename F>
__device__ __forceinline__ T wave_op(T x, F op) {
  return row16_op(xor16_op(xor32_op(x, op), op), op);
}

// Positions per inner step of every partition kernel.  Partitions start on
// multiples of this (relative to the aligned start of the span), so a chunk
// never straddles two partitions.
constexpr int kChunk = 32;

// First position query token i may see.  gllm "feat(backend): sliding-window
// PagedAttention" (#116): window w > 0 shows positions p-w+1 .. p to the
// token at p; w == 0 is unlimited causal.  The query tokens are the last q of
// the L-position context, so token i sits at p = L - q + i.
__host__ __device__ inline int first_visible(int L, int q, int i, int window) {
  const int p = L - q + i;
  return window == 0 ? 0 : max(0, p + 1 - window);
}

// Union of a sequence's visible ranges and its partition grid.
//   [lo, hi)  positions some query token of the sequence can see
//   base      lo rounded down to a chunk boundary; partition j covers
//             [max(lo, base + j*P), min(hi, base + (j+1)*P))
//   nparts    number of non-empty partitions (0 when q == 0)
struct SeqView {
  int lo, hi, base, nparts;
};

__host__ __device__ inline SeqView seq_view(int L, int q, int window, int part_size) {
  SeqView s;
  if (q <= 0 || L <= 0) {
    s.lo = s.hi = L > 0 ? L : 0;
    s.base = s.lo & ~(kChunk - 1);
    s.nparts = 0;
    return s;
  }
  s.lo = first_visible(L, q, 0, window);
  s.hi = L;
  s.base = s.lo & ~(kChunk - 1);
  s.nparts = (s.hi - s.base + part_size - 1) / part_size;
  return s;
}

__host__ __device__ inline void partition_range(const SeqView& s, int j, int part_size,
                                                int* ps, int* pe) {
  *ps = max(s.lo, s.base + j * part_size);
  *pe = min(s.hi, s.base + (j + 1) * part_size);
}

// Physical block holding position t of a sequence whose block-table row is
// `table_row`; block_size = 1 << log2_bs.
__device__ inline int phys_block(const int32_t* __restrict__ table_row, int t, int log2_bs) {
  return table_row[t >> log2_bs];
}

// K cache slab of one (block, KV head): slots in groups of 16, each group a
// [2][D/8][8][8] tile.  Half 0 holds slots 0-3 and 8-11, half 1 slots 4-7
// and 12-15 (the positions one 16-row matrix-core K tile takes from a group);
// in a half, column c (dims 8c .. 8c+7) stores its 8 slots one after another.
// Element offset of (slot, dim 0); dim d adds (d >> 3) * 64 + (d & 7).
__host__ __device__ inline int k_slot_offset(int slot, int D) {
  const int u = slot & 15;
  return (slot >> 4) * (16 * D) + ((u >> 2) & 1) * (8 * D) + ((u & 3) | ((u >> 3) << 2)) * 8;
}

// The same slab addressed in bytes for 16-byte columns (bf16: 8 dims, FP8:
// 16 dims per column); row_bytes = D * element size.  Byte offset of
// (slot, column 0); column c adds 128 * c.
__host__ __device__ inline int k_slot_bytes(int slot, int row_bytes) {
  const int u = slot & 15;
  return (slot >> 4) * (16 * row_bytes) + ((u >> 2) & 1) * (8 * row_bytes) +
         ((u & 3) | ((u >> 3) << 2)) * 16;
}

// Exclusive prefix sum of query_lens[0 .. b) computed by one wave; every lane
// gets the sum.  Gives the first q/out row of sequence b in the packed
// [sum q_b, H_q, D] layout.  In two steps, so that a kernel can request the
// first loads together with its other start-up loads: row_offset_issue
// reads query_lens[lane] (lanes below b), row_offset_finish adds the rest.
__device__ inline int row_offset_issue(const int32_t* __restrict__ query_lens, int b) {
  const int lane = threadIdx.x & 63;
  return lane < b ? query_lens[lane] : 0;
}
__device__ inline int wave_row_offset_finish(int first, const int32_t* __restrict__ query_lens, int b) {
  const int lane = threadIdx.x & 63;
  int s = first;
  if (b > 64) {  // (b is the same on every lane)
    // up to 1024 sequences: all of a lane's loads requested before any is
    // used (one round trip instead of one per 64 sequences); lanes past b
    // re-read the last entry, so no load needs a branch of its own
    int v[15];
#pragma unroll
    for (int c = 1; c < 16; ++c) v[c - 1] = query_lens[min(lane + 64 * c, b - 1)];
#pragma unroll
    for (int c = 1; c < 16; ++c) s += lane + 64 * c < b ? v[c - 1] : 0;
    for (int k = lane + 1024; k < b; k += 64) s += query_lens[k];
  }
  return wave_op(s, [](int x, int y) { return x + y; });
}
__device__ inline int wave_row_offset(const int32_t* __restrict__ query_lens, int b) {
  return wave_row_offset_finish(row_offset_issue(query_lens, b), query_lens, b);
}

// Batches above this size get their row offsets from a prefix array that a
// one-workgroup scan writes into the workspace before the partition kernel
// (below it every workgroup sums query_lens[0 .. b) itself, which costs
// O(B) per workgroup).
constexpr int kScanBatch = 1024;

// First q/out row of sequence b: from the scanned prefix array when there is
// one, else summed by the calling wave.
__device__ inline int row_offset(const int32_t* __restrict__ qoffs,
                                 const int32_t* __restrict__ query_lens, int b) {
  return qoffs ? qoffs[b] : wave_row_offset(query_lens, b);
}
// The same after row_offset_issue (whose loads are wasted when the scanned
// array exists: batches above kScanBatch).
__device__ inline int row_offset_finish(int first, const int32_t* __restrict__ qoffs,
                                        const int32_t* __restrict__ query_lens, int b) {
  return qoffs ? qoffs[b] : wave_row_offset_finish(first, query_lens, b);
}

__device__ inline float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Arguments shared by the partition kernels.
struct PartArgs {
  void* out;                   // [T, H_q, D] (one-shot sequences)
  const void* q;               // [T, H_q, D]
  const void* k_cache;         // [num_blocks, H_kv, bs/16, 2, D/E, 8, E] (E = 8; FP8: 16)
  const void* v_cache;         // [num_blocks, H_kv, bs/E, D, E]
  const int32_t* block_tables; // [B, max_blocks_per_seq]
  const int32_t* seq_lens;     // [B]
  const int32_t* query_lens;   // [B]
  float* ws_m;                 // [S, R] running max, log2 domain, per state slot
  float* ws_l;                 // [S, R] exp-sum
  float* ws_o;                 // [S, R, D] normalised partial output (S state slots:
                               // B * H_kv * NP on the grid schedule, persistent grid
                               // + B * H_kv on the persistent one)
  int* ws_runs;                // [B, H_kv, 2] run count and first state slot per unit
                               // (persistent schedule only)
  float scale_log2;            // scale * log2(e)
  int window;
  int num_q_heads;
  int num_kv_heads;
  int group;                   // G = H_q / H_kv
  int rows;                    // R = G * max_query_len (workspace row stride)
  int num_parts;               // NP (workspace partition stride)
  int part_size;               // P, multiple of kChunk * waves
  int log2_bs;
  int max_blocks_per_seq;
  int batch;
  int row_blocks;              // workgroups per (partition, sequence, KV head), each taking
                               // the next rows_per_block packed rows
  int head_dim;                // D (the vector kernel reads it at run time)
  const float* k_scale;        // FP8 KV: device scalars, K = code * k_scale, V = code * v_scale
  const float* v_scale;        // (null for native caches)
  const float* q_scale;        // FP8 Q: device scalar, Q = code * q_scale (else null)
  const int32_t* qoffs;        // [B] exclusive prefix of query_lens (batches > kScanBatch), or null
};

// Work-item of a partition workgroup.  The grid is 1-D and ordered with the
// row block, then the KV head fastest and the partition slowest: workgroups
// are handed to the 8
// XCDs round-robin by id, so consecutive ids must carry comparable work.
// (With the partition fastest and 8 partitions per sequence, partition j
// would always land on XCD j, and high partitions exist only for long
// sequences.)
struct PartItem {
  int j, h, b, rb;
};

// Row blocks of one (partition, sequence, KV head) read the same K/V.
// Workgroup ids are dealt to the 8 XCDs round-robin, so the row blocks of a
// unit take ids 8 apart: all on one XCD, sharing its L2, while 8 units fill
// the 8 XCDs.  (The grid is padded to whole groups of 8 units; a padded id
// lands on a partition index >= num_parts and exits.)
constexpr int kXcds = 8;
__device__ inline PartItem part_item(const PartArgs& a) {
  const int id = blockIdx.x;
  PartItem it;
  int u = id;
  it.rb = 0;
  if (a.row_blocks > 1) {
    const int rest = id / kXcds;
    it.rb = rest % a.row_blocks;
    u = (rest / a.row_blocks) * kXcds + id % kXcds;
  }
  it.h = u % a.num_kv_heads;
  const int r = u / a.num_kv_heads;
  it.b = r % a.batch;
  it.j = r / a.batch;
  return it;
}

struct ReduceArgs {
  void* out;
  const int32_t* seq_lens;
  const int32_t* query_lens;
  const float* ws_m;
  const float* ws_l;
  const float* ws_o;
  const int* ws_runs;   // per unit (run count, first state slot), or null: every
                        // partition of unit u holds state slot u * NP + j
  int window;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int rows;
  int num_parts;
  int part_size;
  int head_dim;
  const int32_t* qoffs;  // [B] exclusive prefix of query_lens, or null
};

}  // namespace pa
