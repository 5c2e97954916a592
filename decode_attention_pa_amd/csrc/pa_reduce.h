// Log-sum-exp merge of context partitions, and the index-dump kernel.
//
// Merge (executorch PR #18759, split-K reduce; aiter PR #2914, PS reduce over
// max_logits / exp_sums / temporary_output): for one packed row of one
// (sequence, KV head), with partition states (m_j, l_j, o_j) where o_j is the
// partition's normalised output and m_j its max logit in the log2 domain,
//     M = max_j m_j,  w_j = 2^(m_j - M) * l_j  (0 when m_j = -inf),
//     out = sum_j w_j o_j / sum_j w_j.
// A partition in which the row sees nothing has m_j = -inf, l_j = 0, o_j = 0
// and weight 0 (gllm #116, "What changes": a split that the window leaves
// with no positions adds nothing to the combine).  Partitions are summed in a fixed order: results are
// deterministic.
#pragma once

#include "pa_common.h"
#include "pa_valu.h"

namespace pa {

// Output unit = (packed row n, VEC consecutive dims) of one (sequence, KV
// head).  A 256-thread workgroup covers UPW = 256 / GP consecutive units,
// and GP lanes split each unit's partitions (GP = 1, 16 or 32, chosen on the
// host from the state count).  Lane t takes unit t % UPW and partition
// offset t / UPW: neighbouring lanes read neighbouring dims of one partition
// state (UPW * VEC * 4 >= 128 bytes, whole cache lines), and a workgroup's
// lines belong to it alone.  Each thread requests U partitions' states
// before using any.  The GP partial results of a unit are combined by
// a fixed xor butterfly inside each wave, then across the 4 waves through
// shared memory in wave order: results are deterministic.
// Grid: x = unit blocks of UPW units, y = KV head, z = sequence.
// op of x with the lanes lane ^ U, lane ^ 2U, ... lane ^ 32 (U = 8, 16 or 32),
// in that order.
template <int U, typename F>
__device__ __forceinline__ float xor_from(float x, F op) {
  static_assert(U == 8 || U == 16 || U == 32, "lane strides 8, 16, 32");
  if constexpr (U == 8) x = op(x, dpp<kDppXor8>(x));
  if constexpr (U <= 16) x = xor16_op(x, op);
  return xor32_op(x, op);
}

template <int GP>
struct GroupReduce {
  static constexpr int UPW = 256 / GP;
  // GP = 1: nothing to combine.  GP > 1: a unit's lanes are the lanes with
  // the same lane % UPW in all 4 waves (UPW divides 64).
  template <typename F>
  __device__ static float all(float x, float (*lds)[64], F op) {
    if constexpr (GP == 1) {
      return x;
    } else {
      x = xor_from<UPW>(x, op);
      const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
      __syncthreads();  // the previous use of lds is finished
      if (lane < UPW) lds[wave][lane] = x;
      __syncthreads();
      const int u = lane % UPW;
      return op(op(op(lds[0][u], lds[1][u]), lds[2][u]), lds[3][u]);
    }
  }
  // Sums of N values at once: one butterfly per value, one shared-memory
  // round for all of them (waves added in wave order).
  template <int N>
  __device__ static void sum_n(float (&x)[N], float (*lds)[64][N]) {
    if constexpr (GP > 1) {
      const auto add = [](float a, float b) { return a + b; };
#pragma unroll
      for (int e = 0; e < N; ++e) x[e] = xor_from<UPW>(x[e], add);
      const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
      __syncthreads();  // the previous use of lds is finished
      if (lane < UPW)
#pragma unroll
        for (int e = 0; e < N; ++e) lds[wave][lane][e] = x[e];
      __syncthreads();
      const int u = lane % UPW;
#pragma unroll
      for (int e = 0; e < N; ++e) x[e] = ((lds[0][u][e] + lds[1][u][e]) + lds[2][u][e]) + lds[3][u][e];
    }
  }
};

// VEC = 4: a unit is 4 consecutive dims (head dims divisible by 4); VEC = 1:
// one dim.  The head dim itself is a run-time value.
template <typename T, int VEC, int GP>
__global__ __launch_bounds__(256) void lse_reduce(ReduceArgs a) {
  typedef float fvec __attribute__((ext_vector_type(VEC)));
  constexpr int UPW = GroupReduce<GP>::UPW;  // units per workgroup
  constexpr int U = GP == 1 ? 4 : 8;         // partitions in flight per thread per step
  const int D = a.head_dim;
  const int D4 = D / VEC;                    // units per row
  __shared__ float lds[4][64];
  __shared__ float lds_n[4][64][VEC + 1];
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x * UPW + tid % UPW;
  const int gp = tid / UPW;
  const int n = unit / D4, d4 = unit % D4;
  const bool runs = a.ws_runs != nullptr;

  // States of one step: slots base + j0 + u*GP for u < U, those below
  // `bound` and on a workspace row (n < rows); the rest stay neutral.
  float mj[U], lj[U];
  fvec o[U];
  auto load_step = [&](size_t base, int j0, int bound) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j0 + u * GP;
      mj[u] = -INFINITY;
      lj[u] = 0.f;
      o[u] = fvec{};
      if (n < a.rows && jj < bound) {
        const size_t w = (base + jj) * a.rows + n;
        mj[u] = a.ws_m[w];
        lj[u] = a.ws_l[w];
        o[u] = *(const fvec*)(a.ws_o + w * D + d4 * VEC);
      }
    }
  };
  // Grid plan: partition j of unit (b, h) sits at slot (b * H_kv + h) * NP + j
  // whatever the lengths, so the first step's states are requested with the
  // lengths (one dependent round trip less) and masked once they arrive.
  // Slots past this call's partitions hold stale contents, kept out by
  // selects, never by multiplies.
  const size_t grid_base = ((size_t)b * a.num_kv_heads + h) * a.num_parts;
  if (!runs) load_step(grid_base, gp, a.num_parts);

  // One round of independent loads: row offset, lengths, run count.
  const int ro = row_offset_issue(a.query_lens, b);
  const int L = a.seq_lens[b];
  const int q = a.query_lens[b];
  // persistent schedule: the unit's run count and first state slot.  Without
  // it the pair is read from the partial maxima instead (this kernel runs
  // only when they exist) and masked to zero: no branch, so the loads go out
  // with the others.
  const int32_t* rp = runs ? a.ws_runs + 2 * ((size_t)b * a.num_kv_heads + h)
                           : (const int32_t*)a.ws_m;
  const int keep = -(int)runs;  // all ones or zero
  const int2 rs = make_int2(rp[0] & keep, rp[1] & keep);
  const int qoff = row_offset_finish(ro, a.qoffs, a.query_lens, b);  // all lanes still active
  const int G = a.group;
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  // states to merge: one per partition, or the unit's run count
  const int np = runs ? rs.x : (sv.nparts > 1 ? min(sv.nparts, a.num_parts) : 0);
  if (np <= 0) return;  // the partition kernel wrote these rows directly (whole workgroup)
  // Lanes past the last row stay to the end: the combine below synchronises
  // the workgroup.  With GP = 1 there is no combine and they leave now.
  const bool live = n < G * q;
  if (GP == 1 && !live) return;
  // first state slot of the unit: partition j of a grid plan sits at slot
  // unit * NP + j; the persistent runs of a unit at consecutive slots
  const size_t base = runs ? (size_t)rs.y : grid_base;

  // One pass: each thread keeps a running reference max mt over its own
  // partitions (rescaling its sums when it grows), then the group agrees on
  // M = max mt and every thread rescales by 2^(mt - M) before the sums.
  // Every slot below np was written by this call's partition kernel, with
  // finite values (a row that saw nothing stores m = -inf, l = 0, o = 0).
  float mt = -INFINITY;
  fvec acc = {};
  float den = 0.f;
  auto fold = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mj[u] == -INFINITY) continue;  // partition where this row sees nothing
      if (mj[u] > mt) {
        const float r = exp2f(mt - mj[u]);  // 0 while mt = -inf
        acc *= r;
        den *= r;
        mt = mj[u];
      }
      const float f = exp2f(mj[u] - mt) * lj[u];
      acc += f * o[u];
      den += f;
    }
  };
  int j0 = gp;
  if (!runs) {  // the speculative first step: keep this call's live slots
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool use = live && j0 + u * GP < np;
      mj[u] = use ? mj[u] : -INFINITY;
      lj[u] = use ? lj[u] : 0.f;
      o[u] = use ? o[u] : fvec{};
    }
    fold();
    j0 += GP * U;
  }
  for (; j0 < np; j0 += GP * U) {
    // all three requested together: one round trip per step
    load_step(base, j0, live ? np : 0);
    fold();
  }
  const float M = GroupReduce<GP>::all(mt, lds, [](float x, float y) { return fmaxf(x, y); });
  const float r = (mt == -INFINITY) ? 0.f : exp2f(mt - M);
  float sums[VEC + 1];
#pragma unroll
  for (int e = 0; e < VEC; ++e) sums[e] = acc[e] * r;
  sums[VEC] = den * r;
  GroupReduce<GP>::sum_n(sums, lds_n);
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = sums[e];
  den = sums[VEC];
  if (gp != 0 || !live) return;
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int i = n / G, g = n - i * G;
  T* op = (T*)a.out + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D + d4 * VEC;
#pragma unroll
  for (int e = 0; e < VEC; ++e) store_elem<T>(op + e, acc[e] * inv);
}

// Exclusive prefix sum of query_lens[0 .. B) into qoffs (one workgroup of
// 1024 threads: per-thread runs, a wave scan, then the waves in order).
__global__ __launch_bounds__(1024) void scan_row_offsets(const int32_t* __restrict__ query_lens,
                                                         int B, int32_t* __restrict__ qoffs) {
  __shared__ int s_wave[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (B + 1023) / 1024;
  const int k0 = min(B, tid * per), k1 = min(B, k0 + per);
  int cnt = 0;
  for (int k = k0; k < k1; ++k) cnt += query_lens[k];
  int inc = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int run = inc - cnt;
  for (int w = 0; w < wave; ++w) run += s_wave[w];
  for (int k = k0; k < k1; ++k) {
    qoffs[k] = run;
    run += query_lens[k];
  }
}

// Partition lanes per output unit for a given number of states per unit.
inline int reduce_group_lanes(int num_states) {
  return num_states <= 32 ? 1 : (num_states <= 256 ? 16 : 32);
}

struct SpanArgs {
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* query_lens;
  int32_t* seq_info;  // [B, 4]
  int32_t* row_info;  // [T, 2]
  int32_t* blocks;    // [B, max_blocks_per_seq]
  int32_t* parts;     // [B, NP, 2]
  int window;
  int part_size;
  int num_parts;
  int log2_bs;
  int max_blocks_per_seq;
};

// One wave per sequence; uses exactly the helpers of the partition kernels.
__global__ __launch_bounds__(64) void debug_spans(SpanArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int L = a.seq_lens[b], q = a.query_lens[b];
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  const int qoff = wave_row_offset(a.query_lens, b);
  if (lane == 0) {
    a.seq_info[b * 4 + 0] = qoff;
    a.seq_info[b * 4 + 1] = sv.lo;
    a.seq_info[b * 4 + 2] = sv.hi;
    a.seq_info[b * 4 + 3] = sv.nparts;
  }
  for (int i = lane; i < q; i += 64) {
    a.row_info[(qoff + i) * 2 + 0] = first_visible(L, q, i, a.window);
    a.row_info[(qoff + i) * 2 + 1] = L - q + i;
  }
  const int32_t* table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const int bs = 1 << a.log2_bs;
  for (int k = lane; k < a.max_blocks_per_seq; k += 64) {
    const bool seen = sv.nparts > 0 && (long)k * bs < sv.hi && (long)(k + 1) * bs > sv.lo;
    a.blocks[(size_t)b * a.max_blocks_per_seq + k] =
        seen ? phys_block(table, max(k * bs, sv.lo), a.log2_bs) : -1;
  }
  for (int jj = lane; jj < a.num_parts; jj += 64) {
    int ps = sv.hi, pe = sv.hi;
    if (jj < sv.nparts) partition_range(sv, jj, a.part_size, &ps, &pe);
    a.parts[((size_t)b * a.num_parts + jj) * 2 + 0] = ps;
    a.parts[((size_t)b * a.num_parts + jj) * 2 + 1] = pe;
  }
}

// Precondition check (debug aid).  report = {bad length sequences, bad table
// entries, first bad sequence, first bad entry}; check_init clears it on the
// stream first (a kernel, so that the pair can sit in a captured graph).
struct CheckArgs {
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* query_lens;
  int32_t* report;
  int window;
  int log2_bs;
  int max_blocks_per_seq;
  int max_seq_len;
  int max_query_len;
  int num_blocks;
};

__global__ __launch_bounds__(64) void check_init(int32_t* report) {
  if (threadIdx.x < 4) report[threadIdx.x] = threadIdx.x < 2 ? 0 : 0x7fffffff;
}

// One wave per sequence.
__global__ __launch_bounds__(64) void check_inputs(CheckArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int L = a.seq_lens[b], q = a.query_lens[b];
  if (q < 0 || L < 0 || q > L || L > a.max_seq_len || q > a.max_query_len) {
    if (lane == 0) {
      atomicAdd(&a.report[0], 1);
      atomicMin(&a.report[2], b);
    }
    return;
  }
  if (q == 0) return;  // no row: no position is visible
  // union of the rows' visible ranges: [first visible of row 0, L)
  const int k0 = first_visible(L, q, 0, a.window) >> a.log2_bs;
  const int k1 = min((L - 1) >> a.log2_bs, a.max_blocks_per_seq - 1);
  const int32_t* row = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  for (int k = k0 + lane; k <= k1; k += 64) {
    const int id = row[k];
    if (id < 0 || id >= a.num_blocks) {
      atomicAdd(&a.report[1], 1);
      const long long at = (long long)b * a.max_blocks_per_seq + k;
      atomicMin(&a.report[3], (int)min(at, 0x7ffffffeLL));
    }
  }
}

}  // namespace pa
