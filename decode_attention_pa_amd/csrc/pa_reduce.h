// Log-sum-exp merge of context partitions, and the index-dump kernel.
//
// Merge (executorch PR #18759, split-K reduce; aiter PR #2914, PS reduce over
// max_logits / exp_sums / temporary_output): for one packed row of one
// (sequence, KV head), with partition states (m_j, l_j, o_j) where o_j is the
// partition's normalised output and m_j its max logit in the log2 domain,
//     M = max_j m_j,  w_j = 2^(m_j - M) * l_j  (0 when m_j = -inf),
//     out = sum_j w_j o_j / sum_j w_j.
// A partition in which the row sees nothing has m_j = -inf, l_j = 0, o_j = 0
// and weight 0 (gllm #116: a split with no positions "contributes
// nothing").  Partitions are summed in a fixed order: results are
// deterministic.
#pragma once

#include "pa_common.h"
#include "pa_valu.h"

namespace pa {

// Two launch shapes, chosen on the host from the partition count NP:
//
//  * narrow (NP <= kNarrowMaxParts): one 256-thread workgroup per (sequence,
//    KV head); wave w merges rows w, w+4, ...; each lane owns D/64 dims and
//    requests all of its partitions' slices at once.  Few workgroups, one
//    round trip per row.
//  * wide: one workgroup per (32-dim slice, packed row, KV head, sequence);
//    32 partition groups x 8 lanes x float4, several loads in flight per
//    lane, partition groups summed in a fixed order afterwards.  Many lanes
//    per row when a row has hundreds of partitions.
constexpr int kNarrowMaxParts = 32;
constexpr int kReduceSlice = 32;   // dims per wide workgroup
constexpr int kReduceGroups = 32;  // partition groups per wide workgroup

template <typename T, int D>
__global__ __launch_bounds__(256) void lse_reduce_narrow(ReduceArgs a) {
  constexpr int DPL = D / 64;  // dims per lane
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = a.seq_lens[b];
  const int q = a.query_lens[b];
  const int G = a.group;
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  const int np = min(sv.nparts, a.num_parts);
  if (np <= 1) return;  // the partition kernel wrote these rows directly
  const int qoff = wave_row_offset(a.query_lens, b);
  const size_t base = ((size_t)b * a.num_kv_heads + h) * a.num_parts;
  for (int n = wave; n < G * q; n += 4) {
    float mj[kNarrowMaxParts], lj[kNarrowMaxParts];
    float o[kNarrowMaxParts][DPL];
#pragma unroll
    for (int jj = 0; jj < kNarrowMaxParts; ++jj) {
      mj[jj] = -INFINITY;
      lj[jj] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[jj][e] = 0.f;
      if (jj < np) {
        const size_t w = (base + jj) * a.rows + n;
        mj[jj] = a.ws_m[w];
        lj[jj] = a.ws_l[w];
        const float* op = a.ws_o + w * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[jj][e] = op[e];
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kNarrowMaxParts; ++jj) M = fmaxf(M, mj[jj]);
    const float mref = (M == -INFINITY) ? 0.f : M;
    float acc[DPL], den = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
#pragma unroll
    for (int jj = 0; jj < kNarrowMaxParts; ++jj) {
      const float f = (mj[jj] == -INFINITY) ? 0.f : exp2f(mj[jj] - mref) * lj[jj];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += f * o[jj][e];
      den += f;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const int i = n / G, g = n - i * G;
    T* op = (T*)a.out + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_elem<T>(op + e, acc[e] * inv);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void lse_reduce_wide(ReduceArgs a) {
  constexpr int NS = D / kReduceSlice;
  const int slice = blockIdx.x % NS;
  const int n = blockIdx.x / NS;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = a.seq_lens[b];
  const int q = a.query_lens[b];
  const int G = a.group;
  if (n >= G * q) return;
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  const int np = min(sv.nparts, a.num_parts);
  if (np <= 1) return;  // the partition kernel wrote this row directly

  __shared__ float red[4];
  __shared__ f32x4 sacc[kReduceGroups][8];
  __shared__ float sden[kReduceGroups];
  const size_t base = ((size_t)b * a.num_kv_heads + h) * a.num_parts;
  float M = -INFINITY;
  for (int jj = tid; jj < np; jj += 256) M = fmaxf(M, a.ws_m[(base + jj) * a.rows + n]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float mref = (M == -INFINITY) ? 0.f : M;

  const int grp = tid >> 3;        // partition group
  const int d4 = (tid & 7) * 4;    // dims d4 .. d4+3 of the slice
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  constexpr int U = 4;
  for (int j0 = grp; j0 < np; j0 += kReduceGroups * U) {
    float f[U];
    f32x4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j0 + u * kReduceGroups;
      f[u] = 0.f;
      o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jj < np) {
        const size_t w = (base + jj) * a.rows + n;
        const float mj = a.ws_m[w];
        f[u] = (mj == -INFINITY) ? 0.f : exp2f(mj - mref) * a.ws_l[w];
        o[u] = *(const f32x4*)(a.ws_o + w * D + slice * kReduceSlice + d4);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc += f[u] * o[u];
      den += f[u];
    }
  }
  sacc[grp][tid & 7] = acc;
  if ((tid & 7) == 0) sden[grp] = den;
  // every lane of the wave takes part in the prefix sum's shuffles
  const int qoff = wave_row_offset(a.query_lens, b);
  __syncthreads();
  if (tid >= kReduceSlice) return;
  // thread tid finalises dim tid of the slice
  float s = 0.f, tot = 0.f;
#pragma unroll 8
  for (int g = 0; g < kReduceGroups; ++g) {
    s += sacc[g][tid >> 2][tid & 3];
    tot += sden[g];
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int i = n / G, g = n - i * G;
  T* op = (T*)a.out + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D;
  store_elem<T>(op + slice * kReduceSlice + tid, s * inv);
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

}  // namespace pa
