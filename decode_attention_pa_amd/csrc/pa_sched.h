// Persistent schedule shared by the partition kernels: the shares of work
// every workgroup of a resident grid takes, and the runs it makes of them.
#pragma once

#include "pa_common.h"

namespace pa {

// Largest batch the persistent schedule handles (its per-sequence prefix sums
// live in shared memory); larger batches use the grid schedule.
constexpr int kPsMaxBatch = 1024;

// Persistent schedule (aiter PR #2914: "PS" decode): a grid whose
// workgroups are all resident at once (the launcher picks how many per CU,
// at most what fits).  The partitions of all units form one list,
// unit-major ((sequence, KV head), then partition); workgroup w takes the
// contiguous share [w*I/W, (w+1)*I/W) of the I partitions and runs each
// unit's stretch of it as one run.  Shares differ by at most one partition,
// so there is no tail of late workgroups, and a workgroup's set-up is paid
// once per unit it touches rather than once per partition.  A run that is a
// whole unit writes `out`; otherwise it stores its state in slot w + u (w
// its workgroup, u = b * H_kv + h its unit).  Walking the shares in order,
// each (share, unit) pair steps w, u or both up by one, so these slots are
// distinct, those of one unit are consecutive (w_first + u onwards), and
// all lie below W + units: the workspace holds W + units states, whatever
// the partition count.  The unit's last run records its run count and first
// slot for the merge (count 0 when the unit was written directly).
//
// `run(b, h, L, q, qoff, sv, j_first, j_last, state, whole)` is called by
// every thread of the workgroup for each run, in order; it processes
// partitions j_first .. j_last of unit (b, h) as one stretch and stores its
// state in slot `state` (or writes `out` when `whole`).  NT threads.
template <int NT, typename Run>
__device__ __forceinline__ void persistent_shares(const PartArgs& a, Run&& run) {
  constexpr int NW = NT / 64;
  // Multi-wave workgroups keep the sequence lengths the scan reads, which
  // takes a dependent global load off the start of every run (1000 sequences
  // of 256 tokens: 38.4 -> 37.3 us per call).  One-wave workgroups reload
  // them: 4 KB more shared memory would cost them a wave of occupancy.
  constexpr bool kKeepLens = NW > 1;
  __shared__ int s_np[kPsMaxBatch + 1];  // exclusive prefix of partitions per sequence
  __shared__ int s_q[kPsMaxBatch + 1];   // exclusive prefix of query tokens (q/out row)
  __shared__ int s_len[kKeepLens ? kPsMaxBatch : 1];
  __shared__ int s_wave[2][NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.batch;
  // Block-wide exclusive scan of (partitions, query tokens) over sequences.
  const int per = (B + NT - 1) / NT;
  const int k0 = min(B, tid * per), k1 = min(B, k0 + per);
  int cnt_np = 0, cnt_q = 0;
  for (int k = k0; k < k1; ++k) {
    const int q = a.query_lens[k], L = a.seq_lens[k];
    if constexpr (kKeepLens) s_len[k] = L;
    cnt_np += seq_view(L, q, a.window, a.part_size).nparts;
    cnt_q += q;
  }
  int inc_np = cnt_np, inc_q = cnt_q;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t_np = __shfl_up(inc_np, off), t_q = __shfl_up(inc_q, off);
    if (lane >= off) {
      inc_np += t_np;
      inc_q += t_q;
    }
  }
  if (lane == 63) {
    s_wave[0][wave] = inc_np;
    s_wave[1][wave] = inc_q;
  }
  __syncthreads();
  int run_np = inc_np - cnt_np, run_q = inc_q - cnt_q;
  for (int w = 0; w < wave; ++w) {
    run_np += s_wave[0][w];
    run_q += s_wave[1][w];
  }
  for (int k = k0; k < k1; ++k) {
    s_np[k] = run_np;
    s_q[k] = run_q;
    const int q = a.query_lens[k];
    run_np += seq_view(kKeepLens ? s_len[k] : a.seq_lens[k], q, a.window, a.part_size).nparts;
    run_q += q;
  }
  if (tid == NT - 1) {
    s_np[B] = run_np;
    s_q[B] = run_q;
  }
  __syncthreads();

  const int H = a.num_kv_heads;
  const long total = (long)H * s_np[B];
  // Shares over at most `total` workgroups, so that every share is non-empty
  // and a run's ordinal within its unit stays below the unit's partition count.
  const long W = min((long)gridDim.x, total);
  if ((long)blockIdx.x >= W) return;
  long i0 = (long)blockIdx.x * total / W;
  const long i1 = ((long)blockIdx.x + 1) * total / W;
  while (i0 < i1) {
    // sequence of partition i0: the last b with H * s_np[b] <= i0
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long)H * s_np[mid] <= i0) lo = mid;
      else hi = mid - 1;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int np_b = s_np[b + 1] - s_np[b];
    const long rel = i0 - (long)H * s_np[b];
    const int h = __builtin_amdgcn_readfirstlane((int)(rel / np_b));
    const int j1 = __builtin_amdgcn_readfirstlane((int)(rel - (long)h * np_b));
    const int j2 = (int)min((long)np_b - 1, (long)j1 + (i1 - i0) - 1);
    const int L = kKeepLens ? s_len[b] : a.seq_lens[b];
    const int q = s_q[b + 1] - s_q[b];
    const SeqView sv = seq_view(L, q, a.window, a.part_size);
    // ordinal of this run among the unit's runs: this workgroup minus the
    // workgroup whose share holds the unit's first partition (item A);
    // share w starts at floor(w*I/W), so item i lies in share ceil((i+1)W/I)-1
    const long A = (long)H * s_np[b] + (long)h * np_b;
    const long w_first = ((A + 1) * W + total - 1) / total - 1;
    const int slot = (int)((long)blockIdx.x - w_first);
    const bool whole = (j1 == 0 && j2 == np_b - 1);
    const size_t unit = (size_t)b * H + h;
    run(b, h, L, q, s_q[b], sv, j1, j2, (size_t)blockIdx.x + unit, whole);
    // (one-shot plans have no workspace: every unit is whole and no merge runs)
    if (j2 == np_b - 1 && tid == 0 && a.ws_runs != nullptr)
      *(int2*)(a.ws_runs + 2 * unit) = make_int2(whole ? 0 : slot + 1, (int)(w_first + (long)unit));
    __syncthreads();  // the next run reuses the run's shared memory
    i0 += j2 - j1 + 1;
  }
}

}  // namespace pa
