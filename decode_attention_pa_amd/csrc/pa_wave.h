// Partition kernel on the vector ALUs, register-resident (no staging of K or
// V through shared memory): fp32 arithmetic for fp32 or bf16 caches, head
// dims 64, 128 and 256, 4 or 8 packed rows per workgroup.
//
// One workgroup = 4 waves = one context partition of one (sequence, KV head)
// and RB packed rows (row n = i*G + g).  The partition is walked in steps of
// 64 positions; wave w takes steps w, w+4, ...  Per step:
//
//   QK^T  lane t owns position t of the step: it loads that position's key
//         in 16-byte pieces (8-element columns of the tiled K layout) and
//         forms the RB dot products itself, so no cross-lane sum is needed.
//         The query rows stay in registers, 16 values per register (one per
//         lane of a 16-lane row, the same in the wave's four rows), and each
//         product takes its query value by a DPP row broadcast folded into
//         the multiply-add (v_fmac_f32 with row_newbcast).
//   mask  visible iff first_visible(row) <= pos <= row position, pos in the
//         partition; masked scores become -inf by select.
//   online softmax (log2 domain): each row's step max is a wave reduction
//         (row swaps, then DPP inside 16-lane rows); the reference max
//         moves only when a step beats it by more than 2^8 (as on the
//         matrix cores); a row with nothing visible keeps -inf and never
//         evaluates (-inf) - (-inf).
//   PV    for each group of 8 positions the wave reads the group's [D][8] V
//         tile as 16-byte columns, lane t taking columns t, t + 64, ... (each
//         load instruction reads 1 KB contiguous, non-temporal): in bf16 a
//         column is one dim's 8 slots, in fp32 half of them (a lane pair
//         shares a dim and adds its halves at the end).  It accumulates
//         p * v, the step's weights read back from a per-wave shared-memory
//         row (written once per step).
//
// The waves' states are merged in a fixed order at the end (deterministic).
// Output contract as the other partition kernels: a sequence with one
// partition writes `out`, otherwise (max, exp-sum, normalised partial
// output) per row goes to the workspace for the LSE merge.
#pragma once

#include "pa_common.h"
#include "pa_sched.h"
#include "pa_valu.h"

namespace pa {

__device__ inline float wave_max(float x) {
  return wave_op(x, [](float a, float b) { return fmaxf(a, b); });
}

__device__ inline float wave_sum(float x) {
  return wave_op(x, [](float a, float b) { return a + b; });
}

// 8 consecutive elements at p as fp32 (16-byte loads).
template <typename T>
__device__ inline void load8(const T* p, float (&x)[8]);
// Cached 16-byte loads, for K: a key instruction uses half of each line it
// touches and the next one the other half (measured on MI355X, fp32 GQA
// batch: non-temporal K loads 2 % slower; with the earlier V mapping, whose
// loads also leaned on the caches, 36 %).
template <typename V>
__device__ inline V ld16(const V* p) {
  return *p;
}
template <>
__device__ inline void load8<float>(const float* p, float (&x)[8]) {
  const f32x4 a = ld16((const f32x4*)p), b = ld16((const f32x4*)(p + 4));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}
template <>
__device__ inline void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const u32x4 w = ld16((const u32x4*)p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

// One 16-byte column of a V tile as fp32: 4 fp32 or 8 bf16 elements.  V
// instructions read whole lines (1 KB contiguous per instruction), so they
// stream past the caches (measured on MI355X, against cached loads: the
// fp32 GQA batch 202.5 -> 184 us, the bf16 one on this kernel 126 -> 112 us).
template <typename T>
__device__ inline void load_col(const T* p, float (&x)[16 / sizeof(T)]);
template <>
__device__ inline void load_col<float>(const float* p, float (&x)[4]) {
  const f32x4 a = __builtin_nontemporal_load((const f32x4*)p);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = a[e];
}
template <>
__device__ inline void load_col<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const u32x4 w = __builtin_nontemporal_load((const u32x4*)p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

// Dot products with the query values taken by DPP row broadcasts folded
// into the multiply-add: v_fmac_f32_dpp acc, q, k row_newbcast:M adds
// q(lane M of the caller's 16-lane row) * k.  Each block below is one asm
// statement, so nothing is scheduled into it: it opens with two wait states
// (a DPP instruction must not read a register that a vector instruction
// wrote in the two instructions before it), and inside it consecutive
// multiply-adds go to different accumulators (4 or 8 rows apart).  Block
// (H): elements H .. H+7 of a 16-element slice, k0..k7 the key values,
// q_r the row-r query register.
#define PA_FMA(A, Q, K, M) \
  "v_fmac_f32_dpp %" #A ", %" #Q ", %" #K " row_newbcast:" #M " row_mask:0xf bank_mask:0xf\n\t"
#define PA_ROWS4(K, M) PA_FMA(0, 4, K, M) PA_FMA(1, 5, K, M) PA_FMA(2, 6, K, M) PA_FMA(3, 7, K, M)
#define PA_ROWS8(K, M)                                                                       \
  PA_FMA(0, 8, K, M) PA_FMA(1, 9, K, M) PA_FMA(2, 10, K, M) PA_FMA(3, 11, K, M)             \
  PA_FMA(4, 12, K, M) PA_FMA(5, 13, K, M) PA_FMA(6, 14, K, M) PA_FMA(7, 15, K, M)

template <int RB, int H>
__device__ __forceinline__ void dot8(float (&s)[RB], const float (&q)[RB], const float* k);

template <>
__device__ __forceinline__ void dot8<4, 0>(float (&s)[4], const float (&q)[4], const float* k) {
  asm("s_nop 1\n\t" PA_ROWS4(8, 0) PA_ROWS4(9, 1) PA_ROWS4(10, 2) PA_ROWS4(11, 3)
      PA_ROWS4(12, 4) PA_ROWS4(13, 5) PA_ROWS4(14, 6) PA_ROWS4(15, 7)
      : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3])
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]),
        "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]));
}
template <>
__device__ __forceinline__ void dot8<4, 8>(float (&s)[4], const float (&q)[4], const float* k) {
  asm("s_nop 1\n\t" PA_ROWS4(8, 8) PA_ROWS4(9, 9) PA_ROWS4(10, 10) PA_ROWS4(11, 11)
      PA_ROWS4(12, 12) PA_ROWS4(13, 13) PA_ROWS4(14, 14) PA_ROWS4(15, 15)
      : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3])
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]),
        "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]));
}
template <>
__device__ __forceinline__ void dot8<8, 0>(float (&s)[8], const float (&q)[8], const float* k) {
  asm("s_nop 1\n\t" PA_ROWS8(16, 0) PA_ROWS8(17, 1) PA_ROWS8(18, 2) PA_ROWS8(19, 3)
      PA_ROWS8(20, 4) PA_ROWS8(21, 5) PA_ROWS8(22, 6) PA_ROWS8(23, 7)
      : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]), "+v"(s[4]), "+v"(s[5]), "+v"(s[6]),
        "+v"(s[7])
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]),
        "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]));
}
template <>
__device__ __forceinline__ void dot8<8, 8>(float (&s)[8], const float (&q)[8], const float* k) {
  asm("s_nop 1\n\t" PA_ROWS8(16, 8) PA_ROWS8(17, 9) PA_ROWS8(18, 10) PA_ROWS8(19, 11)
      PA_ROWS8(20, 12) PA_ROWS8(21, 13) PA_ROWS8(22, 14) PA_ROWS8(23, 15)
      : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]), "+v"(s[4]), "+v"(s[5]), "+v"(s[6]),
        "+v"(s[7])
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]),
        "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]));
}
#undef PA_ROWS8
#undef PA_ROWS4
#undef PA_FMA

// One run: partitions j_first .. j_last of unit (sequence b, KV head h),
// rows r0 .. r0 + RB - 1 of it, as one stretch of positions taken by the 4
// waves in steps of 64.  With `write_out` (the run is the whole unit) it
// writes `out`; otherwise its state (max, exp-sum, normalised output) goes
// to state slot `state` (R rows per slot).  All waves of the workgroup call
// it with the same arguments, and all return from it.
template <typename T, int D, int RB>
__device__ __forceinline__ void wave_run(const PartArgs& a, int b, int h, int L, int q, int qoff,
                                         const SeqView& sv, int j_first, int j_last, size_t state,
                                         bool write_out, int r0) {
  constexpr int NW = 4;
  // PV reads the [D][8] V tile of a group of 8 positions as 16-byte columns,
  // column c = 64 * i + lane (i < VC), so that each load instruction reads
  // 1 KB contiguous.  Column c holds EPC consecutive slots of dim
  // c * EPC / 8 from slot c * EPC % 8: in bf16 a whole dim (lane owns dims
  // lane + 64 i), in fp32 half of one (lanes 2m and 2m + 1 share dims
  // m + 32 i, each summing 4 of the 8 positions, added at the end).
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int VC = D * 8 / EPC / 64;
  constexpr int NJ = D / 16;  // 16-dim slices of a key
  // Loads in flight per wave: JB 16-element key slices per batch, V groups
  // of 8 positions 4 at a time (measured on MI355X, fp32 GQA batch: 4 and 4
  // beat 2 and 2 by 9 %, and 8 and 8 by 10 %)
  constexpr int JB = 4 < NJ ? 4 : NJ;  // slices per batch of key loads
  __shared__ float p_s[NW][64][RB];
  __shared__ float m_s[NW][RB], l_s[NW][RB];
  __shared__ float o_s[NW - 1][RB][D];

  qoff = __builtin_amdgcn_readfirstlane(qoff);  // uniform: addresses stay scalar
  const int G = a.group;
  const int rows_b = G * q;
  const int ps = max(sv.lo, sv.base + j_first * a.part_size);
  const int pe = min(sv.hi, sv.base + (j_last + 1) * a.part_size);
  const int cb0 = sv.base + j_first * a.part_size;  // multiple of 32
  const int nst = (pe - cb0 + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int log2_bs = a.log2_bs;
  const int bs_mask = (1 << log2_bs) - 1;
  const int32_t* __restrict__ table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const __attribute__((address_space(4))) int32_t* stable =
      (const __attribute__((address_space(4))) int32_t*)table;
  const T* __restrict__ kc = (const T*)a.k_cache;
  const T* __restrict__ vc = (const T*)a.v_cache;
  const size_t slab = (size_t)D << log2_bs;  // elements per (block, head)
  const size_t blk_stride = slab * (size_t)a.num_kv_heads;
  const size_t head_off = slab * (size_t)h;
  const float scale_log2 = a.scale_log2;

  // Query rows in registers as fp32, replicated in each 16-lane row: element
  // 16j + m of row r in qv[r][j] at lane m (zeros past the sequence's rows).
  // Rows: visible interval inside the partition (wave-uniform).
  float qv[RB][NJ];
  int tlo[RB], thi[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int n = r0 + r;
    const int i = n / G, g = n - i * G;
    const T* qrow = (const T*)a.q + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) qv[r][jj] = n < rows_b ? load_elem<T>(qrow + 16 * jj + (lane & 15)) : 0.f;
    tlo[r] = max(ps, first_visible(L, q, i, a.window));
    thi[r] = min(pe - 1, L - q + i);
    if (n >= rows_b || thi[r] < tlo[r]) {
      tlo[r] = 0x7fffffff;
      thi[r] = -1;
    }
  }


  const int slot0 = (lane * EPC) & 7;  // first slot of this lane's columns
  auto vdim = [&](int i) { return ((64 * i + lane) * EPC) >> 3; };
  float mrun[RB], lrun[RB], acc[RB][VC];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    mrun[r] = -INFINITY;
    lrun[r] = 0.f;
#pragma unroll
    for (int i = 0; i < VC; ++i) acc[r][i] = 0.f;
  }

  for (int t = wave; t < nst; t += NW) {
    const int cs = cb0 + 64 * t;
    // QK^T: lane = position
    const int pos = cs + lane;
    const int pc = min(max(pos, ps), pe - 1);  // clamp: never touch blocks outside the span
    const int blk = table[pc >> log2_bs];
    const T* kp = kc + (size_t)blk * blk_stride + head_off + k_slot_offset(pc & bs_mask, D);
    float s[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) s[r] = 0.f;
    // key slices in batches of JB x 16 elements per lane in flight, so that
    // the registers do not grow with the head dim
#pragma unroll
    for (int j0 = 0; j0 < NJ; j0 += JB) {
      float kv[JB][16];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        float lo[8], hi[8];
        load8<T>(kp + (2 * (j0 + jj)) * 64, lo);
        load8<T>(kp + (2 * (j0 + jj) + 1) * 64, hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[jj][e] = lo[e];
          kv[jj][8 + e] = hi[e];
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        float qj[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) qj[r] = qv[r][j0 + jj];
        dot8<RB, 0>(s, qj, &kv[jj][0]);
        dot8<RB, 8>(s, qj, &kv[jj][8]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // mask, online softmax, weights to shared memory
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float x = (uint32_t)(pos - tlo[r]) <= (uint32_t)(thi[r] - tlo[r]) ? s[r] * scale_log2
                                                                              : -INFINITY;
      const float mx = wave_max(x);
      if (mx > mrun[r] + 8.f) {  // wave-uniform
        const float alpha = __builtin_amdgcn_exp2f(mrun[r] - mx);  // 0 while mrun = -inf
        lrun[r] *= alpha;
#pragma unroll
        for (int i = 0; i < VC; ++i) acc[r][i] *= alpha;
        mrun[r] = mx;
      }
      const float mref = (mrun[r] == -INFINITY) ? 0.f : mrun[r];
      const float p = __builtin_amdgcn_exp2f(x - mref);
      lrun[r] += p;
      p_s[wave][lane][r] = p;
    }
    __builtin_amdgcn_wave_barrier();
    // PV: lane = VC columns of each group's V tile; 8 groups of 8 positions
#pragma unroll 4
    for (int gi = 0; gi < 8; ++gi) {
      const int p8 = cs + 8 * gi;
      if (p8 >= pe || p8 + 8 <= ps) continue;  // wave-uniform: the group holds nothing visible
      const int pb = max(p8, ps);
      const int gblk = stable[pb >> log2_bs];
      const T* vt = vc + (size_t)gblk * blk_stride + head_off + (size_t)((p8 & bs_mask) >> 3) * D * 8;
      float v[VC][EPC];
#pragma unroll
      for (int i = 0; i < VC; ++i) load_col<T>(vt + (size_t)(64 * i + lane) * EPC, v[i]);
      if (p8 < ps || p8 + 8 > pe) {
        // edge group: slots outside [ps, pe) may hold anything (NaN): zero by select
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const bool ok = p8 + slot0 + e >= ps && p8 + slot0 + e < pe;
#pragma unroll
          for (int i = 0; i < VC; ++i) v[i][e] = ok ? v[i][e] : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        float pv[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) pv[r] = p_s[wave][8 * gi + slot0 + e][r];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int i = 0; i < VC; ++i) acc[r][i] = fmaf(pv[r], v[i][e], acc[r][i]);
      }
    }
    __builtin_amdgcn_wave_barrier();  // the weights are read before the next step writes them
  }

  // exp-sums across lanes, the halves of each dim (fp32), then the waves'
  // states in a fixed order
#pragma unroll
  for (int r = 0; r < RB; ++r) lrun[r] = wave_sum(lrun[r]);
  if constexpr (EPC < 8) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < VC; ++i) acc[r][i] += dpp<kDppXor1>(acc[r][i]);
  }
  const bool writer = slot0 == 0;  // one lane per dim stores
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      m_s[wave][r] = mrun[r];
      l_s[wave][r] = lrun[r];
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < VC; ++i) o_s[wave - 1][r][vdim(i)] = acc[r][i];  // pairs: equal values
  }
  __syncthreads();
  if (wave != 0) return;  // (every wave returns; wave 0 after the stores below)
  const bool one_shot = write_out;
  const size_t wbase = state * a.rows;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int n = r0 + r;
    if (n >= rows_b) break;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, m_s[w][r]);
    const float mref = (M == -INFINITY) ? 0.f : M;
    const float f0 = __builtin_amdgcn_exp2f(m_s[0][r] - mref);
    float l = l_s[0][r] * f0;
    float o[VC];
#pragma unroll
    for (int i = 0; i < VC; ++i) o[i] = acc[r][i] * f0;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float fw = __builtin_amdgcn_exp2f(m_s[w][r] - mref);
      l += l_s[w][r] * fw;
#pragma unroll
      for (int i = 0; i < VC; ++i) o[i] += fw * o_s[w - 1][r][vdim(i)];
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (one_shot) {
      const int i = n / G, g = n - i * G;
      T* op = (T*)a.out + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D;
      if (writer)
#pragma unroll
        for (int c = 0; c < VC; ++c) store_elem<T>(op + vdim(c), o[c] * inv);
    } else {
      float* op = a.ws_o + (wbase + n) * D;
      if (writer)
#pragma unroll
        for (int c = 0; c < VC; ++c) op[vdim(c)] = o[c] * inv;
      if (lane == 0) {
        a.ws_m[wbase + n] = M;
        a.ws_l[wbase + n] = l;
      }
    }
  }
}

// Grid schedule: one workgroup per (partition, sequence, KV head, row block).
template <typename T, int D, int RB>
__global__ __launch_bounds__(256) void part_wave(PartArgs a) {
  const PartItem it = part_item(a);
  const int ro = row_offset_issue(a.query_lens, it.b);  // travels with the lengths
  const int L = a.seq_lens[it.b];
  const int q = a.query_lens[it.b];
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  if (it.j >= sv.nparts) return;         // past the unit's partitions: no state to store
  const int r0 = it.rb * RB;
  if (r0 >= a.group * q) return;         // no row of this sequence in this block
  const int qoff = __builtin_amdgcn_readfirstlane(row_offset_finish(ro, a.qoffs, a.query_lens, it.b));
  const size_t state = ((size_t)it.b * a.num_kv_heads + it.h) * a.num_parts + it.j;
  wave_run<T, D, RB>(a, it.b, it.h, L, q, qoff, sv, it.j, it.j, state, sv.nparts == 1, r0);
}

// Persistent schedule (persistent_shares): every row of a unit in one
// workgroup (RB >= R).
template <typename T, int D, int RB>
__global__ __launch_bounds__(256) void part_wave_ps(PartArgs a) {
  persistent_shares<256>(a, [&](int b, int h, int L, int q, int qoff, const SeqView& sv, int j1,
                                int j2, size_t state, bool whole) {
    wave_run<T, D, RB>(a, b, h, L, q, qoff, sv, j1, j2, state, whole, 0);
  });
}

}  // namespace pa
