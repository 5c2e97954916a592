// Partition kernel on the vector ALUs: fp32 arithmetic for any element type,
// any head dim D <= 256, any number of packed rows (16 per workgroup).
//
// Used for float32 inputs (no reduced-precision products at all), for head
// dims the matrix-core kernels do not take (gllm #116, "Verification": its
// GPU test also runs head dim 66 through its non-flash kernel), and as a
// forced alternative for bf16.  One 256-thread workgroup handles 16 packed
// rows (row n = i*G + g) of one context partition of one (sequence, KV head);
// the partition is walked in 16-position steps staged through LDS:
//
//   stage   K [16][D] and V [D][16] in fp32 (K from its 16-slot tiles, or one
//           row per slot when D is not a multiple of 8; V from its 8-slot
//           [D][8] tiles); positions outside the partition are stored as
//           zeros, never read from HBM
//   scores  one thread per (row, position): D-term dot product, masked by
//           select to -inf outside the row's visible interval
//   softmax one thread per row: running max (log2 domain), rescale factor,
//           exp-sum; a row with nothing visible keeps max = -inf and never
//           evaluates (-inf) - (-inf)
//   PV      thread d owns output dim d of all 16 rows: acc = acc*alpha + p . v
//
// Output contract is the same as the matrix-core kernel: one-shot sequences
// write `out`, split sequences write (max, exp-sum, normalised partial).
#pragma once

#include "pa_common.h"

namespace pa {

constexpr int kValuRows = 16;   // packed rows per workgroup
constexpr int kValuStep = 16;   // positions staged per step
constexpr int kValuMaxD = 256;  // largest head dim

template <typename T>
__device__ inline float load_elem(const T* p);
template <>
__device__ inline float load_elem<float>(const float* p) { return *p; }
template <>
__device__ inline float load_elem<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }

template <typename T>
__device__ inline void store_elem(T* p, float x);
template <>
__device__ inline void store_elem<float>(float* p, float x) { *p = x; }
template <>
__device__ inline void store_elem<uint16_t>(uint16_t* p, float x) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <typename T>
__global__ __launch_bounds__(256) void part_valu(PartArgs a) {
  constexpr int NT = 256, RB = kValuRows, SUB = kValuStep, DM = kValuMaxD;
  __shared__ float q_s[RB][DM + 1];
  __shared__ float k_s[SUB][DM + 1];
  __shared__ float v_s[DM][SUB + 1];
  __shared__ float p_s[RB][SUB + 1];
  __shared__ float alpha_s[RB];
  __shared__ float lsum_s[RB];
  __shared__ float mmax_s[RB];
  __shared__ int tlo_s[RB], thi_s[RB];

  const PartItem it = part_item(a);
  const int j = it.j, h = it.h, b = it.b;
  const int tid = threadIdx.x;
  const int D = a.head_dim;
  const int L = a.seq_lens[b];
  const int q = a.query_lens[b];
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  if (j >= sv.nparts) return;  // past the unit's partitions: no state to store
  const int G = a.group;
  const int rows_b = G * q;
  const int r0 = it.rb * RB;
  if (r0 >= rows_b) return;    // no row of this sequence in this block
  int ps, pe;
  partition_range(sv, j, a.part_size, &ps, &pe);
  const int cb0 = sv.base + j * a.part_size;
  const int nsub = (pe - cb0 + SUB - 1) / SUB;
  const int qoff = row_offset(a.qoffs, a.query_lens, b);
  const int log2_bs = a.log2_bs;
  const int bs_mask = (1 << log2_bs) - 1;
  const bool k_rows = (D & 7) != 0;  // K layout: one row per slot, else 16-slot tiles
  const int32_t* __restrict__ table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const T* __restrict__ kc = (const T*)a.k_cache;
  const T* __restrict__ vc = (const T*)a.v_cache;
  const size_t slab = (size_t)D << log2_bs;  // elements per (block, head)
  const size_t blk_stride = slab * (size_t)a.num_kv_heads;
  const size_t head_off = slab * (size_t)h;

  for (int e = tid; e < RB * D; e += NT) {
    const int n = e / D, d = e - n * D;
    const int row = r0 + n;
    float x = 0.f;
    if (row < rows_b) {
      const int i = row / G, g = row - i * G;
      x = load_elem<T>((const T*)a.q + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D + d);
    }
    q_s[n][d] = x;
  }
  if (tid < RB) {
    const int row = r0 + tid;
    if (row < rows_b) {
      const int i = row / G;
      tlo_s[tid] = max(ps, first_visible(L, q, i, a.window));
      thi_s[tid] = min(pe - 1, L - q + i);
    } else {
      tlo_s[tid] = 0x7fffffff;
      thi_s[tid] = -1;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;  // owned by thread tid < RB
  float acc[RB];                         // thread tid owns dim tid of every row
#pragma unroll
  for (int n = 0; n < RB; ++n) acc[n] = 0.f;
  const float scale_log2 = a.scale_log2;

  for (int k = 0; k < nsub; ++k) {
    const int cs = cb0 + k * SUB;
    __syncthreads();  // the previous step's readers are done
    {
      // K: thread -> (position r, dims dsl, dsl + 16, ...)
      const int r = tid >> 4, dsl = tid & 15;
      const int pos = cs + r;
      const bool ok = pos >= ps && pos < pe;
      const T* kp = nullptr;
      if (ok) {
        const int slot = pos & bs_mask;
        kp = kc + (size_t)phys_block(table, pos, log2_bs) * blk_stride + head_off +
             (k_rows ? (size_t)slot * D : (size_t)k_slot_offset(slot, D));
      }
      for (int d = dsl; d < D; d += 16)
        k_s[r][d] = ok ? load_elem<T>(kp + (k_rows ? d : (d >> 3) * 64 + (d & 7))) : 0.f;
    }
    {
      // V: thread -> (position r, dims vd, vd + 16, ...); 8-slot [D][8] tiles
      const int r = tid & 15, vd = tid >> 4;
      const int pos = cs + r;
      const bool ok = pos >= ps && pos < pe;
      const T* vp = nullptr;
      if (ok) {
        const int slot = pos & bs_mask;
        vp = vc + (size_t)phys_block(table, pos, log2_bs) * blk_stride + head_off +
             (size_t)(slot >> 3) * D * 8 + (slot & 7);
      }
      for (int d = vd; d < D; d += 16) v_s[d][r] = ok ? load_elem<T>(vp + (size_t)d * 8) : 0.f;
    }
    __syncthreads();
    {
      const int n = tid >> 4, r = tid & 15;
      const int pos = cs + r;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s += q_s[n][d] * k_s[r][d];
      p_s[n][r] = (pos >= tlo_s[n] && pos <= thi_s[n]) ? s * scale_log2 : -INFINITY;
    }
    __syncthreads();
    if (tid < RB) {
      const int n = tid;
      float mx = -INFINITY;
      for (int r = 0; r < SUB; ++r) mx = fmaxf(mx, p_s[n][r]);
      const float mnew = fmaxf(m_run, mx);
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = exp2f(m_run - mref);  // 0 while the row saw nothing
      float sum = 0.f;
      for (int r = 0; r < SUB; ++r) {
        const float e = exp2f(p_s[n][r] - mref);
        p_s[n][r] = e;
        sum += e;
      }
      l_run = l_run * alpha + sum;
      m_run = mnew;
      alpha_s[n] = alpha;
    }
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int n = 0; n < RB; ++n) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < SUB; ++r) s += p_s[n][r] * v_s[tid][r];
        acc[n] = acc[n] * alpha_s[n] + s;
      }
    }
  }
  __syncthreads();
  if (tid < RB) {
    lsum_s[tid] = l_run;
    mmax_s[tid] = m_run;
  }
  __syncthreads();

  if (tid >= D) return;
  const bool one_shot = (sv.nparts == 1);
  const size_t wbase = (((size_t)b * a.num_kv_heads + h) * a.num_parts + j) * a.rows;
#pragma unroll
  for (int n = 0; n < RB; ++n) {
    const int row = r0 + n;
    if (row >= rows_b) break;
    const float l = lsum_s[n];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (one_shot) {
      const int i = row / G, g = row - i * G;
      store_elem<T>((T*)a.out + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D + tid,
                    acc[n] * inv);
    } else {
      a.ws_o[(wbase + row) * D + tid] = acc[n] * inv;
      if (tid == 0) {
        a.ws_m[wbase + row] = mmax_s[n];
        a.ws_l[wbase + row] = l;
      }
    }
  }
}

}  // namespace pa
