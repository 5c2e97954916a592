// Partition kernel on the vector ALUs (any element type; fp32 arithmetic).
//
// Used for float32 inputs (no reduced-precision products at all) and as the
// vector-ALU alternative for bf16.  One 256-thread workgroup handles one
// context partition of one (sequence, KV head); its G*q_b <= 64 packed rows
// (row n = i*G + g) share every K/V chunk, which is staged through LDS:
//
//   stage   K chunk [32][D] and V chunk [D][32] in fp32 (K read from its
//           16-slot tiles, V from its 8-slot [D][8] tiles), positions outside
//           the partition stored as zeros (never read from HBM)
//   scores  one thread per (row, position): D-term dot product, masked by
//           select to -inf outside the row's visible interval
//   softmax one thread per row: running max (log2 domain), rescale factor,
//           exp-sum; all-masked rows keep max = -inf without NaNs
//   PV      one thread per (row, dim) pair group: acc = acc*alpha + p . v
//
// Output contract is the same as the matrix-core kernel: one-shot sequences
// write `out`, split sequences write (max, exp-sum, normalised partial).
#pragma once

#include "pa_common.h"

namespace pa {

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

template <typename T, int D>
__global__ __launch_bounds__(256) void part_valu(PartArgs a) {
  constexpr int NT = 256;
  constexpr int RMAX = 64;
  constexpr int ACC = RMAX * D / NT;
  __shared__ float q_s[RMAX][D + 1];
  __shared__ float k_s[kChunk][D + 1];
  __shared__ float v_s[D][kChunk + 1];
  __shared__ float p_s[RMAX][kChunk + 1];
  __shared__ float alpha_s[RMAX];
  __shared__ float lsum_s[RMAX];
  __shared__ float mmax_s[RMAX];
  __shared__ int tlo_s[RMAX], thi_s[RMAX];

  const PartItem it = part_item(a);
  const int j = it.j, h = it.h, b = it.b;
  const int tid = threadIdx.x;
  const int L = a.seq_lens[b];
  const int q = a.query_lens[b];
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  if (j >= sv.nparts) return;
  int ps, pe;
  partition_range(sv, j, a.part_size, &ps, &pe);
  const int cb0 = sv.base + j * a.part_size;
  const int nck = (pe - cb0 + kChunk - 1) / kChunk;
  const int qoff = wave_row_offset(a.query_lens, b);
  const int G = a.group;
  const int rows_b = G * q;
  const int log2_bs = a.log2_bs;
  const int bs_mask = (1 << log2_bs) - 1;
  const int32_t* __restrict__ table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const T* __restrict__ kc = (const T*)a.k_cache;
  const T* __restrict__ vc = (const T*)a.v_cache;
  const size_t slab = (size_t)D << log2_bs;
  const size_t blk_stride = slab * (size_t)a.num_kv_heads;
  const size_t head_off = slab * (size_t)h;

  for (int e = tid; e < RMAX * D; e += NT) {
    const int n = e / D, d = e - n * D;
    float x = 0.f;
    if (n < rows_b) {
      const int i = n / G, g = n - i * G;
      x = load_elem<T>((const T*)a.q + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D + d);
    }
    q_s[n][d] = x;
  }
  if (tid < RMAX) {
    const int n = tid;
    if (n < rows_b) {
      const int i = n / G;
      tlo_s[n] = max(ps, first_visible(L, q, i, a.window));
      thi_s[n] = min(pe - 1, L - q + i);
    } else {
      tlo_s[n] = 0x7fffffff;
      thi_s[n] = -1;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;  // owned by thread tid < rows_b
  float acc[ACC];
#pragma unroll
  for (int e = 0; e < ACC; ++e) acc[e] = 0.f;
  const float scale_log2 = a.scale_log2;

  for (int k = 0; k < nck; ++k) {
    const int cs = cb0 + k * kChunk;
    __syncthreads();  // previous chunk's readers are done
    {
      // K: thread -> (position r, dims dsl, dsl+8, ...): the 8 threads of a
      // position read 8 consecutive elements of each column of its slot.
      const int r = tid >> 3, dsl = tid & 7;
      const int pos = cs + r;
      const bool ok = pos >= ps && pos < pe;
      const T* kp = nullptr;
      if (ok) kp = kc + (size_t)phys_block(table, pos, log2_bs) * blk_stride + head_off +
                   k_slot_offset(pos & bs_mask, D) + dsl;
      for (int d = dsl; d < D; d += 8) k_s[r][d] = ok ? load_elem<T>(kp + (d >> 3) * 64) : 0.f;
    }
    {
      // V: thread -> (position r, dims vd, vd+8, ...): coalesced along positions.
      const int r = tid & 31, vd = tid >> 5;
      const int pos = cs + r;
      const bool ok = pos >= ps && pos < pe;
      const T* vp = nullptr;
      if (ok) vp = vc + (size_t)phys_block(table, pos, log2_bs) * blk_stride + head_off +
                   (size_t)((pos & bs_mask) >> 3) * (D * 8) + (pos & 7);
      for (int d = vd; d < D; d += 8) v_s[d][r] = ok ? load_elem<T>(vp + d * 8) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < rows_b * kChunk; e += NT) {
      const int n = e >> 5, r = e & 31;
      const int pos = cs + r;
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) s += q_s[n][d] * k_s[r][d];
      p_s[n][r] = (pos >= tlo_s[n] && pos <= thi_s[n]) ? s * scale_log2 : -INFINITY;
    }
    __syncthreads();
    if (tid < rows_b) {
      const int n = tid;
      float mx = -INFINITY;
      for (int r = 0; r < kChunk; ++r) mx = fmaxf(mx, p_s[n][r]);
      const float mnew = fmaxf(m_run, mx);
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = exp2f(m_run - mref);
      float sum = 0.f;
      for (int r = 0; r < kChunk; ++r) {
        const float e = exp2f(p_s[n][r] - mref);
        p_s[n][r] = e;
        sum += e;
      }
      l_run = l_run * alpha + sum;
      m_run = mnew;
      alpha_s[n] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < ACC; ++e) {
      const int pr = tid + NT * e;
      const int n = pr / D, d = pr - n * D;
      if (n < rows_b) {
        float s = 0.f;
#pragma unroll 8
        for (int r = 0; r < kChunk; ++r) s += p_s[n][r] * v_s[d][r];
        acc[e] = acc[e] * alpha_s[n] + s;
      }
    }
  }
  __syncthreads();
  if (tid < rows_b) {
    lsum_s[tid] = l_run;
    mmax_s[tid] = m_run;
  }
  __syncthreads();

  const bool one_shot = (sv.nparts == 1);
  const size_t wbase = (((size_t)b * a.num_kv_heads + h) * a.num_parts + j) * a.rows;
#pragma unroll
  for (int e = 0; e < ACC; ++e) {
    const int pr = tid + NT * e;
    const int n = pr / D, d = pr - n * D;
    if (n >= rows_b) continue;
    const float l = lsum_s[n];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (one_shot) {
      const int i = n / G, g = n - i * G;
      store_elem<T>((T*)a.out + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D + d,
                    acc[e] * inv);
    } else {
      a.ws_o[(wbase + n) * D + d] = acc[e] * inv;
      if (d == 0) {
        a.ws_m[wbase + n] = mmax_s[n];
        a.ws_l[wbase + n] = l;
      }
    }
  }
}

}  // namespace pa
