// Partition kernel on bf16 matrix cores (gfx950 v_mfma_f32_16x16x32_bf16).
//
// One workgroup = NW waves = one context partition of one (sequence, KV
// head).  The G*q_b query rows of the KV head are packed as the N dimension
// of 16-row MFMA tiles (NRT tiles), row n = i*G + g for query token i and
// group member g.  Per 32-position chunk:
//
//   QK^T  S^T[pos, n] = sum_d K[pos, d] * Q[n, d]  — A = K rows straight from
//         HBM (16-byte loads, lane (ln, lg) holds 8 dims of one position),
//         B = Q^T held in registers; two 16-position tiles per chunk.
//   mask  visible iff first_visible(row) <= pos <= row position, and pos in
//         the partition; masked logits become -inf by select, so stale or
//         NaN cache contents never propagate.
//   online softmax (log2 domain): running max per row, rescale factor
//         alpha, exp-sum.  A row with nothing visible so far keeps max = -inf
//         and never evaluates (-inf) - (-inf).
//   PV    O^T[d, n] += sum_pos V^T[d, pos] * P^T[pos, n] — A = V^T columns
//         straight from HBM (the V cache keeps positions contiguous per
//         dim, so 8 positions are one 16-byte load), B = P rounded to bf16.
//
// The two QK tiles map MFMA row 4*lg + j of tile t to chunk position
// 8*lg + 4*t + j, so after QK each lane group lg owns the 8 consecutive
// positions 8*lg .. 8*lg+7 of its row: exactly the B-operand slice PV needs,
// with no data movement between the two products.
//
// Split-K (executorch PR #18759, "split-K flash-decoding"; aiter PR #2914,
// workspace max_logits / exp_sums / temporary_output): a sequence with one
// partition writes `out` directly; otherwise each partition writes its row
// max, exp-sum and normalised partial output for the LSE reduce.
#pragma once

#include "pa_common.h"

namespace pa {

template <int D>
struct MfmaChunk {
  u32x4 k[2][D / 32];  // K: [tile][k-step], 8 bf16 of one position each
  u32x4 v[D / 16];     // V^T: [dim tile], 8 consecutive positions of one dim
};

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

template <int D, int NRT, int NW>
__global__ __launch_bounds__(64 * NW) void part_mfma(PartArgs a) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;

  const int L = a.seq_lens[b];
  const int q = a.query_lens[b];
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  if (j >= sv.nparts) return;  // empty partition: contributes nothing
  int ps, pe;
  partition_range(sv, j, a.part_size, &ps, &pe);
  const int cb0 = sv.base + j * a.part_size;  // chunk-aligned partition start
  const int nck = (pe - cb0 + kChunk - 1) / kChunk;
  const int qoff = wave_row_offset(a.query_lens, b);
  const int G = a.group;
  const int rows_b = G * q;
  const int log2_bs = a.log2_bs;
  const int bs_mask = (1 << log2_bs) - 1;

  const int32_t* __restrict__ table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const uint16_t* __restrict__ kc = (const uint16_t*)a.k_cache;
  const uint16_t* __restrict__ vc = (const uint16_t*)a.v_cache;
  const size_t slab = (size_t)D << log2_bs;                 // elements per (block, head)
  const size_t blk_stride = slab * (size_t)a.num_kv_heads;
  const size_t head_off = slab * (size_t)h;

  // Per-row visible interval inside this partition, and Q^T operands.
  int tlo[NRT], thi[NRT];
  bf16x8 qf[NRT][KS];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int n = rt * 16 + ln;
    if (n < rows_b) {
      const int i = n / G;
      const int g = n - i * G;
      tlo[rt] = max(ps, first_visible(L, q, i, a.window));
      thi[rt] = min(pe - 1, L - q + i);
      const uint16_t* qp =
          (const uint16_t*)a.q + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[rt][s] = as_bf16x8(*(const u32x4*)(qp + (4 * s + lg) * 8));
    } else {
      tlo[rt] = 0x7fffffff;
      thi[rt] = -1;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[rt][s] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }

  auto load = [&](int k, MfmaChunk<D>& r) {
    const int cs = cb0 + k * kChunk;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int pos = cs + 8 * (ln >> 2) + 4 * t + (ln & 3);
      pos = min(max(pos, ps), pe - 1);  // clamp: never touch blocks outside the span
      const int blk = phys_block(table, pos, log2_bs);
      const uint16_t* kp = kc + (size_t)blk * blk_stride + head_off + (size_t)(pos & bs_mask) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) r.k[t][s] = *(const u32x4*)(kp + (4 * s + lg) * 8);
    }
    int p8 = cs + 8 * lg;
    if (p8 + 8 <= ps || p8 >= pe) p8 = ps & ~7;  // wholly outside: read a valid group, zeroed later
    const int vblk = phys_block(table, p8, log2_bs);
    const uint16_t* vp = vc + (size_t)vblk * blk_stride + head_off + (p8 & bs_mask);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      r.v[dt] = *(const u32x4*)(vp + ((size_t)(16 * dt + ln) << log2_bs));
  };

  f32x4 o[NRT][DT];
  float mrun[NRT], lrun[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    mrun[rt] = -INFINITY;
    lrun[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float scale_log2 = a.scale_log2;

  auto compute = [&](int k, const MfmaChunk<D>& r) {
    const int cs = cb0 + k * kChunk;
    const int p8 = cs + 8 * lg;
    u32x4 vv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vv[dt] = r.v[dt];
    if (cs < ps || cs + kChunk > pe) {
      // Edge chunk: zero V entries of positions outside [ps, pe) so that a
      // zero weight never meets a stale (possibly NaN) value.
      u32x4 keep;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int t0 = p8 + 2 * w;
        const uint32_t lo16 = (t0 >= ps && t0 < pe) ? 0x0000ffffu : 0u;
        const uint32_t hi16 = (t0 + 1 >= ps && t0 + 1 < pe) ? 0xffff0000u : 0u;
        keep[w] = lo16 | hi16;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vv[dt] &= keep;
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.k[0][s]), qf[rt][s], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.k[1][s]), qf[rt][s], sb, 0, 0, 0);
      }
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t0 = p8 + e, t1 = p8 + 4 + e;
        x[e] = (t0 >= tlo[rt] && t0 <= thi[rt]) ? sa[e] * scale_log2 : -INFINITY;
        x[4 + e] = (t1 >= tlo[rt] && t1 <= thi[rt]) ? sb[e] * scale_log2 : -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[rt], mx);
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(mrun[rt] - mref);
      mrun[rt] = mnew;
      bf16x8 pb;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 pe16 = (__bf16)__builtin_amdgcn_exp2f(x[e] - mref);
        pb[e] = pe16;
        psum += (float)pe16;  // normalise by the weights PV actually applies
      }
      lrun[rt] = lrun[rt] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[rt][dt] *= alpha;
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vv[dt]), pb, o[rt][dt], 0, 0, 0);
      }
    }
  };

  {
    MfmaChunk<D> cur, nxt;
    int k = wave;
    if (k < nck) load(k, cur);
    while (k < nck) {
      const int kn = k + NW;
      if (kn < nck) load(kn, nxt);  // keep the next chunk's loads in flight
      compute(k, cur);
      cur = nxt;
      k = kn;
    }
  }

#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    lrun[rt] += __shfl_xor(lrun[rt], 16);
    lrun[rt] += __shfl_xor(lrun[rt], 32);
  }

  if constexpr (NW > 1) {
    // Merge the waves' states in a fixed order (deterministic results).
    __shared__ float sm_m[NW][NRT * 16];
    __shared__ float sm_l[NW][NRT * 16];
    __shared__ f32x4 sm_o[NW - 1][NRT][DT][64];
    if (lg == 0) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        sm_m[wave][rt * 16 + ln] = mrun[rt];
        sm_l[wave][rt * 16 + ln] = lrun[rt];
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) sm_o[wave - 1][rt][dt][lane] = o[rt][dt];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int n = rt * 16 + ln;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][n]);
      const float mref = (M == -INFINITY) ? 0.f : M;
      const float f0 = __builtin_amdgcn_exp2f(mrun[rt] - mref);
      float l = lrun[rt] * f0;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= f0;
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float fw = __builtin_amdgcn_exp2f(sm_m[w][n] - mref);
        l += sm_l[w][n] * fw;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] += fw * sm_o[w - 1][rt][dt][lane];
      }
      mrun[rt] = M;
      lrun[rt] = l;
    }
  }

  const bool one_shot = (sv.nparts == 1);
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int n = rt * 16 + ln;
    if (n >= rows_b) continue;
    const float inv = lrun[rt] > 0.f ? 1.f / lrun[rt] : 0.f;
    if (one_shot) {
      const int i = n / G;
      const int g = n - i * G;
      uint16_t* op = (uint16_t*)a.out + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[rt][dt][e] * inv);
        *(bf16x4*)(op + 16 * dt + 4 * lg) = v;
      }
    } else {
      const size_t w = (((size_t)b * a.num_kv_heads + h) * a.num_parts + j) * a.rows + n;
      if (lg == 0) {
        a.ws_m[w] = mrun[rt];
        a.ws_l[w] = lrun[rt];
      }
      float* op = a.ws_o + w * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4*)(op + 16 * dt + 4 * lg) = o[rt][dt] * inv;
    }
  }
}

}  // namespace pa
