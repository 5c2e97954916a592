// Partition kernel on the matrix cores (gfx950 v_mfma_f32_16x16x32_bf16; for
// FP8 queries over an FP8 cache, QK^T on v_mfma_f32_16x16x32_fp8_fp8).
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
//         straight from HBM (the V cache stores 8-slot groups as [D][8]
//         tiles, so 8 positions of one dim are one 16-byte load and a lane
//         group's 16 dims are 256 contiguous bytes), B = P rounded to bf16.
//
// The two QK tiles map MFMA row 4*lg + j of tile t to chunk position
// 8*lg + 4*t + j, so after QK each lane group lg owns the 8 consecutive
// positions 8*lg .. 8*lg+7 of its row: exactly the B-operand slice PV needs,
// with no data movement between the two products.
//
// FP8 caches (KV8): E4M3 codes are loaded as they are (16 dims of K per
// 16-byte load) and converted to bf16 in registers, exactly; the K scale
// joins the logit scale and the V scale the final normalisation.  FP8
// queries (Q8, with KV8 only): Q is loaded as codes and QK^T multiplies code
// by code on the FP8 matrix cores; the Q scale joins the logit scale.
//
// Split-K (executorch PR #18759, "split-K flash-decoding"; aiter PR #2914,
// workspace max_logits / exp_sums / temporary_output): a sequence with one
// partition writes `out` directly; otherwise each partition writes its row
// max, exp-sum and normalised partial output for the LSE reduce.
#pragma once

#include <type_traits>

#include "pa_common.h"
#include "pa_sched.h"

namespace pa {

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ inline u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// 16-byte load of KV data.  STREAM = true marks it non-temporal (streamed past
// the caches): on MI355X such loads sustain ~13 % more bandwidth on a
// block-table gather.  The cached form serves row blocks that read the same
// K/V through L2, and callers whose KV stays in the 256 MB MALL between calls.
template <bool STREAM>
__device__ inline u32x4 ld_kv(const uint8_t* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load((const u32x4*)p);
  else return *(const u32x4*)p;
}
// 8-byte form (8 FP8 values of V).
template <bool STREAM>
__device__ inline u32x2 ld_kv8(const uint8_t* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load((const u32x2*)p);
  else return *(const u32x2*)p;
}

// Eight OCP E4M3 codes (bytes of a, then of b, in memory order) as bf16.
// Exact: every E4M3 value is a bf16 value; the unit scale leaves it as is.
__device__ inline bf16x8 e4m3x8_to_bf16(uint32_t a, uint32_t b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Physical blocks touched by one chunk: the chunk's in-partition positions
// [lo, hi] span at most two blocks (block_size >= 16 >= chunk / 2).  The ids
// are wave-uniform, so they come through the scalar cache (their own wait
// counter: no false dependence on the vector loads in flight).
// A row's reference max is raised only when a chunk beats it by more than
// this (log2 units): weights are then at most 2^8 before normalisation.
constexpr float kRescaleLog2 = 8.f;

// 32-position chunks a wave takes per loop step.  An FP8 chunk is half the
// bytes of a bf16 one, so one-tile FP8 waves of the grid schedule up to head
// dim 128 take two per step: as many bytes in flight per wave as bf16, and
// one softmax update (max exchange, rescale test) per 64 positions
// (measured on MI355X, flushed: a 131072-position FP8 sequence 11.8 -> 11.3
// us, 32 units of 32k 42.1 -> 41.3 us).  The persistent kernel keeps one
// chunk per step: with two it ran 20 % slower (its waits for a step's
// second K rows also covered V loads issued after them).  More row tiles,
// or head dim 256, would lose a wave per SIMD to the extra registers.
constexpr int chunks_per_step(int D, int NRT, bool kv8, bool persistent) {
  return kv8 && NRT == 1 && D <= 128 && !persistent ? 2 : 1;
}

// Resident workgroups per CU the persistent schedule launches (it caps the
// hardware's resident count at this).  One-tile kernels: each wave has one
// 32-position chunk of K and V in flight, and ~64 KB in flight per CU is
// what the HBM gather needs; more resident waves than that only contend
// (measured on MI355X against a full resident set of 3 workgroups per CU:
// the large-block MTP batch 343-350 -> 326 us at one bf16 workgroup per CU,
// the GQA batch 89.6-90.1 -> 87.8-88.5 us; FP8 caches best at two).
// Several row tiles: whatever fits, bounded by 16 waves per CU.  The plan
// sizes the workspace from the same bound.
__host__ __device__ constexpr int ps_wgs_per_cu(int D, int NRT, int NW, bool kv8) {
  return NRT == 1 ? (65536 / (NW * kChunk * 2 * D * (kv8 ? 1 : 2)) > 1
                         ? 65536 / (NW * kChunk * 2 * D * (kv8 ? 1 : 2)) : 1)
                  : (16 / NW > 1 ? 16 / NW : 1);
}

struct ChunkBlocks {
  int first_idx;  // logical block index of the first in-partition position
  int first;      // its physical block
  int second;     // physical block of the last in-partition position
};

// One run: partitions j_first .. j_last of unit (sequence b, KV head h),
// processed as one stretch of positions by the NW waves of the workgroup.
// With `write_out` (the run is the whole unit) it writes `out`; otherwise its
// state (max, exp-sum, normalised output) goes to workspace state slot
// `state` (R rows per slot).  All waves of the workgroup call this with the same arguments.
// KV8: K and V hold OCP E4M3 codes (16 per 16-byte column / V row) that are
// converted to bf16 in registers; the K scale folds into the logit scale and
// the V scale into the output normalisation.  With 16 dims per K column, one
// 16-byte load feeds two k-steps: k-step 2c + x of lane group lg takes dims
// 16 * (4c + lg) + 8x .. +7, and Q^T is loaded in the same order (a
// contraction may visit its index in any order, as long as both operands
// agree).
template <int D, int NRT, int NW, bool STREAM, bool KV8, bool Q8, bool PS>
__device__ __forceinline__ void mfma_run(const PartArgs& a, int b, int h, int L, int q, int qoff,
                                         const SeqView& sv, int j_first, int j_last, size_t state,
                                         bool write_out, int r0 = 0) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int ES = KV8 ? 1 : 2;        // bytes per cached element
  constexpr int KL = KV8 ? KS / 2 : KS;  // 16-byte K loads per tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int ps = max(sv.lo, sv.base + j_first * a.part_size);
  const int pe = min(sv.hi, sv.base + (j_last + 1) * a.part_size);
  const int cb0 = sv.base + j_first * a.part_size;  // chunk-aligned run start
  const int nck = (pe - cb0 + kChunk - 1) / kChunk;
  const int G = a.group;
  const int rows_b = G * q;
  const int log2_bs = a.log2_bs;
  const int bs_mask = (1 << log2_bs) - 1;

  const int32_t* __restrict__ table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  // The block table is read-only for the whole call: through the constant
  // address space, uniform indices become scalar loads (their own wait
  // counter).  As vector loads, waiting for a block id would also wait for
  // the K/V loads issued before it and drain the pipeline every chunk.
  const __attribute__((address_space(4))) int32_t* stable =
      (const __attribute__((address_space(4))) int32_t*)table;
  const uint8_t* __restrict__ kc = (const uint8_t*)a.k_cache;
  const uint8_t* __restrict__ vc = (const uint8_t*)a.v_cache;
  const size_t slab = ((size_t)D * ES) << log2_bs;          // bytes per (block, head)
  const size_t blk_stride = slab * (size_t)a.num_kv_heads;
  const size_t head_off = slab * (size_t)h;

  static_assert(!Q8 || KV8, "an FP8 query goes with an FP8 KV cache");
  // Q^T operand of one k-step: 8 bf16 values, or 8 E4M3 codes (FP8 query).
  using QOp = std::conditional_t<Q8, uint64_t, bf16x8>;
  // V^T registers of one dim tile: 8 bf16 values, or 8 E4M3 codes.
  using VReg = std::conditional_t<KV8, u32x2, u32x4>;
  constexpr int CPS = chunks_per_step(D, NRT, KV8, PS);  // 32-position chunks per loop step

  // Per-row visible interval inside this partition, and Q^T operands.
  int tlo[NRT], thi[NRT];
  QOp qf[NRT][KS];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int n = r0 + rt * 16 + ln;
    if (n < rows_b) {
      const int i = n / G;
      const int g = n - i * G;
      tlo[rt] = max(ps, first_visible(L, q, i, a.window));
      thi[rt] = min(pe - 1, L - q + i);
      if (thi[rt] < tlo[rt]) {  // row sees nothing in this partition
        tlo[rt] = 0x7fffffff;
        thi[rt] = -1;
      }
      const size_t qrow = ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int d0 = KV8 ? 16 * (4 * (s >> 1) + lg) + 8 * (s & 1) : 8 * (4 * s + lg);
        if constexpr (Q8)  // 8 codes = 8 bytes at dim d0 of the row
          qf[rt][s] = *(const uint64_t*)((const uint8_t*)a.q + qrow + d0);
        else
          qf[rt][s] = as_bf16x8(*(const u32x4*)((const uint16_t*)a.q + qrow + d0));
      }
    } else {
      tlo[rt] = 0x7fffffff;
      thi[rt] = -1;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if constexpr (Q8)
          qf[rt][s] = 0;
        else
          qf[rt][s] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      }
    }
  }

  // Per tile, the intersection of its real rows' visible intervals
  // (wave-uniform): a chunk inside it is seen whole by every real row and
  // needs no mask.  Rows past the sequence's rows do not constrain it: their
  // scores are never stored.
  int tlo_all[NRT], thi_all[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const bool real = r0 + rt * 16 + ln < rows_b;
    const int lo_ = row16_op(real ? tlo[rt] : INT32_MIN, [](int x, int y) { return max(x, y); });
    const int hi_ = row16_op(real ? thi[rt] : INT32_MAX, [](int x, int y) { return min(x, y); });
    tlo_all[rt] = __builtin_amdgcn_readfirstlane(lo_);
    thi_all[rt] = __builtin_amdgcn_readfirstlane(hi_);
  }

  auto blocks_of = [&](int k) {
    const int cs = cb0 + k * kChunk;
    const int lo = max(cs, ps);
    const int hi = min(cs + kChunk - 1, pe - 1);
    ChunkBlocks cb;
    cb.first_idx = __builtin_amdgcn_readfirstlane(lo >> log2_bs);
    const int second_idx = __builtin_amdgcn_readfirstlane(hi >> log2_bs);
    cb.first = stable[cb.first_idx];
    cb.second = stable[second_idx];
    return cb;
  };
  // K rows: lane (ln, lg) of tile t holds position 8*(ln/4) + 4*t + ln%4 of
  // the chunk and, per load, the 16-byte column 4*c + lg of it (bf16: the
  // dims of k-step c; FP8: those of k-steps 2c and 2c+1).  In the tiled K
  // layout that is place ln%8 of half t of 16-slot group ln/8: each load
  // instruction reads two runs of 512 contiguous bytes.
  // `dummy` (wave-uniform): the loads only keep the wait counts static past
  // the last chunk; every lane then reads the same 16 bytes, so they cost one
  // line instead of the chunk (non-temporal loads would fetch it again).
  auto load_k = [&](int k, const ChunkBlocks& cb, u32x4 (&kr)[2][KL], bool dummy) {
    const int cs = cb0 + k * kChunk;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int pos = cs + 8 * (ln >> 2) + 4 * t + (ln & 3);
      pos = min(max(pos, ps), pe - 1);  // clamp: never touch blocks outside the span
      const int blk = (pos >> log2_bs) == cb.first_idx ? cb.first : cb.second;
      const int in_slab = dummy ? 0 : k_slot_bytes(pos & bs_mask, D * ES) + lg * 128;
      const uint8_t* kp = kc + (size_t)(dummy ? cb.first : blk) * blk_stride + head_off + in_slab;
#pragma unroll
      for (int c = 0; c < KL; ++c) kr[t][c] = ld_kv<STREAM>(kp + (dummy ? 0 : c * 512));
    }
  };
  // V^T columns: lane (ln, lg) holds dim 16*dt + ln, positions 8*lg .. +7.
  // The registers hold the cache's own bytes (FP8: 8 codes per dim tile,
  // converted only when PV takes them).
  // bf16: 8-slot group = a [D][8] tile, one 16-byte load; the 16 lanes of a
  // lane group read 256 contiguous bytes.  FP8: 16-slot group = a [D][16]
  // tile, the 8 bytes of half lg % 2 of the dim's row; lane groups 2j and
  // 2j+1 together read 256 contiguous bytes.
  auto load_v = [&](int k, const ChunkBlocks& cb, VReg (&vr)[DT], bool dummy) {
    const int cs = cb0 + k * kChunk;
    int p8 = cs + 8 * lg;
    if (p8 + 8 <= ps || p8 >= pe) p8 = max(cs, ps) & ~7;  // wholly outside: any valid group, zeroed later
    else p8 = max(p8, ps & ~7);
    const int blk = dummy ? cb.first : ((p8 >> log2_bs) == cb.first_idx ? cb.first : cb.second);
    const uint8_t* vb = vc + (size_t)blk * blk_stride + head_off;
    if constexpr (KV8) {
      const uint8_t* vp = vb + (dummy ? 0 : ((p8 & bs_mask) >> 4) * (D * 16) + ln * 16 + (p8 & 8));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vr[dt] = ld_kv8<STREAM>(vp + (dummy ? 0 : 256 * dt));
    } else {
      const uint8_t* vp = vb + (dummy ? 0 : ((p8 & bs_mask) >> 3) * (D * 16) + ln * 16);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vr[dt] = ld_kv<STREAM>(vp + (dummy ? 0 : 256 * dt));
    }
  };
  // FP8 A operand of k-step s of tile t: its 8 E4M3 codes as they were loaded
  auto k_codes = [&](const u32x4 (&kr)[2][KL], int t, int s) -> uint64_t {
    const u32x4& w = kr[t][s >> 1];
    return (s & 1) ? ((uint64_t)w[3] << 32 | w[2]) : ((uint64_t)w[1] << 32 | w[0]);
  };
  // bf16 A operand of k-step s of tile t
  auto k_operand = [&](const u32x4 (&kr)[2][KL], int t, int s) -> bf16x8 {
    if constexpr (KV8) {
      const u32x4& w = kr[t][s >> 1];
      return (s & 1) ? e4m3x8_to_bf16(w[2], w[3]) : e4m3x8_to_bf16(w[0], w[1]);
    } else {
      return as_bf16x8(kr[t][s]);
    }
  };

  // Exp-sums of the rounded weights: at head dims up to 128, one more
  // matrix-core product per chunk and tile, ones^T P, which sums each row's
  // weights over the chunk's 32 positions (every lane receives its row's
  // sum); at 256 (no registers to spare) each lane sums its own 8 weights
  // and the lane groups are added at the end.
  constexpr bool LSUM = D <= 128;
  const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                       (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
  f32x4 o[NRT][DT];
  f32x4 lacc[NRT];
  float mrun[NRT], lrun[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    mrun[rt] = -INFINITY;
    lrun[rt] = 0.f;
    lacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float scale_log2 = a.scale_log2;
  float v_scale = 1.f;
  if constexpr (KV8) {
    scale_log2 *= *a.k_scale;
    v_scale = *a.v_scale;
  }
  if constexpr (Q8) scale_log2 *= *a.q_scale;
  // The logit scale folds into the exponent's argument: scores stay raw
  // through the mask and the max (a positive factor commutes with both, in
  // rounding too) and each weight is exp2(fma(s, scale, -m)), one vector
  // instruction per score fewer.  A negative scale goes into the query's
  // sign bits (exact); a zero one becomes the smallest normal, which leaves
  // every weight at exactly 1 and keeps masked scores at -inf.
  if (scale_log2 < 0.f) {
    scale_log2 = -scale_log2;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if constexpr (Q8) qf[rt][s] ^= 0x8080808080808080ull;  // E4M3 sign bits
        else qf[rt][s] = as_bf16x8(as_u32x4(qf[rt][s]) ^ 0x80008000u);
      }
  }
  scale_log2 = fmaxf(scale_log2, 1.17549435e-38f);

  // Software pipeline, one step deep: the next step's K rows are requested
  // as soon as QK has consumed the current ones, its V columns as soon as PV
  // has; block ids run two steps ahead through the scalar cache.  Loads are
  // issued unconditionally (after its last step a wave issues one-line dummy
  // loads, and so does a step's chunk past the run's end) so that the wait
  // counts are the same on every path.  Wave w takes steps w, w + NW, ...;
  // step t covers chunks CPS*t .. CPS*t + CPS - 1.
  const int nst = (nck + CPS - 1) / CPS;
  // (with one chunk per step every chunk of a step below nst is in the run)
  auto step_blocks = [&](int t, ChunkBlocks (&cb)[CPS]) {
#pragma unroll
    for (int c = 0; c < CPS; ++c) cb[c] = blocks_of(CPS == 1 ? t : min(t * CPS + c, nck - 1));
  };
  auto beyond = [&](int t, int c) { return CPS > 1 && t * CPS + c >= nck; };
  int t = wave;
  u32x4 kr[CPS][2][KL];
  VReg vr[CPS][DT];
  ChunkBlocks nb[CPS];
#pragma unroll
  for (int c = 0; c < CPS; ++c) nb[c] = ChunkBlocks{0, 0, 0};
  if (t < nst) {
    ChunkBlocks cb[CPS];
    step_blocks(t, cb);
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      load_k(t * CPS + c, cb[c], kr[c], beyond(t, c));
      load_v(t * CPS + c, cb[c], vr[c], beyond(t, c));
    }
    step_blocks(min(t + NW, nst - 1), nb);
  }
  for (; t < nst; t += NW) {
    const bool past = t + NW >= nst;  // no next step for this wave
    const int tn = min(t + NW, nst - 1);
    bf16x8 pb[CPS][NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      // visible iff tlo <= pos <= thi, as one unsigned comparison (rows that
      // see nothing have tlo = 2^31 - 1, thi = -1: no pos >= 0 passes)
      const uint32_t span = (uint32_t)(thi[rt] - tlo[rt]);
      float x[CPS][8];
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if constexpr (Q8) {  // E4M3 x E4M3 products, fp32 accumulation
            sa = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)k_codes(kr[c], 0, s), (long)qf[rt][s],
                                                           sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)k_codes(kr[c], 1, s), (long)qf[rt][s],
                                                           sb, 0, 0, 0);
          } else {
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(kr[c], 0, s), qf[rt][s], sa, 0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(kr[c], 1, s), qf[rt][s], sb, 0, 0, 0);
          }
        }
        const int cs = cb0 + (t * CPS + c) * kChunk;
        if (cs >= tlo_all[rt] && cs + kChunk - 1 <= thi_all[rt]) {
          // every real row sees the whole chunk
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[c][e] = sa[e];
            x[c][4 + e] = sb[e];
          }
        } else {
          const int p8 = cs + 8 * lg;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[c][e] = (uint32_t)(p8 + e - tlo[rt]) <= span ? sa[e] : -INFINITY;
            x[c][4 + e] = (uint32_t)(p8 + 4 + e - tlo[rt]) <= span ? sb[e] : -INFINITY;
          }
        }
      }
      float mx;
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
        const float mc = fmaxf(fmaxf(fmaxf(x[c][0], x[c][1]), fmaxf(x[c][2], x[c][3])),
                               fmaxf(fmaxf(x[c][4], x[c][5]), fmaxf(x[c][6], x[c][7])));
        mx = c == 0 ? mc : fmaxf(mx, mc);
      }
      {
        const auto fmax = [](float x, float y) { return fmaxf(x, y); };
        mx = xor32_op(xor16_op(mx, fmax), fmax) * scale_log2;  // to the log2 domain
      }
      // Lazy rescaling: the reference max of a row moves only when the step
      // max exceeds it by more than kRescaleLog2 (or it is still -inf), so
      // weights stay <= 2^kRescaleLog2 and the accumulators are rescaled on
      // few steps instead of every step.  Any reference gives the exact
      // final result: (m, l, o) stay consistent with one another.
      const bool grow = mx > mrun[rt] + kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        // alpha is exactly 1 for rows that keep their reference (never
        // (-inf) - (-inf)), and 0 for a row leaving -inf
        const float alpha = grow ? __builtin_amdgcn_exp2f(mrun[rt] - mx) : 1.f;
        if constexpr (LSUM) lacc[rt] *= alpha;
        else lrun[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
        mrun[rt] = grow ? mx : mrun[rt];
      }
      const float mref = (mrun[rt] == -INFINITY) ? 0.f : mrun[rt];
      float psum = 0.f;
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 pe16 = (__bf16)__builtin_amdgcn_exp2f(fmaf(x[c][e], scale_log2, -mref));
          pb[c][rt][e] = pe16;
          // normalise by the weights PV actually applies
          if constexpr (!LSUM) psum += (float)pe16;
        }
      }
      if constexpr (!LSUM) lrun[rt] += psum;
    }
#pragma unroll
    for (int c = 0; c < CPS; ++c) load_k(tn * CPS + c, nb[c], kr[c], past || beyond(tn, c));
    ChunkBlocks nb2[CPS];
    step_blocks(min(t + 2 * NW, nst - 1), nb2);
    // Keep V-dependent work below this point: the V columns are the last
    // loads to arrive, and waiting for them earlier would serialise the
    // next step's K requests behind them.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      const int cs = cb0 + (t * CPS + c) * kChunk;
      const int p8 = cs + 8 * lg;
      if (cs < ps || cs + kChunk > pe) {
        // Edge chunk: zero V entries of positions outside [ps, pe) so that a
        // zero weight never meets a stale, possibly NaN, value (an E4M3 code
        // of 0 is +0).
        if constexpr (KV8) {
          u32x2 keep;
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            uint32_t m = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t0 = p8 + 4 * w + e;
              m |= (t0 >= ps && t0 < pe) ? 0xffu << (8 * e) : 0u;
            }
            keep[w] = m;
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) vr[c][dt] &= keep;
        } else {
          u32x4 keep;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int t0 = p8 + 2 * w;
            const uint32_t lo16 = (t0 >= ps && t0 < pe) ? 0x0000ffffu : 0u;
            const uint32_t hi16 = (t0 + 1 >= ps && t0 + 1 < pe) ? 0xffff0000u : 0u;
            keep[w] = lo16 | hi16;
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) vr[c][dt] &= keep;
        }
      }
      if constexpr (KV8) {  // each dim tile converted just before its products
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 vop = e4m3x8_to_bf16(vr[c][dt][0], vr[c][dt][1]);
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
            o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[c][rt], o[rt][dt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vr[c][dt]), pb[c][rt], o[rt][dt],
                                                                0, 0, 0);
      }
      if constexpr (LSUM) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
          lacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[c][rt], lacc[rt], 0, 0, 0);
      }
    }
    // Request the next V columns only after PV has read these registers
    // (no second register copy of the step).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < CPS; ++c) load_v(tn * CPS + c, nb[c], vr[c], past || beyond(tn, c));
#pragma unroll
    for (int c = 0; c < CPS; ++c) nb[c] = nb2[c];
  }

#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    if constexpr (LSUM) {
      lrun[rt] = lacc[rt][0];
    } else {
      const auto add = [](float x, float y) { return x + y; };
      lrun[rt] = xor32_op(xor16_op(lrun[rt], add), add);
    }
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
    if (wave == 0) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int n = rt * 16 + ln;  // row within the block (shared-memory index)
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
  }

  if (wave == 0) {
    const bool one_shot = write_out;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int n = r0 + rt * 16 + ln;
      if (n >= rows_b) continue;
      const float inv = lrun[rt] > 0.f ? v_scale / lrun[rt] : 0.f;
      if (one_shot) {
        const int i = n / G;
        const int g = n - i * G;
        uint16_t* op =
            (uint16_t*)a.out + ((size_t)(qoff + i) * a.num_q_heads + (size_t)h * G + g) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[rt][dt][e] * inv);
          *(bf16x4*)(op + 16 * dt + 4 * lg) = v;
        }
      } else {
        const size_t w = state * a.rows + n;
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
}

// Grid schedule: one workgroup per (partition, sequence, KV head).
template <int D, int NRT, int NW, bool STREAM, bool KV8, bool Q8>
__global__ __launch_bounds__(64 * NW) void part_mfma(PartArgs a) {
  const PartItem it = part_item(a);
  const int ro = row_offset_issue(a.query_lens, it.b);  // travels with the lengths
  const int L = a.seq_lens[it.b];
  const int q = a.query_lens[it.b];
  const SeqView sv = seq_view(L, q, a.window, a.part_size);
  if (it.j >= sv.nparts) return;  // past the unit's partitions: no state to store
  const int r0 = it.rb * 16 * NRT;                // first packed row of this block
  if (r0 >= a.group * q) return;                 // no row of this sequence is in it
  const int qoff = row_offset_finish(ro, a.qoffs, a.query_lens, it.b);
  const size_t state = ((size_t)it.b * a.num_kv_heads + it.h) * a.num_parts + it.j;
  mfma_run<D, NRT, NW, STREAM, KV8, Q8, false>(a, it.b, it.h, L, q, qoff, sv, it.j, it.j, state,
                                               sv.nparts == 1, r0);
}

// Persistent schedule (persistent_shares in pa_sched.h) on the matrix cores.
template <int D, int NRT, int NW, bool STREAM, bool KV8, bool Q8>
__global__ __launch_bounds__(64 * NW) void part_mfma_ps(PartArgs a) {
  persistent_shares<64 * NW>(a, [&](int b, int h, int L, int q, int qoff, const SeqView& sv, int j1,
                                    int j2, size_t state, bool whole) {
    mfma_run<D, NRT, NW, STREAM, KV8, Q8, true>(a, b, h, L, q, qoff, sv, j1, j2, state, whole);
  });
}

}  // namespace pa
