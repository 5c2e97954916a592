// C ABI of the paged-attention decode library: validation, launch plan,
// kernel dispatch.  Declarations and the full contract: include/pa_decode.h.
#include "pa_decode.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "pa_common.h"
#include "pa_launch.h"
#include "pa_pack.h"
#include "pa_probe.h"
#include "pa_reduce.h"
#include "pa_valu.h"

namespace pa_host {

// Resident workgroups of a kernel on the current device (workgroups per CU
// cached per kernel; the kernels are the same code on every gfx950 device).
int resident_wgs(const void* fn, int threads, int cus) {
  static std::mutex lock;
  static const void* keys[64];
  static int per_cu_of[64];
  std::lock_guard<std::mutex> guard(lock);
  int i = 0;
  for (; i < 64 && keys[i] != nullptr; ++i)
    if (keys[i] == fn) return per_cu_of[i] * cus;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (i < 64) {
    keys[i] = fn;
    per_cu_of[i] = per_cu;
  }
  return per_cu * cus;
}

}  // namespace pa_host

namespace {

using pa_host::Launch;
using pa_host::launch_part;

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool log_enabled() {
  static const int on = [] {
    const char* v = std::getenv("PA_LOG");
    return (v && v[0] && v[0] != '0') ? 1 : 0;
  }();
  return on != 0;
}

int ilog2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Host-visible argument checks shared by every entry point.
// Packed rows (G * max_query_len) one call may carry per KV head: mixed
// batches of prefill chunks and decode rows, in blocks of 16 to 64 rows.
constexpr int kMaxRows = 1024;

// Register-resident vector kernels on the persistent schedule: whether
// automatic plans take it (as on the matrix cores), and the workgroups per
// CU its grid may hold; the launcher caps them at what fits (3 at head dim
// 128).  Measured on MI355X: the fp32 GQA batch 214-219 -> 202 us (kernel)
// with every resident workgroup, 204 with 2 per CU, 227 with 1; the bf16
// GQA batch on the vector kernel 140 -> 126 us.
constexpr bool kWavePersistentAuto = true;
constexpr int kWavePsPerCu = 8;

// Head dims with matrix-core kernels (whole 32-dim k-steps, instantiated).
bool mfma_head_dim(int D) { return D == 64 || D == 128 || D == 256; }

pa_status check_shape(const pa_dims* d, int32_t window, int32_t num_kv_heads, int32_t block_size) {
  if (!d) return fail(PA_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 0 || d->batch > 65535)
    return fail(PA_ERR_INVALID_ARG, "batch %d outside [0, 65535]", d->batch);
  if (d->dtype != PA_F32 && d->dtype != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "dtype %d is neither PA_F32 nor PA_BF16", d->dtype);
  if (d->kv_format != PA_KV_NATIVE && d->kv_format != PA_KV_FP8_E4M3)
    return fail(PA_ERR_INVALID_ARG, "kv_format %d unknown", d->kv_format);
  if (d->kv_format == PA_KV_FP8_E4M3 && d->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "an FP8 KV cache needs bf16 q and out");
  if (d->head_dim < 1 || d->head_dim > pa::kValuMaxD)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d outside [1, %d]", d->head_dim, pa::kValuMaxD);
  if (d->kv_format == PA_KV_FP8_E4M3 && !mfma_head_dim(d->head_dim))
    return fail(PA_ERR_UNSUPPORTED, "an FP8 KV cache needs head_dim 64, 128 or 256");
  if (d->q_format != PA_Q_NATIVE && d->q_format != PA_Q_FP8_E4M3)
    return fail(PA_ERR_INVALID_ARG, "q_format %d unknown", d->q_format);
  if (d->q_format == PA_Q_FP8_E4M3 && d->kv_format != PA_KV_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "an FP8 query needs an FP8 KV cache");
  if (num_kv_heads < 1 || num_kv_heads > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d outside [1, 65535]", num_kv_heads);
  if (d->num_q_heads < 1 || d->num_q_heads % num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                d->num_q_heads, num_kv_heads);
  if (ilog2_exact(block_size) < 4 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d must be a power of two in [16, 1024]", block_size);
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d is negative", window);
  if (d->max_query_len < 1) return fail(PA_ERR_INVALID_ARG, "max_query_len %d < 1", d->max_query_len);
  if (d->max_seq_len < d->max_query_len)
    return fail(PA_ERR_INVALID_ARG, "max_seq_len %d < max_query_len %d", d->max_seq_len,
                d->max_query_len);
  if (d->max_blocks_per_seq < cdiv(d->max_seq_len, block_size))
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d < ceil(max_seq_len %d / block_size %d)",
                d->max_blocks_per_seq, d->max_seq_len, block_size);
  if (d->num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks %d < 1", d->num_blocks);
  const int64_t rows = (int64_t)(d->num_q_heads / num_kv_heads) * d->max_query_len;
  if (rows > kMaxRows)
    return fail(PA_ERR_UNSUPPORTED, "rows per KV head G*max_query_len = %lld exceeds %d",
                (long long)rows, kMaxRows);
  return PA_OK;
}

// Workspace of a split plan: state slots (each R rows) of max, exp-sum and
// normalised output, 256-byte aligned regions; the persistent schedule adds
// a (run count, first slot) pair per unit.  Slots: one per (unit, partition)
// on the grid schedule, persistent grid + units on the persistent one.
// Workspace: partial states of split plans (none for one-shot plans), the
// persistent schedule's per-unit run records, and for batches above
// kScanBatch the scanned row offsets.
struct WsLayout {
  uint64_t states;  // state rows (slots x R)
  uint64_t off_l, off_o, off_runs, off_qoffs, total;
};

WsLayout workspace_layout(const pa_plan& r, const pa_dims& d, int hkv) {
  WsLayout w;
  const uint64_t units = (uint64_t)d.batch * hkv;
  const uint64_t slots = r.one_shot ? 0 : (r.persistent ? (uint64_t)r.ps_grid + units : units * r.num_parts);
  w.states = slots * r.rows;
  w.off_l = align256(w.states * 4);
  w.off_o = w.off_l + align256(w.states * 4);
  w.off_runs = w.off_o + align256(w.states * d.head_dim * 4);
  w.off_qoffs = w.off_runs + (r.persistent && !r.one_shot ? align256(units * 8) : 0);
  w.total = w.off_qoffs + (d.batch > pa::kScanBatch ? align256((uint64_t)d.batch * 4) : 0);
  return w;
}

pa_status make_plan(const pa_dims* d, int32_t window, int32_t hkv, int32_t bs, int32_t num_cus,
                    const pa_options* o, pa_plan* p) {
  pa_status st = check_shape(d, window, hkv, bs);
  if (st != PA_OK) return st;
  if (!p) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
  if (num_cus < 1) return fail(PA_ERR_INVALID_ARG, "num_cus %d < 1", num_cus);
  pa_plan r = {};
  const int G = d->num_q_heads / hkv;
  r.rows = G * d->max_query_len;
  r.span_max = window ? (int32_t)std::min<int64_t>(d->max_seq_len, (int64_t)window + d->max_query_len - 1)
                      : d->max_seq_len;
  const int path_req = o ? o->path : PA_PATH_AUTO;
  if (path_req < PA_PATH_AUTO || path_req > PA_PATH_VALU_LDS)
    return fail(PA_ERR_INVALID_ARG, "path %d unknown", path_req);
  if (path_req == PA_PATH_AUTO) {
    // fp32 inputs never take reduced-precision products: the vector ALUs.
    // For bf16 the matrix cores, which measured faster than the vector
    // kernels on MI355X at every row count (R = 4 included).
    r.path = (d->dtype == PA_F32 || !mfma_head_dim(d->head_dim)) ? PA_PATH_VALU : PA_PATH_MFMA;
  } else {
    r.path = path_req;
  }
  // the register-resident vector kernel is instantiated at head dims 64, 128
  // and 256; other head dims stage K and V through shared memory
  if (r.path == PA_PATH_VALU && !mfma_head_dim(d->head_dim)) r.path = PA_PATH_VALU_LDS;
  if (r.path == PA_PATH_MFMA && d->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "the matrix-core path needs bf16 inputs");
  if (r.path == PA_PATH_MFMA && !mfma_head_dim(d->head_dim))
    return fail(PA_ERR_UNSUPPORTED, "the matrix-core path takes head_dim 64, 128 or 256");
  if (r.path != PA_PATH_MFMA && d->kv_format == PA_KV_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "an FP8 KV cache needs the matrix-core path");
  if (r.path == PA_PATH_MFMA) {
    // Row tiles (16 rows each) per workgroup: all rows when they fit in 64
    // (D = 256: one tile, for registers); beyond that blocks of 64 rows at
    // D = 64 and 32 rows at D = 128 (2 waves per SIMD at 212 VGPRs, and still
    // faster on MI355X than one-tile blocks, which read K/V twice as often:
    // 61 against 66-70 us on a 128-row batch).
    const int need = (r.rows + 15) / 16;
    const int cap = d->head_dim == 256 ? 1 : (r.rows <= 64 ? 4 : (d->head_dim == 64 ? 4 : 2));
    r.row_tiles = std::min(need, cap);
    const int w_req = o ? o->waves : 0;
    if (w_req) {
      if (w_req != 1 && w_req != 2 && w_req != 4)
        return fail(PA_ERR_INVALID_ARG, "waves %d must be 1, 2 or 4", w_req);
      // two row tiles also run with 4 waves (each K/V load feeds both tiles)
      if (w_req * r.row_tiles > (r.row_tiles == 2 ? 8 : 4))
        return fail(PA_ERR_UNSUPPORTED, "waves %d x row tiles %d not instantiated", w_req,
                    r.row_tiles);
      r.waves = w_req;
    } else {
      r.waves = r.row_tiles == 1 ? 4 : (r.row_tiles == 2 ? 2 : 1);
    }
    r.block_rows = 16 * r.row_tiles;
  } else if (r.path == PA_PATH_VALU) {
    r.waves = 4;  // 256-thread workgroup
    r.row_tiles = 0;
    // rows per workgroup: 4 or 8 (the scores of a step take one register
    // per row, and at least 4 independent accumulators keep the broadcast
    // multiply-adds free of read-after-write waits; fewer real rows leave
    // zero rows, which cost arithmetic but no memory traffic)
    r.block_rows = r.rows <= 4 ? 4 : 8;
  } else {
    r.waves = 4;  // 256-thread workgroup
    r.row_tiles = pa::kValuRows / 16;
    r.block_rows = pa::kValuRows;
  }
  r.row_blocks = (r.rows + r.block_rows - 1) / r.block_rows;
  const int64_t span_cover = (int64_t)r.span_max + pa::kChunk - 1;  // span plus alignment slack
  const int64_t units = (int64_t)d->batch * hkv;
  const int sched_req = o ? o->schedule : 0;
  if (sched_req < 0 || sched_req > 2) return fail(PA_ERR_INVALID_ARG, "schedule %d unknown", sched_req);
  if (sched_req == 2) {
    if (r.path != PA_PATH_MFMA && r.path != PA_PATH_VALU)
      return fail(PA_ERR_UNSUPPORTED,
                  "the persistent schedule needs the matrix-core or register-resident vector path");
    if (d->batch > pa::kPsMaxBatch)
      return fail(PA_ERR_UNSUPPORTED, "the persistent schedule handles batch <= %d", pa::kPsMaxBatch);
    if (r.row_blocks > 1)
      return fail(PA_ERR_UNSUPPORTED, "the persistent schedule needs all rows in one workgroup");
  }
  // Persistent schedule (measured on MI355X: +3-5 % on many-unit split
  // shapes, slightly slower for one (sequence, head) or one-shot calls):
  // matrix-core or register-resident vector path, at least 64 (sequence, KV
  // head) units, batch that fits its shared-memory prefix sums, a span long
  // enough to split, and every row of a unit in one workgroup.
  const bool ps_path = r.path == PA_PATH_MFMA || (r.path == PA_PATH_VALU && kWavePersistentAuto);
  const bool ps_auto = ps_path && units >= 64 && d->batch <= pa::kPsMaxBatch &&
                       span_cover > 8 * pa::kChunk && r.row_blocks == 1;
  r.persistent = sched_req == 2 ? 1 : (sched_req == 1 ? 0 : (ps_auto ? 1 : 0));
  const int p_req = o ? o->part_size : 0;
  if (p_req) {
    if (p_req < pa::kChunk || p_req % pa::kChunk)
      return fail(PA_ERR_INVALID_ARG, "part_size %d must be a positive multiple of %d", p_req,
                  pa::kChunk);
    r.part_size = p_req;
  } else if (r.persistent) {
    // Persistent schedule: consecutive partitions of a unit inside one
    // workgroup's share are merged on the fly, so partitions only set how
    // finely the shares balance the work.  About 1/16 of a share (estimated
    // with every unit at the longest span and 3 resident workgroups per CU),
    // 4..64 chunks: finer costs workspace slots, not runs (measured on
    // MI355X: GQA 32 x 8192 at 4-6 chunks is 0-5 % faster than at 17).
    const int64_t share = cdiv(units * cdiv(span_cover, pa::kChunk), 3 * (int64_t)num_cus);
    int64_t pc = cdiv(share, 16);
    pc = std::max<int64_t>(pc, 4);
    pc = std::min<int64_t>(pc, 64);
    r.part_size = (int32_t)(pc * pa::kChunk);
  } else {
    // Enough partitions for ~8 workgroups per CU if every (sequence, KV
    // head) had the longest span (real batches average less), counting
    // each row block as a workgroup, with partitions of 8..128 chunks
    // (4.. at head dim 256: the same K/V bytes per workgroup): longer ones
    // amortise each workgroup's set-up and keep the partial states small,
    // shorter ones would multiply the LSE merge's work.
    // One-tile plans on the matrix cores size the grid by bytes in flight
    // instead: each wave has one 32-position chunk of K and V in flight, so
    // about 64 KB per CU takes 65536 / chunk-bytes waves per CU (4 at head
    // dim 128 in bf16, 8 over an FP8 cache or at head dim 64, 2 at head dim
    // 256).  Measured on MI355X, flushed, against the 8-per-CU split: a
    // 131072-position bf16 sequence 29.5 -> 27.9 us per call; 32 units of
    // 32k 91-93 -> 84.5 us (bf16) and 47 -> 42 us (FP8); 4 units of 64k
    // 37.5 -> 36.1 (bf16) and 18.0-18.7 -> 16.0-16.5 us (FP8, kernel).
    const int64_t chunks = cdiv(span_cover, pa::kChunk);
    const int64_t wgs_per_part = std::max<int64_t>(units * r.row_blocks, 1);
    const bool by_bytes = r.path == PA_PATH_MFMA && r.row_tiles == 1 && r.row_blocks == 1;
    int64_t pc;
    if (by_bytes) {
      const bool kv8 = d->kv_format == PA_KV_FP8_E4M3;
      const int64_t chunk_bytes = (int64_t)pa::kChunk * 2 * d->head_dim * (kv8 ? 1 : 2) *
                                  pa::chunks_per_step(d->head_dim, 1, kv8, false);  // bytes per wave step
      const int64_t waves_per_cu = std::max<int64_t>(1, 65536 / chunk_bytes);
      const int64_t nw = d->head_dim == 256 ? 2 : r.waves;  // split plans at D = 256 run 2 waves
      const int64_t wgs = std::max<int64_t>(1, waves_per_cu * num_cus / nw);
      const int64_t want = std::max<int64_t>(1, cdiv(wgs, wgs_per_part));
      // rounded down, so that the longest unit fills its share of the CUs
      // (131072 positions in bf16: 256 partitions of 16 chunks)
      pc = std::max<int64_t>(1, chunks / want);
    } else {
      const int64_t want = std::max<int64_t>(1, cdiv(8 * (int64_t)num_cus, wgs_per_part));
      pc = cdiv(chunks, want);
      // Many rows per unit: each partition's states (R rows of D + 2 fp32,
      // written, then read by the merge) against the K/V it reads, kept to
      // about 1/6: P >= 24 R (D + 2) / (D s), as long as the longest units
      // still give two workgroups per CU.  On the 128-row batch (R = 128,
      // bf16) that is 49 chunks instead of 33: 60 -> 52 us per call on its
      // mixed lengths, and 56 -> 46 / 38 -> 34.5 us with uniform contexts of
      // 4096 / 2048 (fewer, longer partitions).
      const int64_t s_kv = d->kv_format == PA_KV_FP8_E4M3 ? 1 : (d->dtype == PA_F32 ? 4 : 2);
      const int64_t p_state = cdiv(24 * (int64_t)r.rows * (d->head_dim + 2), (int64_t)d->head_dim * s_kv);
      const int64_t pc_fill = chunks * wgs_per_part / (2 * (int64_t)num_cus);
      pc = std::max<int64_t>(pc, std::min<int64_t>(cdiv(p_state, pa::kChunk), pc_fill));
    }
    pc = std::max<int64_t>(pc, d->head_dim == 256 ? 4 : 8);
    pc = std::min<int64_t>(pc, 128);
    r.part_size = (int32_t)(pc * pa::kChunk);
  }
  // KV load form.  Within a call each K/V byte is read by one workgroup,
  // unless row blocks split the rows (then they share it through L2).
  // Across calls a decode step reads every layer's cache once, so the 256 MB
  // MALL holds no layer's cache from one step to the next: non-temporal
  // loads (measured on MI355X: 6.8 vs 6.0 TB/s on 4 KB block gathers, 6 %
  // faster on a 67 MB cache read from HBM) unless the call re-reads K/V.
  const int loads_req = o ? o->loads : 0;
  if (loads_req < 0 || loads_req > 2) return fail(PA_ERR_INVALID_ARG, "loads %d unknown", loads_req);
  r.num_parts = (int32_t)std::max<int64_t>(1, cdiv(span_cover, r.part_size));
  if (r.num_parts == 1) r.part_size = (int32_t)(cdiv(span_cover, pa::kChunk) * pa::kChunk);
  r.one_shot = r.num_parts == 1;
  if (r.one_shot && sched_req != 2) r.persistent = 0;
  const int w_req = o ? o->waves : 0;
  if (r.path == PA_PATH_MFMA && w_req == 0) {
    // Grid plans with few waves in flight, one-shot with under 16 waves per
    // CU: two row tiles run as one workgroup of 4 waves (each K/V load feeds
    // both tiles: half the load instructions and workgroups); more tiles go
    // to one-tile blocks of 4 waves.  Measured on MI355X, 512 sliding-window
    // MTP units of 32 rows: 1024 workgroups x 4 waves were 10 % faster per
    // call than 512 x 2, and 512 x 4 with both tiles ties with them (8.2-8.4
    // us per call warm, 12.4-12.8 flushed; the same HBM traffic, as the
    // second block's reads hit L2).
    if (!r.persistent && r.one_shot && r.row_tiles > 1 && d->head_dim != 256 &&
        units * r.row_blocks * r.waves < 16 * (int64_t)num_cus) {
      if (r.row_tiles == 2) {
        r.waves = 4;
      } else {
        r.row_tiles = 1;
        r.waves = 4;
        r.block_rows = 16;
        r.row_blocks = (r.rows + 15) / 16;
      }
    }
    // Split plans at head dim 256 (~250 VGPRs, one or two waves per SIMD):
    // 2 waves per workgroup, so that twice as many workgroups share the CUs
    // (a long single sequence: 15 % faster than 4 waves; a 32-sequence GQA
    // batch on the persistent schedule: 5 %).
    if (!r.one_shot && d->head_dim == 256) r.waves = 2;
  }
  const bool reread = r.row_blocks > 1;
  r.streaming = r.path != PA_PATH_MFMA ? 0 : (loads_req == 2 ? 1 : (loads_req == 1 ? 0 : !reread));
  r.ps_grid = 0;
  if (r.persistent) {
    const bool kv8 = d->kv_format == PA_KV_FP8_E4M3;
    r.ps_grid = (r.path == PA_PATH_VALU ? kWavePsPerCu
                                        : pa::ps_wgs_per_cu(d->head_dim, r.row_tiles, r.waves, kv8)) *
                num_cus;
  }
  r.workspace_bytes = workspace_layout(r, *d, hkv).total;
  *p = r;
  return PA_OK;
}

std::atomic<int> g_cu_count[64];

pa_status device_cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(PA_ERR_HIP, "device ordinal %d out of range", dev);
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return PA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

pa_status run(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_lens,
              float scale, int32_t window, int32_t hkv, int32_t bs, const pa_dims* d,
              void* workspace, size_t workspace_bytes, void* stream, const pa_options* o) {
  pa_status st = check_shape(d, window, hkv, bs);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_lens)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "out, q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(query_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
  if (workspace && !aligned(workspace, 256))
    return fail(PA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const bool kv8 = d->kv_format == PA_KV_FP8_E4M3;
  if (kv8) {
    // aiter PR #2914 review: FP8 caches without their scales must be refused,
    // not decoded with a default
    if (!o || !o->k_scale || !o->v_scale)
      return fail(PA_ERR_INVALID_ARG,
                  "an FP8 KV cache needs k_scale and v_scale (pa_decode_ex, pa_options)");
    if (!aligned(o->k_scale, 4) || !aligned(o->v_scale, 4))
      return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be 4-byte aligned");
  }
  const bool q8 = d->q_format == PA_Q_FP8_E4M3;
  if (q8) {
    // aiter PR #2914 review: an FP8 query without its scale must be refused
    if (!o || !o->q_scale)
      return fail(PA_ERR_INVALID_ARG, "an FP8 query needs q_scale (pa_decode_ex, pa_options)");
    if (!aligned(o->q_scale, 4))
      return fail(PA_ERR_INVALID_ARG, "q_scale must be 4-byte aligned");
  }
  if (d->batch == 0) return PA_OK;
  int cus = 0;
  st = device_cu_count(&cus);
  if (st != PA_OK) return st;
  pa_plan p;
  st = make_plan(d, window, hkv, bs, cus, o, &p);
  if (st != PA_OK) return st;
  if (p.workspace_bytes && (!workspace || workspace_bytes < p.workspace_bytes))
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes given, %llu needed", workspace ? workspace_bytes : 0,
                (unsigned long long)p.workspace_bytes);
  if (log_enabled())
    std::fprintf(stderr,
                 "[pa_decode] B=%d Hq=%d Hkv=%d D=%d bs=%d w=%d kv8=%d q8=%d R=%d span_max=%d path=%s "
                 "P=%d NP=%d waves=%d row_tiles=%d row_blocks=%d one_shot=%d persistent=%d "
                 "ps_grid=%d streaming=%d ws=%llu cus=%d\n",
                 d->batch, d->num_q_heads, hkv, d->head_dim, bs, window, (int)kv8, (int)q8, p.rows,
                 p.span_max, p.path == PA_PATH_MFMA ? "mfma" : (p.path == PA_PATH_VALU ? "valu" : "valu-lds"), p.part_size, p.num_parts,
                 p.waves, p.row_tiles, p.row_blocks, p.one_shot, p.persistent, p.ps_grid, p.streaming,
                 (unsigned long long)p.workspace_bytes, cus);

  const WsLayout wl = workspace_layout(p, *d, hkv);
  char* ws = (char*)workspace;
  pa::PartArgs a = {};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_lens = query_lens;
  a.ws_m = p.one_shot ? nullptr : (float*)ws;
  a.ws_l = p.one_shot ? nullptr : (float*)(ws + wl.off_l);
  a.ws_o = p.one_shot ? nullptr : (float*)(ws + wl.off_o);
  a.ws_runs = (p.one_shot || !p.persistent) ? nullptr : (int*)(ws + wl.off_runs);
  a.qoffs = d->batch > pa::kScanBatch ? (const int32_t*)(ws + wl.off_qoffs) : nullptr;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.window = window;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = hkv;
  a.group = d->num_q_heads / hkv;
  a.rows = p.rows;
  a.num_parts = p.num_parts;
  a.part_size = p.part_size;
  a.log2_bs = ilog2_exact(bs);
  a.max_blocks_per_seq = d->max_blocks_per_seq;
  a.batch = d->batch;
  a.k_scale = kv8 ? o->k_scale : nullptr;
  a.v_scale = kv8 ? o->v_scale : nullptr;
  a.q_scale = q8 ? o->q_scale : nullptr;
  a.row_blocks = p.row_blocks;
  a.head_dim = d->head_dim;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  const Launch L = {s, o ? (hipEvent_t)o->event_begin : nullptr,
                   o ? (hipEvent_t)o->event_end : nullptr};
  if (a.qoffs) {
    hipLaunchKernelGGL(pa::scan_row_offsets, dim3(1), dim3(1024), 0, s, query_lens, d->batch,
                       (int32_t*)a.qoffs);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "row offset scan launch");
  }
  const uint64_t units = (uint64_t)p.num_parts * hkv * d->batch;  // (partition, seq, head)
  const uint64_t nwg = p.row_blocks > 1
                           ? (units + pa::kXcds - 1) / pa::kXcds * pa::kXcds * p.row_blocks
                           : units;
  if (nwg > 0x7fffffffull) return fail(PA_ERR_UNSUPPORTED, "grid of %llu workgroups too large", (unsigned long long)nwg);
  // persistent plans launch at most the plan's grid bound (the kernel caps
  // it further at what fits on the device at once)
  const dim3 grid(p.persistent ? (uint32_t)p.ps_grid : (uint32_t)nwg);
  const int nrt = p.row_tiles;
  bool ok = true;
  if (p.path == PA_PATH_MFMA) {
    switch (d->head_dim) {
      case 64: ok = pa_host::launch_mfma_64(nrt, p.waves, grid, p.persistent, p.streaming, kv8, q8, cus, L, a); break;
      case 128: ok = pa_host::launch_mfma_128(nrt, p.waves, grid, p.persistent, p.streaming, kv8, q8, cus, L, a); break;
      default: ok = pa_host::launch_mfma_256(nrt, p.waves, grid, p.persistent, p.streaming, kv8, q8, cus, L, a); break;
    }
  } else if (p.path == PA_PATH_VALU) {
    ok = pa_host::launch_wave(d->dtype == PA_F32, d->head_dim, p.block_rows, grid, p.persistent,
                              cus, L, a);
  } else if (d->dtype == PA_F32) {
    launch_part(pa::part_valu<float>, grid, dim3(256), L, a);
  } else {
    launch_part(pa::part_valu<uint16_t>, grid, dim3(256), L, a);
  }
  if (!ok)
    return fail(PA_ERR_UNSUPPORTED, "no kernel for %d row tiles / %d rows x %d waves", nrt,
                p.block_rows, p.waves);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "partition kernel launch");
  if (!p.one_shot) {
    pa::ReduceArgs r = {};
    r.out = out;
    r.seq_lens = seq_lens;
    r.query_lens = query_lens;
    r.ws_m = a.ws_m;
    r.ws_l = a.ws_l;
    r.ws_o = a.ws_o;
    r.ws_runs = a.ws_runs;
    r.window = window;
    r.num_q_heads = d->num_q_heads;
    r.num_kv_heads = hkv;
    r.group = a.group;
    r.rows = p.rows;
    r.num_parts = p.num_parts;
    r.part_size = p.part_size;
    r.head_dim = d->head_dim;
    r.qoffs = a.qoffs;
    // persistent: a unit has one state per workgroup share it crosses;
    // balanced units cross about (grid / units) + 2 shares (a lone long unit
    // crosses them all)
    const int64_t bh = (int64_t)d->batch * hkv;
    const int64_t ps_runs = ((int64_t)p.ps_grid + bh - 1) / bh + 2;
    const int gp = pa::reduce_group_lanes(
        p.persistent ? (int)std::min<int64_t>(p.num_parts, ps_runs) : p.num_parts);
    const int vec = d->head_dim % 4 == 0 ? 4 : 1;  // dims per merge unit
    const int units = p.rows * (d->head_dim / vec);
    const dim3 rgrid((units + 256 / gp - 1) / (256 / gp), hkv, d->batch);
#define PA_REDUCE(T, V)                                                                     \
  switch (gp) {                                                                            \
    case 1: hipLaunchKernelGGL((pa::lse_reduce<T, V, 1>), rgrid, dim3(256), 0, s, r); break; \
    case 16: hipLaunchKernelGGL((pa::lse_reduce<T, V, 16>), rgrid, dim3(256), 0, s, r); break; \
    default: hipLaunchKernelGGL((pa::lse_reduce<T, V, 32>), rgrid, dim3(256), 0, s, r); break; \
  }
    if (d->dtype == PA_F32) {
      if (vec == 4) { PA_REDUCE(float, 4) } else { PA_REDUCE(float, 1) }
    } else {
      if (vec == 4) { PA_REDUCE(uint16_t, 4) } else { PA_REDUCE(uint16_t, 1) }
    }
#undef PA_REDUCE
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "reduce kernel launch");
  }
  return PA_OK;
}

// Workspace of pa_decode_noalloc: a fixed device array instead of
// caller-owned memory, for callers that cannot allocate.  Each GPU the
// library runs on holds its own copy until the process ends; in host code
// the array's name is only a stand-in, so its device address is looked up
// once per device (with that device current) and kept.
constexpr size_t kScratchBytes = size_t(64) << 20;

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_lock;
void* g_scratch_ptr[64];

// Device address of `scratch` on the current device.
pa_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(PA_ERR_HIP, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> guard(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(PA_ERR_HIP, "scratch address %p unusable", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_plan_compute(const pa_dims* dims, int32_t window, int32_t num_kv_heads,
                          int32_t block_size, int32_t num_cus, const pa_options* opts,
                          pa_plan* plan) {
  return make_plan(dims, window, num_kv_heads, block_size, num_cus, opts, plan);
}

pa_status pa_decode_workspace_size_ex(const pa_dims* dims, int32_t window, int32_t num_kv_heads,
                                      int32_t block_size, const pa_options* opts, size_t* bytes) {
  if (!bytes) return fail(PA_ERR_INVALID_ARG, "bytes is NULL");
  pa_status st = check_shape(dims, window, num_kv_heads, block_size);
  if (st != PA_OK) return st;
  int cus = 0;
  st = device_cu_count(&cus);
  if (st != PA_OK) return st;
  pa_plan p;
  st = make_plan(dims, window, num_kv_heads, block_size, cus, opts, &p);
  if (st != PA_OK) return st;
  *bytes = (size_t)p.workspace_bytes;
  return PA_OK;
}

pa_status pa_decode_workspace_size(const pa_dims* dims, int32_t window, int32_t num_kv_heads,
                                   int32_t block_size, size_t* bytes) {
  return pa_decode_workspace_size_ex(dims, window, num_kv_heads, block_size, nullptr, bytes);
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    const int32_t* query_lens, float scale, int32_t window,
                    int32_t num_kv_heads, int32_t block_size, const pa_dims* dims,
                    void* workspace, size_t workspace_bytes, void* hip_stream) {
  return run(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, scale, window,
             num_kv_heads, block_size, dims, workspace, workspace_bytes, hip_stream, nullptr);
}

pa_status pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* seq_lens,
                       const int32_t* query_lens, float scale, int32_t window,
                       int32_t num_kv_heads, int32_t block_size, const pa_dims* dims,
                       void* workspace, size_t workspace_bytes, void* hip_stream,
                       const pa_options* opts) {
  return run(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, scale, window,
             num_kv_heads, block_size, dims, workspace, workspace_bytes, hip_stream, opts);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            const int32_t* query_lens, float scale, int32_t window,
                            int32_t num_kv_heads, int32_t block_size, const pa_dims* dims,
                            void* hip_stream, const pa_options* opts) {
  pa_status st = check_shape(dims, window, num_kv_heads, block_size);
  if (st != PA_OK) return st;
  if (dims->batch == 0) return PA_OK;
  int cus = 0;
  st = device_cu_count(&cus);
  if (st != PA_OK) return st;
  pa_plan p;
  st = make_plan(dims, window, num_kv_heads, block_size, cus, opts, &p);
  if (st != PA_OK) return st;
  if (p.workspace_bytes > kScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "this plan needs %llu bytes of workspace, more than the %zu-byte static scratch "
                "of pa_decode_noalloc; call pa_decode with a workspace instead",
                (unsigned long long)p.workspace_bytes, kScratchBytes);
  void* ws = nullptr;
  if (p.workspace_bytes) {
    st = scratch_address(&ws);
    if (st != PA_OK) return st;
  }
  return run(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, scale, window,
             num_kv_heads, block_size, dims, ws, ws ? kScratchBytes : 0, hip_stream, opts);
}

size_t pa_noalloc_scratch_bytes(void) { return kScratchBytes; }

pa_status pa_pack_kv_cache(const void* k_rows, const void* v_rows, void* k_cache, void* v_cache,
                           const int32_t* block_ids, int32_t num_ids, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                           int32_t dtype, int32_t kv_format, void* hip_stream) {
  if (!k_rows || !v_rows || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID_ARG, "a cache pointer is NULL");
  if (!aligned(k_rows, 16) || !aligned(v_rows, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "cache pointers must be 16-byte aligned");
  if (block_ids && !aligned(block_ids, 4)) return fail(PA_ERR_INVALID_ARG, "block_ids must be 4-byte aligned");
  if (dtype != PA_F32 && dtype != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "dtype %d is neither PA_F32 nor PA_BF16", dtype);
  if (kv_format != PA_KV_NATIVE && kv_format != PA_KV_FP8_E4M3)
    return fail(PA_ERR_INVALID_ARG, "kv_format %d unknown", kv_format);
  if (num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks %d < 1", num_blocks);
  if (num_kv_heads < 1 || num_kv_heads > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d outside [1, 65535]", num_kv_heads);
  if (ilog2_exact(block_size) < 4 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d must be a power of two in [16, 1024]", block_size);
  if (head_dim < 1 || head_dim > pa::kValuMaxD)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d outside [1, %d]", head_dim, pa::kValuMaxD);
  if (block_ids && num_ids < 0) return fail(PA_ERR_INVALID_ARG, "num_ids %d < 0", num_ids);
  const char* kr = (const char*)k_rows;
  const char* kc = (const char*)k_cache;
  const int es = kv_format == PA_KV_FP8_E4M3 ? 1 : (dtype == PA_F32 ? 4 : 2);
  const uint64_t bytes = (uint64_t)num_blocks * num_kv_heads * block_size * head_dim * es;
  const char* vr = (const char*)v_rows;
  const char* vc = (const char*)v_cache;
  auto overlap = [bytes](const char* x, const char* y) { return x < y + bytes && y < x + bytes; };
  if (overlap(kr, kc) || overlap(vr, vc) || overlap(kr, vc) || overlap(vr, kc))
    return fail(PA_ERR_INVALID_ARG, "the row-layout and tiled caches must not overlap");
  const int n = block_ids ? num_ids : num_blocks;  // grid x (up to 2^31 - 1), heads on y
  if (n == 0) return PA_OK;
  pa::PackArgs a = {};
  a.k_rows = (const uint8_t*)k_rows;
  a.v_rows = (const uint8_t*)v_rows;
  a.k_cache = (uint8_t*)k_cache;
  a.v_cache = (uint8_t*)v_cache;
  a.block_ids = block_ids;
  a.num_blocks = num_blocks;
  a.num_kv_heads = num_kv_heads;
  a.log2_bs = ilog2_exact(block_size);
  a.head_dim = head_dim;
  a.es = es;
  hipLaunchKernelGGL(pa::pack_kv, dim3(n, num_kv_heads), dim3(256), 0, (hipStream_t)hip_stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "pack_kv launch");
  return PA_OK;
}

pa_status pa_debug_spans(const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* query_lens, int32_t window, int32_t num_kv_heads,
                         int32_t block_size, const pa_dims* dims, const pa_options* opts,
                         int32_t* seq_info, int32_t* row_info, int32_t* blocks, int32_t* parts,
                         void* hip_stream) {
  pa_status st = check_shape(dims, window, num_kv_heads, block_size);
  if (st != PA_OK) return st;
  if (!block_tables || !seq_lens || !query_lens || !seq_info || !row_info || !blocks || !parts)
    return fail(PA_ERR_INVALID_ARG, "a pointer is NULL");
  if (dims->batch == 0) return PA_OK;
  int cus = 0;
  st = device_cu_count(&cus);
  if (st != PA_OK) return st;
  pa_plan p;
  st = make_plan(dims, window, num_kv_heads, block_size, cus, opts, &p);
  if (st != PA_OK) return st;
  pa::SpanArgs a = {};
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_lens = query_lens;
  a.seq_info = seq_info;
  a.row_info = row_info;
  a.blocks = blocks;
  a.parts = parts;
  a.window = window;
  a.part_size = p.part_size;
  a.num_parts = p.num_parts;
  a.log2_bs = ilog2_exact(block_size);
  a.max_blocks_per_seq = dims->max_blocks_per_seq;
  hipLaunchKernelGGL(pa::debug_spans, dim3(dims->batch), dim3(64), 0, (hipStream_t)hip_stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "debug_spans launch");
  return PA_OK;
}

pa_status pa_check_inputs(const int32_t* block_tables, const int32_t* seq_lens,
                          const int32_t* query_lens, int32_t window, int32_t num_kv_heads,
                          int32_t block_size, const pa_dims* dims, int32_t* report,
                          void* hip_stream) {
  pa_status st = check_shape(dims, window, num_kv_heads, block_size);
  if (st != PA_OK) return st;
  if (!block_tables || !seq_lens || !query_lens || !report)
    return fail(PA_ERR_INVALID_ARG, "a pointer is NULL");
  if (!aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(query_lens, 4) ||
      !aligned(report, 4))
    return fail(PA_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
  const hipStream_t s = (hipStream_t)hip_stream;
  hipLaunchKernelGGL(pa::check_init, dim3(1), dim3(64), 0, s, report);
  if (dims->batch > 0) {
    pa::CheckArgs a = {};
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.query_lens = query_lens;
    a.report = report;
    a.window = window;
    a.log2_bs = ilog2_exact(block_size);
    a.max_blocks_per_seq = dims->max_blocks_per_seq;
    a.max_seq_len = dims->max_seq_len;
    a.max_query_len = dims->max_query_len;
    a.num_blocks = dims->num_blocks;
    hipLaunchKernelGGL(pa::check_inputs, dim3(dims->batch), dim3(64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "check_inputs launch");
  return PA_OK;
}

pa_status pa_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t sink_len,
                         int32_t layout, int32_t* workgroups, void* hip_stream) {
  if (!src || !sink || !workgroups) return fail(PA_ERR_INVALID_ARG, "a pointer is NULL");
  if (!aligned(src, 16) || bytes % 16)
    return fail(PA_ERR_INVALID_ARG, "src must be 16-byte aligned and bytes a multiple of 16");
  if (!aligned(sink, 4)) return fail(PA_ERR_INVALID_ARG, "sink must be 4-byte aligned");
  if (sink_len < 1) return fail(PA_ERR_INVALID_ARG, "sink_len %d < 1", sink_len);
  if (layout != 0 && layout != 1) return fail(PA_ERR_INVALID_ARG, "layout %d unknown", layout);
  const uint64_t n16 = bytes / 16;
  const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>(sink_len, cdiv((int64_t)n16, 256)));
  const hipStream_t s = (hipStream_t)hip_stream;
  if (layout == 1)
    hipLaunchKernelGGL(pa::stream_read<true>, dim3((uint32_t)wgs), dim3(256), 0, s,
                       (const pa::u32x4*)src, n16, sink);
  else
    hipLaunchKernelGGL(pa::stream_read<false>, dim3((uint32_t)wgs), dim3(256), 0, s,
                       (const pa::u32x4*)src, n16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "stream_read launch");
  *workgroups = (int32_t)wgs;
  return PA_OK;
}

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: valid request not implemented";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime error";
  }
  return "unknown pa_status";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
