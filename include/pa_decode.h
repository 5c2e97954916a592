/*
 * pa_decode.h - paged-attention decode on AMD Instinct MI355X (gfx950).
 *
 * A few query tokens per sequence attend over a KV cache held in fixed-size
 * physical blocks that a per-sequence block table names.  The operation
 * follows the interface of gllm "feat(backend): sliding-window
 * PagedAttention" (#116), "What changes — Interface":
 *     PagedAttention(dst, q, kCache, vCache, blockTables, seqLens,
 *                    queryLens, scale, window)
 * with its window rule (summary): a positive window w limits the query at
 * position p to the w positions ending at p (p-w+1 to p); w = 0 leaves
 * causal attention unlimited.  Query heads map onto KV heads by integer
 * division by the group size H_q / H_kv (executorch PR #18759, review of
 * sdpa_decode_splitk: native grouped-query attention).
 * Multi-token queries (aiter PR #2914 "Pa gluon swa mtp opt": sliding-window
 * MTP decode) are the trailing query_lens[b] positions of the context and
 * are causal among themselves.  Long contexts are cut into partitions whose
 * (max logit, exp-sum, partial output) a second kernel merges by
 * log-sum-exp (executorch PR #18759 "split-K flash-decoding"; aiter PR #2914
 * workspace buffers max_logits / exp_sums / temporary_output).
 *
 * Definition.  For sequence b with context length L_b = seq_lens[b] (the
 * query tokens included) and q_b = query_lens[b] query tokens, query token
 * i in [0, q_b) sits at position p = L_b - q_b + i.  Query head h_q uses KV
 * head h = h_q / G, G = H_q / H_kv.  Its visible positions are
 * [lo, p] with lo = 0 if window == 0 else max(0, p - window + 1).  With
 * s_t = scale * <q, k_t>, out = sum_t softmax(s)_t * v_t.
 *
 * Memory layouts (row-major, contiguous, all device memory):
 *   q, out        [T, H_q, D], T = sum_b q_b; sequence b owns rows
 *                 qoff_b .. qoff_b + q_b - 1, qoff_b = q_0 + ... + q_{b-1}
 *   k_cache       [num_blocks, H_kv, block_size/16, 2, D/E, 8, E] with E = 8 for
 *                 bf16 and fp32 and E = 16 for FP8: slots grouped by 16; slot s
 *                 of a group lives in half (s >> 2) & 1 at place
 *                 (s & 3) | ((s >> 3) << 2), i.e. half 0 holds slots 0-3 and
 *                 8-11, half 1 slots 4-7 and 12-15; each half is a [D/E][8][E]
 *                 tile (column of E dims, place, dim within the column).  For
 *                 bf16 and FP8 a column of one slot is 16 contiguous bytes and a
 *                 column of a half 128.  Head dims that are not a multiple of 8
 *                 (vector path only) keep one row per slot: [num_blocks, H_kv,
 *                 block_size, D]
 *   v_cache       [num_blocks, H_kv, block_size/8, D, 8]: slots grouped by 8;
 *                 slot s of a block lives at [s/8][d][s%8] (a [D, 8] tile per
 *                 group: 16 contiguous bytes hold one dim of 8 consecutive
 *                 positions).  FP8: groups of 16, [block_size/16][D][16]
 *   block_tables  int32 [B, max_blocks_per_seq]; position t of sequence b
 *                 lives in physical block block_tables[b][t / block_size] at
 *                 slot t % block_size
 *   seq_lens, query_lens   int32 [B]
 * q and out share one element type (pa_dims.dtype); k_cache and v_cache share
 * it too, or hold FP8 codes (pa_dims.kv_format); over an FP8 cache q may hold
 * FP8 codes as well (pa_dims.q_format, [T, H_q, D] bytes).
 *
 * Device-side preconditions (not checked on the hot path; violating them is
 * undefined behaviour):  0 <= q_b <= L_b <= max_seq_len, q_b <= max_query_len,
 * and block_tables[b][k] in [0, num_blocks) for every k < ceil(L_b/block_size)
 * that holds a visible position.  Table entries beyond those, cache slots
 * at or past L_b, and blocks no row can see are never used: they may hold
 * anything, NaN included.
 *
 * Ownership and streams.  The caller owns every buffer, the workspace too;
 * the library allocates and frees nothing.  Work is enqueued on the given HIP
 * stream (NULL = the default stream); no call synchronises the host or reads
 * device memory from the host.  Calls are reentrant; calls that share one
 * workspace must be ordered on one stream.
 *
 * Errors.  No call throws.  Every host-visible argument is validated before
 * any HIP call; a failing call returns a status and leaves a thread-local
 * message readable through pa_last_error().
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or shape */
  PA_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement */
  PA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  PA_ERR_HIP = 4            /* a HIP runtime call failed (message has the HIP error) */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,               /* IEEE binary32 */
  PA_BF16 = 1               /* bfloat16 */
} pa_dtype;

/* Element format of k_cache and v_cache. */
typedef enum pa_kv_format {
  PA_KV_NATIVE = 0,         /* K and V in pa_dims.dtype */
  PA_KV_FP8_E4M3 = 1        /* OCP E4M3 codes (one byte) with per-tensor scales: value =
                               code * (*k_scale) for K, code * (*v_scale) for V.  bf16
                               q/out and the matrix-core path only.  aiter PR #2914
                               (review of pa_decode_gluon): an FP8 cache must come with
                               its key / value scales, and calls without them are
                               rejected (PA_ERR_INVALID_ARG) */
} pa_kv_format;

/* Element format of q. */
typedef enum pa_q_format {
  PA_Q_NATIVE = 0,          /* q in pa_dims.dtype */
  PA_Q_FP8_E4M3 = 1         /* OCP E4M3 codes (one byte) with a per-tensor scale: value =
                               code * (*q_scale); out stays bf16.  Needs an FP8 KV cache
                               (QK^T then runs on the FP8 matrix cores) and the
                               matrix-core path.  aiter PR #2914 (review of
                               pa_decode_gluon): an FP8 query must come with its query
                               scale, and a call without it is rejected
                               (PA_ERR_INVALID_ARG) */
} pa_q_format;

/* Shapes a raw-pointer interface cannot infer.  All host-side values. */
typedef struct pa_dims {
  int32_t batch;              /* B >= 0 */
  int32_t num_q_heads;        /* H_q, a multiple of num_kv_heads */
  int32_t head_dim;           /* D in [1, 256]; the matrix-core path (bf16 and FP8 caches)
                                 takes 64, 128 and 256, the vector path any D */
  int32_t max_query_len;      /* upper bound on query_lens[b], >= 1 */
  int32_t max_seq_len;        /* upper bound on seq_lens[b], >= 1 */
  int32_t max_blocks_per_seq; /* row stride of block_tables, >= ceil(max_seq_len/block_size) */
  int32_t num_blocks;         /* physical blocks in each cache, >= 1 */
  int32_t dtype;              /* pa_dtype of out (and of q, k_cache, v_cache when native) */
  int32_t kv_format;          /* pa_kv_format of k_cache and v_cache */
  int32_t q_format;           /* pa_q_format of q */
} pa_dims;

/* Kernel families for the partition step. */
typedef enum pa_path {
  PA_PATH_AUTO = 0,
  PA_PATH_VALU = 1,           /* vector ALUs, register-resident: lane = position for QK^T,
                                 lane = output dims for PV, up to 8 rows per workgroup;
                                 fp32 or bf16 caches at head dims 64, 128 and 256 (other
                                 head dims fall back to PA_PATH_VALU_LDS) */
  PA_PATH_MFMA = 2,           /* bf16 matrix cores (16-row tiles); bf16 only */
  PA_PATH_VALU_LDS = 3        /* vector ALUs with K and V staged through shared memory,
                                 16 rows per workgroup; any head dim up to 256 */
} pa_path;

/* Launch plan: a pure function of the arguments below and the CU count. */
typedef struct pa_plan {
  int32_t path;               /* PA_PATH_VALU, PA_PATH_MFMA or PA_PATH_VALU_LDS */
  int32_t rows;               /* R = G * max_query_len rows per KV head */
  int32_t block_rows;         /* packed rows per workgroup (row_blocks = ceil(R / block_rows)) */
  int32_t span_max;           /* longest windowed span over the batch bound */
  int32_t part_size;          /* positions per partition, a multiple of 32 */
  int32_t num_parts;          /* partition-grid extent per (sequence, KV head) */
  int32_t waves;              /* 64-lane waves per partition workgroup */
  int32_t one_shot;           /* 1: a single partition writes out directly */
  int32_t persistent;         /* 1: persistent schedule (resident grid, balanced partition
                                 shares); 0: one workgroup per partition */
  int32_t row_tiles;          /* 16-row tiles of packed rows per workgroup */
  int32_t row_blocks;         /* workgroups that split the R rows of one partition */
  int32_t streaming;          /* 1: KV loads are non-temporal (each K/V byte is read by one
                                 workgroup); 0: cached loads (row blocks share K/V through
                                 L2, or forced).  Matrix-core path only (0 on the vector
                                 path) */
  int32_t ps_grid;            /* persistent schedule: most workgroups its grid may hold
                                 (fewer when fewer fit on the device at once); 0 otherwise */
  uint64_t workspace_bytes;   /* bytes pa_decode needs in `workspace`: partial states
                                 of split plans, B*H_kv*num_parts slots on the grid
                                 schedule, ps_grid + B*H_kv slots on the persistent one
                                 (R rows of D + 2 floats each), plus 8 bytes per
                                 (sequence, KV head) on the persistent schedule, plus 4
                                 bytes per sequence for batches above 1024 (row offsets
                                 scanned once per call); 0 for one-shot plans of up to
                                 1024 sequences */
} pa_plan;

/* Optional controls for pa_decode_ex / pa_plan_compute (zero = automatic). */
typedef struct pa_options {
  int32_t path;               /* pa_path; AUTO picks by dtype and R */
  int32_t part_size;          /* force the partition size (multiple of 32), 0 = auto */
  int32_t waves;              /* force waves per workgroup (1, 2 or 4), 0 = auto */
  int32_t schedule;           /* 0 = auto, 1 = one workgroup per partition, 2 = persistent
                                 (matrix-core path, batch <= 1024) */
  int32_t loads;              /* KV loads on the matrix-core path: 0 = auto (non-temporal
                                 unless row blocks re-read K/V), 1 = cached (for callers
                                 whose KV stays in the 256 MB last-level cache from one
                                 call to the next), 2 = non-temporal */
  void* event_begin;          /* hipEvent_t (created, timing enabled) stamped with the
                                 partition kernel's start, or NULL; with either event
                                 set the kernel is launched by hipExtLaunchKernel, which
                                 binds the events to that dispatch */
  void* event_end;            /* hipEvent_t stamped with the partition kernel's end */
  const float* k_scale;       /* PA_KV_FP8_E4M3: device pointer to the K scale (one float,
                                 4-byte aligned); required then, ignored otherwise */
  const float* v_scale;       /* PA_KV_FP8_E4M3: device pointer to the V scale */
  const float* q_scale;       /* PA_Q_FP8_E4M3: device pointer to the Q scale (one float,
                                 4-byte aligned); required then, ignored otherwise */
} pa_options;

/*
 * Computes the launch plan without touching a device.  `num_cus` is the
 * compute-unit count the heuristic sizes the grid for (256 on MI355X).
 * Returns PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED for arguments pa_decode
 * would reject.  `opts` may be NULL.
 */
pa_status pa_plan_compute(const pa_dims* dims, int32_t window, int32_t num_kv_heads,
                          int32_t block_size, int32_t num_cus, const pa_options* opts,
                          pa_plan* plan);

/*
 * Workspace bytes pa_decode needs for these arguments on the current HIP
 * device (its CU count is read once per device and cached).  0 means no
 * workspace is needed (one partition per sequence).
 */
pa_status pa_decode_workspace_size(const pa_dims* dims, int32_t window, int32_t num_kv_heads,
                                   int32_t block_size, size_t* bytes);
pa_status pa_decode_workspace_size_ex(const pa_dims* dims, int32_t window, int32_t num_kv_heads,
                                      int32_t block_size, const pa_options* opts, size_t* bytes);

/*
 * Paged-attention decode: writes out[T, H_q, D].  With the environment
 * variable PA_LOG set (and not "0"), each call prints its plan to stderr.
 *   out, q, k_cache, v_cache   device pointers, non-NULL, 16-byte aligned,
 *              layouts above (the library cannot see T on the host: a
 *              caller whose batch has no query tokens at all, T = 0, has
 *              nothing to compute and need not call)
 *   block_tables, seq_lens, query_lens   device int32 arrays, 4-byte aligned
 *   scale      finite logit scale
 *   window     0 (unlimited causal) or the window length in positions
 *   workspace  device scratch of at least pa_decode_workspace_size() bytes,
 *              256-byte aligned; may be NULL when that size is 0
 * pa_decode keeps the argument list of the interface it follows, which has
 * no place for FP8 scales: a call on an FP8 cache or with FP8 queries (whose
 * scales must be given, never defaulted) returns PA_ERR_INVALID_ARG and must
 * go through pa_decode_ex with pa_options.k_scale / v_scale / q_scale.
 *   hip_stream hipStream_t or NULL
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    const int32_t* query_lens, float scale, int32_t window,
                    int32_t num_kv_heads, int32_t block_size, const pa_dims* dims,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

/* pa_decode with explicit plan controls and optional timing events. */
pa_status pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* seq_lens,
                       const int32_t* query_lens, float scale, int32_t window,
                       int32_t num_kv_heads, int32_t block_size, const pa_dims* dims,
                       void* workspace, size_t workspace_bytes, void* hip_stream,
                       const pa_options* opts);

/*
 * pa_decode_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  The partial states live in a static
 * device array of pa_noalloc_scratch_bytes() bytes (64 MiB) that each GPU
 * the library runs on holds until the process ends; no call allocates or
 * frees anything.  A plan whose workspace (pa_decode_workspace_size_ex)
 * exceeds it returns PA_ERR_WORKSPACE before any launch.  Nothing in the
 * scratch has to start at zero: every byte a call reads was written by the
 * same call.  All calls on one GPU share the array, so calls that may
 * overlap on one GPU (different streams, other threads, other processes'
 * copies excepted) race and must be ordered by the caller, e.g. on one
 * stream.  Other arguments and errors as pa_decode_ex.
 */
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            const int32_t* query_lens, float scale, int32_t window,
                            int32_t num_kv_heads, int32_t block_size, const pa_dims* dims,
                            void* hip_stream, const pa_options* opts);

/* Size in bytes of pa_decode_noalloc's static scratch. */
size_t pa_noalloc_scratch_bytes(void);

/*
 * Repacks a paged KV cache held one row per slot, k_rows and v_rows
 * [num_blocks, H_kv, block_size, D] (the plain layout of gllm #116 "What
 * changes — Interface"), into the tiled k_cache / v_cache layouts above, on
 * the given stream: a byte permutation, so the values are bit-identical.
 *   block_ids  device int32 array of the num_ids physical blocks to repack
 *              (ids outside [0, num_blocks) are skipped), or NULL for all
 *              num_blocks blocks; blocks not repacked are left untouched
 *   dtype, kv_format   element type as in pa_dims (fp32, bf16 or E4M3 codes)
 * Head dims off the column grid (not a multiple of 8, or of 16 for FP8) keep
 * one row per slot in K, so K is copied as it is.  All four caches are
 * device memory, 16-byte aligned, and the row-layout caches must not
 * overlap the tiled ones.  The library allocates nothing; errors as
 * pa_decode.
 */
pa_status pa_pack_kv_cache(const void* k_rows, const void* v_rows, void* k_cache, void* v_cache,
                           const int32_t* block_ids, int32_t num_ids, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                           int32_t dtype, int32_t kv_format, void* hip_stream);

/*
 * Index dump for bit-exact checks: runs the device index helpers the
 * partition kernels use and writes, into device int32 arrays,
 *   seq_info  [B, 4]   qoff_b, lo_b, hi_b (union of visible ranges [lo_b, hi_b)),
 *                      number of non-empty partitions of sequence b
 *   row_info  [T, 2]   per query token: first visible position lo_i and its
 *                      own position p_i
 *   blocks    [B, max_blocks_per_seq]   physical block id the kernels read for
 *                      logical block k, or -1 if no visible position is in it
 *   parts     [B, num_parts, 2]   [start, end) of each partition (empty: start == end)
 * for the plan `opts` selects (num_parts from pa_plan_compute).  The kernel
 * reads only seq_lens, query_lens and table entries that hold visible
 * positions.
 */
pa_status pa_debug_spans(const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* query_lens, int32_t window, int32_t num_kv_heads,
                         int32_t block_size, const pa_dims* dims, const pa_options* opts,
                         int32_t* seq_info, int32_t* row_info, int32_t* blocks,
                         int32_t* parts, void* hip_stream);

/*
 * Debug aid, off the hot path: checks on the device the preconditions
 * pa_decode relies on but cannot see from the host (the lengths and the
 * block-table rows of the call, as gllm #116 "What changes — Interface"
 * passes them), so that a caller can have bad inputs reported instead of
 * read (executorch PR #18759 review: arguments the kernel cannot serve
 * should fail clearly).  Writes into `report`, a caller-owned device
 * int32[4]:
 *   report[0]  sequences with q_b < 0, L_b < 0, q_b > L_b, L_b > max_seq_len
 *              or q_b > max_query_len
 *   report[1]  block-table entries outside [0, num_blocks) among those of
 *              logical blocks that hold a visible position of their sequence
 *   report[2]  smallest b counted in report[0], INT32_MAX if none
 *   report[3]  smallest b * max_blocks_per_seq + k counted in report[1],
 *              INT32_MAX if none
 * Sequences counted in report[0] are not scanned for table entries.  The
 * kernels read seq_lens, query_lens and only table entries k <
 * min(ceil(L_b / block_size), max_blocks_per_seq); read `report` once the
 * stream has completed the call.  Host-visible arguments are validated as
 * for pa_decode.
 */
pa_status pa_check_inputs(const int32_t* block_tables, const int32_t* seq_lens,
                          const int32_t* query_lens, int32_t window, int32_t num_kv_heads,
                          int32_t block_size, const pa_dims* dims, int32_t* report,
                          void* hip_stream);

/*
 * Diagnostic: a streaming read of `bytes` (a multiple of 16) from device
 * memory at `src` (16-byte aligned), with the same 16-byte non-temporal
 * loads as the partition kernels, enqueued on `hip_stream`: the HBM read
 * rate a plain kernel reaches, to set the partition kernels' achieved
 * bandwidth against.  `layout` 0: the workgroups interleave over the buffer
 * (grid stride); 1: each reads one contiguous slab.  It launches
 * min(sink_len, ceil(bytes / 4096)) workgroups of 256 threads (count
 * returned in *workgroups); workgroup w writes the XOR of the 32-bit words
 * it read to sink[w] (device memory, 4-byte aligned), so the XOR of
 * sink[0 .. *workgroups) is the XOR of every word read.  Nothing else is
 * written.  PA_ERR_INVALID_ARG for NULL pointers, misalignment, an unknown
 * layout or sink_len < 1.
 */
pa_status pa_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t sink_len,
                         int32_t layout, int32_t* workgroups, void* hip_stream);

/* Static description of a status code. */
const char* pa_status_string(pa_status status);

/* Message of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
