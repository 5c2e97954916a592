// Host-side launch of the matrix-core partition kernels, shared by the
// translation units that instantiate them (one per head dim, compiled in
// parallel) and by the entry points in pa_decode.hip.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pa_common.h"
#include "pa_mfma.h"

namespace pa_host {

// Resident workgroups of a kernel on the current device, all CUs together
// (defined in pa_decode.hip: one cache for the whole library).
int resident_wgs(const void* fn, int threads, int cus);

// Stream of a call and the caller's timing events.  With events, the
// partition kernel is launched through hipExtLaunchKernel, which stamps them
// with that dispatch's own start and end (the interval a kernel trace
// reports), not with the times the stream reached two separate markers.
struct Launch {
  hipStream_t s;
  hipEvent_t begin, end;
};

template <typename K>
void launch_part(K kernel, dim3 grid, dim3 block, const Launch& L, const pa::PartArgs& a) {
  if (L.begin || L.end)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, L.s, L.begin, L.end, 0, a);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, L.s, a);
}

template <int D, int NRT, int NW, bool STREAM, bool KV8, bool Q8>
void launch_mfma_inst(dim3 grid, bool persistent, int cus, const Launch& L, const pa::PartArgs& a) {
  if (persistent) {
    // grid.x: the plan's bound on the persistent grid (it sized the
    // workspace for that many workgroups); never more than fit at once
    const void* fn = (const void*)pa::part_mfma_ps<D, NRT, NW, STREAM, KV8, Q8>;
    const dim3 pgrid((unsigned)std::min<int64_t>(resident_wgs(fn, 64 * NW, cus), (int64_t)grid.x));
    launch_part(pa::part_mfma_ps<D, NRT, NW, STREAM, KV8, Q8>, pgrid, dim3(64 * NW), L, a);
  } else {
    launch_part(pa::part_mfma<D, NRT, NW, STREAM, KV8, Q8>, grid, dim3(64 * NW), L, a);
  }
}

template <int D, bool STREAM, bool KV8, bool Q8>
bool launch_mfma_shape(int nrt, int nw, dim3 grid, bool persistent, int cus, const Launch& L,
                       const pa::PartArgs& a) {
  if constexpr (D == 256) {  // one row tile (the plan never asks for more)
    switch (nrt * 8 + nw) {
      case 1 * 8 + 1: launch_mfma_inst<D, 1, 1, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
      case 1 * 8 + 2: launch_mfma_inst<D, 1, 2, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
      case 1 * 8 + 4: launch_mfma_inst<D, 1, 4, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
      default: return false;
    }
  } else {
  switch (nrt * 8 + nw) {
    case 1 * 8 + 1: launch_mfma_inst<D, 1, 1, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
    case 1 * 8 + 2: launch_mfma_inst<D, 1, 2, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
    case 1 * 8 + 4: launch_mfma_inst<D, 1, 4, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
    case 2 * 8 + 1: launch_mfma_inst<D, 2, 1, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
    case 2 * 8 + 2: launch_mfma_inst<D, 2, 2, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
    case 2 * 8 + 4: launch_mfma_inst<D, 2, 4, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
    case 3 * 8 + 1: launch_mfma_inst<D, 3, 1, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
    case 4 * 8 + 1: launch_mfma_inst<D, 4, 1, STREAM, KV8, Q8>(grid, persistent, cus, L, a); return true;
    default: return false;
  }
  }
}

template <int D>
inline bool launch_mfma(int nrt, int nw, dim3 grid, bool persistent, bool streaming, bool kv8, bool q8,
                 int cus, const Launch& L, const pa::PartArgs& a) {
  if (q8)
    return streaming ? launch_mfma_shape<D, true, true, true>(nrt, nw, grid, persistent, cus, L, a)
                     : launch_mfma_shape<D, false, true, true>(nrt, nw, grid, persistent, cus, L, a);
  if (kv8)
    return streaming ? launch_mfma_shape<D, true, true, false>(nrt, nw, grid, persistent, cus, L, a)
                     : launch_mfma_shape<D, false, true, false>(nrt, nw, grid, persistent, cus, L, a);
  return streaming ? launch_mfma_shape<D, true, false, false>(nrt, nw, grid, persistent, cus, L, a)
                   : launch_mfma_shape<D, false, false, false>(nrt, nw, grid, persistent, cus, L, a);
}


// One instantiation per head dim, each in its own translation unit.
bool launch_mfma_64(int nrt, int nw, dim3 grid, bool persistent, bool streaming, bool kv8, bool q8,
                    int cus, const Launch& L, const pa::PartArgs& a);
bool launch_mfma_128(int nrt, int nw, dim3 grid, bool persistent, bool streaming, bool kv8, bool q8,
                     int cus, const Launch& L, const pa::PartArgs& a);
bool launch_mfma_256(int nrt, int nw, dim3 grid, bool persistent, bool streaming, bool kv8, bool q8,
                     int cus, const Launch& L, const pa::PartArgs& a);

// Register-resident vector kernels (pa_wave_kernels.hip): fp32 or bf16
// caches, head dims 64, 128 and 256, 4 or 8 rows per workgroup, grid or
// persistent schedule.
bool launch_wave(bool f32, int D, int block_rows, dim3 grid, bool persistent, int cus,
                 const Launch& L, const pa::PartArgs& a);

}  // namespace pa_host
