// Matrix-core partition kernels at head dim 256: every (row tiles, waves,
// load form, KV format, query format) instantiation and its launcher.
#include "pa_launch.h"

namespace pa_host {

bool launch_mfma_256(int nrt, int nw, dim3 grid, bool persistent, bool streaming, bool kv8, bool q8,
                    int cus, const Launch& L, const pa::PartArgs& a) {
  return launch_mfma<256>(nrt, nw, grid, persistent, streaming, kv8, q8, cus, L, a);
}

}  // namespace pa_host
