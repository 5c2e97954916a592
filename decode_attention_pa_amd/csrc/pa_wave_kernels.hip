// Register-resident vector-ALU partition kernels: every (element type, head
// dim, rows per workgroup) instantiation and its launcher.
#include "pa_launch.h"
#include "pa_wave.h"

namespace pa_host {

namespace {

template <typename T, int D, int RB>
void launch_inst(dim3 grid, bool persistent, int cus, const Launch& L, const pa::PartArgs& a) {
  if (persistent) {
    // grid.x: the plan's bound on the persistent grid; never more than fit at once
    const void* fn = (const void*)pa::part_wave_ps<T, D, RB>;
    const dim3 pgrid((unsigned)std::min<int64_t>(resident_wgs(fn, 256, cus), (int64_t)grid.x));
    launch_part(pa::part_wave_ps<T, D, RB>, pgrid, dim3(256), L, a);
  } else {
    launch_part(pa::part_wave<T, D, RB>, grid, dim3(256), L, a);
  }
}

template <typename T, int D>
bool launch_rows(int block_rows, dim3 grid, bool persistent, int cus, const Launch& L,
                 const pa::PartArgs& a) {
  switch (block_rows) {
    case 4: launch_inst<T, D, 4>(grid, persistent, cus, L, a); return true;
    case 8: launch_inst<T, D, 8>(grid, persistent, cus, L, a); return true;
    default: return false;
  }
}

template <typename T>
bool launch_dim(int D, int block_rows, dim3 grid, bool persistent, int cus, const Launch& L,
                const pa::PartArgs& a) {
  switch (D) {
    case 64: return launch_rows<T, 64>(block_rows, grid, persistent, cus, L, a);
    case 128: return launch_rows<T, 128>(block_rows, grid, persistent, cus, L, a);
    case 256: return launch_rows<T, 256>(block_rows, grid, persistent, cus, L, a);
    default: return false;
  }
}

}  // namespace

bool launch_wave(bool f32, int D, int block_rows, dim3 grid, bool persistent, int cus,
                 const Launch& L, const pa::PartArgs& a) {
  return f32 ? launch_dim<float>(D, block_rows, grid, persistent, cus, L, a)
             : launch_dim<uint16_t>(D, block_rows, grid, persistent, cus, L, a);
}

}  // namespace pa_host
