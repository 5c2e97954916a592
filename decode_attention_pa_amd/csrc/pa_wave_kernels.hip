// Register-resident vector-ALU partition kernels: every (element type, head
// dim, rows per workgroup) instantiation and its launcher.
#include "pa_launch.h"
#include "pa_wave.h"

namespace pa_host {

namespace {

template <typename T, int D>
bool launch_rows(int block_rows, dim3 grid, const Launch& L, const pa::PartArgs& a) {
  switch (block_rows) {
    case 4: launch_part(pa::part_wave<T, D, 4>, grid, dim3(256), L, a); return true;
    case 8: launch_part(pa::part_wave<T, D, 8>, grid, dim3(256), L, a); return true;
    default: return false;
  }
}

template <typename T>
bool launch_dim(int D, int block_rows, dim3 grid, const Launch& L, const pa::PartArgs& a) {
  switch (D) {
    case 64: return launch_rows<T, 64>(block_rows, grid, L, a);
    case 128: return launch_rows<T, 128>(block_rows, grid, L, a);
    case 256: return launch_rows<T, 256>(block_rows, grid, L, a);
    default: return false;
  }
}

}  // namespace

bool launch_wave(bool f32, int D, int block_rows, dim3 grid, const Launch& L, const pa::PartArgs& a) {
  return f32 ? launch_dim<float>(D, block_rows, grid, L, a)
             : launch_dim<uint16_t>(D, block_rows, grid, L, a);
}

}  // namespace pa_host
