// Weight packing: row-major bf16 matrices -> 16x32 MFMA fragment tiles.
//
// The expert GEMMs stream every weight element once from HBM into the A
// operand of a 16x16x32 bf16 MFMA, where lane l (r = l & 15, g = l >> 4)
// holds row r, columns 8g..8g+7 of a 16-row x 32-column tile.  Storing each
// tile as 1 KB in exactly that lane order makes every wave-wide load one
// contiguous 1 KB access (64 lanes x 16 B).  Tiles of a matrix [R, C] are
// ordered row-tile-major: tile (rt, kt) starts at element (rt*(C/32)+kt)*512,
// so a wave that walks K inside one row tile reads consecutive kilobytes.
#include "smoe_internal.h"

namespace smoe {

// One thread copies one lane's 16 bytes of one tile.  Source matrix m, row
// i, column j sits at src[m * mat_stride + i * ld + j], so a matrix can also
// be a column slice of a wider one.
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ src,
                                                   uint16_t* __restrict__ dst, int rows, int cols,
                                                   long long ld, long long mat_stride,
                                                   long long total_lanes) {
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  if (id >= total_lanes) return;
  const int l = (int)(id & 63);
  const long long tile = id >> 6;                 // over all matrices
  const int ktiles = cols / 32;
  const long long tiles_per_mat = (long long)(rows / 16) * ktiles;
  const long long mat = tile / tiles_per_mat;
  const long long t_in = tile % tiles_per_mat;
  const int rt = (int)(t_in / ktiles), kt = (int)(t_in % ktiles);
  const int r = l & 15, g = l >> 4;
  const uint16_t* s = src + mat * mat_stride + (long long)(rt * 16 + r) * ld + kt * 32 + 8 * g;
  *reinterpret_cast<u32x4*>(dst + (size_t)tile * 512 + l * 8) = *reinterpret_cast<const u32x4*>(s);
}

hipError_t launch_pack(const uint16_t* src, uint16_t* dst, int n_mats, int rows, int cols,
                       long long ld, long long mat_stride, hipStream_t s) {
  const long long lanes = (long long)n_mats * (rows / 16) * (cols / 32) * 64;
  const long long blocks = (lanes + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, rows, cols,
                     ld, mat_stride, lanes);
  return hipGetLastError();
}

}  // namespace smoe
