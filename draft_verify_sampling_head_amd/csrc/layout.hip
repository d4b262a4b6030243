// Weight layout conversion: W2 as the method defines it, r x V (row i holds
// the contribution of rank component i to every vocabulary entry), into the
// W2t [V][r] layout the draft kernels read (each vocabulary entry's r values
// contiguous, so a compute unit's slice of entries loads as whole rows into
// its MFMA operand registers and a chunk's 128 entries are 128 contiguous
// rows).  A weight update converts once; the draft then reads W2t every round.
//
// The transpose moves 64 x 64 tiles through LDS: a workgroup of 256 threads
// reads a tile of W2 row by row (coalesced along V) and writes it row by row
// of W2t (coalesced along r); the LDS tile has a padded row so the column
// reads do not collide in the banks.  Pure data movement: element bits are
// copied unchanged, for 2-byte (bf16) and 4-byte (fp32) elements alike.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dspark.h"
#include "launch.hpp"

namespace dspark {
namespace {

constexpr int kTile = 64;       // tile edge (elements)
constexpr int kTT = 256;        // threads per workgroup

template <typename E>
__global__ __launch_bounds__(kTT) void k_transpose(const E* __restrict__ src, E* __restrict__ dst,
                                                   int rows, int cols) {
  // src [rows][cols] -> dst [cols][rows]; blockIdx.x tiles cols, blockIdx.y rows
  __shared__ E tile[kTile][kTile + 1];
  const int c0 = blockIdx.x * kTile, r0 = blockIdx.y * kTile;
  const int tx = threadIdx.x & (kTile - 1), ty = threadIdx.x / kTile;   // 64 x 4
  for (int i = ty; i < kTile; i += kTT / kTile) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[(int64_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < kTile; i += kTT / kTile) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) dst[(int64_t)c * rows + r] = tile[tx][i];
  }
}

}  // namespace
}  // namespace dspark

extern "C" dspark_status dspark_w2_transpose(int r, int V, const void* W2, void* W2t,
                                             dspark_dtype W_dt, hipStream_t stream) {
  DSPARK_ABI_RANGE();
  using namespace dspark;
  if (r < 0 || V < 1) return DSPARK_E_INVALID;
  if (W_dt != DSPARK_F32 && W_dt != DSPARK_BF16) return DSPARK_E_INVALID;
  if (r == 0) return DSPARK_OK;
  if (!W2 || !W2t) return DSPARK_E_INVALID;
  const char* a = static_cast<const char*>(W2);
  const char* b = static_cast<const char*>(W2t);
  const int64_t bytes = (int64_t)r * V * (W_dt == DSPARK_BF16 ? 2 : 4);
  if (a < b + bytes && b < a + bytes) return DSPARK_E_INVALID;      // overlapping buffers
  const dim3 grid((V + kTile - 1) / kTile, (r + kTile - 1) / kTile);
  if (grid.y > 65535u) return DSPARK_E_UNSUPPORTED;
  if (W_dt == DSPARK_BF16)
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(kTT), 0, stream,
                       static_cast<const uint16_t*>(W2), static_cast<uint16_t*>(W2t), r, V);
  else
    hipLaunchKernelGGL(k_transpose<uint32_t>, grid, dim3(kTT), 0, stream,
                       static_cast<const uint32_t*>(W2), static_cast<uint32_t*>(W2t), r, V);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_E_HIP;
}
