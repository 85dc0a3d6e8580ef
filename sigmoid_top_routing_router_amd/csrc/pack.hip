// k-block-major copies of the routed gate and up weights.
//
// The tile engine reads an expert's B operand one 64-wide k-block at a time:
// 128 bytes of each of 256 rows per stage.  Row-major [E][h][d] puts those
// pieces d * 2 bytes apart; [E][d/64][h][64] puts the pieces of one stage
// (and of one k-set of the weight-streaming kernel) next to each other, so
// each stage reads whole runs of DRAM pages.  The arithmetic is unchanged:
// the kernels read the same values in the same order, only from other
// addresses.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// One thread per 16-byte piece of the output, written in order: piece o is
// lane-chunk o % 8 of row (o / 8) % rows of k-block (o / (8 rows)) % (cols /
// 64) of matrix o / (8 rows cols / 64).
__global__ __launch_bounds__(256) void pack_kblocks_kernel(const uint4* __restrict__ w,
                                                           int64_t pieces, int rows, int kbs,
                                                           uint4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < pieces; o += stride) {
    const int c8 = (int)(o & 7);
    const int64_t rest = o >> 3;
    const int r = (int)(rest % rows);
    const int64_t rest2 = rest / rows;
    const int kb = (int)(rest2 % kbs);
    const int64_t e = rest2 / kbs;
    // input piece: row r of matrix e, columns 64 kb + 8 c8 .. +7
    const int64_t in = ((e * rows + r) * kbs + kb) * 8 + c8;
    out[o] = w[in];
  }
}

hipError_t launch_pack_kblocks(const uint16_t* w, int64_t E, int rows, int cols, uint16_t* out,
                               hipStream_t stream) {
  const int64_t pieces = E * (int64_t)rows * (cols / 8);
  if (pieces <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_kblocks_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(w), pieces, rows, cols / 64,
                     reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
