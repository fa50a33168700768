// Tiled int8 weight layout used by the expert kernels.
//
// A row-major int8 matrix [rows, cols] (rows % 16 == 0, cols % 64 == 0) is
// stored as 1 KiB blocks of 16 rows x 64 columns:
//   block (rg, ks) = rows 16*rg .. +16, columns 64*ks .. +64, at block index
//   rg * (cols/64) + ks, i.e. the blocks of one 16-row group are consecutive;
//   inside a block, byte (r, c) sits at 256*(c/16) + 16*r + (c%16).
// So lane l of a wavefront reading the block's 16-byte piece l gets row l%16,
// columns 16*(l/16) .. +16 -- exactly the operand a 16x16x32 MFMA lane needs
// for two reduction steps -- and a wave streams a 16-row group as one
// contiguous run of (cols/64) KiB. With (out, in) expert weights
// [E, out, in] = rows E*out, every 16-row group stays inside one expert.
//
// Packing is a pure byte permutation done once at load time; one thread
// moves one 16-byte piece (reads 16 bytes of a source row, writes the packed
// piece in order, so the writes are fully coalesced).
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void pack_rows_kernel(const int8_t* __restrict__ src, long rows, int cols,
                                                        int8_t* __restrict__ dst) {
  const long piece = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long pieces = rows * cols / 16;
  if (piece >= pieces) return;
  const long block = piece >> 6;
  const int l = (int)(piece & 63);
  const int kblocks = cols >> 6;
  const long rg = block / kblocks;
  const int ks = (int)(block - rg * kblocks);
  const long row = rg * 16 + (l & 15);
  const int col = ks * 64 + 16 * (l >> 4);
  const uint4 v = *reinterpret_cast<const uint4*>(src + row * cols + col);
  *reinterpret_cast<uint4*>(dst + piece * 16) = v;
}

}  // namespace

hipError_t launch_pack_rows(long rows, int cols, const int8_t* src, int8_t* dst, hipStream_t stream) {
  const long pieces = rows * cols / 16;
  if (pieces == 0) return hipSuccess;
  const long blocks = (pieces + 255) / 256;
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, rows, cols, dst);
  return hipGetLastError();
}

}  // namespace moe
