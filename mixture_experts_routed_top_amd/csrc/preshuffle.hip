// One-time, load-time relayout of expert weights into matrix-core operand
// order (the preshuffle that the FlyDSL-in-JAX talk summary runs once when the
// weights are loaded, 8:14). A byte permutation; each thread moves one 16-byte
// piece.
//
// Fragment = 32 output rows x 64 reduction bytes (one 32x32 matrix-core step:
// 64 e4m3fn or 32 bf16 values), 2 KB, stored as two 1 KB pieces. In piece pc,
// lane l (16 bytes at l*16) holds row l%32 and reduction bytes
// (l/32)*32 + pc*16 .. +15, so a wave loads one piece as one contiguous,
// fully coalesced block and each lane receives exactly its operand register.
// MXFP8 uses bytes pc*32 + (l/32)*16 .. +15 instead: the scaled instruction
// applies the scale of lane r (r < 32) to what lanes r and r+32 hold in their
// first 16-byte piece and the scale of lane r+32 to their second pieces, so
// each piece must be one 32-value block of the row. MXFP4 (E2M1 codes, two
// per byte) has one-piece fragments of 32 rows x 32 bytes (64 values): lane l
// holds row l%32 and the fragment's bytes (l/32)*16 .. +15, the instruction's
// own order for a 4-bit operand (lane l's 32 values form its scale block).
// Fragments are ordered by 32-row block, then by reduction block. For
// gate/up, composite row c of an expert is row (c/64)*32 + c%32 of W1 when
// (c/32) is even and of W3 when it is odd.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

__global__ __launch_bounds__(256) void preshuffle_kernel(PreshuffleArgs a) {
  const bool fp4 = a.mx_order == 2;
  const int fbytes = fp4 ? 1024 : 2048;          // bytes per fragment
  const int64_t kblocks = a.K_bytes / (fbytes / 32);
  const int64_t per_expert = (int64_t)a.R * a.K_bytes;
  const int64_t n16 = per_expert * a.E / 16;
  const int64_t rows_src = a.src1 ? a.R / 2 : a.R;  // rows of each source matrix
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < n16;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = u * 16;
    const int64_t e = b / per_expert;
    const int64_t rem = b % per_expert;
    const int64_t f = rem / fbytes;
    const int in = (int)(rem % fbytes);
    const int pc = in / 1024, lane = (in % 1024) / 16;
    const int64_t rb = f / kblocks, kb = f % kblocks;
    const int64_t c = rb * 32 + lane % 32;
    const uint8_t* src = a.src0;
    int64_t row = c;
    if (a.src1) {
      row = (c / 64) * 32 + c % 32;
      if ((c / 32) % 2) src = a.src1;
    }
    const int64_t kbyte = fp4 ? kb * 32 + (lane / 32) * 16
                              : kb * 64 + (a.mx_order ? pc * 32 + (lane / 32) * 16
                                                      : (lane / 32) * 32 + pc * 16);
    const int64_t sb = (e * rows_src + row) * a.K_bytes + kbyte;
    *reinterpret_cast<uint4*>(a.dst + b) = *reinterpret_cast<const uint4*>(src + sb);
  }
}

// MXFP8 weight scales: one E8M0 code per row and 32 reduction values. Output
// byte o of an expert: j = o % 4 (which of four row blocks), lane = (o/4) % 64,
// fragment kb = (o/256) % KB, block group g = o / (256*KB); it is the code of
// composite row (4g + j)*32 + lane%32, value block 2*kb + lane/32. A lane of a
// GEMM wave then loads the codes of its four (or two) row blocks for one
// fragment as one 32-bit (16-bit) word, and the matrix-core instruction picks
// the byte.
__global__ __launch_bounds__(256) void preshuffle_mx_scales_kernel(PreshuffleArgs a) {
  const int64_t nb = a.K_bytes / 32;               // codes per row
  const int64_t kblocks = a.K_bytes / 64;
  const int64_t per_expert = (int64_t)a.R * nb;
  const int64_t n = per_expert * a.E;
  const int64_t rows_src = a.src1 ? a.R / 2 : a.R;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = o / per_expert, rem = o % per_expert;
    const int j = (int)(rem % 4), lane = (int)(rem / 4 % 64);
    const int64_t kb = rem / 256 % kblocks, g = rem / (256 * kblocks);
    const int64_t c = (4 * g + j) * 32 + lane % 32;
    const uint8_t* src = a.src0;
    int64_t row = c;
    if (a.src1) {
      row = (c / 64) * 32 + c % 32;
      if ((c / 32) % 2) src = a.src1;
    }
    a.dst[o] = src[(e * rows_src + row) * nb + 2 * kb + lane / 32];
  }
}

hipError_t launch_preshuffle_mx_scales(const PreshuffleArgs& a, hipStream_t st) {
  int64_t n = (int64_t)a.R * (a.K_bytes / 32) * a.E;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(preshuffle_mx_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_preshuffle(const PreshuffleArgs& a, hipStream_t st) {
  int64_t n16 = (int64_t)a.R * a.K_bytes * a.E / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(preshuffle_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
