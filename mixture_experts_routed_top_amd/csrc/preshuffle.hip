// One-time, load-time relayout of expert weights into matrix-core operand
// order (the "einmaliger Load-Time-Preshuffle" of the FlyDSL-in-JAX talk
// summary, 8:14). A byte permutation; each thread moves one 16-byte piece.
//
// Fragment = 16 output rows x KE reduction columns (one MFMA K step: KE = 32
// bf16 or 128 e4m3fn). Inside a fragment, lane l holds row l%16 and the
// columns [(l/16)*KE/4, (l/16+1)*KE/4), lanes stored one after another, so a
// wave loads a whole fragment as one contiguous, fully coalesced block and each
// lane receives exactly its operand registers. Fragments are ordered by 16-row
// block, then by K block. For gate/up, composite row c of an expert is row
// (c/32)*16 + c%16 of W1 when (c/16) is even and of W3 when it is odd.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

__global__ __launch_bounds__(256) void preshuffle_kernel(PreshuffleArgs a) {
  const int LB = a.KE / 4 * a.es;  // bytes per lane
  const int64_t frag_bytes = 64 * (int64_t)LB;
  const int64_t kblocks = a.K / a.KE;
  const int64_t per_expert = (int64_t)a.R * a.K * a.es;
  const int64_t n16 = per_expert * a.E / 16;
  const int64_t rows_src = a.src1 ? a.R / 2 : a.R;  // rows of each source matrix
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < n16;
       u += (int64_t)gridDim.x * blockDim.x) {
    int64_t b = u * 16;
    int64_t e = b / per_expert;
    int64_t rem = b % per_expert;
    int64_t f = rem / frag_bytes;
    int64_t in = rem % frag_bytes;
    int lane = (int)(in / LB);
    int part = (int)(in % LB);  // byte offset inside the lane's chunk (multiple of 16)
    int64_t rb = f / kblocks, kb = f % kblocks;
    int64_t c = rb * 16 + lane % 16;
    const uint8_t* src = a.src0;
    int64_t row = c;
    if (a.src1) {
      row = (c / 32) * 16 + c % 16;
      if ((c / 16) % 2) src = a.src1;
    }
    int64_t k0 = kb * a.KE + (lane / 16) * (a.KE / 4);
    int64_t sb = ((e * rows_src + row) * a.K + k0) * a.es + part;
    *reinterpret_cast<uint4*>(a.dst + b) = *reinterpret_cast<const uint4*>(src + sb);
  }
}

hipError_t launch_preshuffle(const PreshuffleArgs& a, hipStream_t st) {
  int64_t n16 = (int64_t)a.R * a.K * a.es * a.E / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(preshuffle_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
