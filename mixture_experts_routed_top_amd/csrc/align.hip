// Grouping of token-slots by expert, padded to the M-tile: a stable counting
// sort (the "dynamic expert sizes" of the routed MoE GEMM in the FlyDSL-in-JAX
// talk summary, 5:56).
//
// One workgroup of 1024 threads. Pass 1 counts slots per expert with LDS
// integer atomics (order free). One thread scans the padded counts. Pass 2
// walks the slots in 1024-slot chunks in ascending order; inside a chunk a
// slot's rank among equal experts comes from a wave ballot (lanes are in
// ascending slot order) plus the counts of the lower waves, so the result is
// exactly the stable order. Integer work only: bit-exact by construction.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(AlignArgs a) {
  __shared__ int cnt[64];
  __shared__ int off[65];
  __shared__ int base[64];
  __shared__ int wcnt[kAlignWaves][64];
  __shared__ int bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, E = a.E, bm = a.bm;

  if (tid < 64) cnt[tid] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int s = tid; s < S; s += kAlignThreads) {
    int e = a.ids[s];
    if (e < 0 || e >= E)
      bad = 1;
    else
      atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (bad) {  // invalid ids: publish an empty grouping so nothing downstream runs
    if (tid == 0) *a.total = 0;
    return;
  }
  if (tid == 0) {
    int pos = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = pos;
      pos += (cnt[e] + bm - 1) / bm * bm;
    }
    off[E] = pos;
    *a.total = pos;
  }
  __syncthreads();
  if (tid < E) {
    a.count[tid] = cnt[tid];
    a.offset[tid] = off[tid];
    base[tid] = off[tid];
  }
  if (tid == 0) a.offset[E] = off[E];

  // Tile experts and pad sentinels.
  const int total = off[E];
  for (int i = tid; i < total / bm; i += kAlignThreads) {
    int e = 0;
    while (off[e + 1] <= i * bm) ++e;
    a.tile_expert[i] = e;
  }
  for (int p = tid; p < total; p += kAlignThreads) {
    int e = 0;
    while (off[e + 1] <= p) ++e;
    if (p - off[e] >= cnt[e]) a.sorted_slot[p] = S;
  }
  __syncthreads();

  // Stable scatter.
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < S; c0 += kAlignThreads) {
    const int s = c0 + tid;
    const int e = s < S ? a.ids[s] : -1;
    int rank = 0;
    for (int ee = 0; ee < E; ++ee) {
      unsigned long long m = __ballot(e == ee);
      if (e == ee) rank = __popcll(m & lt);
      if (lane == 0) wcnt[wave][ee] = __popcll(m);
    }
    __syncthreads();
    if (tid < E) {
      int run = base[tid];
      for (int w = 0; w < kAlignWaves; ++w) {
        int c = wcnt[w][tid];
        wcnt[w][tid] = run;
        run += c;
      }
      base[tid] = run;
    }
    __syncthreads();
    if (e >= 0) a.sorted_slot[wcnt[wave][e] + rank] = s;
    __syncthreads();
  }
}

hipError_t launch_align(const AlignArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
