// Grouping of token-slots by expert, padded to the M-tile: a stable counting
// sort (the "dynamic expert sizes" of the routed MoE GEMM in the FlyDSL-in-JAX
// talk summary, 5:56). Integer work only: bit-exact by construction. Three
// kernels by size, each one workgroup:
//  - align_small_kernel (S <= 128 slots, decode): one wave, ids in registers,
//    counts and ranks from ballots, offsets from a shuffle scan
//    (align_device.h);
//  - align_runs_kernel (S <= 32768, E <= 16): each thread takes a contiguous
//    run of slots and counts it in packed 16-bit counters; one exclusive scan
//    of those over the 1024 threads gives every slot its stable rank
//    (align_device.h);
//  - align_kernel (the rest): 1024 threads, slot c*1024 + t of each 1024-slot
//    chunk c on thread t. Pass 1 counts slots per expert with wave ballots (one
//    LDS integer atomic per wave and expert). Pass 2 walks the chunks in
//    ascending order: inside a chunk a slot's rank among equal experts is a
//    wave ballot (lanes are in ascending slot order) plus the counts of the
//    lower waves, which one lane per (expert, wave) pair obtains with a 16-lane
//    shuffle scan; so the result is exactly the stable order.
#include "align_device.h"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;  // 16
constexpr int kIdsInRegs = 32;                   // chunks held in registers (S <= 32768)

__global__ __launch_bounds__(kAlignThreads) void align_kernel(AlignArgs a) {
  __shared__ int cnt[64];
  __shared__ int off[65];
  __shared__ int base[64];
  __shared__ int wcnt[kAlignWaves][64];
  __shared__ int bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, E = a.E, bm = a.bm;
  const int nchunks = (S + kAlignThreads - 1) / kAlignThreads;

  int idv[kIdsInRegs];
#pragma unroll
  for (int i = 0; i < kIdsInRegs; ++i) {
    const int s = i * kAlignThreads + tid;  // clamped load, then select: no branches
    const int v = a.ids[min(s, S - 1)];
    idv[i] = s < S ? v : -1;
  }
  auto id_of = [&](int i) {  // id of slot i*1024 + tid (-1 past the end)
    const int s = i * kAlignThreads + tid;
    return s < S ? a.ids[s] : -1;
  };

  if (tid < 64) cnt[tid] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  // Per-wave counts from ballots: one LDS atomic per wave and expert instead
  // of one per slot on a few hot counters.
  int mine = 0;  // this lane's count for expert `lane` (lanes e < E)
  bool anybad = false;
  auto count = [&](int i, int e) {
    anybad |= i * kAlignThreads + tid < S && (e < 0 || e >= E);
    for (int ee = 0; ee < E; ++ee) {
      const int c = __popcll(__ballot(e == ee));
      if (lane == ee) mine += c;
    }
  };
#pragma unroll
  for (int i = 0; i < kIdsInRegs; ++i)
    if (i < nchunks) count(i, idv[i]);
  for (int i = kIdsInRegs; i < nchunks; ++i) count(i, id_of(i));
  if (anybad) bad = 1;
  if (lane < E && mine) atomicAdd(&cnt[lane], mine);
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

  // Stable scatter, one chunk at a time. Destinations are kept in registers
  // and every global store is issued after the chunk loop: on this
  // architecture stores and loads share one completion counter, so a store
  // inside the loop would make later waits wait for it too.
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int se = tid >> 4, sw = tid & 15;  // scan lane: expert se, wave sw
  auto rank_of = [&](int e) {  // destination row of this thread's slot (or -1)
    int rank = 0;
    for (int ee = 0; ee < E; ++ee) {
      const unsigned long long m = __ballot(e == ee);
      if (e == ee) rank = __popcll(m & lt);
      if (lane == 0) wcnt[wave][ee] = __popcll(m);
    }
    __syncthreads();
    // Exclusive scan of the per-wave counts of each expert over the 16 waves
    // (the 16 lanes of one expert sit in one wave), added to the expert's
    // running base; the last wave's lane advances the base.
    if (se < E) {
      const int v = wcnt[sw][se];
      int incl = v;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int o = __shfl_up(incl, d, 16);
        if (sw >= d) incl += o;
      }
      const int b = base[se];
      wcnt[sw][se] = b + incl - v;
      if (sw == 15) base[se] = b + incl;
    }
    __syncthreads();
    const int dst = e >= 0 ? wcnt[wave][e] + rank : -1;
    __syncthreads();
    return dst;
  };
#pragma unroll
  for (int i = 0; i < kIdsInRegs; ++i)  // each id is replaced by its destination row
    if (i < nchunks) idv[i] = rank_of(idv[i]);

  // Tile experts and pad sentinels (fewer than block_m pad rows per expert),
  // then the slots of the chunks.
  for (int e = 0; e < E; ++e) {
    const int o0 = off[e], o1 = off[e + 1];
    for (int i = o0 / bm + tid; i < o1 / bm; i += kAlignThreads) a.tile_expert[i] = e;
    const int p = o0 + cnt[e] + tid;
    if (p < o1) a.sorted_slot[p] = S;
  }
#pragma unroll
  for (int i = 0; i < kIdsInRegs; ++i)
    if (i < nchunks && idv[i] >= 0) a.sorted_slot[idv[i]] = i * kAlignThreads + tid;
  // Batches beyond the register-held chunks (more than 32768 slots).
  for (int i = kIdsInRegs; i < nchunks; ++i) {
    const int d = rank_of(id_of(i));
    if (d >= 0) a.sorted_slot[d] = i * kAlignThreads + tid;
  }
}

// Small groupings: one wave (align_small).
__global__ __launch_bounds__(64) void align_small_kernel(AlignArgs a) {
  align_small(a, threadIdx.x);
}

// Prefill-size groupings with few experts: runs of up to 32 slots on 1024
// threads (align_runs).
constexpr int kRunSlots = 32;
constexpr int kRunMaxSlots = kRunSlots * kAlignThreads;

template <int W>
__global__ __launch_bounds__(kAlignThreads) void align_runs_kernel(AlignArgs a) {
  __shared__ __align__(16) AlignRunsLds<kAlignThreads, kRunSlots> lds;
  align_runs<W, kAlignThreads, kRunSlots>(a, lds);
}

hipError_t launch_align(const AlignArgs& a, hipStream_t st) {
  if (a.S <= kSmallSlots)
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(64), 0, st, a);
  else if (a.S <= kRunMaxSlots && a.E <= 8)
    hipLaunchKernelGGL(align_runs_kernel<4>, dim3(1), dim3(kAlignThreads), 0, st, a);
  else if (a.S <= kRunMaxSlots && a.E <= 16)
    hipLaunchKernelGGL(align_runs_kernel<8>, dim3(1), dim3(kAlignThreads), 0, st, a);
  else
    hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
