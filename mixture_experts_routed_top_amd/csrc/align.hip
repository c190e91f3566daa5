// Grouping of token-slots by expert, padded to the M-tile: a stable counting
// sort (the per-expert group sizes that change with every batch in the routed
// MoE GEMM of the FlyDSL-in-JAX talk summary, 5:56). Integer work only:
// bit-exact by construction. Three
// kernels by size, each one workgroup:
//  - align_small_kernel (S <= 128 slots, decode): one wave, ids in registers,
//    counts and ranks from ballots, offsets from a shuffle scan;
//  - align_runs_kernel (S <= 32768, E <= 16): each thread takes a contiguous
//    run of slots and counts it in packed 16-bit counters; one exclusive scan
//    of those over the 1024 threads gives every slot its stable rank;
//  - align_kernel (the rest): 1024 threads, slot c*1024 + t of each 1024-slot
//    chunk c on thread t. Pass 1 counts slots per expert with wave ballots (one
//    LDS integer atomic per wave and expert). Pass 2 walks the chunks in
//    ascending order: inside a chunk a slot's rank among equal experts is a
//    wave ballot (lanes are in ascending slot order) plus the counts of the
//    lower waves, which one lane per (expert, wave) pair obtains with a 16-lane
//    shuffle scan; so the result is exactly the stable order.
#include "align_small.h"
#include "moe_device.h"
#include "moe_launch.h"

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

// Small groupings (S <= kSmallSlots): one wave, align_small_wave.
__global__ __launch_bounds__(64) void align_small_kernel(AlignArgs a) {
  align_small_wave(a, a.ids, threadIdx.x);
}

// Prefill-size groupings with few experts (S <= kRunSlots * 1024, E <= 16):
// thread t owns a contiguous run of slots, so one block-wide scan replaces the
// per-chunk ballots. The ids go through LDS as bytes (coalesced loads, then
// each thread copies its run into registers); a thread counts its run in
// packed 16-bit counters (expert e in half e%2 of word e/2: counts stay below
// 2^16 since S <= 32768); an exclusive scan of those words over the threads
// gives every thread, for every expert, the number of earlier slots; its
// slots then go to offset[e] + that number + the rank inside its run, in
// ascending order, which is the stable order. The grouping is assembled in
// LDS (over the ids, which are in registers by then) and written out in
// order: one workgroup's scattered 4-byte global stores touched a cache line
// each and were the kernel's largest cost.
constexpr int kRunSlots = 32;                     // slots per thread at most
constexpr int kRunMaxSlots = kRunSlots * kAlignThreads;
constexpr int kRunWords = 8;                      // packed counter words at most (E <= 16)
constexpr int kRunMaxRows = kRunMaxSlots + 16 * 255;  // capacity at E <= 16, block_m <= 256

// W packed counter words: experts 0 .. 2W-1 (4 words for E <= 8, else 8).
template <int W>
__global__ __launch_bounds__(kAlignThreads) void align_runs_kernel(AlignArgs a) {
  // ids as bytes first, then the grouped rows (capacity ints) in the same space
  __shared__ __align__(16) int rows[kRunMaxRows];
  uint8_t* const ids8 = reinterpret_cast<uint8_t*>(rows);
  __shared__ uint32_t wtot[kAlignWaves][W];  // per-wave totals, then wave prefixes
  __shared__ int cnt[2 * W];
  __shared__ int off[2 * W + 1];
  __shared__ int bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, E = a.E, bm = a.bm;
  const int nchunks = (S + kAlignThreads - 1) / kAlignThreads;
  if (tid == 0) bad = 0;
  __syncthreads();
  {
    bool anybad = false;
#pragma unroll
    for (int i = 0; i < kRunSlots; ++i) {
      if (i >= nchunks) break;                // uniform: the chunks present
      const int s = i * kAlignThreads + tid;  // clamped load, then select
      const int v = a.ids[min(s, S - 1)];
      if (s < S) {
        anybad |= v < 0 || v >= E;
        ids8[s] = (uint8_t)v;
      }
    }
    if (anybad) bad = 1;
  }
  __syncthreads();
  if (bad) {  // invalid ids: an empty grouping, nothing downstream runs
    if (tid == 0) *a.total = 0;
    return;
  }
  // This thread's run: slots [r0, r0 + n4) clipped to S, n4 a multiple of 4,
  // copied into registers four ids per word (slots past S read as 0, unused).
  const int n4 = ((nchunks + 3) / 4) * 4;
  const int r0 = tid * n4;
  uint32_t idw[kRunSlots / 4];
#pragma unroll
  for (int q = 0; q < kRunSlots / 4; ++q)
    idw[q] = 4 * q < n4 ? *reinterpret_cast<const uint32_t*>(ids8 + r0 + 4 * q) : 0u;
  auto run_id = [&](int i) { return (int)((idw[i / 4] >> (8 * (i % 4))) & 0xffu); };
  uint32_t cntw[W];
#pragma unroll
  for (int w = 0; w < W; ++w) cntw[w] = 0;
#pragma unroll
  for (int i = 0; i < kRunSlots; ++i) {
    if (i >= n4 || r0 + i >= S) break;
    const int e = run_id(i);
    const uint32_t inc = (e & 1) ? 0x10000u : 1u;
#pragma unroll
    for (int w = 0; w < W; ++w) cntw[w] += (e >> 1) == w ? inc : 0u;
  }
  // Exclusive scan of the packed words over the threads (thread order = slot
  // order): inside each wave with shuffles, then over the 16 wave totals.
  uint32_t excl[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    uint32_t x = cntw[w];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(x, d, 64);
      if (lane >= d) x += o;
    }
    excl[w] = x - cntw[w];
    if (lane == 63) wtot[wave][w] = x;
  }
  __syncthreads();  // also: every run is in registers, so the id bytes may be overwritten
  if (tid < W) {  // wave prefixes in place, and the expert counts from the grand total
    uint32_t acc = 0;
    for (int w = 0; w < kAlignWaves; ++w) {
      const uint32_t t = wtot[w][tid];
      wtot[w][tid] = acc;
      acc += t;
    }
    cnt[2 * tid] = (int)(acc & 0xffffu);
    cnt[2 * tid + 1] = (int)(acc >> 16);
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < W; ++w) excl[w] += wtot[wave][w];
  if (tid == 0) {  // padded offsets
    int pos = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = pos;
      pos += (cnt[e] + bm - 1) / bm * bm;
    }
    off[E] = pos;
    *a.total = pos;
  }
  __syncthreads();
  if (tid < E) a.count[tid] = cnt[tid];
  if (tid <= E) a.offset[tid] = off[tid];
  // Tile experts (global) and pad sentinels (fewer than block_m pad rows per
  // expert, in LDS).
  for (int e = 0; e < E; ++e) {
    const int o0 = off[e], o1 = off[e + 1];
    for (int i = o0 / bm + tid; i < o1 / bm; i += kAlignThreads) a.tile_expert[i] = e;
    const int p = o0 + cnt[e] + tid;
    if (p < o1) rows[p] = S;
  }
  // Stable scatter of this thread's run into LDS.
#pragma unroll
  for (int i = 0; i < kRunSlots; ++i) {
    const int sl = r0 + i;
    if (i >= n4 || sl >= S) break;
    const int e = run_id(i);
    uint32_t word = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) word = (e >> 1) == w ? excl[w] : word;
    const int rank = (int)((e & 1) ? (word >> 16) : (word & 0xffffu));
    rows[off[e] + rank] = sl;
    const uint32_t inc = (e & 1) ? 0x10000u : 1u;
#pragma unroll
    for (int w = 0; w < W; ++w) excl[w] += (e >> 1) == w ? inc : 0u;
  }
  __syncthreads();
  // The grouping in order: consecutive threads write consecutive rows.
  const int total = off[E];
  for (int p = tid; p < total; p += kAlignThreads) a.sorted_slot[p] = rows[p];
}

hipError_t launch_align(const AlignArgs& a, hipStream_t st) {
  if (a.S <= kSmallSlots)
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(64), 0, st, a);
  else if (a.S <= kRunMaxSlots && a.E <= 8)
    hipLaunchKernelGGL(align_runs_kernel<4>, dim3(1), dim3(kAlignThreads), 0, st, a);
  else if (a.S <= kRunMaxSlots && a.E <= 2 * kRunWords)
    hipLaunchKernelGGL(align_runs_kernel<kRunWords>, dim3(1), dim3(kAlignThreads), 0, st, a);
  else
    hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
