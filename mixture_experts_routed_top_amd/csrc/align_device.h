// Device bodies of the grouping of token-slots by expert (the stable counting
// sort padded to the M-tile; the "dynamic expert sizes" of the routed MoE GEMM
// in the FlyDSL-in-JAX talk summary, 5:56). They run either as their own
// one-workgroup kernels (align.hip) or inside the last-arriving workgroup of
// the router launch (route.hip), which reads the ids the other workgroups
// wrote. Integer work only: bit-exact by construction.
#pragma once

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// Small groupings (S <= kSmallSlots, decode batches): the counting sort on one
// wave, in registers. Lane l holds slot 64*i + l of each 64-slot chunk i; lane
// e (< E) keeps expert e's count, offset and running base. No LDS and no
// barriers: the cost is a few ballots per chunk and expert, so it grows with
// the chunks (measured: 5.1 us at 32 slots, 6.1 at 128, 8.2 at 256, 36 at
// 2048 as its own kernel).
constexpr int kSmallSlots = 128;
constexpr int kSmallChunks = kSmallSlots / 64;

__device__ __forceinline__ void align_small(const AlignArgs& a, int lane) {
  const int S = a.S, E = a.E, bm = a.bm;
  const int nchunks = (S + 63) / 64;
  int idv[kSmallChunks];
#pragma unroll
  for (int i = 0; i < kSmallChunks; ++i) {
    const int s = i * 64 + lane;  // clamped load, then select: no branches
    const int v = a.ids[min(s, S - 1)];
    idv[i] = s < S ? v : -1;
  }
  // Counts (lane e: expert e), and a check of every id.
  int cnt = 0;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < kSmallChunks; ++i) {
    if (i >= nchunks) break;
    const int e = idv[i];
    bad |= i * 64 + lane < S && (e < 0 || e >= E);
    for (int ee = 0; ee < E; ++ee) {
      const int c = __popcll(__ballot(e == ee));
      if (lane == ee) cnt += c;
    }
  }
  if (__ballot(bad)) {  // invalid ids: an empty grouping, nothing downstream runs
    if (lane == 0) *a.total = 0;
    return;
  }
  // Padded offsets: exclusive scan of the padded counts over lanes 0..E-1.
  const int padded = lane < E ? (cnt + bm - 1) / bm * bm : 0;
  int incl = padded;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  const int off = incl - padded;
  const int total = __shfl(incl, 63, 64);
  if (lane < E) {
    a.count[lane] = cnt;
    a.offset[lane] = off;
  }
  if (lane == 0) {
    a.offset[E] = total;
    *a.total = total;
  }
  // Tile experts and pad sentinels (fewer than block_m pad rows per expert).
  for (int e = 0; e < E; ++e) {
    const int o0 = __shfl(off, e, 64), o1 = __shfl(incl, e, 64);
    const int c = __shfl(cnt, e, 64);
    for (int i = o0 / bm + lane; i < o1 / bm; i += 64) a.tile_expert[i] = e;
    for (int p = o0 + c + lane; p < o1; p += 64) a.sorted_slot[p] = S;
  }
  // Stable scatter, chunk by chunk: a slot's row is its expert's running base
  // plus the number of lower lanes of the chunk with the same expert.
  const unsigned long long lt = (1ull << lane) - 1ull;
  int base = off;  // lane e: next row of expert e
#pragma unroll
  for (int i = 0; i < kSmallChunks; ++i) {
    if (i >= nchunks) break;
    const int e = idv[i];
    const int b = __shfl(base, e < 0 ? 0 : e, 64);  // the expert's base before this chunk
    int rank = 0;
    for (int ee = 0; ee < E; ++ee) {
      const unsigned long long m = __ballot(e == ee);
      if (e == ee) rank = __popcll(m & lt);
      if (lane == ee) base += __popcll(m);
    }
    if (e >= 0) a.sorted_slot[b + rank] = i * 64 + lane;
  }
}

// Groupings with few experts (S <= NT * RUN, E <= 2W): thread t owns a
// contiguous run of slots, so one block-wide scan replaces per-chunk ballots.
// The ids go through LDS as bytes (coalesced loads, then each thread copies
// its run into registers); a thread counts its run in packed 16-bit counters
// (expert e in half e%2 of word e/2: counts stay below 2^16 since
// S <= 32768); an exclusive scan of those words over the threads gives every
// thread, for every expert, the number of earlier slots; its slots then go to
// offset[e] + that number + the rank inside its run, in ascending order, which
// is the stable order. The grouping is assembled in LDS (over the ids, which
// are in registers by then) and written out in order: one workgroup's
// scattered 4-byte global stores touched a cache line each and were the
// kernel's largest cost.
template <int NT, int RUN>
struct AlignRunsLds {
  static constexpr int kRows = NT * RUN + 16 * 255;  // capacity at E <= 16, block_m <= 256
  int rows[kRows];  // ids as bytes first, then the grouped rows
  uint32_t wtot[NT / 64][8];  // per-wave totals, then wave prefixes
  int cnt[16];
  int off[17];
  int bad;
};

template <int W, int NT, int RUN>
__device__ __forceinline__ void align_runs(const AlignArgs& a, AlignRunsLds<NT, RUN>& L) {
  static_assert(W <= 8 && RUN % 4 == 0 && NT * RUN <= 32768, "run layout");
  constexpr int NW = NT / 64;
  uint8_t* const ids8 = reinterpret_cast<uint8_t*>(L.rows);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, E = a.E, bm = a.bm;
  const int nchunks = (S + NT - 1) / NT;
  if (tid == 0) L.bad = 0;
  __syncthreads();
  {
    bool anybad = false;
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
      if (i >= nchunks) break;      // uniform: the chunks present
      const int s = i * NT + tid;   // clamped load, then select
      const int v = a.ids[min(s, S - 1)];
      if (s < S) {
        anybad |= v < 0 || v >= E;
        ids8[s] = (uint8_t)v;
      }
    }
    if (anybad) L.bad = 1;
  }
  __syncthreads();
  if (L.bad) {  // invalid ids: an empty grouping, nothing downstream runs
    if (tid == 0) *a.total = 0;
    return;
  }
  // This thread's run: slots [r0, r0 + n4) clipped to S, n4 a multiple of 4,
  // copied into registers four ids per word (slots past S read as 0, unused).
  const int n4 = ((nchunks + 3) / 4) * 4;
  const int r0 = tid * n4;
  uint32_t idw[RUN / 4];
#pragma unroll
  for (int q = 0; q < RUN / 4; ++q)
    idw[q] = 4 * q < n4 ? *reinterpret_cast<const uint32_t*>(ids8 + r0 + 4 * q) : 0u;
  auto run_id = [&](int i) { return (int)((idw[i / 4] >> (8 * (i % 4))) & 0xffu); };
  uint32_t cntw[W];
#pragma unroll
  for (int w = 0; w < W; ++w) cntw[w] = 0;
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (i >= n4 || r0 + i >= S) break;
    const int e = run_id(i);
    const uint32_t inc = (e & 1) ? 0x10000u : 1u;
#pragma unroll
    for (int w = 0; w < W; ++w) cntw[w] += (e >> 1) == w ? inc : 0u;
  }
  // Exclusive scan of the packed words over the threads (thread order = slot
  // order): inside each wave with shuffles, then over the wave totals.
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
    if (lane == 63) L.wtot[wave][w] = x;
  }
  __syncthreads();  // also: every run is in registers, so the id bytes may be overwritten
  if (tid < W) {  // wave prefixes in place, and the expert counts from the grand total
    uint32_t acc = 0;
    for (int w = 0; w < NW; ++w) {
      const uint32_t t = L.wtot[w][tid];
      L.wtot[w][tid] = acc;
      acc += t;
    }
    L.cnt[2 * tid] = (int)(acc & 0xffffu);
    L.cnt[2 * tid + 1] = (int)(acc >> 16);
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < W; ++w) excl[w] += L.wtot[wave][w];
  if (tid == 0) {  // padded offsets
    int pos = 0;
    for (int e = 0; e < E; ++e) {
      L.off[e] = pos;
      pos += (L.cnt[e] + bm - 1) / bm * bm;
    }
    L.off[E] = pos;
    *a.total = pos;
  }
  __syncthreads();
  if (tid < E) a.count[tid] = L.cnt[tid];
  if (tid <= E) a.offset[tid] = L.off[tid];
  // Tile experts (global) and pad sentinels (fewer than block_m pad rows per
  // expert, in LDS).
  for (int e = 0; e < E; ++e) {
    const int o0 = L.off[e], o1 = L.off[e + 1];
    for (int i = o0 / bm + tid; i < o1 / bm; i += NT) a.tile_expert[i] = e;
    for (int p = o0 + L.cnt[e] + tid; p < o1; p += NT) L.rows[p] = S;
  }
  // Stable scatter of this thread's run into LDS.
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    const int sl = r0 + i;
    if (i >= n4 || sl >= S) break;
    const int e = run_id(i);
    uint32_t word = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) word = (e >> 1) == w ? excl[w] : word;
    const int rank = (int)((e & 1) ? (word >> 16) : (word & 0xffffu));
    L.rows[L.off[e] + rank] = sl;
    const uint32_t inc = (e & 1) ? 0x10000u : 1u;
#pragma unroll
    for (int w = 0; w < W; ++w) excl[w] += (e >> 1) == w ? inc : 0u;
  }
  __syncthreads();
  // The grouping in order: consecutive threads write consecutive rows.
  const int total = L.off[E];
  for (int p = tid; p < total; p += NT) a.sorted_slot[p] = L.rows[p];
}

}  // namespace moe
