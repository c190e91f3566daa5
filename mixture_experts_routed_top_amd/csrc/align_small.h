// The one-wave counting sort of small groupings (decode batches), shared by
// the align kernel and the route kernel that groups tiny batches in the same
// launch: the per-expert group sizes that change with every batch in the
// routed MoE GEMM of the FlyDSL-in-JAX talk summary (5:56). Integer work only.
#pragma once
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// Small groupings (S <= kSmallSlots, decode batches): the same counting sort
// on one wave, in registers. Lane l holds slot 64*i + l of each 64-slot chunk
// i; lane e (< E) keeps expert e's count, offset and running base. No LDS and
// no barriers: the cost is a few ballots per chunk and expert, so it grows
// with the chunks (measured: 5.1 us at 32 slots, 6.1 at 128, 8.2 at 256, 36 at
// 2048), while align_runs_kernel takes 6.3-6.8 us from 512 to 2048 slots.
// The ids come from `ids` (global memory, or LDS when the routing of the same
// workgroup left them there); the other arrays are a's.
constexpr int kSmallSlots = 128;
constexpr int kSmallChunks = kSmallSlots / 64;

__device__ __forceinline__ void align_small_wave(const AlignArgs& a, const int32_t* ids, int lane) {
  const int S = a.S, E = a.E, bm = a.bm;
  const int nchunks = (S + 63) / 64;
  int idv[kSmallChunks];
#pragma unroll
  for (int i = 0; i < kSmallChunks; ++i) {
    const int s = i * 64 + lane;  // clamped load, then select: no branches
    const int v = ids[min(s, S - 1)];
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

}  // namespace moe
