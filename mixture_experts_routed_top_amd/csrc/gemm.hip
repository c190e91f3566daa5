// Grouped expert GEMMs of the routed MoE layer on gfx950 matrix cores: stage 1
// (gather-on-load + gate/up GEMM + SwiGLU) and stage 2 (down GEMM + weighted
// per-slot scatter), plus the FP8 requantisation of the intermediate and the
// fixed-order combine. The fusion of gather, group GEMM, SwiGLU and scatter is
// the routed MoE GEMM of the FlyDSL-in-JAX talk summary (5:56); the tiling
// here is this library's own.
//
// Matrix-core roles. The A operand of v_mfma_f32_32x32x64_f8f6f4 (FP8) or of
// two v_mfma_f32_32x32x16_bf16 (BF16) is a fragment of 32 expert-weight rows
// (output features) by 64 reduction bytes; the B operand is the same shape cut
// from 32 token rows. Lane l supplies row l%32 and the 32 reduction bytes
// starting at (l/32)*32, held as two 16-byte pieces; accumulator register i of
// lane l is then output feature 8*(i/4) + 4*(l/32) + i%4 of token l%32. (The
// instruction itself pairs K differently: lanes r and r+32 together hold its
// first 32 values in their first pieces. Any order shared by both operands
// gives the same sums; the MXFP8 path, whose scales follow the instruction's
// own grouping, stores piece pc of lane l as bytes 32*pc + 16*(l/32).) The
// MXFP4 path (E2M1 weights, two per byte, against MXFP8 tokens) has a
// one-piece weight fragment of 32 rows x 32 bytes: lane l holds row l%32 and
// the 32 values 32*(l/32) .. +31 of the fragment's 64, in order, which pair
// with the token values of the MXFP8 order and take lane l's scale.
//
// Workgroup = 4 waves. Each wave owns NF weight fragments along the features
// (NF*32 rows; for stage 1 gate blocks and the matching up blocks, so the
// SwiGLU pairs sit in the same lane) and all MT token fragments of the tile;
// KSPLIT waves may split the reduction instead of the features (decode
// shapes), and a launch may split the reduction over KG workgroups (stage 2
// decode). Prefill tiles are 128 tokens x 512 features. Weights stream from HBM
// straight into registers, NB-1 pipeline stages ahead (the preshuffle made each
// piece of a fragment one contiguous 1 KB block); tokens are gathered by row
// (sorted_slot) into registers and written to LDS in fragment order, three
// buffers deep, so the matrix-core reads are contiguous 16-byte-per-lane blocks
// with no bank conflicts.
//
// Tile order: XCD-contiguous runs of logical tiles, grouped so that the tiles
// sharing an expert's weights run together (tile_coords). Decode shapes index
// only the live tiles, from the device-side padded total. Stage 2 at prefill
// sizes cuts the tiles of a partial last round of workgroups into reduction
// pieces (tail_plan, tail_reduce_kernel). Stage 1 stages its bf16 output tile
// in LDS and writes whole row segments non-temporally.
#include "moe_device.h"
#include "moe_launch.h"

#include <cmath>

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPiece = 1024;  // one fragment piece: 64 lanes x 16 B
constexpr int kFrag = 2048;   // one fragment: 32 rows x 64 reduction bytes

// One 32x32 step over 64 reduction bytes. ws and xs carry the E8M0 block
// scales of the MXFP8 path (byte OA of ws for the weight operand, byte OB of
// xs for the token operand: lane l's byte scales its 32 values); the other
// element types ignore them. The instruction reads the scale from byte 0 of
// its register whatever its byte-select field says, so the byte is shifted
// down first.
template <int DT>
struct Mma;
template <>
struct Mma<1> {  // e4m3fn x e4m3fn, 32x32x64, unscaled form
  template <int OA, int OB>
  static __device__ __forceinline__ f32x16 run(const uint4 (&w)[2], const uint4 (&x)[2],
                                               f32x16 c, int, int) {
    i32x8 a = {(int)w[0].x, (int)w[0].y, (int)w[0].z, (int)w[0].w,
               (int)w[1].x, (int)w[1].y, (int)w[1].z, (int)w[1].w};
    i32x8 b = {(int)x[0].x, (int)x[0].y, (int)x[0].z, (int)x[0].w,
               (int)x[1].x, (int)x[1].y, (int)x[1].z, (int)x[1].w};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};
template <>
struct Mma<2> {  // e4m3fn x e4m3fn with E8M0 block scales (MXFP8), 32x32x64
  template <int OA, int OB>
  static __device__ __forceinline__ f32x16 run(const uint4 (&w)[2], const uint4 (&x)[2],
                                               f32x16 c, int ws, int xs) {
    i32x8 a = {(int)w[0].x, (int)w[0].y, (int)w[0].z, (int)w[0].w,
               (int)w[1].x, (int)w[1].y, (int)w[1].z, (int)w[1].w};
    i32x8 b = {(int)x[0].x, (int)x[0].y, (int)x[0].z, (int)x[0].w,
               (int)x[1].x, (int)x[1].y, (int)x[1].z, (int)x[1].w};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        a, b, c, 0, 0, 0, (int)((uint32_t)ws >> (8 * OA)), 0, (int)((uint32_t)xs >> (8 * OB)));
  }
};
template <>
struct Mma<3> {  // E2M1 weights x e4m3fn tokens with E8M0 block scales (MXFP4), 32x32x64
  template <int OA, int OB>
  static __device__ __forceinline__ f32x16 run(const uint4 (&w)[1], const uint4 (&x)[2],
                                               f32x16 c, int ws, int xs) {
    // The E2M1 operand occupies the first four registers; the rest are unread.
    i32x8 a = {(int)w[0].x, (int)w[0].y, (int)w[0].z, (int)w[0].w, 0, 0, 0, 0};
    i32x8 b = {(int)x[0].x, (int)x[0].y, (int)x[0].z, (int)x[0].w,
               (int)x[1].x, (int)x[1].y, (int)x[1].z, (int)x[1].w};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        a, b, c, 4, 0, 0, (int)((uint32_t)ws >> (8 * OA)), 0, (int)((uint32_t)xs >> (8 * OB)));
  }
};
template <>
struct Mma<0> {  // bf16: one 32x32x16 per piece
  template <int OA, int OB>
  static __device__ __forceinline__ f32x16 run(const uint4 (&w)[2], const uint4 (&x)[2],
                                               f32x16 c, int, int) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[0]),
                                                __builtin_bit_cast(bf16x8, x[0]), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[1]),
                                                   __builtin_bit_cast(bf16x8, x[1]), c, 0, 0, 0);
  }
};

template <int V>
struct IntC {
  static constexpr int value = V;
};

// f(IntC<0>), ..., f(IntC<N-1>), unrolled at compile time.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<N, I + 1>(f);
  }
}

// Buffer offset of a pad row: past the end of any activation buffer (those are
// limited to 2 GiB), so a raw buffer load from it returns zeros.
constexpr uint32_t kPadOffset = 0x80000000u;

// LDS slot swizzle of the token tile. The 16-byte column c (0..3) of a row's
// 64-byte window goes to piece c&1, slot s = row + 32*(c>>1) (MXFP8: piece
// c>>1, slot row + 32*(c&1)), stored at slot s ^ lds_swz(c). The four columns
// of a row (written by four adjacent lanes) then land in different bank
// groups, for both 8- and 16-lane LDS passes: over 2 rows x 4 columns the
// slots differ mod 8, over 4 rows x 4 columns mod 16 (a piece is 64 slots, so
// the piece does not change a slot's bank group). Readers apply the same
// permutation (it keeps bit 5 of the slot, so it is a bijection inside each
// piece).
__device__ __forceinline__ int lds_swz(int c) { return 4 * (c & 1) + 10 * (c >> 1); }


template <int MT, int KSPLIT, int CK>
constexpr int gemm_lds_bytes() {
  return 3 * KSPLIT * (CK / 64) * MT * kFrag;  // three token buffers
}

// Logical tile -> (row tile, feature tile): groups of group_m row tiles sweep
// the feature tiles, so that co-resident workgroups of one XCD share weight
// slabs and token rows in its L2. n_m row tiles in all.
__device__ __forceinline__ void tile_coords(int logical, int n_m, int group_m, int n_ntiles,
                                            int& mtile, int& ntile) {
  const int per_group = group_m * n_ntiles;
  const int grp = logical / per_group, rem = logical % per_group;
  const int gm = min(group_m, n_m - grp * group_m);
  mtile = grp * group_m + rem % gm;
  ntile = rem / gm;
}

// Plan of a stage-2 launch over n_live tiles with `round` workgroups per
// round: the last, partial round's `tail` tiles are cut into `split` pieces
// along the reduction (at most max_split, at most kTailPieces pieces, at most
// one piece per chunk) when that gives at least two per tile; the first
// n_full tiles run whole.
struct TailPlan {
  int n_full, tail, split;
};
__device__ __forceinline__ TailPlan tail_plan(int n_live, int round, int max_split,
                                              int nchunks) {
  TailPlan p{n_live, 0, 1};
  const int t = round > 0 ? n_live % round : 0;
  if (max_split < 2 || t == 0) return p;
  int s = min(min(max_split, round / t), min(kTailPieces / t, nchunks));
  if (s < 2) return p;
  p.n_full = n_live - t;
  p.tail = t;
  p.split = s;
  return p;
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp; the
// product is rounded to bf16 or requantised right after).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// The E2M1 decode tile of stage 1 (one token fragment, four weight fragments
// per wave) is held to the 256 registers that two waves per SIMD leave each.
template <int DT, int STAGE, int MT, int NF, int KSPLIT, int NB, int CK>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(DT == 3 && MT == 1 && NF == 4 ? 2 : 1, 8)))
void gemm_kernel(GemmArgs a) {
  constexpr int kSub = CK / 64;          // fragments along the reduction per stage
  constexpr int kChunk = CK;             // reduction bytes per pipeline stage
  constexpr int WN = 4 / KSPLIT;         // waves along the features
  constexpr int WGN = WN * NF * 32;      // composite rows (features) per workgroup
  constexpr int BMT = 32 * MT;           // token rows per tile
  constexpr int PPT = KSPLIT * kSub * MT / 2;  // 16-byte token pieces per thread per stage
  constexpr int LDS = gemm_lds_bytes<MT, KSPLIT, CK>();
  constexpr int BUF = LDS / 3;           // one token buffer
  constexpr int NSTEP = kSub * MT;       // token fragments per wave per stage
  static_assert(NSTEP % 2 == 0, "the stage barrier sits between two halves");
  static_assert(PPT >= 1 && KSPLIT * kSub * MT % 2 == 0, "staging layout");
  constexpr int NACC = MT * NF * 16;     // accumulator floats per lane
  static_assert(NF == 2 || NF == 4, "weight fragments per wave (gate/up pairs)");
  static_assert(KSPLIT == 1 || (KSPLIT - 1) * WN * NACC * 64 * 4 <= LDS, "reduction space");
  static_assert(WN * BMT * 4 <= LDS, "amax space");
  static_assert(NB >= 2 && NB <= 4, "weight pipeline depth");

  // MXFP8 and MXFP4 (block-scaled tokens): the E8M0 codes of the tile's
  // token rows over this workgroup's reduction range sit after the token
  // buffers for the main loop, laid out [column][token][fragment] (a column
  // covers 32 reduction values), so that one LDS read gives a lane the codes
  // of all MT fragments in one column.
  constexpr bool MX = DT == 2 || DT == 3;
  // Weight fragment: two 1 KB pieces, or one for E2M1 (32 rows x 32 bytes).
  constexpr int WP = DT == 3 ? 1 : 2;
  constexpr int WFRAG = WP * kPiece;
  constexpr int XCOLS = MX ? (STAGE == 1 ? kMxMaxH : kMxMaxI) / 32 + 16 : 0;
  constexpr int XST = XCOLS * BMT;
  // Token buffers (reused by the epilogue), then the column scales of this
  // workgroup's features (FP8), staged once so that the epilogue reads LDS.
  constexpr int SCL = DT == 1 ? WGN : 0;
  // Stage 1 stages its bf16 output tile here after the main loop (rows of
  // WGN/2 columns, padded by 8 bytes so that the 32 rows one write covers
  // fall in different banks), reusing the token buffers, and keeps the row
  // maxima of the FP8 epilogue past it.
  constexpr int SP = WGN + 8;                               // staging row pitch, bytes
  constexpr int STG = STAGE == 1 ? BMT * SP : 0;
  constexpr int MAIN = LDS + XST;  // main loop: token buffers and the MXFP8 code tile
  constexpr int LDSX = (MAIN > STG ? MAIN : STG) + (STAGE == 1 && DT == 1 ? WN * BMT * 4 : 0);
  __shared__ __align__(16) uint8_t lds[LDSX + SCL * 4];
  float* const scl = reinterpret_cast<float*>(lds + LDSX);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wk = wave / WN;

  const int S = a.T * a.k;
  const int Kb = a.K_bytes;                    // reduction bytes of a full row
  const int Kw = Kb / (KSPLIT * a.kg);         // reduction bytes per wave
  int nchunks = Kw / kChunk;

  // Tile order: XCD-contiguous runs of logical tiles (xcd_remap), grouped as
  // tile_coords describes.
  int kg = 0, mtile, ntile, total, e_raw;
  int piece = -1, tail_idx = 0, n_tail = 0;  // stage-2 tail piece of this workgroup
  int cbegin = 0;                            // first reduction chunk
  if (a.tail_split == 0 && !a.live_order) {
    const int logical = xcd_remap(blockIdx.x, a.n_mtiles * a.n_ntiles * a.kg);
    kg = logical % a.kg;
    tile_coords(logical / a.kg, a.n_mtiles, a.group_m, a.n_ntiles, mtile, ntile);
    // The grouping's size and this tile's expert are read together (the
    // expert index is in bounds for any tile of the launch), then the tile
    // exits if it lies past the padded total.
    total = *a.total_padded;
    e_raw = a.tile_expert[mtile * BMT / a.bm];
    if (mtile * BMT >= total) return;
  } else {
    // Live tiles only, first in launch order (the padded total is a multiple
    // of the tile rows). With few live row tiles (decode), a launch over the
    // capacity would interleave them with exiting workgroups in a fixed
    // pattern that the hardware's round-robin placement maps onto a subset of
    // the CUs. Stage 2 also cuts the partial last round's tiles into pieces
    // along the reduction (kg is 1 then).
    total = *a.total_padded;
    const int n_m = total / BMT;
    const TailPlan pl = tail_plan(n_m * a.n_ntiles * a.kg, a.round, a.tail_split, nchunks);
    const int b = blockIdx.x;
    int logical;
    if (b < pl.n_full) {
      logical = xcd_remap(b, pl.n_full);
    } else {
      const int pi = b - pl.n_full;
      if (pi >= pl.tail * pl.split) return;
      tail_idx = pi % pl.tail;
      piece = pi / pl.tail;
      n_tail = pl.tail;
      logical = pl.n_full + tail_idx;
      cbegin = piece * nchunks / pl.split;
      nchunks = (piece + 1) * nchunks / pl.split - cbegin;
    }
    kg = logical % a.kg;
    tile_coords(logical / a.kg, n_m, a.group_m, a.n_ntiles, mtile, ntile);
    e_raw = a.tile_expert[mtile * BMT / a.bm];
  }
  const int row0 = mtile * BMT;
  const int e = e_raw;
  const int kbase = (kg * KSPLIT) * Kw + cbegin * kChunk;  // first reduction byte of this workgroup

  // Token pieces this thread stages each stage. Piece q (thread tid, slot j):
  // 16-byte column c = q%4 of the 64-byte window, row r = (q/4)%32 of fragment
  // m = (q/128)%MT, reduction sub-block s = (q/(128*MT))%kSub, wave split ks.
  // Rows are read through a raw buffer descriptor: a pad row gets an offset
  // past the end of the buffer, which the hardware returns as zeros, so the
  // load needs no branch.
  const __amdgpu_buffer_rsrc_t xrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.X, (short)0, (int)a.x_bytes, 0x00020000);
  uint32_t xoff[PPT];
  int loff[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int q = tid + 256 * j;
    const int c = q & 3, r = (q >> 2) & 31, m = (q >> 7) % MT;
    const int s = (q / (128 * MT)) % kSub, ks = q / (128 * MT * kSub);
    const int p = row0 + m * 32 + r;
    // Stage 1 gathers token rows; stage 2 reads intermediate rows in place.
    // Pad rows (sentinel slot) are not read at all.
    const int slot = a.sorted_slot[p];
    const uint32_t row = STAGE == 1 ? div_k(min(slot, S - 1), a.k_magic) : (uint32_t)p;
    const uint32_t rowbase = slot < S ? row * (uint32_t)Kb : kPadOffset;  // select, no branch
    xoff[j] = rowbase + (uint32_t)(kbase + ks * Kw + s * 64 + c * 16);
    // Column c goes to piece c&1 of lane half c>>1 (MXFP8: piece c>>1 of lane
    // half c&1, so that each piece is one 32-value scale block).
    const int pce = MX ? (c >> 1) : (c & 1), hlf = MX ? (c & 1) : (c >> 1);
    loff[j] = ((ks * kSub + s) * MT + m) * kFrag + pce * kPiece +
              ((r + 32 * hlf) ^ lds_swz(c)) * 16;
  }

  // This wave's weight fragments: composite row blocks rb0 .. rb0+NF-1;
  // reduction blocks from this wave's split on.
  const int64_t RB = a.N / 32, KB = Kb / 64;
  const int rb0 = ntile * (WGN / 32) + wn * NF;
  const uint8_t* wbase = a.W + (((int64_t)e * RB + rb0) * KB + (kbase + wk * Kw) / 64) * WFRAG +
                         lane * 16;
  const int64_t wfrag_stride = KB * WFRAG;  // next row block
  // MXFP8 weight codes of this wave's row blocks: per fragment one 32-bit
  // (NF = 4) or 16-bit (NF = 2) word per lane whose byte f belongs to row
  // block rb0 + f (rb0 is a multiple of NF).
  const uint8_t* wsp = nullptr;
  if constexpr (MX)
    wsp = a.w_mx + (((int64_t)e * (RB / 4) + rb0 / 4) * KB + (kbase + wk * Kw) / 64) * 256 +
          lane * 4 + (rb0 & 3);

  f32x16 acc[MT][NF];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][f][i] = 0.0f;

  uint4 xr[2][PPT];             // token prefetch, by chunk parity
  uint4 wbuf[NB][kSub][NF][WP];  // weight prefetch: [stage][sub-block][fragment][piece]
  uint32_t wsr[NB][kSub];       // MXFP8 weight codes, staged like the weights
  uint32_t xsr[2][kSub];        // MXFP8 token codes, by chunk parity

  auto load_x = [&](int c, uint4 (&x)[PPT]) {
#pragma unroll
    for (int j = 0; j < PPT; ++j)
      x[j] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, xoff[j] + (uint32_t)c * kChunk, 0, 0));
  };
  auto store_x = [&](int buf, const uint4 (&x)[PPT]) {
#pragma unroll
    for (int j = 0; j < PPT; ++j)
      *reinterpret_cast<uint4*>(lds + buf * BUF + loff[j]) = x[j];
  };
  auto load_w1 = [&](int c, int s, int f, int pc, uint4& w) {
    w = *reinterpret_cast<const uint4*>(wbase + f * wfrag_stride +
                                        ((int64_t)c * kSub + s) * WFRAG + pc * kPiece);
  };
  auto load_ws = [&](int c, int sb, uint32_t& r) {
    const uint8_t* p = wsp + ((int64_t)c * kSub + sb) * 256;
    if constexpr (NF == 4)
      r = *reinterpret_cast<const uint32_t*>(p);
    else
      r = *reinterpret_cast<const uint16_t*>(p);
  };
  auto load_w = [&](int c, uint4 (&w)[kSub][NF][WP]) {
#pragma unroll
    for (int s = 0; s < kSub; ++s)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int pc = 0; pc < WP; ++pc) load_w1(c, s, f, pc, w[s][f][pc]);
  };
  // Column whose bytes this lane's piece 0 / piece 1 holds, and their slots.
  const int rc0 = MX ? (lane >> 5) : 2 * (lane >> 5), rc1 = MX ? 2 + (lane >> 5) : 1 + 2 * (lane >> 5);
  const int rd0 = (lane ^ lds_swz(rc0)) * 16;           // piece 0 slot of this lane
  const int rd1 = kPiece + (lane ^ lds_swz(rc1)) * 16;  // piece 1
  auto read_frag = [&](int buf, int t, uint4 (&x)[2]) {
    const uint8_t* pp = lds + buf * BUF + (wk * NSTEP + t) * kFrag;
    x[0] = *reinterpret_cast<const uint4*>(pp + rd0);
    x[1] = *reinterpret_cast<const uint4*>(pp + rd1);
  };
  // MXFP8 token codes of chunk c: per sub-block one word whose byte m is the
  // code of fragment m's row (this lane's token) in this lane's column.
  int xs_lane = 0;  // byte offset of this lane's column of chunk 0 in the code tile
  auto read_xs = [&](int c, uint32_t (&r)[kSub]) {
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb) {
      const uint8_t* p = lds + LDS + xs_lane + (c * (kChunk / 32) + 2 * sb) * BMT;
      if constexpr (MT == 4)
        r[sb] = *reinterpret_cast<const uint32_t*>(p);
      else if constexpr (MT == 2)
        r[sb] = *reinterpret_cast<const uint16_t*>(p);
      else
        r[sb] = *p;
    }
  };

  // One pipeline stage for chunk c (u = c mod the unroll period). Its token
  // fragments sit in LDS buffer c%3, fragment 0 already in registers. In
  // order: the MFMAs of each fragment, each preceded by the LDS read of the
  // next one (the last step reads fragment 0 of chunk c+1 from buffer
  // (c+1)%3); the global prefetches (tokens of chunk c+3, weights of chunk
  // c+NB-1; indices clamped at the last chunk, so there are no branches and
  // the load counters stay exact) spread one by one between the MFMAs; and,
  // halfway, the workgroup barrier followed by the LDS write of the tokens of
  // chunk c+2 into buffer (c+2)%3. The barrier sits behind queued MFMAs and
  // orders: every wave's reads of buffer (c+2)%3 (chunk c-1) before its
  // overwrite, and every wave's writes of buffer (c+1)%3 (made in stage c-1)
  // before the first read of chunk c+1.
  uint4 xf[2][2];
  auto step = [&](int c, auto u_const) {
    constexpr int u = decltype(u_const)::value;
    constexpr int NWL = PPT + kSub * NF * WP;  // token and weight loads
    constexpr int NLOAD = NWL + (MX ? kSub : 0);
    constexpr int NM = NSTEP * NF;
    const int last = nchunks - 1;
    const int cx = min(c + 3, last), cw = min(c + NB - 1, last);
    auto issue = [&](auto j_const) {
      constexpr int j = decltype(j_const)::value;
      if constexpr (j < PPT) {
        xr[(u + 1) & 1][j] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, xoff[j] + (uint32_t)cx * kChunk,
                                                         0, 0));
      } else if constexpr (j < NWL) {
        constexpr int q = j - PPT, s = q / (NF * WP), f = (q / WP) % NF, pc = q % WP;
        load_w1(cw, s, f, pc, wbuf[(u + NB - 1) % NB][s][f][pc]);
      } else {
        load_ws(cw, j - NWL, wsr[(u + NB - 1) % NB][j - NWL]);
      }
    };
    static_for<NSTEP>([&](auto t_const) {
      constexpr int t = decltype(t_const)::value;
      if constexpr (t + 1 < NSTEP)
        read_frag(u % 3, t + 1, xf[(t + 1) & 1]);
      else
        read_frag((u + 1) % 3, 0, xf[(t + 1) & 1]);
      if constexpr (MX && t == 0) read_xs(min(c + 1, last), xsr[(u + 1) & 1]);
      constexpr int s = t / MT, m = t % MT;
      static_for<NF>([&](auto f_const) {
        constexpr int f = decltype(f_const)::value;
        acc[m][f] = Mma<DT>::template run<f, m>(wbuf[u % NB][s][f], xf[t & 1], acc[m][f],
                                                (int)wsr[u % NB][s], (int)xsr[u & 1][s]);
        constexpr int mi = t * NF + f;
        static_for<NLOAD>([&](auto j_const) {
          constexpr int j = decltype(j_const)::value;
          if constexpr (j * NM / NLOAD == mi) issue(j_const);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      if constexpr (t == NSTEP / 2 - 1) {
        __syncthreads();
        store_x((u + 2) % 3, xr[u & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };

  // Epilogue inputs, fetched now so that their latency hides behind the main
  // loop: per output row of this lane (token tok of each fragment m) its
  // scale factor, and the workgroup's column scales into LDS. The loads are
  // unconditional (pad rows read a clamped index and are masked in the
  // epilogue), so nothing here waits for memory.
  const int tok = lane & 31, fq = (lane >> 5) * 4;
  float rsc[MT];   // stage 1: token scale; stage 2: routing weight x row scale
  int rslot[MT];   // slot of the row (S for pad rows)
#pragma unroll
  for (int m = 0; m < MT; ++m) rslot[m] = a.sorted_slot[row0 + m * 32 + tok];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int sc = min(rslot[m], S - 1);
    if constexpr (STAGE == 1)
      rsc[m] = DT == 1 ? a.x_scale[div_k(sc, a.k_magic)] : 1.0f;
    else
      rsc[m] = (a.unit_w ? 1.0f : a.topk_w[sc]) *
               (DT == 1 ? a.x_scale[row0 + m * 32 + tok] : 1.0f);
  }
  // Column scales of this workgroup's features (FP8): loaded after the
  // pipeline's first loads, kept in registers through the main loop and
  // written to LDS after it, so no wait is spent on them.
  constexpr int NSC = DT == 1 ? (WGN + 255) / 256 : 1;
  float colsc[NSC];
  auto load_colsc = [&]() {
#pragma unroll
    for (int u = 0; u < NSC; ++u) {
      const int i = min(tid + 256 * u, WGN - 1);
      if constexpr (STAGE == 1) {
        const int half = WGN / 2;  // intermediate columns of this workgroup
        colsc[u] = a.w_scale[(size_t)e * 2 * a.I + (i / half) * a.I + ntile * half + i % half];
      } else {
        colsc[u] = a.w_scale[(size_t)e * a.N + ntile * WGN + i];
      }
    }
  };

  // Prologue: weights of chunks 0..NB-2; tokens of chunks 0 and 1 in LDS
  // buffers 0 and 1, chunk 2 in registers; fragment 0 of chunk 0 read.
  {
    const int last = nchunks - 1;
#pragma unroll
    for (int u = 0; u < NB - 1; ++u) {
      load_w(min(u, last), wbuf[u]);
      if constexpr (MX)
#pragma unroll
        for (int sb = 0; sb < kSub; ++sb) load_ws(min(u, last), sb, wsr[u][sb]);
    }
    load_x(0, xr[0]);
    load_x(min(1, last), xr[1]);
    if constexpr (DT == 1) load_colsc();
    if constexpr (MX) {
      // The code tile: row r of the tile (fragment r/32, token r%32), columns
      // gstart .. cend of the E8M0 codes of its X row (this workgroup's
      // reduction range, gstart rounded down to a multiple of 8), in 8-byte
      // loads. Pad rows read past the buffer, as zeros (their values are zero
      // too).
      const int col0 = kbase >> 5, gstart = col0 & ~7;
      const int cend = (kbase + (KSPLIT - 1) * Kw + nchunks * kChunk) >> 5;
      const int ng = (cend - gstart + 7) >> 3;
      const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)a.x_mx, (short)0, (int)(a.x_bytes >> 5), 0x00020000);
      auto code_base = [&](int r) {  // buffer offset of tile row r's first code
        const int slot = a.sorted_slot[row0 + r];
        const uint32_t srow =
            STAGE == 1 ? div_k(min(slot, S - 1), a.k_magic) : (uint32_t)(row0 + r);
        return slot < S ? srow * (uint32_t)(Kb >> 5) + (uint32_t)gstart : kPadOffset;
      };
      if constexpr (MT == 4) {
        // Thread: token t's four rows (t + 32f, fragment f) over 8 columns at a
        // time; a 4x4 byte transpose in registers makes each column's word
        // (fragment f in byte f), stored with one 32-bit LDS write.
        const int t = tid & 31;
        uint32_t sb[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) sb[f] = code_base(32 * f + t);
        uint32_t* dstw = reinterpret_cast<uint32_t*>(lds + LDS) + t;  // column c: word c*32 + t
        constexpr int BATCH = 4;  // column groups per thread in flight
        for (int g0 = tid >> 5; g0 < ng; g0 += 8 * BATCH) {
          uint2 v[BATCH][4];
#pragma unroll
          for (int j = 0; j < BATCH; ++j)
#pragma unroll
            for (int f = 0; f < 4; ++f)
              v[j][f] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                      srsrc, sb[f] + 8u * (uint32_t)(g0 + 8 * j), 0, 0));
#pragma unroll
          for (int j = 0; j < BATCH; ++j) {
            const int g = g0 + 8 * j;
            if (g < ng) {
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const int sh = 8 * (i & 3);
                uint32_t w = 0;
#pragma unroll
                for (int f = 0; f < 4; ++f)
                  w |= (((i < 4 ? v[j][f].x : v[j][f].y) >> sh) & 0xffu) << (8 * f);
                dstw[(8 * g + i) * 32] = w;
              }
            }
          }
        }
      } else {
        const int r = tid % BMT;
        const uint32_t sbase = code_base(r);
        uint8_t* dst = lds + LDS + (r & 31) * MT + (r >> 5);
        constexpr int GS = 256 / BMT, BATCH = 8;
        for (int g0 = tid / BMT; g0 < ng; g0 += GS * BATCH) {
          uint2 v[BATCH];
#pragma unroll
          for (int j = 0; j < BATCH; ++j)
            v[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                 srsrc, sbase + 8u * (uint32_t)(g0 + GS * j), 0, 0));
#pragma unroll
          for (int j = 0; j < BATCH; ++j) {
            const int g = g0 + GS * j;
            if (g < ng) {
#pragma unroll
              for (int i = 0; i < 8; ++i)
                dst[(8 * g + i) * BMT] = (uint8_t)((i < 4 ? v[j].x : v[j].y) >> (8 * (i & 3)));
            }
          }
        }
      }
      xs_lane = (col0 - gstart + wk * (Kw >> 5) + (lane >> 5)) * BMT + (lane & 31) * MT;
    }
    store_x(0, xr[0]);
    store_x(1, xr[1]);
    load_x(min(2, last), xr[0]);
    __syncthreads();
    read_frag(0, 0, xf[0]);
    if constexpr (MX) read_xs(0, xsr[0]);
  }

  // Steady state, unrolled by the period P = lcm(2, 3, NB) (token registers
  // alternate by 2, LDS buffers cycle by 3, weight stages by NB) so that every
  // buffer index is static; then at most P-1 guarded tail stages.
  constexpr int P = NB == 4 ? 12 : 6;
  int c0 = 0;
  for (; c0 + P <= nchunks; c0 += P) static_for<P>([&](auto u) { step(c0 + decltype(u)::value, u); });
  static_for<P - 1>([&](auto u) {
    if (c0 + decltype(u)::value < nchunks) step(c0 + decltype(u)::value, u);
  });
  if constexpr (DT == 1) {
#pragma unroll
    for (int u = 0; u < NSC; ++u)
      if (WGN % 256 == 0 || tid + 256 * u < WGN) scl[tid + 256 * u] = colsc[u];
  }
  __syncthreads();  // all LDS reads done before the epilogue reuses the space; scales visible

  if constexpr (KSPLIT > 1) {
    // Fixed-order reduction of the wave splits: split 0 + split 1 + split 2 + ...
    float* red = reinterpret_cast<float*>(lds);
    if (wk > 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            red[(((wk - 1) * WN + wn) * NACC + (m * NF + f) * 16 + i) * 64 + lane] = acc[m][f][i];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int sp = 1; sp < KSPLIT; ++sp)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              acc[m][f][i] += red[(((sp - 1) * WN + wn) * NACC + (m * NF + f) * 16 + i) * 64 + lane];
    }
    __syncthreads();  // the amax step below reuses the same LDS
  }

  if constexpr (STAGE == 1 && DT == 0) {
    if (a.epi == 1) {
      // Backward recompute: the gate and up pre-activations in bf16, g to
      // columns i, u to columns I + i of the row (pad rows are not written).
      if (wk != 0) return;
      uint16_t* gu = reinterpret_cast<uint16_t*>(a.out);
      const int ib0 = rb0 / 2;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (rslot[m] >= S) continue;
        uint16_t* row = gu + (size_t)(row0 + m * 32 + tok) * 2 * a.I;
#pragma unroll
        for (int qg = 0; qg < NF / 2 * 4; ++qg) {
          const int q = qg / 4, g = qg % 4;
          const int i0 = (ib0 + q) * 32 + 8 * g + fq;
          const f32x16& ga = acc[m][2 * q];
          const f32x16& ua = acc[m][2 * q + 1];
          *reinterpret_cast<uint2*>(row + i0) =
              make_uint2(f32x2_to_bf16x2(ga[4 * g], ga[4 * g + 1]),
                         f32x2_to_bf16x2(ga[4 * g + 2], ga[4 * g + 3]));
          *reinterpret_cast<uint2*>(row + a.I + i0) =
              make_uint2(f32x2_to_bf16x2(ua[4 * g], ua[4 * g + 1]),
                         f32x2_to_bf16x2(ua[4 * g + 2], ua[4 * g + 3]));
        }
      }
      return;
    }
    if (a.epi == 2) {
      // Backward of the SwiGLU: acc holds z = W2^T dout of the row's token
      // (features i of fragment f: (rb0 + f) * 32 + ...). With the row's
      // routing weight w, the forward's a = act and the recomputed g, u:
      //   <z, a> over these columns -> dwpart (the routing weight's gradient),
      //   da = w z, dg = da u s (1 + g (1 - s)), du = da g s, s = sigmoid(g).
      float* wsum = reinterpret_cast<float*>(lds);  // [WN][BMT] partial dot products
      uint16_t* dgu = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int slot = rslot[m];
        float dsum = 0.0f;
        if (wk == 0 && slot < S) {
          const size_t p = (size_t)(row0 + m * 32 + tok);
          const float w = a.topk_w[slot];
          const uint16_t* arow = a.act_in + p * a.I;
          const uint16_t* grow = a.gu + p * 2 * a.I;
          uint16_t* drow = dgu + p * 2 * a.I;
          // All of the fragment's a, g, u loads go out before its first store:
          // interleaved with the dg, du stores (which the compiler cannot
          // prove apart from them) they waited one round trip each (bf16
          // Mixtral backward, T=8192: 13.0 -> 12.75 ms; staging these rows
          // through LDS for whole-row accesses instead was no faster).
          uint2 av4[NF][4], gv4[NF][4], uv4[NF][4];
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int i0 = (rb0 + f) * 32 + 8 * g + fq;
              av4[f][g] = *reinterpret_cast<const uint2*>(arow + i0);
              gv4[f][g] = *reinterpret_cast<const uint2*>(grow + i0);
              uv4[f][g] = *reinterpret_cast<const uint2*>(grow + a.I + i0);
            }
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int i0 = (rb0 + f) * 32 + 8 * g + fq;
              const uint2 av = av4[f][g], gv = gv4[f][g], uv = uv4[f][g];
              const uint32_t aw[2] = {av.x, av.y}, gw[2] = {gv.x, gv.y}, uw[2] = {uv.x, uv.y};
              float dg[4], du[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int sh = 16 * (r & 1);
                const float z = acc[m][f][4 * g + r];
                const float av_r = bf16_bits_to_f32((aw[r >> 1] >> sh) & 0xffffu);
                const float gg = bf16_bits_to_f32((gw[r >> 1] >> sh) & 0xffffu);
                const float uu = bf16_bits_to_f32((uw[r >> 1] >> sh) & 0xffffu);
                dsum = fmaf(z, av_r, dsum);
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gg));
                const float da = w * z;
                dg[r] = da * uu * sg * (1.0f + gg * (1.0f - sg));
                du[r] = da * gg * sg;
              }
              *reinterpret_cast<uint2*>(drow + i0) =
                  make_uint2(f32x2_to_bf16x2(dg[0], dg[1]), f32x2_to_bf16x2(dg[2], dg[3]));
              *reinterpret_cast<uint2*>(drow + a.I + i0) =
                  make_uint2(f32x2_to_bf16x2(du[0], du[1]), f32x2_to_bf16x2(du[2], du[3]));
            }
        }
        // lane halves hold the same row, then the waves along the features
        dsum = dsum + __shfl_xor(dsum, 32, 64);
        if (wk == 0 && lane < 32) wsum[wn * BMT + m * 32 + lane] = dsum;
      }
      __syncthreads();
      for (int r = tid; r < BMT; r += 256) {
        const int slot = a.sorted_slot[row0 + r];
        if (slot >= S) continue;
        float v = wsum[r];
#pragma unroll
        for (int w = 1; w < WN; ++w) v = v + wsum[w * BMT + r];
        a.dwpart[(size_t)slot * a.n_ntiles + ntile] = v;
      }
      return;
    }
  }
  if constexpr (STAGE == 1) {
    // SwiGLU epilogue: fragment 2q is gate block ib0+q, fragment 2q+1 the
    // matching up block.
    uint16_t* act = reinterpret_cast<uint16_t*>(a.out);
    const int ib0 = rb0 / 2;
    const int col0 = ntile * (WGN / 2);  // first intermediate column of this workgroup
    float amax[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      amax[m] = 0.0f;
      if (wk != 0) continue;
      const float xs = rslot[m] < S ? rsc[m] : 0.0f;  // pad rows: act = 0
#pragma unroll
      for (int qg = 0; qg < NF / 2 * 4; ++qg) {
        const int q = qg / 4, g = qg % 4;
        const int i0 = (ib0 + q) * 32 + 8 * g + fq;
        float gs[4] = {xs, xs, xs, xs}, us[4] = {xs, xs, xs, xs};
        if constexpr (DT == 1) {
          const float4 g4 = *reinterpret_cast<const float4*>(scl + (i0 - col0));
          const float4 u4 = *reinterpret_cast<const float4*>(scl + WGN / 2 + (i0 - col0));
          gs[0] *= g4.x; gs[1] *= g4.y; gs[2] *= g4.z; gs[3] *= g4.w;
          us[0] *= u4.x; us[1] *= u4.y; us[2] *= u4.z; us[3] *= u4.w;
        }
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = acc[m][2 * q][4 * g + r] * gs[r];
          const float uv = acc[m][2 * q + 1][4 * g + r] * us[r];
          h[r] = silu(gv) * uv;
        }
        if constexpr (DT == 0) {
          // Training forward: the pre-activations for the backward, stored as
          // the backward's recompute (epi 1) stores them.
          if (a.gu_out && rslot[m] < S) {
            const f32x16& ga = acc[m][2 * q];
            const f32x16& ua = acc[m][2 * q + 1];
            uint16_t* grow = a.gu_out + (size_t)(row0 + m * 32 + tok) * 2 * a.I;
            *reinterpret_cast<uint2*>(grow + i0) =
                make_uint2(f32x2_to_bf16x2(ga[4 * g], ga[4 * g + 1]),
                           f32x2_to_bf16x2(ga[4 * g + 2], ga[4 * g + 3]));
            *reinterpret_cast<uint2*>(grow + a.I + i0) =
                make_uint2(f32x2_to_bf16x2(ua[4 * g], ua[4 * g + 1]),
                           f32x2_to_bf16x2(ua[4 * g + 2], ua[4 * g + 3]));
          }
        }
        // The row maximum is taken on the fp32 values, before their bf16
        // storage rounding (the requantisation clamps the few stored values
        // that round above it).
        amax[m] = fmaxf(amax[m],
                        fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3]))));
        *reinterpret_cast<uint2*>(lds + (m * 32 + tok) * SP + (i0 - col0) * 2) =
            make_uint2(f32x2_to_bf16x2(h[0], h[1]), f32x2_to_bf16x2(h[2], h[3]));
      }
    }
    // The tile leaves in whole row segments of WGN bytes: each wave store
    // covers 64 x 16 contiguous-per-row bytes, full cache lines, written
    // non-temporally (the intermediate is read back only by the next step).
    __syncthreads();
    {
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      constexpr int CPR = WGN / 16;  // 16-byte chunks per row
#pragma unroll
      for (int i = tid; i < BMT * CPR; i += 256) {
        const int r = i / CPR, c = i % CPR;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + r * SP + c * 16);
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4_t*>(act + (size_t)(row0 + r) * a.I + col0 + c * 8));
      }
    }
    if constexpr (DT == 1) {
      // Partial row maxima over this workgroup's columns: lane halves, then waves.
      float* wmax = reinterpret_cast<float*>(lds + (LDS > STG ? LDS : STG));
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float v = fmaxf(amax[m], __shfl_xor(amax[m], 32, 64));
        if (wk == 0 && lane < 32) wmax[wn * BMT + m * 32 + lane] = v;
      }
      __syncthreads();
      for (int r = tid; r < BMT; r += 256) {
        float v = wmax[r];
#pragma unroll
        for (int w = 1; w < WN; ++w) v = fmaxf(v, wmax[w * BMT + r]);
        a.amax_part[(size_t)(row0 + r) * a.n_ntiles + ntile] = v;
      }
    }
  } else {
    // Down-projection epilogue: weighted per-slot partials, one writer per element.
    if (wk != 0) return;
    float* part = reinterpret_cast<float*>(a.out) + (size_t)kg * S * a.N;
    // A tail piece writes its tile-local partial instead: rows of the tile,
    // columns of the workgroup, in the piece's slice of the tail space.
    float* const tp = a.tail_part + (size_t)(piece * n_tail + tail_idx) * BMT * WGN;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int slot = rslot[m];
      if (slot >= S) continue;
      const float sc = rsc[m];
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int h0 = (rb0 + f) * 32 + 8 * g + fq;
          float ws[4] = {1.f, 1.f, 1.f, 1.f};
          if constexpr (DT == 1) {
            const float4 w4 = *reinterpret_cast<const float4*>(scl + (h0 - ntile * WGN));
            ws[0] = w4.x; ws[1] = w4.y; ws[2] = w4.z; ws[3] = w4.w;
          }
          float4 o;
          o.x = acc[m][f][4 * g + 0] * ws[0] * sc;
          o.y = acc[m][f][4 * g + 1] * ws[1] * sc;
          o.z = acc[m][f][4 * g + 2] * ws[2] * sc;
          o.w = acc[m][f][4 * g + 3] * ws[3] * sc;
          if (piece < 0)
            *reinterpret_cast<float4*>(part + (size_t)slot * a.N + h0) = o;
          else
            *reinterpret_cast<float4*>(tp + (size_t)(m * 32 + tok) * WGN + (h0 - ntile * WGN)) = o;
        }
    }
  }
}

// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void quant_act_kernel(QuantArgs a) {
  __shared__ float red[4];
  const int p = blockIdx.x;
  if (p >= *a.total_padded) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const uint16_t* row = a.act + (size_t)p * a.I;
  // The row's first chunks are loaded before the row maximum is known, so
  // that their latency overlaps the maxima's (rows of up to 8 * 2048 values
  // come entirely from these registers).
  constexpr int kPre = 8;
  uint4 pre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int c = tid + 256 * j;
    if (c < a.I / 8) pre[j] = *reinterpret_cast<const uint4*>(row + c * 8);
  }
  float m = 0.0f;
  for (int i = tid; i < a.nparts; i += 256) m = fmaxf(m, a.amax_part[(size_t)p * a.nparts + i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m > 0.0f ? m / 448.0f : 1.0f;
  const float inv = 1.0f / s;  // for the correctly rounded quotients (quant_div)
  if (tid == 0) a.act_scale[p] = s;
  uint8_t* q = a.act_q + (size_t)p * a.I;
  auto convert = [&](int c, const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = quant_div(bf16_bits_to_f32(w[i] & 0xffffu), s, inv);
      f[2 * i + 1] = quant_div(bf16_bits_to_f32(w[i] >> 16), s, inv);
    }
    *reinterpret_cast<uint2*>(q + c * 8) =
        make_uint2(f32x4_to_e4m3(f[0], f[1], f[2], f[3]), f32x4_to_e4m3(f[4], f[5], f[6], f[7]));
  };
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int c = tid + 256 * j;
    if (c < a.I / 8) convert(c, pre[j]);
  }
  for (int c = tid + 256 * kPre; c < a.I / 8; c += 256)
    convert(c, *reinterpret_cast<const uint4*>(row + c * 8));
}

// MX block quantisation of the bf16 intermediate (MXFP8 stage 2): one thread
// per block of 32 values of a row p < total_padded; the block maximum sets the
// shared exponent (mx_exponent), codes = e4m3fn(clamp(v * 2^-x)).
__global__ __launch_bounds__(256) void quant_act_mx_kernel(QuantMxArgs a) {
  const int nb = a.I / 32;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t p = i / nb;
  const int b = (int)(i % nb);
  if (p >= *a.total_padded) return;
  const uint4* src = reinterpret_cast<const uint4*>(a.act + (size_t)p * a.I + (size_t)b * 32);
  uint4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = src[j];
  float f[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[8 * j + 2 * q] = bf16_bits_to_f32(w[q] & 0xffffu);
      f[8 * j + 2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(f[j]));
  const int x = mx_exponent(m);
  const float inv = mx_inv_scale(x);
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    c[j] = f32x4_to_e4m3(clamp448(f[4 * j] * inv), clamp448(f[4 * j + 1] * inv),
                         clamp448(f[4 * j + 2] * inv), clamp448(f[4 * j + 3] * inv));
  uint4* dq = reinterpret_cast<uint4*>(a.act_q + (size_t)p * a.I + (size_t)b * 32);
  dq[0] = make_uint4(c[0], c[1], c[2], c[3]);
  dq[1] = make_uint4(c[4], c[5], c[6], c[7]);
  a.act_mx[(size_t)p * nb + b] = (uint8_t)(x + 127);
}

// out[t,:] = bf16( sum_j sum_g part[g][t*k+j][:] ), j ascending, then split g ascending.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int64_t n4 = (int64_t)a.T * a.H / 4;
  const size_t split = (size_t)a.T * a.k * a.H;
  if (*a.total_padded == 0) {  // empty grouping (invalid ids): no partial was written
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x)
      *reinterpret_cast<uint2*>(a.out + (size_t)i * 4) = make_uint2(0u, 0u);
    return;
  }
  const int n = a.k * a.kg;  // partials per output, summed in the order u = j*kg + g
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i * 4 / a.H, h = i * 4 % a.H;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    // Eight partials are loaded before any is added, so their latencies overlap.
    constexpr int B = 8;
    for (int u0 = 0; u0 < n; u0 += B) {
      float4 v[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int u = u0 + b, j = u / a.kg, g = u % a.kg;
        if (u < n)
          v[b] = *reinterpret_cast<const float4*>(a.part + g * split +
                                                  ((size_t)t * a.k + j) * a.H + h);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (u0 + b >= n) break;
        if (u0 + b == 0) {
          s = v[b];
        } else {
          s.x = s.x + v[b].x;
          s.y = s.y + v[b].y;
          s.z = s.z + v[b].z;
          s.w = s.w + v[b].w;
        }
      }
    }
    *reinterpret_cast<uint2*>(a.out + (size_t)t * a.H + h) =
        make_uint2(f32x2_to_bf16x2(s.x, s.y), f32x2_to_bf16x2(s.z, s.w));
  }
}

// part[slot][h] of the tail tiles = sum over pieces p = 0, 1, ... in order of
// tail_part[p][tile][row][col]; one float4 per thread and step.
__global__ __launch_bounds__(256) void tail_reduce_kernel(TailReduceArgs a) {
  const int total = *a.total_padded;
  const int n_m = total / a.bmt;
  const TailPlan pl = tail_plan(n_m * a.n_ntiles, a.round, a.tail_split, a.nchunks);
  if (pl.split < 2) return;
  const int c4n = a.wgn / 4;
  const int64_t items = (int64_t)pl.tail * a.bmt * c4n;
  const size_t piece_stride = (size_t)pl.tail * a.bmt * a.wgn;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c4 = (int)(i % c4n), r = (int)(i / c4n % a.bmt), ti = (int)(i / ((int64_t)c4n * a.bmt));
    int mtile, ntile;
    tile_coords(pl.n_full + ti, n_m, a.group_m, a.n_ntiles, mtile, ntile);
    const int slot = a.sorted_slot[mtile * a.bmt + r];
    if (slot >= a.S) continue;
    const float* src = a.tail_part + ((size_t)ti * a.bmt + r) * a.wgn + c4 * 4;
    float4 acc = *reinterpret_cast<const float4*>(src);
    for (int p = 1; p < pl.split; ++p) {
      const float4 v = *reinterpret_cast<const float4*>(src + p * piece_stride);
      acc.x = acc.x + v.x;
      acc.y = acc.y + v.y;
      acc.z = acc.z + v.z;
      acc.w = acc.w + v.w;
    }
    *reinterpret_cast<float4*>(a.part + (size_t)slot * a.N + ntile * a.wgn + c4 * 4) = acc;
  }
}

// ---------------------------------------------------------------------------
// Host side: configuration choice and dispatch.

namespace {

// Expected live row tiles of a grouping of T tokens with k distinct experts
// each: the expected number of experts that get a slot, E(1 - (1 - k/E)^T)
// for uniform routing, rounded up, and at least the tiles the slots fill.
int64_t live_mtiles(int T, int k, int E, int tile_rows) {
  const int64_t S = (int64_t)T * k;
  const int64_t by_slots = (S + tile_rows - 1) / tile_rows;
  const double active = E * (1.0 - std::pow(1.0 - (double)k / E, (double)T));
  const int64_t by_experts = (int64_t)std::ceil(active - 1e-6);
  return by_slots > by_experts ? by_slots : by_experts;
}

// Workgroups of a decode-shaped stage-2 launch that MI355X runs at once (two
// per CU on 256 CUs): the reduction split aims for one full round of them.
constexpr int64_t kDecodeRound = 512;
// The same for the 128 x 512 prefill tile (one workgroup per CU).
constexpr int64_t kPrefillRound = 256;

// Pipeline shape of a (mt, nf, ksplit) triple: 128-byte stages (every stage
// has an even number of token fragments per wave, and each token row is
// fetched as whole 128-byte lines), weights three stages deep. The bf16 and
// FP8 prefill tiles, whose 128 accumulator registers per lane leave room for
// two stages of 16 weight pieces, keep 128-byte stages two deep; the MX
// prefill tiles 64-byte stages three deep. Measured on the Mixtral prefill,
// T=8192: FP8 2.70 -> 2.62 ms per layer call with 128-byte stages two deep
// (the cache lines fetched per flop and the stage barriers halve; a
// three-deep ring of 128-byte stages spills), MXFP8 3.04 -> 3.14 ms and MXFP4
// 2.57 -> 2.62 ms with them.
void set_pipeline(GemmCfg& c, int dt) {
  const bool prefill = c.ksplit == 1 && c.mt * c.nf >= 16;
  c.ck = prefill && dt >= 2 ? 64 : 128;
  c.nb = prefill && dt <= 1 ? 2 : 3;
  c.wg_n = (4 / c.ksplit) * c.nf * 32;
  c.tail_split = 0;
  c.round = 0;
}

}  // namespace

GemmCfg stage1_cfg(int dt, int T, int k, int E, int H, int I, int bm) {
  GemmCfg c;
  c.mt = (bm >= 128 ? 128 : bm) / 32;
  c.nf = c.mt == 4 && (2 * I) % 512 == 0 ? 4 : 2;  // prefill: 128 x 128 per wave
  c.ksplit = 1;
  c.kg = 1;
  // Decode shapes (one 32-row fragment per tile): split the reduction over the
  // waves so that a workgroup covers 64 features and the launch fills the chip
  // (E2M1 weights: 128 features, the same weight bytes per workgroup; the
  // kernel then needs all 256 registers of two waves per SIMD).
  if (c.mt == 1 && (H * (dt == 0 ? 2 : 1)) % (4 * 128) == 0) {
    c.ksplit = 4;
    if (dt == 3) c.nf = 4;
    // FP8 and MXFP8: two waves along the reduction instead (128 features,
    // half as many workgroups, twice the work each) when those workgroups fit
    // one round or every expert is expected to be live (the weights of all
    // experts streamed in fewer, longer workgroups). Measured on the Mixtral
    // shape, median per layer call: FP8 T=1 91.0 -> 89.4 us, T=16 273.6 ->
    // 271.5, T=64 278.9 -> 274.2, and at T=4 (five live experts, 1120
    // workgroups: a thin last round) 182.9 -> 184.2, so it keeps four; MXFP8
    // T=16 282.5 -> 277.8; bf16 T=16 486.7 -> 491.7, so bf16 keeps four.
    if (dt == 1 || dt == 2) {
      const int64_t live = live_mtiles(T, k, E, 32);
      if (live * (2 * (int64_t)I / 128) <= kDecodeRound || live >= E) c.ksplit = 2;
    }
  }
  set_pipeline(c, dt);
  return c;
}

GemmCfg stage2_cfg(int dt, int T, int k, int E, int H, int I, int bm) {
  GemmCfg c;
  c.mt = (bm >= 128 ? 128 : bm) / 32;
  c.nf = c.mt == 4 && H % 512 == 0 ? 4 : 2;
  c.ksplit = 1;
  c.kg = 1;
  const int kbytes = I * (dt == 0 ? 2 : 1);
  if (H % 256 != 0) {
    c.ksplit = 2;  // 128 features per workgroup
    c.nf = 2;
    if (c.mt > 2) c.mt = 2;
  }
  if (c.mt == 1 && kbytes % (4 * 128) == 0) {
    c.ksplit = 4;
    // When the live workgroups do not fill a round, split the reduction over
    // workgroups too (each split g adds a partial, summed in order): FP8 until
    // they fill two rounds, with at most four splits; the others until they
    // fill one. Measured on the Mixtral shape, FP8 decode: T=1 102 -> 98 us
    // with 4 splits instead of 7; T=4 (five live experts, 320 workgroups
    // unsplit) 185 -> 183 us with 4 splits instead of 2 (1.25 rounds); T=16
    // and T=64 fill a round unsplit (2 splits: no gain). MXFP4 (half the
    // weight bytes per workgroup) at T=4: 2 splits, 4 were 3.6 us slower.
    const int chunks = kbytes / (4 * 128);
    const int64_t base = live_mtiles(T, k, E, 32) * (H / (32 * c.nf));
    const int64_t target = dt == 1 ? 2 * kDecodeRound : kDecodeRound;
    const int max_kg = dt == 1 ? 4 : 16;
    if (base < kDecodeRound) {
      for (int cand = 2; cand <= max_kg; ++cand) {
        if (chunks % cand) continue;
        if (base * c.kg >= target) break;
        c.kg = cand;
      }
    }
  }
  set_pipeline(c, dt);
  if (c.mt == 4 && c.nf == 4 && c.ksplit == 1 && c.kg == 1) {
    // Prefill tiles are long (the whole reduction of 128 rows x 512 features).
    // When a quarter round of resident workgroups holds them all (small
    // batches on 128-row tiles), split the reduction over workgroups until
    // the round is full, with at least 16 chunks per split; otherwise cut a
    // partial last round into pieces (tail_split). Measured, FP8 on the
    // Mixtral shape: T=256 325 -> 319 us and T=512 453 -> 443 us with 4
    // splits; at T=1024 two splits were slower than the pieces (636 -> 649).
    const int chunks = kbytes / c.ck;
    const int64_t tiles = live_mtiles(T, k, E, 128) * (H / c.wg_n);
    for (int cand = 2; cand <= 64; ++cand) {
      if (chunks % cand || chunks / cand < 16) continue;
      if (tiles * cand > kPrefillRound) break;
      c.kg = cand;
    }
    if (c.kg < 4) c.kg = 1;
    if (c.kg == 1) {
      c.tail_split = 8;
      c.round = (int)kPrefillRound;
    }
  }
  return c;
}

bool gemm_cfg_ok(int dt, int stage, const GemmCfg& c, int N, int K) {
  const int64_t kbytes = (int64_t)K * (dt == 0 ? 2 : 1);
  if (c.mt != 1 && c.mt != 2 && c.mt != 4) return false;
  if (c.nf != 2 && !(c.nf == 4 && c.mt == 4 && c.ksplit == 1) &&
      !(dt == 3 && stage == 1 && c.nf == 4 && c.mt == 1 && c.ksplit == 4))
    return false;
  if (N % c.wg_n) return false;
  if (kbytes % ((int64_t)c.ksplit * c.kg * c.ck)) return false;
  if (stage == 1 && (c.kg != 1 || c.tail_split != 0)) return false;
  if (c.tail_split != 0 && (c.ksplit != 1 || c.kg != 1 || c.round < 1)) return false;
  const bool prefill = c.ksplit == 1 && c.mt * c.nf >= 16;
  if (c.ck != (prefill && dt >= 2 ? 64 : 128)) return false;
  if (c.nb != (prefill && dt <= 1 ? 2 : 3)) return false;
  if (c.ksplit == 4) return c.mt == 1;
  if (c.ksplit == 2) return c.mt <= 2;
  return c.ksplit == 1;
}

namespace {

template <int DT, int STAGE, int MT, int NF, int KSPLIT, int NB, int CK>
hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  int64_t blocks = (int64_t)a.n_mtiles * a.n_ntiles * a.kg;
  // The tail pieces take the place of the tail tiles: at most min(round,
  // kTailPieces) more workgroups.
  if (a.tail_split > 0) blocks += a.round < kTailPieces ? a.round : kTailPieces;
  hipLaunchKernelGGL((gemm_kernel<DT, STAGE, MT, NF, KSPLIT, NB, CK>), dim3((unsigned)blocks),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DT, int STAGE>
hipError_t launch_dt_stage(const GemmCfg& c, const GemmArgs& a, hipStream_t st) {
  if constexpr (DT == 3 && STAGE == 1)
    if (c.ksplit == 4 && c.nf == 4) return launch_one<DT, STAGE, 1, 4, 4, 3, 128>(a, st);
  if (c.ksplit == 4) return launch_one<DT, STAGE, 1, 2, 4, 3, 128>(a, st);
  if (c.ksplit == 2)
    return c.mt == 1 ? launch_one<DT, STAGE, 1, 2, 2, 3, 128>(a, st)
                     : launch_one<DT, STAGE, 2, 2, 2, 3, 128>(a, st);
  if (c.nf == 4) {
    if constexpr (DT <= 1)
      return launch_one<DT, STAGE, 4, 4, 1, 2, 128>(a, st);
    else
      return launch_one<DT, STAGE, 4, 4, 1, 3, 64>(a, st);
  }
  switch (c.mt) {
    case 1: return launch_one<DT, STAGE, 1, 2, 1, 3, 128>(a, st);
    case 2: return launch_one<DT, STAGE, 2, 2, 1, 3, 128>(a, st);
    case 4: return launch_one<DT, STAGE, 4, 2, 1, 3, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch(int dt, int stage, const GemmCfg& c, const GemmArgs& a, hipStream_t st) {
  if (dt == 0)
    return stage == 1 ? launch_dt_stage<0, 1>(c, a, st) : launch_dt_stage<0, 2>(c, a, st);
  if (dt == 2)
    return stage == 1 ? launch_dt_stage<2, 1>(c, a, st) : launch_dt_stage<2, 2>(c, a, st);
  if (dt == 3)
    return stage == 1 ? launch_dt_stage<3, 1>(c, a, st) : launch_dt_stage<3, 2>(c, a, st);
  return stage == 1 ? launch_dt_stage<1, 1>(c, a, st) : launch_dt_stage<1, 2>(c, a, st);
}

}  // namespace

hipError_t launch_gemm(int dt, int stage, const GemmCfg& c, const GemmArgs& a, hipStream_t st) {
  if (!gemm_cfg_ok(dt, stage, c, a.N, a.K_bytes / (dt == 0 ? 2 : 1))) return hipErrorInvalidValue;
  if (c.tail_split != a.tail_split ||
      (a.tail_split > 0 && (a.round != c.round || !a.tail_part)))
    return hipErrorInvalidValue;
  return dispatch(dt, stage, c, a, st);
}

hipError_t launch_tail_reduce(const TailReduceArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(tail_reduce_kernel, dim3(1024), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_quant_act(const QuantArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(quant_act_kernel, dim3(a.cap), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_quant_act_mx(const QuantMxArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.cap * (a.I / 32);
  hipLaunchKernelGGL(quant_act_mx_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  int64_t n4 = (int64_t)a.T * a.H / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
