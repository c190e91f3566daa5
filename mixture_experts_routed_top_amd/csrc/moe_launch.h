// Host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct AlignArgs {
  const int32_t* ids;  // [S]
  int S, E, bm;
  int32_t* sorted_slot;
  int32_t* tile_expert;
  int32_t* count;
  int32_t* offset;
  int32_t* total;
};
hipError_t launch_align(const AlignArgs& a, hipStream_t st);
// Largest grouping the router launch can build in its last-arriving workgroup
// (256 threads, runs of up to 8 slots); larger ones take launch_align.
constexpr int kFusedAlignSlots = 2048;

struct RouteArgs {
  const uint16_t* x;         // bf16 [T,H]
  const uint16_t* w_router;  // bf16 [E,H]
  const float* bias;         // [E] or null
  int T, H, E, k;
  int32_t* topk_ids;         // [T,k]
  float* topk_w;             // [T,k]
  float* logits;             // [T,E] or null
  uint8_t* x_q;              // [T,H] or null
  float* x_scale;            // [T] (per-token FP8)
  uint8_t* x_mx;             // [T][H/32] E8M0 codes (MXFP8: x_q holds block-scaled codes), or null
  // Grouping built by the last workgroup to finish (ticket != null; the ids
  // are topk_ids; T*k <= kFusedAlignSlots, at most 16 experts). The ticket is
  // one int that is zero on entry; the last workgroup resets it.
  AlignArgs al;
  int32_t* ticket;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

// Byte relayout of one row-major [R, K] matrix per expert into fragment order.
// For the gate/up pair (two sources) composite rows alternate 32-row blocks.
struct PreshuffleArgs {
  const uint8_t* src0;  // W1 or W2, [E][rows][K] elements
  const uint8_t* src1;  // W3, or null for W2
  uint8_t* dst;
  int E, R;             // R: composite rows per expert (2I or H)
  int64_t K_bytes;      // reduction length in bytes (multiple of 64; E2M1: of 32)
  int mx_order;         // 0: plain, 1: MXFP8 byte order, 2: E2M1 fragments (see preshuffle_kernel)
};
hipError_t launch_preshuffle(const PreshuffleArgs& a, hipStream_t st);
// The E8M0 block scales of the same matrices ([E][rows][K/32] codes, K_bytes =
// K for e4m3fn) into the order the GEMM reads them: per expert, groups of four
// 32-row blocks, then reduction fragment (64 values), then lane l (row l%32 of
// each block, 32-value block l/32 of the fragment), then the four blocks.
hipError_t launch_preshuffle_mx_scales(const PreshuffleArgs& a, hipStream_t st);

// Kernel configuration of a grouped GEMM stage, chosen on the host from the
// shapes; the same choice sizes the FP8 amax partials.
struct GemmCfg {
  int mt;      // 32-row token fragments per tile (tile rows = 32 * mt, dividing block_m)
  int nf;      // 32-row weight fragments per wave (2 or 4: gate/up pairs in stage 1)
  int ksplit;  // waves splitting the reduction inside a workgroup (1 or 4)
  int kg;      // workgroups splitting the reduction (stage 2 only; partials summed in order)
  int nb;      // weight pipeline depth (register stages)
  int ck;      // reduction bytes per pipeline stage (64 or 128)
  int wg_n;    // features (composite rows) per workgroup = (4 / ksplit) * nf * 32
  int tail_split;  // stage 2: most pieces a tile of the last, partial round is cut into (0: off)
  int round;   // stage 2 with tail_split: workgroups per round the tail plan assumes (a
               // constant of the configuration, so that the plan, and with it the output
               // bits, depend on the shapes only)
};

// Tiles of a partial last round of a stage-2 launch are cut along the
// reduction into pieces, so that the round fills the device; the last piece
// of a tile to finish sums the pieces' partials in piece order. At most
// kTailPieces pieces per launch (workspace). A round is GemmCfg::round workgroups: the
// MI355X's 256 compute units times the workgroups of the configuration one
// of them holds.
constexpr int kTailPieces = 256;
GemmCfg stage1_cfg(int dt, int T, int k, int E, int H, int I, int bm);
GemmCfg stage2_cfg(int dt, int T, int k, int E, int H, int I, int bm);
// Whether a configuration can run a stage with N output features and reduction length K.
bool gemm_cfg_ok(int dt, int stage, const GemmCfg& c, int N, int K);

struct GemmArgs {
  const uint8_t* X;        // stage 1: x / x_q [T][K] (rows gathered by token); stage 2: act
                           // bf16 [cap][I] (BF16 and FP8: FP8 requantises it as it loads it)
                           // or the MX codes act_q [cap][I]
  const float* x_scale;    // FP8 stage 1: per-token activation scale
  const uint8_t* W;        // preshuffled weights
  const float* w_scale;    // FP8: s13 [E][2][I] (stage 1) or s2 [E][H] (stage 2)
  const uint8_t* x_mx;     // MXFP8/MXFP4: E8M0 codes of X's rows, [rows of X][K/32]
  const uint8_t* w_mx;     // MXFP8/MXFP4: preshuffled E8M0 weight codes (launch_preshuffle_mx_scales)
  const int32_t* sorted_slot;
  const int32_t* tile_expert;
  const int32_t* total_padded;
  const float* topk_w;     // stage 2
  void* out;               // stage 1: act bf16 [cap][I]; stage 2: part fp32 [kg][T*k][H]
  float* amax_part;        // FP8 [cap][nparts] row maxima over stage 1's feature tiles
                           // (stage 1 writes them, stage 2 reduces them to the row scale)
  int nparts;
  int T, k, N, I, cap, bm;
  int K_bytes;             // reduction bytes of one row in the matrix-core format (H or I
                           // times the element size; FP8 stage 2: I, its source rows are 2I)
  int64_t x_bytes;         // size of X in bytes (< 2 GiB): loads past it read zeros
  int n_mtiles, n_ntiles;  // row tiles (32*mt rows) and feature tiles (wg_n rows)
  int kg, group_m;         // reduction split over workgroups; M-tiles per schedule group
  uint64_t k_magic;        // ceil(2^35 / k): slot / k as a multiply
  float* tail_part;        // stage 2 tail pieces: [kTailPieces][32*mt][wg_n] (tail_split > 0)
  int round;               // GemmCfg::round
  int tail_split;          // GemmCfg::tail_split
  int live_order;          // index the live tiles first (decode shapes) instead of the capacity
  // Stage 2 combine: out[t,:] = bf16(sum_j sum_g part[g][t*k+j][:]) by the last
  // workgroup to finish each (token, feature tile); tickets [T][n_ntiles] and,
  // with tail pieces, tile_tickets [kTailPieces]: zero on entry, left zero.
  uint16_t* y;             // bf16 [T][N]
  int32_t* tickets;
  int32_t* tile_tickets;
};
hipError_t launch_gemm(int dt, int stage, const GemmCfg& c, const GemmArgs& a, hipStream_t st);

// MXFP8 stage 2 prologue: the MX block quantisation of every row p < total of
// the bf16 intermediate (32 values per E8M0 code).
struct QuantMxArgs {
  const uint16_t* act;     // bf16 [cap][I]
  int cap, I;
  const int32_t* total_padded;
  uint8_t* act_q;          // [cap][I] e4m3fn codes
  uint8_t* act_mx;         // [cap][I/32] E8M0 codes
};
hipError_t launch_quant_act_mx(const QuantMxArgs& a, hipStream_t st);

// Token-scale tile of the MXFP8 GEMMs: the E8M0 columns (32 reduction values
// each) a workgroup covers, plus 16 for alignment. Stage 1 reduces over H
// (at most 8192), stage 2 over I (at most 16384).
constexpr int kMxMaxH = 8192;
constexpr int kMxMaxI = 16384;

}  // namespace moe
