// Host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

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
};
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

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
// Route, then align the routed ids (g.ids == a.topk_ids): one launch for
// batches of at most kTinyRouteTokens tokens (H <= 4096), two otherwise.
// Measured, FP8 Mixtral decode: T=1 92.7 -> 91.0 us per layer call; at T=4
// the single workgroup (all four tokens' W_r rows through one CU) made the
// call 1.5 us slower than the two launches, so only single tokens take it.
constexpr int kTinyRouteTokens = 1;
hipError_t launch_route_align(const RouteArgs& a, const AlignArgs& g, hipStream_t st);

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
// reduction into pieces, so that the round fills the device; the pieces'
// partials are summed in piece order by tail_reduce. At most kTailPieces
// pieces per launch (workspace). A round is GemmCfg::round workgroups: the
// MI355X's 256 compute units times the workgroups of the configuration one
// of them holds.
constexpr int kTailPieces = 256;
GemmCfg stage1_cfg(int dt, int T, int k, int E, int H, int I, int bm);
GemmCfg stage2_cfg(int dt, int T, int k, int E, int H, int I, int bm);
// Whether a configuration can run a stage with N output features and reduction length K.
bool gemm_cfg_ok(int dt, int stage, const GemmCfg& c, int N, int K);

struct GemmArgs {
  const uint8_t* X;        // stage 1: x / x_q [T][K] (rows gathered by token); stage 2: act / act_q [cap][K]
  const float* x_scale;    // FP8: per-token (stage 1) or per-row (stage 2) activation scale
  const uint8_t* W;        // preshuffled weights
  const float* w_scale;    // FP8: s13 [E][2][I] (stage 1) or s2 [E][H] (stage 2)
  const uint8_t* x_mx;     // MXFP8/MXFP4: E8M0 codes of X's rows, [rows of X][K/32]
  const uint8_t* w_mx;     // MXFP8/MXFP4: preshuffled E8M0 weight codes (launch_preshuffle_mx_scales)
  const int32_t* sorted_slot;
  const int32_t* tile_expert;
  const int32_t* total_padded;
  const float* topk_w;     // stage 2
  void* out;               // stage 1: act bf16 [cap][I]; stage 2: part fp32 [kg][T*k][H]
  float* amax_part;        // stage 1 FP8: [cap][N/wg_n]
  int T, k, N, I, cap, bm;
  int K_bytes;             // reduction bytes of one row (H or I times the element size)
  int64_t x_bytes;         // size of X in bytes (< 2 GiB): loads past it read zeros
  int n_mtiles, n_ntiles;  // row tiles (32*mt rows) and feature tiles (wg_n rows)
  int kg, group_m;         // reduction split over workgroups; M-tiles per schedule group
  uint64_t k_magic;        // ceil(2^35 / k): slot / k as a multiply
  float* tail_part;        // stage 2 tail pieces: [kTailPieces][32*mt][wg_n] (tail_split > 0)
  int round;               // GemmCfg::round
  // Backward pass (BF16 only): epi 1 = stage 1 writes the gate and up
  // pre-activations g, u to out (bf16 [cap][2I]: g in columns 0..I-1, u in
  // I..2I-1) instead of the SwiGLU; epi 2 = stage 1 over W2^T and the gathered
  // output gradient rows computes z = W2^T dout and writes dg, du to out (bf16
  // [cap][2I]) from act_in, gu and topk_w, and each row's partial <z, act>
  // over the workgroup's columns to dwpart [T*k][n_ntiles]; unit_w = stage 2
  // weighs every row by 1 instead of its routing weight.
  int epi;
  const uint16_t* act_in;
  const uint16_t* gu;
  uint16_t* gu_out;        // BF16 forward stage 1: also stores g, u as epi 1 does, or null
  float* dwpart;
  int unit_w;
  int tail_split;          // GemmCfg::tail_split
  int live_order;          // index the live tiles first (decode shapes) instead of the capacity
};
hipError_t launch_gemm(int dt, int stage, const GemmCfg& c, const GemmArgs& a, hipStream_t st);

// Sum of the tail pieces of a stage-2 launch, in piece order, into the per-slot
// partials (the same tile plan as the GEMM, from the device-side total).
struct TailReduceArgs {
  const float* tail_part;
  const int32_t* sorted_slot;
  const int32_t* total_padded;
  float* part;             // [T*k][N]
  int S, N, bmt, wgn, n_ntiles, group_m, round, tail_split, nchunks;
};
hipError_t launch_tail_reduce(const TailReduceArgs& a, hipStream_t st);

// FP8 stage 2 prologue: per-row amax from the partials, scale, requantise.
struct QuantArgs {
  const uint16_t* act;     // bf16 [cap][I]
  const float* amax_part;  // [cap][nparts] (row-major: a row's partial maxima together)
  int nparts, cap, I;
  const int32_t* total_padded;
  uint8_t* act_q;          // [cap][I]
  float* act_scale;        // [cap]
};
hipError_t launch_quant_act(const QuantArgs& a, hipStream_t st);

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

// out[t,:] = bf16(sum_j sum_g part[g][t*k+j,:]), j ascending, then g ascending.
struct CombineArgs {
  const float* part;  // [kg][T*k][H]
  const int32_t* total_padded;  // 0: an empty grouping (invalid ids), the output is zero
  int T, k, H, kg;
  uint16_t* out;      // [T][H]
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// --- backward pass (bf16) ---

// Load-time relayout of the transposed weights (mode 0: W2^T [E][I rows][H];
// mode 1: [W1^T | W3^T] [E][H rows][2I]) into the bf16 fragment order.
struct PreshuffleTArgs {
  const uint16_t* w1;  // [E][I][H]
  const uint16_t* w3;  // [E][I][H]
  const uint16_t* w2;  // [E][H][I]
  uint16_t* dst;
  int E, H, I, mode;
};
hipError_t launch_preshuffle_t(const PreshuffleTArgs& a, hipStream_t st);

// C[e][m][n] = sum over the rows p of expert e (offset[e] .. offset[e+1]) of
// A[p][m] B[p][n]; rows m < m_split go to C0 [E][m_split][N], the rest to C1
// [E][M - m_split][N]. a_mode/b_mode: 0 = the grouped row p; 1 = the token row
// of its slot (A: times the slot's routing weight).
struct WgradArgs {
  const uint16_t* A;
  const uint16_t* B;
  int a_stride, b_stride;      // elements per row
  int a_mode, b_mode;
  int64_t a_bytes, b_bytes;    // buffer sizes (< 2 GiB)
  int M, N, E, m_split;
  const int32_t* offset;       // [E+1]
  const int32_t* sorted_slot;
  const float* topk_w;
  int S;
  uint64_t k_magic;
  float* C0;
  float* C1;
};
hipError_t launch_wgrad(const WgradArgs& a, hipStream_t st);

// Grouped operand rows of the weight gradients: for each padded row p of the
// grouping (slot s = sorted_slot[p], token t = s / k), xg[p] = x[t] and
// wdg[p] = bf16(topk_w[s] * dout[t]); pad rows get zeros there and in dgu.
struct GatherArgs {
  const uint16_t* x;           // bf16 [T][H]
  const uint16_t* dout;        // bf16 [T][H]
  const float* topk_w;         // [T*k]
  const int32_t* sorted_slot;  // [capacity]
  const int32_t* total;        // [1]
  int H, I, S, cap;
  uint64_t k_magic;
  uint16_t* xg;                // bf16 [capacity][H]
  uint16_t* wdg;               // bf16 [capacity][H]
  uint16_t* dgu;               // bf16 [capacity][2I]: pad rows zeroed
};
hipError_t launch_bwd_gather(const GatherArgs& a, hipStream_t st);

// Router gradient and dx (bwd_dl_kernel, bwd_dx_kernel, bwd_router_kernel).
struct BwdArgs {
  int T, H, k, E, nparts, kg;
  const float* dwpart;     // [T*k][nparts]
  const float* topk_w;     // [T*k]
  const int32_t* ids;      // [T*k]
  const float* part;       // [kg][T*k][H] per-slot W1^T dg + W3^T du (kg reduction splits)
  const uint16_t* w_router;  // bf16 [E][H]
  const uint16_t* x;       // bf16 [T][H]
  float* dl;               // [T*k]
  float* dx;               // [T][H]
  float* dw_router;        // [E][H]
  float* dbias;            // [E] or null
  const int32_t* sorted_slot;  // [capacity] grouped rows (slot, or T*k for a pad row)
  const int32_t* offset;   // [E+1] padded row offset of each expert's group
  const int32_t* total;    // [1] padded rows in use
  int bm, ntiles;          // rows per tile (block_m); tiles of the capacity
  uint64_t k_magic;        // ceil(2^35 / k): slot / k as a multiply (div_k)
  float* rpart;            // [ntiles][H] router-gradient partials, then [ntiles] bias partials
};
hipError_t launch_bwd_router(const BwdArgs& a, hipStream_t st);

}  // namespace moe
