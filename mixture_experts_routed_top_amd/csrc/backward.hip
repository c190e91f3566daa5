// Backward pass of the bf16 routed MoE layer (the custom VJP the FlyDSL-in-JAX
// talk summary names as its next step, "Ausblick und Roadmap" 10:07): the
// gradients of x, W1, W3, W2, the router weights and the router bias for an
// output gradient dout, with the forward's top-k selection held fixed.
//
// Per grouped row p (slot s = t*k + j of expert e, routing weight w):
//   g, u  = W1 x_t, W3 x_t            (recomputed: stage 1 with epilogue 1)
//   z     = W2^T dout_t               (stage 1 over W2^T, epilogue 2, which also
//   dg/du = w z (.) SwiGLU'(g, u)      forms <z, a> and the SwiGLU gradient)
//   part_s = W1^T dg + W3^T du         (stage 2 over [W1^T | W3^T], weight 1)
//   dl    = w (dw - sum_i w_i dw_i),  dw_j = <z_j, a_j>   (bwd_dl_kernel)
//   dx_t  = sum_j part_{t,j} + sum_j dl_j W_r[e_j]        (bwd_dx_kernel)
//   dW_r[e], db[e] = sums over the slots of e of dl x_t, dl (per tile of
//                    grouped rows, then over the tiles: bwd_router_*_kernel)
//   dW2[e]  = sum_p (w dout_t) a_p^T,  dW1|dW3[e] = sum_p [dg|du]_p x_t^T
//                                       (wgrad_kernel: reductions over the rows
//                                        of each expert's group)
// Every sum runs in a fixed order: the results are reproducible bit for bit.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// --- load-time relayout of the transposed weights ---------------------------

// bf16 fragment order (as preshuffle_kernel) of a transposed expert matrix:
// mode 0 (W2^T, rows i < I, reduction over h < H): element (i, h) = W2[e][h][i];
// mode 1 ([W1^T | W3^T], rows h < H, reduction over k < 2I): element (h, k) =
// W1[e][k][h] for k < I, W3[e][k - I][h] after. One thread per 16-byte piece
// (8 values gathered with a stride of a source row).
__global__ __launch_bounds__(256) void preshuffle_t_kernel(PreshuffleTArgs a) {
  const int R = a.mode == 0 ? a.I : a.H;       // rows of the transposed matrix
  const int K = a.mode == 0 ? a.H : 2 * a.I;   // its reduction length
  const int64_t kblocks = K / 32;              // 32 bf16 per 64-byte fragment row
  const int64_t per_expert = (int64_t)R * K;   // elements
  const int64_t n8 = per_expert * a.E / 8;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < n8;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t el = u * 8;
    const int64_t e = el / per_expert, rem = el % per_expert;
    const int64_t f = rem / 1024;                // fragment: 32 rows x 32 values
    const int in = (int)(rem % 1024);
    const int pc = in / 512, lane = (in % 512) / 8;
    const int64_t rb = f / kblocks, kb = f % kblocks;
    const int64_t c = rb * 32 + lane % 32;
    const int64_t k0 = kb * 32 + (lane / 32) * 16 + pc * 8;
    uint16_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t k = k0 + q;
      if (a.mode == 0)
        v[q] = a.w2[(e * a.H + k) * a.I + c];
      else
        v[q] = k < a.I ? a.w1[(e * a.I + k) * a.H + c] : a.w3[(e * a.I + (k - a.I)) * a.H + c];
    }
    uint4 o;
    o.x = v[0] | ((uint32_t)v[1] << 16);
    o.y = v[2] | ((uint32_t)v[3] << 16);
    o.z = v[4] | ((uint32_t)v[5] << 16);
    o.w = v[6] | ((uint32_t)v[7] << 16);
    *reinterpret_cast<uint4*>(a.dst + el) = o;
  }
}

hipError_t launch_preshuffle_t(const PreshuffleTArgs& a, hipStream_t st) {
  const int64_t n8 = (int64_t)a.E * a.H * a.I * (a.mode == 0 ? 1 : 2) / 8;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(preshuffle_t_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// --- weight gradients: reductions over each expert's rows --------------------

// C[e][m][n] = sum over the padded rows p of expert e of A[p][m] * B[p][n] (pad
// rows and rows of no slot add zero), fp32 accumulation on the bf16 matrix
// cores, rows in ascending order. A rows are the grouped rows themselves
// (a_mode 0) or the token row of the row's slot scaled by its routing weight
// and rounded to bf16 (a_mode 1); B rows are grouped rows (0) or token rows (1).
//
// Workgroup tile 128 (m) x 128 (n), four waves of 64 x 64; 64 rows per step.
// The rows arrive m- (n-) contiguous, the matrix cores want the reduction
// contiguous: each thread loads an 8-row x 8-column block, transposes it in
// registers, and writes 8 rows of 8 reduction values to LDS ([m][64 rows],
// 16-byte column groups XOR-swizzled, wg_swz). Two LDS buffers: the next
// step's blocks load while this step's matrix-core work runs.
constexpr int kWgTile = 128;
constexpr int kWgRows = 64;
constexpr int kWgLdsHalf = kWgTile * kWgRows * 2;  // one operand of one buffer, bytes

// Byte offset of 16-byte column group cg of row `row` in an operand tile. The
// group is XORed with (row ^ row/8) % 8: the eight rows a matrix-core read
// takes at once (consecutive rows) and the eight a transposed block write
// takes at once (rows 8 apart) each spread over all banks.
__device__ __forceinline__ int wg_swz(int row, int cg) {
  return row * (kWgRows * 2) + ((cg ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// 8x8 transpose of bf16: in[r] holds columns 0..7 of row r; out[c] rows 0..7 of column c.
__device__ __forceinline__ void transpose8(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t w[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    w[r][0] = in[r].x;
    w[r][1] = in[r].y;
    w[r][2] = in[r].z;
    w[r][3] = in[r].w;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // value c of rows 2j and 2j+1: low or high half of word c/2
      const uint32_t lo = w[2 * j][c / 2], hi = w[2 * j + 1][c / 2];
      o[j] = (c & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)   // high halves
                     : __builtin_amdgcn_perm(hi, lo, 0x05040100u);  // low halves
    }
    out[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void wgrad_kernel(WgradArgs a) {
  __shared__ __align__(16) uint8_t lds[2][2][kWgLdsHalf];  // [buffer][A, B]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int mtiles = a.M / kWgTile, ntiles = a.N / kWgTile;
  const int e = blockIdx.x / (mtiles * ntiles);
  const int rem = blockIdx.x % (mtiles * ntiles);
  const int mt = rem / ntiles, nt = rem % ntiles;
  const int r0 = a.offset[e], r1 = a.offset[e + 1];
  const int S = a.S;

  // This thread's 8x8 block of one operand: operand B for threads 128..255.
  const bool isB = tid >= 128;
  const int bt = tid & 127;
  const int cblk = bt % 16, rblk = bt / 16;  // 16 column blocks x 8 row blocks
  const uint16_t* src = isB ? a.B : a.A;
  const int stride = isB ? a.b_stride : a.a_stride;
  const int mode = isB ? a.b_mode : a.a_mode;
  const int col0 = (isB ? nt : mt) * kWgTile + cblk * 8;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)src, (short)0, (int)(isB ? a.b_bytes : a.a_bytes), 0x00020000);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  uint4 blk[8];
  // Loads of step c's block: row p = r0 + c*64 + rblk*8 + q; rows past the
  // group, pad rows and (a_mode 1) their weights read as zero.
  auto load = [&](int c) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int p = r0 + c * kWgRows + rblk * 8 + q;
      const int slot = p < r1 ? a.sorted_slot[p] : S;
      const uint32_t row = mode == 0 ? (uint32_t)p : div_k(min(slot, S - 1), a.k_magic);
      const uint32_t off = slot < S ? (row * (uint32_t)stride + (uint32_t)col0) * 2u : 0x80000000u;
      blk[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
      if (!isB && mode == 1) {  // dout row times the routing weight, back to bf16
        const float w = slot < S ? a.topk_w[slot] : 0.0f;
        uint32_t x[4] = {blk[q].x, blk[q].y, blk[q].z, blk[q].w};
#pragma unroll
        for (int h = 0; h < 4; ++h)
          x[h] = f32x2_to_bf16x2(bf16_bits_to_f32(x[h] & 0xffffu) * w,
                                 bf16_bits_to_f32(x[h] >> 16) * w);
        blk[q] = make_uint4(x[0], x[1], x[2], x[3]);
      }
    }
  };
  auto store = [&](int buf) {
    uint4 t[8];
    transpose8(blk, t);
    uint8_t* base = lds[buf][isB ? 1 : 0];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      *reinterpret_cast<uint4*>(base + wg_swz(cblk * 8 + cc, rblk)) = t[cc];
  };

  const int nsteps = (r1 - r0 + kWgRows - 1) / kWgRows;
  if (nsteps > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int c = 0; c < nsteps; ++c) {
    const int buf = c & 1;
    if (c + 1 < nsteps) load(c + 1);
    const uint8_t* At = lds[buf][0];
    const uint8_t* Bt = lds[buf][1];
#pragma unroll
    for (int ks = 0; ks < kWgRows / 16; ++ks) {
      const int cg = ks * 2 + (lane >> 5);  // 16-byte group of 8 rows this lane supplies
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = *reinterpret_cast<const bf16x8*>(At + wg_swz(wm * 64 + i * 32 + (lane & 31), cg));
        bv[i] = *reinterpret_cast<const bf16x8*>(Bt + wg_swz(wn * 64 + i * 32 + (lane & 31), cg));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (c + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j][q]: m = wm*64 + i*32 + 8*(q/4) + 4*(lane/32) + q%4, n = wn*64 + j*32 + lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = mt * kWgTile + wm * 64 + i * 32 + 8 * (q / 4) + 4 * (lane >> 5) + (q & 3);
      float* crow = m < a.m_split
                        ? a.C0 + (int64_t)e * a.m_split * a.N + (int64_t)m * a.N
                        : a.C1 + (int64_t)e * (a.M - a.m_split) * a.N +
                              (int64_t)(m - a.m_split) * a.N;
#pragma unroll
      for (int j = 0; j < 2; ++j) crow[nt * kWgTile + wn * 64 + j * 32 + (lane & 31)] = acc[i][j][q];
    }
}

// The same reduction in 256 x 256 workgroup tiles (M and N multiples of 256)
// for operands whose rows are the grouped rows themselves (a_mode = b_mode =
// 0: the token rows are gathered beforehand, bwd_gather_kernel). A stage is
// 32 rows; each thread loads four 16-byte row chunks per stage (a wave loads
// two whole rows of the tile per instruction), and four stages are in flight
// in registers. Stages go to LDS row-major, each row's 16-byte chunks
// XOR-permuted by the row (chunk c at c ^ 4 (row mod 4)), so that the
// transposing reads below are conflict free; two LDS buffers. The matrix cores
// take 8 consecutive rows of one column per lane, which ds_read_b64_tr_b16
// delivers from the row-major tile: in each 16-lane group, lane 4j + q reads 4
// columns of row j, and lane i receives column i of the 4 rows. Eight waves
// of 128 (m) x 64 (n); tiles in launch order (the hardware deals them round
// robin over the XCDs, so all XCDs work on one expert at a time, whose
// operands then fit the Infinity Cache), in groups of four m-tiles with m
// fastest.
constexpr int kWg2Tile = 256;
constexpr int kWg2GroupM = 4;
constexpr int kWlRows = 32;                      // rows per stage
constexpr int kWlHalf = kWlRows * kWg2Tile * 2;  // one operand of one stage, bytes

typedef short wl_v4s __attribute__((ext_vector_type(4)));

// Byte offset of (row, column) in a stage's operand tile.
__device__ __forceinline__ int wl_addr(int row, int col) {
  return row * (kWg2Tile * 2) + (((col >> 3) ^ (4 * (row & 3))) << 4) + (col & 7) * 2;
}

// The matrix-core operand of rows k0 .. k0 + 15 and columns c0 .. c0 + 31 for
// this lane (column c0 + lane % 32, rows k0 + 8 (lane / 32) + 0..7).
__device__ __forceinline__ bf16x8 wl_frag(const uint8_t* tile, int k0, int c0, int lane) {
  const int g = lane >> 4, t = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (t >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (t & 3);
  typedef __attribute__((address_space(3))) wl_v4s* lds_v4s;
  const wl_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(tile + wl_addr(row, col)));
  const wl_v4s hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(tile + wl_addr(row + 4, col)));
  const wl_v4s v8[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v8);
}

struct WlStage {
  uint4 v[4];
};

__global__ __launch_bounds__(512) void wgrad_lds_kernel(WgradArgs a) {
  __shared__ __align__(16) uint8_t lds[2][2][kWlHalf];  // [buffer][A, B]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int mtiles = a.M / kWg2Tile, ntiles = a.N / kWg2Tile;
  const int per_e = mtiles * ntiles;
  const int L = blockIdx.x;
  const int e = L / per_e, r = L % per_e;
  const int g = r / (kWg2GroupM * ntiles), rg = r % (kWg2GroupM * ntiles);
  const int gm = min(kWg2GroupM, mtiles - g * kWg2GroupM);
  const int mt = g * kWg2GroupM + rg % gm, nt = rg / gm;
  const int r0 = a.offset[e], r1 = a.offset[e + 1];

  // Loader role: threads 0..255 operand A, 256..511 operand B; chunk t + 256 u
  // (u = 0..3) of the stage's 32 rows x 32 chunks: row (t + 256 u) / 32,
  // chunk position t % 32.
  const int opnd = tid >> 8;
  const int t = tid & 255;
  const int stride = opnd ? a.b_stride : a.a_stride;
  const int colbase = (opnd ? nt : mt) * kWg2Tile + (t & 31) * 8;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(opnd ? a.B : a.A), (short)0, (int)(opnd ? a.b_bytes : a.a_bytes), 0x00020000);
  auto load = [&](int s, WlStage& R) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = (t >> 5) + 8 * u;
      const int p = r0 + s * kWlRows + row;
      const uint32_t off =
          p < r1 ? ((uint32_t)p * (uint32_t)stride + (uint32_t)colbase) * 2u : 0x80000000u;
      R.v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    }
  };
  auto store = [&](int buf, const WlStage& R) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = (t >> 5) + 8 * u;
      *reinterpret_cast<uint4*>(lds[buf][opnd] + row * (kWg2Tile * 2) +
                                (((t & 31) ^ (4 * (row & 3))) << 4)) = R.v[u];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  auto compute = [&](int buf) {
    const uint8_t* At = lds[buf][0];
    const uint8_t* Bt = lds[buf][1];
#pragma unroll
    for (int ks = 0; ks < kWlRows / 16; ++ks) {
      bf16x8 av[4], bv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = wl_frag(At, ks * 16, wm * 128 + i * 32, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = wl_frag(Bt, ks * 16, wn * 64 + j * 32, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };

  // Stage s is computed from LDS buffer s % 2. Register stage s % 4 receives
  // stage s three steps before, and is written to LDS at the end of step
  // s - 1, behind the barrier that follows the last step reading that buffer.
  // The guards (not breaks) keep the four register stages in registers; the
  // barriers run on every path (n is the same for the whole workgroup).
  const int n = (r1 - r0 + kWlRows - 1) / kWlRows;
  WlStage R0, R1, R2, R3;
  if (n > 0) load(0, R0);
  if (n > 1) load(1, R1);
  if (n > 2) load(2, R2);
  if (n > 0) store(0, R0);
  __syncthreads();
  for (int c = 0; c < n; c += 4) {
    if (c + 3 < n) load(c + 3, R3);
    compute(0);
    if (c + 1 < n) store(1, R1);
    __syncthreads();
    if (c + 4 < n) load(c + 4, R0);
    if (c + 1 < n) compute(1);
    if (c + 2 < n) store(0, R2);
    __syncthreads();
    if (c + 5 < n) load(c + 5, R1);
    if (c + 2 < n) compute(0);
    if (c + 3 < n) store(1, R3);
    __syncthreads();
    if (c + 6 < n) load(c + 6, R2);
    if (c + 3 < n) compute(1);
    if (c + 4 < n) store(0, R0);
    __syncthreads();
  }

  // acc[i][j][q]: m = wm*128 + i*32 + 8*(q/4) + 4*(lane/32) + q%4, n = wn*64 + j*32 + lane%32
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = mt * kWg2Tile + wm * 128 + i * 32 + 8 * (q / 4) + 4 * (lane >> 5) + (q & 3);
      float* crow = m < a.m_split
                        ? a.C0 + (int64_t)e * a.m_split * a.N + (int64_t)m * a.N
                        : a.C1 + (int64_t)e * (a.M - a.m_split) * a.N +
                              (int64_t)(m - a.m_split) * a.N;
#pragma unroll
      for (int j = 0; j < 2; ++j) crow[nt * kWg2Tile + wn * 64 + j * 32 + (lane & 31)] = acc[i][j][q];
    }
}

// xg, wdg rows and the zeroed pad rows of dgu (GatherArgs). One 16-byte chunk
// of one row per thread and step.
__global__ __launch_bounds__(256) void bwd_gather_kernel(GatherArgs a) {
  const int total = a.total[0];
  const int cpr = a.H / 8;                 // chunks per token row
  const int cpr2 = 2 * a.I / 8;            // chunks per dgu row
  const int64_t n = (int64_t)total * cpr;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(i / cpr), c = (int)(i % cpr);
    const int slot = a.sorted_slot[p];
    uint4 xv = make_uint4(0, 0, 0, 0), dv = make_uint4(0, 0, 0, 0);
    if (slot < a.S) {
      const size_t t = div_k(slot, a.k_magic);
      xv = *reinterpret_cast<const uint4*>(a.x + t * a.H + c * 8);
      const uint4 d = *reinterpret_cast<const uint4*>(a.dout + t * a.H + c * 8);
      const float w = a.topk_w[slot];
      const uint32_t in[4] = {d.x, d.y, d.z, d.w};
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        o[h] = f32x2_to_bf16x2(bf16_bits_to_f32(in[h] & 0xffffu) * w,
                               bf16_bits_to_f32(in[h] >> 16) * w);
      dv = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      for (int cc = c; cc < cpr2; cc += cpr)  // pad row: zero its dg, du
        *reinterpret_cast<uint4*>(a.dgu + (size_t)p * 2 * a.I + cc * 8) = make_uint4(0, 0, 0, 0);
    }
    *reinterpret_cast<uint4*>(a.xg + (size_t)p * a.H + c * 8) = xv;
    *reinterpret_cast<uint4*>(a.wdg + (size_t)p * a.H + c * 8) = dv;
  }
}

hipError_t launch_bwd_gather(const GatherArgs& a, hipStream_t st) {
  int64_t blocks = ((int64_t)a.cap * (a.H / 8) + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(bwd_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradArgs& a, hipStream_t st) {
  if (a.M % kWg2Tile == 0 && a.N % kWg2Tile == 0 && a.a_mode == 0 && a.b_mode == 0) {
    const int64_t blocks = (int64_t)a.E * (a.M / kWg2Tile) * (a.N / kWg2Tile);
    hipLaunchKernelGGL(wgrad_lds_kernel, dim3((unsigned)blocks), dim3(512), 0, st, a);
    return hipGetLastError();
  }
  if (a.M % kWgTile || a.N % kWgTile) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.E * (a.M / kWgTile) * (a.N / kWgTile);
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// --- router gradient and dx ---------------------------------------------------

// dl[t*k+j] = w_j (dw_j - sum_i w_i dw_i), dw_j = sum over the feature tiles of
// dwpart[t*k+j][.] in order. One thread per token.
__global__ __launch_bounds__(256) void bwd_dl_kernel(BwdArgs a) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.T) return;
  float dw[8], sw = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    const float* p = a.dwpart + (size_t)(t * a.k + j) * a.nparts;
    float v = p[0];
    for (int i = 1; i < a.nparts; ++i) v = v + p[i];
    dw[j] = v;
    sw = fmaf(a.topk_w[t * a.k + j], v, sw);
  }
  for (int j = 0; j < a.k; ++j) a.dl[t * a.k + j] = a.topk_w[t * a.k + j] * (dw[j] - sw);
}

// dx[t][h] = sum_j sum_g part[g][t*k+j][h] (j ascending, then the reduction
// split g) + sum_j dl[t*k+j] W_r[e_j][h] (j ascending). One float4 per thread
// and step.
__global__ __launch_bounds__(256) void bwd_dx_kernel(BwdArgs a) {
  const int64_t n4 = (int64_t)a.T * a.H / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i * 4 / a.H, h = i * 4 % a.H;
    const size_t split = (size_t)a.T * a.k * a.H;
    float4 s = *reinterpret_cast<const float4*>(a.part + (size_t)t * a.k * a.H + h);
    for (int u = 1; u < a.k * a.kg; ++u) {  // u = j*kg + g: slot j, reduction split g
      const int j = u / a.kg, g = u % a.kg;
      const float4 v =
          *reinterpret_cast<const float4*>(a.part + g * split + ((size_t)t * a.k + j) * a.H + h);
      s.x = s.x + v.x;
      s.y = s.y + v.y;
      s.z = s.z + v.z;
      s.w = s.w + v.w;
    }
    for (int j = 0; j < a.k; ++j) {
      const float d = a.dl[t * a.k + j];
      const uint2 wv = *reinterpret_cast<const uint2*>(
          a.w_router + (size_t)a.ids[t * a.k + j] * a.H + h);
      s.x = fmaf(d, bf16_bits_to_f32(wv.x & 0xffffu), s.x);
      s.y = fmaf(d, bf16_bits_to_f32(wv.x >> 16), s.y);
      s.z = fmaf(d, bf16_bits_to_f32(wv.y & 0xffffu), s.z);
      s.w = fmaf(d, bf16_bits_to_f32(wv.y >> 16), s.w);
    }
    *reinterpret_cast<float4*>(a.dx + (size_t)t * a.H + h) = s;
  }
}

// dW_r[e][h] = sum over the slots s of expert e of dl[s] x[s/k][h], db[e] the
// same sum of dl: first one partial per tile of block_m grouped rows (rows in
// ascending order; a tile holds one expert's rows), then, per expert, its
// tiles' partials in ascending order. Partial block: (tile, 512 columns), two
// columns per thread.
constexpr int kRouterCols = 512;

__global__ __launch_bounds__(256) void bwd_router_part_kernel(BwdArgs a) {
  const int tile = blockIdx.x;
  const int p0 = tile * a.bm;
  if (p0 >= a.total[0]) return;
  const int h = blockIdx.y * kRouterCols + 2 * threadIdx.x;
  const int S = a.T * a.k;
  float acc0 = 0.0f, acc1 = 0.0f, bacc = 0.0f;
  for (int p = p0; p < p0 + a.bm; ++p) {
    const int slot = a.sorted_slot[p];
    if ((unsigned)slot >= (unsigned)S) continue;  // pad row
    const float d = a.dl[slot];
    bacc = bacc + d;
    if (h < a.H) {
      const uint32_t xv = *reinterpret_cast<const uint32_t*>(
          a.x + (size_t)div_k((uint32_t)slot, a.k_magic) * a.H + h);
      acc0 = fmaf(d, bf16_bits_to_f32(xv & 0xffffu), acc0);
      acc1 = fmaf(d, bf16_bits_to_f32(xv >> 16), acc1);
    }
  }
  if (h < a.H)
    *reinterpret_cast<float2*>(a.rpart + (size_t)tile * a.H + h) = make_float2(acc0, acc1);
  if (blockIdx.y == 0 && threadIdx.x == 0) a.rpart[(size_t)a.ntiles * a.H + tile] = bacc;
}

__global__ __launch_bounds__(256) void bwd_router_sum_kernel(BwdArgs a) {
  const int e = blockIdx.y;
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  const int tb = a.offset[e] / a.bm, te = a.offset[e + 1] / a.bm;
  if (h < a.H) {
    float acc = 0.0f;
    for (int t = tb; t < te; ++t) acc = acc + a.rpart[(size_t)t * a.H + h];
    a.dw_router[(size_t)e * a.H + h] = acc;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.dbias) {
    float b = 0.0f;
    for (int t = tb; t < te; ++t) b = b + a.rpart[(size_t)a.ntiles * a.H + t];
    a.dbias[e] = b;
  }
}

hipError_t launch_bwd_router(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dl_kernel, dim3((a.T + 255) / 256), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t blocks = ((int64_t)a.T * a.H / 4 + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(bwd_dx_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_router_part_kernel, dim3(a.ntiles, (a.H + kRouterCols - 1) / kRouterCols),
                     dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_router_sum_kernel, dim3((a.H + 255) / 256, a.E), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
