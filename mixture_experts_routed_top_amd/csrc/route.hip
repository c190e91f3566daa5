// Router logits, top-k, renormalised routing weights and the per-token FP8 or
// per-block MXFP8 quantisation of x (the top-2 routing of the Mixtral layer in
// the FlyDSL-in-JAX talk summary, 8:14; the MX format of the PyTorch FlyDSL
// backend news item, "Grenzen und Folgen für Anwender").
//
// Fixed logit order (part of the layer's contract, so that ids can be compared
// bit for bit): element h goes to partial (h/8) mod 64; each partial adds its
// products in ascending h; the 64 partials are folded with p[l] += p[l+off]
// for off = 32..1. Lane l of a wave owns the 8-element chunks c = l, l+64, ...,
// which is exactly partial l, so each lane's running sum is that partial and
// the fold is a shuffle tree. A lane keeps its chunks of the token row in
// registers (16-byte loads, at most kMaxChunks per lane: H <= 64*8*kMaxChunks).
//
// Three launch shapes:
//  - a single token routed and grouped in one launch (moe_route_align): one
//    workgroup of eight waves, one expert each; then wave 0 selects the top-k
//    and groups the slots while wave 1 quantises the row;
//  - small batches: one workgroup per token; its eight waves (four for H >
//    4096) split the experts so that all loads of the token are in flight at
//    once, then wave 0 selects the top-k while wave 1 quantises the row;
//  - large batches (E <= 16): one wave per two tokens (four for H <= 2048),
//    W_r staged once per workgroup in LDS (batched 16-byte copies), the
//    experts' logits folded together (fold_many); for E <= 8 and H <= 4096,
//    W_r is staged as fp32 and each wave prefetches its next rows.
#include "align_small.h"
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kRouteLdsBytes = 64 * 1024;  // W_r staged in LDS when it fits
constexpr int kMaxChunks = 16;             // 8-element chunks per lane (H <= 8192)

__device__ __forceinline__ void unpack8(uint4 q, float v[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

// (value, index) ordering of the top-k: larger value first, then lower index.
__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// Lane exchanges without the LDS crossbar. dpp<CTRL>(v): v from another lane
// of the same 16-lane row (CTRL: 0xB1 / 0x4E quad permutes = lane ^ 1 / ^ 2,
// 0x141 / 0x140 half-row / row mirror, 0x128 rotate by 8 = lane ^ 8,
// 0x101..0x104 shift: lane l reads l + 1..4, 0 where that leaves the row).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Row swaps of two registers: swap32 exchanges the upper 32 lanes of a with the
// lower 32 lanes of b; swap16 exchanges the odd 16-lane rows of a with the
// even rows of b. Afterwards lane l of a and of b hold the two values that
// lanes l and l ^ 32 (l ^ 16) of a held, if l is in the lower half (an even
// row), and those of b otherwise.
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r =
      __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Largest of a non-negative value over the wave, in every lane: in-row
// reduction by DPP, then the four row results (max is exact in any order).
__device__ __forceinline__ float wave_max_nonneg(float m) {
  m = fmaxf(m, dpp<0xB1>(m));
  m = fmaxf(m, dpp<0x4E>(m));
  m = fmaxf(m, dpp<0x141>(m));
  m = fmaxf(m, dpp<0x140>(m));
  const int i = __float_as_int(m);
  const int r0 = __builtin_amdgcn_readlane(i, 0), r1 = __builtin_amdgcn_readlane(i, 16);
  const int r2 = __builtin_amdgcn_readlane(i, 32), r3 = __builtin_amdgcn_readlane(i, 48);
  // non-negative floats order like their bit patterns
  return __int_as_float(max(max(r0, r1), max(r2, r3)));
}

// This lane's partial of one logit: its chunks in ascending order, products
// added one by one (a bf16 x bf16 product is exact in fp32).
template <int NCH>
__device__ __forceinline__ float lane_partial(const uint4 (&xv)[NCH], const uint16_t* wrow,
                                              int lane, int nchunk) {
  uint4 wv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    if (lane + 64 * i < nchunk)
      wv[i] = *reinterpret_cast<const uint4*>(wrow + (size_t)(lane + 64 * i) * 8);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (lane + 64 * i < nchunk) {
      float xf[8], wf[8];
      unpack8(xv[i], xf);
      unpack8(wv[i], wf);
#pragma unroll
      for (int j = 0; j < 8; ++j) s = s + xf[j] * wf[j];
    }
  }
  return s;
}

__device__ __forceinline__ float fold64(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_down(v, off, 64);
  return __shfl(v, 0, 64);
}

// Top-k over the logits held by lanes e < E (lane e holds logit e), weights,
// outputs (lane 0 writes).
// With lds_ids, lane 0 also leaves the ids there, at t*k + j.
__device__ __forceinline__ void select_topk(const RouteArgs& a, int t, int lane, float mine,
                                            int32_t* lds_ids = nullptr) {
  const int E = a.E, k = a.k;
  int off0 = 32;
  while (off0 > 1 && off0 >= E) off0 >>= 1;
  if (a.logits && lane < E) a.logits[(size_t)t * E + lane] = mine;
  bool taken = lane >= E;
  float top_l[8];
  int top_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv = taken ? -__builtin_inff() : mine;
    int bi = taken ? 1 << 20 : lane;
    // Candidates sit in lanes e < E <= 2*off0, so the butterfly starts at off0:
    // lanes 0 .. 2*off0-1 then all hold the best pair (lane 0 writes).
    for (int off = off0; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    top_l[j] = bv;
    top_i[j] = bi;
    if (lane == bi) taken = true;
  }
  if (lane == 0) {
    float num[8], den = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      num[j] = expf(top_l[j] - top_l[0]);
      den += num[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      a.topk_ids[(size_t)t * k + j] = top_i[j];
      a.topk_w[(size_t)t * k + j] = num[j] / den;
      if (lds_ids) lds_ids[t * k + j] = top_i[j];
    }
  }
}

// Per-token FP8 quantisation from the row chunks held in registers:
// s = amax/448 (1 if zero), code = e4m3fn(clamp(x/s)), fp32 divide. lane_amax
// is this lane's largest |x| over its chunks; the row maximum is its fold.
template <int NCH>
__device__ __forceinline__ void quantise_row_amax(const RouteArgs& a, int t, int lane, int nchunk,
                                                  const uint4 (&xv)[NCH], float lane_amax) {
  const float amax = wave_max_nonneg(lane_amax);
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (lane == 0) a.x_scale[t] = s;
  // Correctly rounded x / s from one reciprocal per row (quant_div).
  const float r = 1.0f / s;
  auto qdiv = [&](float x) { return quant_div(x, s, r); };
  uint8_t* qr = a.x_q + (size_t)t * a.H;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunk) {
      float xf[8];
      unpack8(xv[i], xf);
      const uint32_t lo = f32x4_to_e4m3(qdiv(xf[0]), qdiv(xf[1]), qdiv(xf[2]), qdiv(xf[3]));
      const uint32_t hi = f32x4_to_e4m3(qdiv(xf[4]), qdiv(xf[5]), qdiv(xf[6]), qdiv(xf[7]));
      *reinterpret_cast<uint2*>(qr + (size_t)c * 8) = make_uint2(lo, hi);
    }
  }
}

template <int NCH>
__device__ __forceinline__ void quantise_row(const RouteArgs& a, int t, int lane, int nchunk,
                                             const uint4 (&xv)[NCH]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (lane + 64 * i < nchunk) {
      float xf[8];
      unpack8(xv[i], xf);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(xf[j]));
    }
  }
  quantise_row_amax<NCH>(a, t, lane, nchunk, xv, amax);
}

// MX block quantisation of the token row (MXFP8): each block of 32 values is
// four consecutive 8-value chunks, held by four adjacent lanes (chunk c on lane
// c mod 64), so the block maximum is two lane exchanges away. H is a multiple
// of 128, so the four lanes of a block are all in range or all out.
template <int NCH>
__device__ __forceinline__ void quantise_row_mx(const RouteArgs& a, int t, int lane, int nchunk,
                                                const uint4 (&xv)[NCH]) {
  uint8_t* qr = a.x_q + (size_t)t * a.H;
  uint8_t* sr = a.x_mx + (size_t)t * (a.H / 32);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    float xf[8];
    unpack8(xv[i], xf);  // zeros past the row (load_row)
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(xf[j]));
    m = fmaxf(m, dpp<0xB1>(m));  // lane ^ 1
    m = fmaxf(m, dpp<0x4E>(m));  // lane ^ 2
    const int x = mx_exponent(m);
    const float inv = mx_inv_scale(x);
    if (c < nchunk) {
      const uint32_t lo = f32x4_to_e4m3(clamp448(xf[0] * inv), clamp448(xf[1] * inv),
                                        clamp448(xf[2] * inv), clamp448(xf[3] * inv));
      const uint32_t hi = f32x4_to_e4m3(clamp448(xf[4] * inv), clamp448(xf[5] * inv),
                                        clamp448(xf[6] * inv), clamp448(xf[7] * inv));
      *reinterpret_cast<uint2*>(qr + (size_t)c * 8) = make_uint2(lo, hi);
      if ((lane & 3) == 0) sr[c / 4] = (uint8_t)(x + 127);
    }
  }
}

// Per-token (FP8) or per-block (MXFP8) quantisation of the row.
template <int NCH>
__device__ __forceinline__ void quantise(const RouteArgs& a, int t, int lane, int nchunk,
                                         const uint4 (&xv)[NCH]) {
  if (a.x_mx)
    quantise_row_mx<NCH>(a, t, lane, nchunk, xv);
  else
    quantise_row<NCH>(a, t, lane, nchunk, xv);
}

// The row's chunks c = lane + 64 i, zero past the row. Every load is issued
// (from a clamped address) and the zeros are selected afterwards, so the
// loads are all in flight together instead of one guarded load at a time.
template <int NCH>
__device__ __forceinline__ void load_row(const uint16_t* xr, int lane, int nchunk,
                                         uint4 (&xv)[NCH]) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    const uint4 v = *reinterpret_cast<const uint4*>(xr + (size_t)min(c, nchunk - 1) * 8);
    xv[i] = c < nchunk ? v : make_uint4(0, 0, 0, 0);
  }
}

// One workgroup of W waves per token (eight; four for rows past 4096 values,
// whose chunk registers would not fit two waves per SIMD); wave w computes the
// logits of experts w, w+W, ... (for W experts every W_r row is requested at
// once), then wave 0 takes the top-k while wave 1 quantises the row.
template <int NCH>
constexpr int block_waves() { return NCH <= 8 ? 8 : 4; }

template <int NCH>
__global__ __launch_bounds__(64 * block_waves<NCH>()) void route_block_kernel(RouteArgs a) {
  constexpr int W = block_waves<NCH>();
  __shared__ float logit[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nchunk = a.H / 8;
  for (int t = blockIdx.x; t < a.T; t += gridDim.x) {
    uint4 xv[NCH];
    load_row<NCH>(a.x + (size_t)t * a.H, lane, nchunk, xv);
    for (int e = wave; e < a.E; e += W) {
      float l = fold64(lane_partial<NCH>(xv, a.w_router + (size_t)e * a.H, lane, nchunk));
      if (a.bias) l = l + a.bias[e];
      if (lane == 0) logit[e] = l;
    }
    __syncthreads();
    if (wave == 0)
      select_topk(a, t, lane, lane < a.E ? logit[lane] : -__builtin_inff());
    else if (wave == 1 && a.x_q)
      quantise<NCH>(a, t, lane, nchunk, xv);
    __syncthreads();  // logit is rewritten for the next token
  }
}

// Tiny batches (T <= kTinyRouteTokens) with their grouping in the same launch:
// one workgroup of 8T waves. Each of waves 8t .. 8t+7 loads token t's row
// together with the W_r row of one expert (experts w, w+8, ... past eight) and
// folds that logit; after a barrier wave 8t takes the top-k and then sorts
// the T*k slots (align_small_wave) from the ids the top-k left in LDS, while
// wave 8t+1 quantises the row. The workgroup barrier and the wave's own order
// sequence the steps, so no synchronisation between workgroups is needed;
// the grouping is read by the next launch only. This saves a single-token
// decode call one launch.
template <int NCH>
__global__ __launch_bounds__(512 * kTinyRouteTokens) void route_align_tiny_kernel(RouteArgs a,
                                                                                 AlignArgs g) {
  __shared__ float logit[kTinyRouteTokens][64];
  __shared__ int32_t ids[kTinyRouteTokens * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = wave >> 3, w8 = wave & 7;  // blockDim = 512 * T: t < T
  const int nchunk = a.H / 8;
  uint4 xv[NCH];
  load_row<NCH>(a.x + (size_t)t * a.H, lane, nchunk, xv);
  for (int e = w8; e < a.E; e += 8) {
    float l = fold64(lane_partial<NCH>(xv, a.w_router + (size_t)e * a.H, lane, nchunk));
    if (a.bias) l = l + a.bias[e];
    if (lane == 0) logit[t][e] = l;
  }
  __syncthreads();
  static_assert(kTinyRouteTokens == 1, "the grouping below reads one token's ids");
  if (w8 == 0) {
    select_topk(a, t, lane, lane < a.E ? logit[t][lane] : -__builtin_inff(), ids);
    // The ids are in LDS from lane 0 of this same wave, whose LDS accesses
    // complete in order: a wave-scope fence suffices, and the grouping does
    // not wait for the quantisation running in wave 1.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    align_small_wave(g, ids, lane);
  } else if (w8 == 1 && a.x_q) {
    quantise<NCH>(a, t, lane, nchunk, xv);
  }
}

// The fixed fold (p[l] += p[l+off], off = 32 .. 1) of M experts' lane partials
// at once (M a power of two, 2 <= M <= 16). While an expert's partials still
// span several lanes, each step keeps half of the experts in the lower lanes
// of a pair and half in the upper ones, so one exchange serves two experts:
// lower lane l and upper lane l+off both form p[l] + p[l+off] (an fp32 sum is
// the same either way round), for the experts they keep. After log2(M) steps
// every lane holds one expert and the last steps are a plain butterfly. Each
// expert sees exactly the canonical pairs, so its logit is bit-identical to
// fold64's; the result for expert e sits in lane fold_lane<M>(e).
template <int M>
__device__ __forceinline__ int fold_lane(int e) {
  int l = 0;
#pragma unroll
  for (int b = 0; (1 << b) < M; ++b)  // bit b of e (from the top) picks lane bit 5-b
    if (e & (M >> (b + 1))) l |= 32 >> b;
  return l;
}

// One transposed step at distance OFF over the first 2*HALF values.
template <int HALF, int OFF, int M>
__device__ __forceinline__ void fold_step(float (&v)[M], int lane) {
  const bool up = (lane & OFF) != 0;
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float keep = up ? v[HALF + i] : v[i];
    const float send = up ? v[i] : v[HALF + i];
    const float recv = __shfl_xor(send, OFF, 64);
    v[i] = up ? recv + keep : keep + recv;  // p[lower] + p[upper]
  }
  if constexpr (HALF > 1) fold_step<HALF / 2, OFF / 2, M>(v, lane);
}

template <int M>
__device__ __forceinline__ float fold_many(float (&v)[M], int lane) {
  static_assert(M >= 2 && M <= 16 && (M & (M - 1)) == 0, "experts folded together");
  fold_step<M / 2, 32, M>(v, lane);
  float r = v[0];
#pragma unroll
  for (int off = 32 / M; off >= 1; off >>= 1) {
    const float o = __shfl_xor(r, off, 64);
    r = (lane & off) ? o + r : r + o;
  }
  return r;
}

// TPW tokens per wave at once; W_r in LDS. The TPW rows are loaded together,
// then each W_r chunk is read from LDS and converted once for all TPW tokens;
// each (token, expert) sum still adds its products in ascending h.
template <int NCH, int MAXE, int TPW>
__global__ __launch_bounds__(256) void route_wave_kernel(RouteArgs a) {
  extern __shared__ __align__(16) uint16_t wr_lds[];
  const int lane = threadIdx.x & 63;
  const int nchunk = a.H / 8;
  {
    // Stage W_r: 16 independent 16-byte loads per thread in flight per batch.
    const int n16 = a.E * a.H / 8;
    const uint4* src = reinterpret_cast<const uint4*>(a.w_router);
    uint4* dst = reinterpret_cast<uint4*>(wr_lds);
    for (int b = 0; b < n16; b += 256 * 16) {
      uint4 tmp[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tmp[i] = src[min(b + (int)threadIdx.x + 256 * i, n16 - 1)];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int idx = b + threadIdx.x + 256 * i;
        if (idx < n16) dst[idx] = tmp[i];
      }
    }
    __syncthreads();
  }
  const int waves_total = gridDim.x * (blockDim.x / 64);
  for (int t0 = (blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)) * TPW; t0 < a.T;
       t0 += waves_total * TPW) {
    uint4 xv[TPW][NCH];
#pragma unroll
    for (int u = 0; u < TPW; ++u)  // rows past T repeat the last one (not written)
      load_row<NCH>(a.x + (size_t)min(t0 + u, a.T - 1) * a.H, lane, nchunk, xv[u]);
    float acc[TPW][MAXE];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int e = 0; e < MAXE; ++e) acc[u][e] = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunk) {
        float xf[TPW][8];
#pragma unroll
        for (int u = 0; u < TPW; ++u) unpack8(xv[u][i], xf[u]);
#pragma unroll
        for (int e = 0; e < MAXE; ++e) {
          if (e < a.E) {
            float wf[8];
            unpack8(*reinterpret_cast<const uint4*>(wr_lds + (size_t)e * a.H + (size_t)c * 8), wf);
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
              float s = acc[u][e];
#pragma unroll
              for (int j = 0; j < 8; ++j) s = s + xf[u][j] * wf[j];
              acc[u][e] = s;
            }
          }
        }
      }
    }
    const int src_lane = fold_lane<MAXE>(lane < MAXE ? lane : 0);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = t0 + u;
      const float folded = fold_many<MAXE>(acc[u], lane);
      float mine = __shfl(folded, src_lane, 64);  // lane e < E: logit of expert e
      if (a.bias && lane < a.E) mine = mine + a.bias[lane];
      if (lane >= a.E) mine = -__builtin_inff();
      if (t < a.T) {
        select_topk(a, t, lane, mine);
        if (a.x_q) quantise<NCH>(a, t, lane, nchunk, xv[u]);
      }
    }
  }
}

// Large batches with E <= 8 and H <= 4096: W_r staged once per workgroup in
// LDS as fp32, in two planes (the first and the last four values of every
// 8-element chunk, so that a wave's 16-byte reads of one plane are contiguous
// and need no conversion per token), expert e's chunks at a fixed stride of
// 64 * NCH (so every read address is one register plus an immediate), eight
// waves per workgroup. Each wave takes TPW tokens per pass and loads the rows
// of its next pass before computing the current one; its first rows are
// requested before W_r is staged. The FP8 row maxima are taken in the logit
// loop from the values unpacked there. The fold and the top-k exchange values
// through row swaps and DPP moves rather than LDS permutes. Sums, folds, top-k
// and quantisation are those of the kernels above, bit for bit.
constexpr int kWideWaves = 8;

template <int NCH, int TPW>
__device__ __forceinline__ void load_rows(const RouteArgs& a, int t0, int lane, int nchunk,
                                          uint4 (&xv)[TPW][NCH]) {
#pragma unroll
  for (int u = 0; u < TPW; ++u)  // rows past T repeat the last one (not written)
    load_row<NCH>(a.x + (size_t)min(t0 + u, a.T - 1) * a.H, lane, nchunk, xv[u]);
}

// fold_many<8> with its exchanges done by row swaps and DPP moves: the steps
// at distance 32 and 16 are exactly what swap32 / swap16 leave in a register
// pair (each lane then adds the two values it holds), the step at 8 is a
// rotate within the row, and the last three steps need the correct sum only
// in lanes l = 0 mod 8, which read lane l + off. The pairs added are the
// canonical ones, so each logit is bit-identical to fold64's; expert e's sits
// in lane fold_lane<8>(e).
__device__ __forceinline__ float fold8_swaps(float (&v)[8], int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    swap32(v[i], v[4 + i]);
    v[i] = v[i] + v[4 + i];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    swap16(v[i], v[2 + i]);
    v[i] = v[i] + v[2 + i];
  }
  const bool up = (lane & 8) != 0;
  const float keep = up ? v[1] : v[0], send = up ? v[0] : v[1];
  float r = keep + dpp<0x128>(send);
  r = r + dpp<0x104>(r);
  r = r + dpp<0x102>(r);
  r = r + dpp<0x101>(r);
  return r;
}

// Order-preserving integer key of a finite float (larger value, larger key);
// -0 is taken as +0 first, so equal values get equal keys. Key 0 is below
// every finite value's.
__device__ __forceinline__ unsigned order_key(float v) {
  const unsigned b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ unsigned dppu(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}

// Largest / smallest over each group of eight lanes (quad permutes, then the
// half-row mirror, which pairs the two quads of a group).
__device__ __forceinline__ unsigned max8(unsigned m) {
  m = max(m, dppu<0xB1>(m));
  m = max(m, dppu<0x4E>(m));
  return max(m, dppu<0x141>(m));
}
__device__ __forceinline__ unsigned min8(unsigned m) {
  m = min(m, dppu<0xB1>(m));
  m = min(m, dppu<0x4E>(m));
  return min(m, dppu<0x141>(m));
}

// select_topk for E <= 8 from the folded logits r (expert e's in lane
// fold_lane<8>(e)): lane e < E takes expert e's logit plus its bias and an
// integer key of it; each of the k rounds finds the largest key over lanes
// 0..7, then the lowest lane holding it (the lower index wins a tie), and
// retires that lane. Lane 0 writes ids and weights, lanes e < E the logits.
__device__ __forceinline__ void select_topk8(const RouteArgs& a, int t, int lane, float r) {
  const int E = a.E, k = a.k;
  float lv = __shfl(r, fold_lane<8>(lane & 7), 64);
  if (a.bias && lane < E) lv = lv + a.bias[lane];
  if (a.logits && lane < E) a.logits[(size_t)t * E + lane] = lv;
  unsigned key = lane < E ? order_key(lv) : 0u;
  float top_l[8];
  int top_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const unsigned m = max8(key);
    const unsigned w = __builtin_amdgcn_readfirstlane(min8(key == m ? (unsigned)lane : 8u));
    top_i[j] = (int)w;
    top_l[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), w));
    if ((unsigned)lane == w) key = 0u;
  }
  if (lane == 0) {
    float num[8], den = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      num[j] = expf(top_l[j] - top_l[0]);
      den += num[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      a.topk_ids[(size_t)t * k + j] = top_i[j];
      a.topk_w[(size_t)t * k + j] = num[j] / den;
    }
  }
}

template <int NCH, int TPW>
__device__ __forceinline__ void route_rows(const RouteArgs& a, const float4* plo,
                                           const float4* phi, int t0, int lane, int nchunk,
                                           const uint4 (&xv)[TPW][NCH]) {
  float acc[TPW][8], amax[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    amax[u] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
  }
  // Experts past E have zero planes: their sums stay +0 and are masked after
  // the fold, so the expert loop needs no branch and a chunk's eight W_r reads
  // are issued together. The chunk guard (lanes past the row, only where H is
  // not a multiple of 512) also keeps each chunk a block of its own, so the
  // compiler does not hoist every read of the pass (512 values per lane).
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunk) {
      float xf[TPW][8];
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        unpack8(xv[u][i], xf[u]);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax[u] = fmaxf(amax[u], fabsf(xf[u][j]));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 lo = plo[e * (64 * NCH) + c], hi = phi[e * (64 * NCH) + c];
        const float wf[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          float s = acc[u][e];
#pragma unroll
          for (int j = 0; j < 8; ++j) s = s + xf[u][j] * wf[j];
          acc[u][e] = s;
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = t0 + u;
    const float r = fold8_swaps(acc[u], lane);
    if (t < a.T) {
      select_topk8(a, t, lane, r);
      if (a.x_q) {
        if (a.x_mx)
          quantise_row_mx<NCH>(a, t, lane, nchunk, xv[u]);
        else
          quantise_row_amax<NCH>(a, t, lane, nchunk, xv[u], amax[u]);
      }
    }
  }
}

template <int NCH, int TPW>
__global__ __launch_bounds__(64 * kWideWaves) void route_wide_kernel(RouteArgs a) {
  constexpr int kPlane = 8 * NCH * 64;  // chunks of E <= 8 rows of H <= 512 * NCH
  __shared__ float4 wl[2 * kPlane];
  const int lane = threadIdx.x & 63;
  const int nchunk = a.H / 8;
  const int step = gridDim.x * kWideWaves * TPW;
  int t0 = (blockIdx.x * kWideWaves + (threadIdx.x >> 6)) * TPW;
  uint4 xa[TPW][NCH], xb[TPW][NCH];
  if (t0 < a.T) load_rows<NCH, TPW>(a, t0, lane, nchunk, xa);
  {
    // Stage W_r: plane index e * 64 * NCH + c holds chunk c of expert e's row
    // (the first four values in the low plane, the last four in the high
    // one), zero for c >= H/8 or e >= E; NCH 16-byte loads per thread.
    const uint4* src = reinterpret_cast<const uint4*>(a.w_router);
    uint4 tmp[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int at = threadIdx.x + 64 * kWideWaves * i;  // < kPlane
      const int e = at / (64 * NCH), c = at % (64 * NCH);
      tmp[i] = e < a.E && c < nchunk ? src[e * nchunk + c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int at = threadIdx.x + 64 * kWideWaves * i;
      float f[8];
      unpack8(tmp[i], f);
      wl[at] = make_float4(f[0], f[1], f[2], f[3]);
      wl[kPlane + at] = make_float4(f[4], f[5], f[6], f[7]);
    }
    __syncthreads();
  }
  const float4* plo = wl;
  const float4* phi = wl + kPlane;
  while (t0 < a.T) {  // wave-uniform: t0 is the same for all lanes of a wave
    const int t1 = t0 + step;
    if (t1 < a.T) load_rows<NCH, TPW>(a, t1, lane, nchunk, xb);
    route_rows<NCH, TPW>(a, plo, phi, t0, lane, nchunk, xa);
    if (t1 >= a.T) break;
    const int t2 = t1 + step;
    if (t2 < a.T) load_rows<NCH, TPW>(a, t2, lane, nchunk, xa);
    route_rows<NCH, TPW>(a, plo, phi, t1, lane, nchunk, xb);
    t0 = t2;
  }
}

namespace {

template <int NCH>
hipError_t launch_nch(const RouteArgs& a, hipStream_t st) {
  const size_t wbytes = (size_t)a.E * a.H * 2;
  if constexpr (NCH <= 8) {
    if (a.T >= 1024 && a.E <= 8) {
      // One workgroup per CU (128 KiB of LDS at H = 4096), two per CU below;
      // one token per wave and pass (more, shorter passes overlap the row
      // loads with the arithmetic better than two tokens per pass).
      constexpr int TPW = 1;
      const int cap = NCH <= 4 ? 512 : 256;
      int blocks = (a.T + kWideWaves * TPW - 1) / (kWideWaves * TPW);
      if (blocks > cap) blocks = cap;
      hipLaunchKernelGGL((route_wide_kernel<NCH, TPW>), dim3(blocks), dim3(64 * kWideWaves), 0,
                         st, a);
      return hipGetLastError();
    }
  }
  if (a.T >= 1024 && a.E <= 16 && wbytes <= (size_t)kRouteLdsBytes) {
    // W_r fits in LDS: TPW tokens per wave per pass, two workgroups per CU
    // (the LDS limit), so at most 512 workgroups each staging W_r once.
    constexpr int TPW = NCH <= 4 ? 4 : 2;
    int blocks = (a.T + 4 * TPW - 1) / (4 * TPW);
    if (blocks > 512) blocks = 512;
    if (a.E <= 8)
      hipLaunchKernelGGL((route_wave_kernel<NCH, 8, TPW>), dim3(blocks), dim3(256), wbytes, st, a);
    else
      hipLaunchKernelGGL((route_wave_kernel<NCH, 16, TPW>), dim3(blocks), dim3(256), wbytes, st,
                         a);
  } else {
    const int blocks = a.T < 4096 ? a.T : 4096;
    hipLaunchKernelGGL((route_block_kernel<NCH>), dim3(blocks), dim3(64 * block_waves<NCH>()), 0,
                       st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_align(const RouteArgs& a, const AlignArgs& g, hipStream_t st) {
  const int nch = (a.H / 8 + 63) / 64;
  if (a.T >= 1 && a.T <= kTinyRouteTokens && a.k <= 8 && g.S <= kSmallSlots && nch <= 8) {
    const dim3 block(512 * a.T);
    if (nch <= 4)
      hipLaunchKernelGGL((route_align_tiny_kernel<4>), dim3(1), block, 0, st, a, g);
    else
      hipLaunchKernelGGL((route_align_tiny_kernel<8>), dim3(1), block, 0, st, a, g);
    return hipGetLastError();
  }
  hipError_t err = launch_route(a, st);
  if (err != hipSuccess) return err;
  return launch_align(g, st);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const int nch = (a.H / 8 + 63) / 64;  // chunks per lane
  if (nch <= 4) return launch_nch<4>(a, st);
  if (nch <= 8) return launch_nch<8>(a, st);
  if (nch <= kMaxChunks) return launch_nch<kMaxChunks>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
