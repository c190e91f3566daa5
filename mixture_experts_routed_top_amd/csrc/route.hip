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
// Two launch shapes:
//  - small batches: one workgroup per token; its four waves split the experts
//    (expert e on wave e%4) so that all loads of the token are in flight at
//    once, then wave 0 selects the top-k and quantises the row;
//  - large batches (E <= 16): one wave per two tokens (four for H <= 2048),
//    W_r staged once per workgroup in LDS (batched 16-byte copies), the
//    experts' logits folded together (fold_many).
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
__device__ __forceinline__ void select_topk(const RouteArgs& a, int t, int lane, float mine) {
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
    }
  }
}

// Per-token FP8 quantisation from the row chunks held in registers:
// s = amax/448 (1 if zero), code = e4m3fn(clamp(x/s)), fp32 divide.
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
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
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
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
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

template <int NCH>
__device__ __forceinline__ void load_row(const uint16_t* xr, int lane, int nchunk,
                                         uint4 (&xv)[NCH]) {
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    xv[i] = lane + 64 * i < nchunk
                ? *reinterpret_cast<const uint4*>(xr + (size_t)(lane + 64 * i) * 8)
                : make_uint4(0, 0, 0, 0);
}

// One workgroup per token; wave w computes the logits of experts w, w+4, ...
template <int NCH>
__global__ __launch_bounds__(256) void route_block_kernel(RouteArgs a) {
  __shared__ float logit[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nchunk = a.H / 8;
  for (int t = blockIdx.x; t < a.T; t += gridDim.x) {
    uint4 xv[NCH];
    load_row<NCH>(a.x + (size_t)t * a.H, lane, nchunk, xv);
    for (int e = wave; e < a.E; e += 4) {
      float l = fold64(lane_partial<NCH>(xv, a.w_router + (size_t)e * a.H, lane, nchunk));
      if (a.bias) l = l + a.bias[e];
      if (lane == 0) logit[e] = l;
    }
    __syncthreads();
    if (wave == 0) {
      select_topk(a, t, lane, lane < a.E ? logit[lane] : -__builtin_inff());
      if (a.x_q) quantise<NCH>(a, t, lane, nchunk, xv);
    }
    __syncthreads();
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

namespace {

template <int NCH>
hipError_t launch_nch(const RouteArgs& a, hipStream_t st) {
  const size_t wbytes = (size_t)a.E * a.H * 2;
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
    hipLaunchKernelGGL((route_block_kernel<NCH>), dim3(blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const int nch = (a.H / 8 + 63) / 64;  // chunks per lane
  if (nch <= 4) return launch_nch<4>(a, st);
  if (nch <= 8) return launch_nch<8>(a, st);
  if (nch <= kMaxChunks) return launch_nch<kMaxChunks>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
