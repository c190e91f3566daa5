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
//  - large batches (E <= 16): one wave per token, W_r staged once per
//    workgroup in LDS (batched 16-byte copies), several tokens per workgroup.
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
  if (a.logits && lane < E) a.logits[(size_t)t * E + lane] = mine;
  bool taken = lane >= E;
  float top_l[8];
  int top_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv = taken ? -__builtin_inff() : mine;
    int bi = taken ? 1 << 20 : lane;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
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
  // Correctly rounded x / s from one reciprocal per row (Markstein): with
  // r = RN(1/s), q0 = RN(x*r) is within one ulp of x/s, the remainder
  // x - s*q0 is exact in one fma, and RN(q0 + rem*r) is RN(x/s) whenever the
  // quotient is a normal number; smaller quotients encode to (signed) zero
  // either way, and copysign keeps the sign of a zero x.
  const float r = 1.0f / s;
  auto qdiv = [&](float x) {
    const float q0 = x * r;
    return clamp448(copysignf(fmaf(fmaf(-q0, s, x), r, q0), x));
  };
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

// One wave per token; W_r in LDS. All experts accumulate together (chunk by
// chunk, each expert's sum still in ascending h), so the LDS reads and FMAs of
// different experts overlap.
template <int NCH, int MAXE>
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
  for (int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); t < a.T; t += waves_total) {
    uint4 xv[NCH];
    load_row<NCH>(a.x + (size_t)t * a.H, lane, nchunk, xv);
    float acc[MAXE];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunk) {
        float xf[8];
        unpack8(xv[i], xf);
#pragma unroll
        for (int e = 0; e < MAXE; ++e) {
          if (e < a.E) {
            float wf[8];
            unpack8(*reinterpret_cast<const uint4*>(wr_lds + (size_t)e * a.H + (size_t)c * 8), wf);
            float s = acc[e];
#pragma unroll
            for (int j = 0; j < 8; ++j) s = s + xf[j] * wf[j];
            acc[e] = s;
          }
        }
      }
    }
    float mine = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
      if (e < a.E) {
        float l = fold64(acc[e]);
        if (a.bias) l = l + a.bias[e];
        if (lane == e) mine = l;
      }
    }
    select_topk(a, t, lane, mine);
    if (a.x_q) quantise<NCH>(a, t, lane, nchunk, xv);
  }
}

namespace {

template <int NCH>
hipError_t launch_nch(const RouteArgs& a, hipStream_t st) {
  const size_t wbytes = (size_t)a.E * a.H * 2;
  if (a.T >= 1024 && a.E <= 16 && wbytes <= (size_t)kRouteLdsBytes) {
    // W_r fits in LDS: about 4 tokens per wave, so staging it is amortised.
    int blocks = (a.T + 15) / 16;
    if (blocks > 2048) blocks = 2048;
    if (a.E <= 8)
      hipLaunchKernelGGL((route_wave_kernel<NCH, 8>), dim3(blocks), dim3(256), wbytes, st, a);
    else
      hipLaunchKernelGGL((route_wave_kernel<NCH, 16>), dim3(blocks), dim3(256), wbytes, st, a);
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
