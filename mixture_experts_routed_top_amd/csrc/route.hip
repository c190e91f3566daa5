// Router logits, top-k, renormalised routing weights and the per-token FP8
// quantisation of x (the top-2 routing of the Mixtral layer in the FlyDSL-in-JAX
// talk summary, 8:14).
//
// One wavefront per token. Lane l owns the 8-element chunks c = l, l+64, ...
// of the row, which is exactly the partial-sum assignment of the layer's
// fixed logit order (element h -> partial (h/8) mod 64), so each lane's
// running sum is that partial; the 64 partials are folded with shuffles at
// offsets 32..1. Chunks are 16-byte loads: one wave reads 1 KB contiguous.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// W_r staged in LDS when it fits (Mixtral: 8 x 4096 x 2 B = 64 KB).
constexpr int kRouteLdsBytes = 64 * 1024;

__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  uint4 q = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
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

template <int MAXE, bool LDS_W>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  extern __shared__ __align__(16) uint16_t wr_lds[];
  const int lane = threadIdx.x & 63;
  const int H = a.H, E = a.E, k = a.k;
  const int nchunk = H / 8;

  if constexpr (LDS_W) {
    const int n16 = E * H / 8;  // 16-byte pieces of W_r
    for (int i = threadIdx.x; i < n16; i += blockDim.x)
      reinterpret_cast<uint4*>(wr_lds)[i] = reinterpret_cast<const uint4*>(a.w_router)[i];
    __syncthreads();
  }
  const uint16_t* wr = LDS_W ? wr_lds : a.w_router;

  const int waves_total = gridDim.x * (blockDim.x / 64);
  for (int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); t < a.T; t += waves_total) {
    const uint16_t* xr = a.x + (size_t)t * H;
    float acc[MAXE];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) acc[e] = 0.0f;
    float amax = 0.0f;

    for (int c = lane; c < nchunk; c += 64) {
      float xv[8];
      load8(xr + c * 8, xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(xv[i]));
#pragma unroll
      for (int e = 0; e < MAXE; ++e) {
        if (e < E) {
          float wv[8];
          load8(wr + (size_t)e * H + c * 8, wv);
          float s = acc[e];
#pragma unroll
          for (int i = 0; i < 8; ++i) s = s + xv[i] * wv[i];  // product exact in fp32
          acc[e] = s;
        }
      }
    }

    // Fold the 64 partials: p[l] += p[l+off], off = 32..1; lane 0 ends with the logit.
    float mine = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
      if (e < E) {
        float v = acc[e];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_down(v, off, 64);
        float l = __shfl(v, 0, 64);
        if (a.bias) l = l + a.bias[e];
        if (lane == e) mine = l;
      }
    }
    if (a.logits && lane < E) a.logits[(size_t)t * E + lane] = mine;

    // k rounds of a wave-wide argmax over the lanes e < E not yet taken.
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
        float ov = __shfl_xor(bv, off, 64);
        int oi = __shfl_xor(bi, off, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
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

    if (a.x_q) {
      // amax over the row (exact, order free), scale, then the fp32 divide.
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
      if (lane == 0) a.x_scale[t] = s;
      uint8_t* qr = a.x_q + (size_t)t * H;
      for (int c = lane; c < nchunk; c += 64) {
        float xv[8];
        load8(xr + c * 8, xv);
        uint32_t lo = f32x4_to_e4m3(clamp448(xv[0] / s), clamp448(xv[1] / s),
                                    clamp448(xv[2] / s), clamp448(xv[3] / s));
        uint32_t hi = f32x4_to_e4m3(clamp448(xv[4] / s), clamp448(xv[5] / s),
                                    clamp448(xv[6] / s), clamp448(xv[7] / s));
        *reinterpret_cast<uint2*>(qr + c * 8) = make_uint2(lo, hi);
      }
    }
  }
}

template <int MAXE>
static hipError_t launch_route_e(const RouteArgs& a, hipStream_t st) {
  const size_t wbytes = (size_t)a.E * a.H * 2;
  const int blocks_needed = (a.T + 3) / 4;
  if (wbytes <= (size_t)kRouteLdsBytes) {
    // Enough tokens per workgroup to amortise staging W_r in LDS.
    int blocks = blocks_needed < 1024 ? blocks_needed : 1024;
    hipLaunchKernelGGL((route_kernel<MAXE, true>), dim3(blocks), dim3(256), wbytes, st, a);
  } else {
    int blocks = blocks_needed < 4096 ? blocks_needed : 4096;
    hipLaunchKernelGGL((route_kernel<MAXE, false>), dim3(blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.E <= 8) return launch_route_e<8>(a, st);
  if (a.E <= 16) return launch_route_e<16>(a, st);
  if (a.E <= 32) return launch_route_e<32>(a, st);
  return launch_route_e<64>(a, st);
}

}  // namespace moe
