// Grouped expert GEMMs of the routed MoE layer on gfx950 matrix cores: stage 1
// (gather-on-load + gate/up GEMM + SwiGLU) and stage 2 (down GEMM + weighted
// per-slot scatter), plus the FP8 requantisation of the intermediate and the
// fixed-order combine. The fusion of gather, group GEMM, SwiGLU and scatter is
// the routed MoE GEMM of the FlyDSL-in-JAX talk summary (5:56); the tiling
// here is this library's own.
//
// Roles: the matrix-core A operand is a 16-row block of (preshuffled) expert
// weights, the B operand a 16-token block of activations, so each lane's four
// accumulators are four consecutive output features of one token:
//   acc[feature 4*(lane/16) + r][token lane%16], r = 0..3.
// A workgroup is 4 waves. Waves split the tile's features (and, for decode
// shapes, the reduction); all waves share the token tile, which is staged
// through LDS in 256-byte-per-row chunks (double buffered; the gather of
// token rows happens in that load). Weight fragments go straight from HBM to
// registers: the preshuffle made each wave's fragment one contiguous block.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

template <int DT>
struct Frag;
template <>
struct Frag<0> {  // bf16, v_mfma_f32_16x16x32_bf16: 8 values (16 B) per lane
  static constexpr int ES = 2, KE = 32, WV = 1;
  static __device__ __forceinline__ f32x4 mma(const uint4* w, const uint4* x, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[0]),
                                                   __builtin_bit_cast(bf16x8, x[0]), c, 0, 0, 0);
  }
};
template <>
struct Frag<1> {  // e4m3fn, v_mfma_f32_16x16x128_f8f6f4 (both formats fp8): 32 B per lane
  static constexpr int ES = 1, KE = 128, WV = 2;
  static __device__ __forceinline__ f32x4 mma(const uint4* w, const uint4* x, f32x4 c) {
    i32x8 a = {(int)w[0].x, (int)w[0].y, (int)w[0].z, (int)w[0].w,
               (int)w[1].x, (int)w[1].y, (int)w[1].z, (int)w[1].w};
    i32x8 b = {(int)x[0].x, (int)x[0].y, (int)x[0].z, (int)x[0].w,
               (int)x[1].x, (int)x[1].y, (int)x[1].z, (int)x[1].w};
    // format codes 0/0 = e4m3 for A and B; scale operands 0 select the unscaled form.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

constexpr int kChunk = 256;           // bytes of reduction per row per LDS stage
constexpr int kRowBytes = kChunk + 16;  // padded LDS row: conflict-free 16-B reads

template <int DT, int MT, int KSPLIT>
constexpr int gemm_lds_bytes() {
  return 2 * KSPLIT * 16 * MT * kRowBytes;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <int DT, int STAGE, int MT, int NI, int KSPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  using F = Frag<DT>;
  constexpr int ES = F::ES, KE = F::KE, WV = F::WV;
  constexpr int KB = KE * ES;          // bytes per row per k-step (64 / 128)
  constexpr int LB = KB / 4;           // bytes per lane per operand (16 / 32)
  constexpr int KS = kChunk / KB;      // k-steps per chunk (4 / 2)
  constexpr int CE = kChunk / ES;      // elements per chunk (128 / 256)
  constexpr int BM = 16 * MT;
  constexpr int WN = 4 / KSPLIT;       // waves along features
  constexpr int WGN = WN * NI * 16;    // features per workgroup
  constexpr int PIECES = KSPLIT * BM * 16;
  constexpr int PPT = PIECES / 256;    // 16-byte activation pieces per thread per chunk
  constexpr int LDS = gemm_lds_bytes<DT, MT, KSPLIT>();
  static_assert(PIECES % 256 == 0, "tile too small for the staging layout");
  static_assert(STAGE == 2 || (NI % 2 == 0 && KSPLIT == 1), "stage 1 pairs gate/up blocks");
  static_assert(KSPLIT == 1 || (KSPLIT - 1) * WN * MT * NI * 4 * 64 * 4 <= LDS, "reduction space");
  static_assert(STAGE == 2 || DT == 0 || WN * BM * 4 <= LDS, "amax space");

  __shared__ __align__(16) uint8_t lds[LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wk = wave / WN;

  const int ntiles = a.n_mtiles * a.n_ntiles;
  const int logical = xcd_remap(blockIdx.x, ntiles);
  const int mtile = logical % a.n_mtiles, ntile = logical / a.n_mtiles;
  const int total = *a.total_padded;
  const int row0 = mtile * BM;
  if (row0 >= total) return;
  const int e = a.tile_expert[mtile];
  const int S = a.T * a.k;
  const int Kw = a.K / KSPLIT;  // reduction elements per wave
  const int nchunks = Kw / CE;

  // Activation pieces this thread stages each chunk (row gather happens here).
  const uint8_t* src[PPT];
  int loff[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int q = tid + 256 * j;
    const int ks = q / (BM * 16), r = (q / 16) % BM, c16 = q % 16;
    const int p = row0 + r;
    const uint8_t* rowp;
    if constexpr (STAGE == 1) {
      const int slot = a.sorted_slot[p];
      rowp = slot < S ? a.X + (size_t)(slot / a.k) * a.K * ES : nullptr;
    } else {
      rowp = a.X + (size_t)p * a.K * ES;
    }
    src[j] = rowp ? rowp + (size_t)ks * Kw * ES + c16 * 16 : nullptr;
    loff[j] = (ks * BM + r) * kRowBytes + c16 * 16;
  }

  // This wave's weight fragments: feature blocks rb0 .. rb0+NI-1, K blocks of its split.
  const size_t kblocks = (size_t)a.K / KE;
  const int rb0 = (ntile * WGN + wn * NI * 16) / 16;
  const uint8_t* wbase = a.W + (size_t)e * a.N * a.K * ES +
                         ((size_t)rb0 * kblocks + (size_t)wk * (Kw / KE)) * 64 * LB + lane * LB;

  f32x4 acc[MT][NI];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NI; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 xr[PPT];
  uint4 wc[KS][NI][WV], wx[KS][NI][WV];

  auto load_x = [&](int c) {
#pragma unroll
    for (int j = 0; j < PPT; ++j)
      xr[j] = src[j] ? *reinterpret_cast<const uint4*>(src[j] + (size_t)c * kChunk)
                     : make_uint4(0, 0, 0, 0);
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < PPT; ++j)
      *reinterpret_cast<uint4*>(lds + buf * (LDS / 2) + loff[j]) = xr[j];
  };
  auto load_w = [&](int c, uint4 (&w)[KS][NI][WV]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int n = 0; n < NI; ++n)
#pragma unroll
        for (int v = 0; v < WV; ++v)
          w[ks][n][v] = *reinterpret_cast<const uint4*>(
              wbase + ((size_t)n * kblocks + (size_t)c * KS + ks) * 64 * LB + v * 16);
  };
  auto compute = [&](int buf, uint4 (&w)[KS][NI][WV]) {
    const uint8_t* xl = lds + buf * (LDS / 2) + wk * BM * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        uint4 xf[WV];
        const uint8_t* pp = xl + (m * 16 + (lane & 15)) * kRowBytes + ks * KB + (lane >> 4) * LB;
#pragma unroll
        for (int v = 0; v < WV; ++v) xf[v] = *reinterpret_cast<const uint4*>(pp + 16 * v);
#pragma unroll
        for (int n = 0; n < NI; ++n) acc[m][n] = F::mma(w[ks][n], xf, acc[m][n]);
      }
    }
  };

  load_x(0);
  load_w(0, wc);
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) {
      load_x(c + 1);
      load_w(c + 1, wx);
    }
    compute(c & 1, wc);
    if (more) store_x((c + 1) & 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int n = 0; n < NI; ++n)
#pragma unroll
          for (int v = 0; v < WV; ++v) wc[ks][n][v] = wx[ks][n][v];
    }
  }

  if constexpr (KSPLIT > 1) {
    // Fixed-order reduction of the reduction splits: wave 0's sum, + split 1, + split 2, ...
    float* red = reinterpret_cast<float*>(lds);
    constexpr int NV = MT * NI * 4;
    if (wk > 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NI; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[(((wk - 1) * WN + wn) * NV + (m * NI + n) * 4 + r) * 64 + lane] = acc[m][n][r];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int s = 1; s < KSPLIT; ++s)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NI; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[m][n][r] += red[(((s - 1) * WN + wn) * NV + (m * NI + n) * 4 + r) * 64 + lane];
  }

  const int tok = lane & 15, fq = (lane >> 4) * 4;
  if constexpr (STAGE == 1) {
    // SwiGLU epilogue: gate block 2j and up block 2j+1 hold the same act columns.
    uint16_t* act = reinterpret_cast<uint16_t*>(a.out);
    const float* sg = DT == 1 ? a.w_scale + (size_t)e * 2 * a.I : nullptr;
    float amax[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int p = row0 + m * 16 + tok;
      float xs = 1.0f;
      if constexpr (DT == 1) {
        const int slot = a.sorted_slot[p];
        xs = slot < S ? a.x_scale[slot / a.k] : 0.0f;
      }
      amax[m] = 0.0f;
#pragma unroll
      for (int j = 0; j < NI / 2; ++j) {
        const int i0 = (ntile * WGN + wn * NI * 16) / 2 + j * 16 + fq;
        float gs[4] = {1.f, 1.f, 1.f, 1.f}, us[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (DT == 1) {
          float4 g4 = *reinterpret_cast<const float4*>(sg + i0);
          float4 u4 = *reinterpret_cast<const float4*>(sg + a.I + i0);
          gs[0] = g4.x * xs; gs[1] = g4.y * xs; gs[2] = g4.z * xs; gs[3] = g4.w * xs;
          us[0] = u4.x * xs; us[1] = u4.y * xs; us[2] = u4.z * xs; us[3] = u4.w * xs;
        }
        uint32_t b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float g = acc[m][2 * j][r] * gs[r];
          const float u = acc[m][2 * j + 1][r] * us[r];
          b[r] = f32_to_bf16_bits(silu(g) * u);
          amax[m] = fmaxf(amax[m], fabsf(bf16_bits_to_f32(b[r])));
        }
        *reinterpret_cast<uint2*>(act + (size_t)p * a.I + i0) =
            make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
    }
    if constexpr (DT == 1) {
      // Partial row maxima of this workgroup's columns: lanes, then waves.
      float* wmax = reinterpret_cast<float*>(lds);
      __syncthreads();  // LDS reuse after the main loop's last reads
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float v = amax[m];
        v = fmaxf(v, __shfl_xor(v, 16, 64));
        v = fmaxf(v, __shfl_xor(v, 32, 64));
        if (lane < 16) wmax[wn * BM + m * 16 + lane] = v;
      }
      __syncthreads();
      if (tid < BM) {
        float v = wmax[tid];
#pragma unroll
        for (int w = 1; w < WN; ++w) v = fmaxf(v, wmax[w * BM + tid]);
        a.amax_part[(size_t)(row0 + tid) * a.n_ntiles + ntile] = v;
      }
    }
  } else {
    // Down-projection epilogue: weighted per-slot partials, one writer per element.
    float* part = reinterpret_cast<float*>(a.out);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int p = row0 + m * 16 + tok;
      const int slot = a.sorted_slot[p];
      if (slot >= S) continue;
      float sc = a.topk_w[slot];
      if constexpr (DT == 1) sc *= a.x_scale[p];
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int h0 = ntile * WGN + wn * NI * 16 + n * 16 + fq;
        float ws[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (DT == 1) {
          float4 w4 = *reinterpret_cast<const float4*>(a.w_scale + (size_t)e * a.N + h0);
          ws[0] = w4.x; ws[1] = w4.y; ws[2] = w4.z; ws[3] = w4.w;
        }
        float4 o;
        o.x = acc[m][n][0] * ws[0] * sc;
        o.y = acc[m][n][1] * ws[1] * sc;
        o.z = acc[m][n][2] * ws[2] * sc;
        o.w = acc[m][n][3] * ws[3] * sc;
        *reinterpret_cast<float4*>(part + (size_t)slot * a.N + h0) = o;
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
  float m = 0.0f;
  for (int i = tid; i < a.nparts; i += 256) m = fmaxf(m, a.amax_part[(size_t)p * a.nparts + i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m > 0.0f ? m / 448.0f : 1.0f;
  const float inv = 1.0f / s;
  if (tid == 0) a.act_scale[p] = s;
  const uint16_t* row = a.act + (size_t)p * a.I;
  uint8_t* q = a.act_q + (size_t)p * a.I;
  for (int c = tid; c < a.I / 8; c += 256) {
    uint4 v = *reinterpret_cast<const uint4*>(row + c * 8);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = clamp448(bf16_bits_to_f32(w[i] & 0xffffu) * inv);
      f[2 * i + 1] = clamp448(bf16_bits_to_f32(w[i] >> 16) * inv);
    }
    *reinterpret_cast<uint2*>(q + c * 8) =
        make_uint2(f32x4_to_e4m3(f[0], f[1], f[2], f[3]), f32x4_to_e4m3(f[4], f[5], f[6], f[7]));
  }
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int64_t n4 = (int64_t)a.T * a.H / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i * 4 / a.H, h = i * 4 % a.H;
    float4 s = *reinterpret_cast<const float4*>(a.part + ((size_t)t * a.k) * a.H + h);
    for (int j = 1; j < a.k; ++j) {
      float4 v = *reinterpret_cast<const float4*>(a.part + ((size_t)t * a.k + j) * a.H + h);
      s.x = s.x + v.x;
      s.y = s.y + v.y;
      s.z = s.z + v.z;
      s.w = s.w + v.w;
    }
    *reinterpret_cast<uint2*>(a.out + (size_t)t * a.H + h) =
        make_uint2(f32_to_bf16_bits(s.x) | (f32_to_bf16_bits(s.y) << 16),
                   f32_to_bf16_bits(s.z) | (f32_to_bf16_bits(s.w) << 16));
  }
}

// ---------------------------------------------------------------------------

GemmCfg stage1_cfg(int dt, int T, int k, int E, int H, int I, int bm) {
  (void)dt; (void)T; (void)k; (void)E; (void)H; (void)I;
  GemmCfg c;
  c.mt = bm / 16;
  c.ni = 4;
  c.ksplit = 1;
  c.wg_n = 4 * c.ni * 16;
  return c;
}

GemmCfg stage2_cfg(int dt, int T, int k, int E, int H, int I, int bm) {
  (void)T; (void)k; (void)E;
  const int ce = dt == 0 ? 128 : 256;
  GemmCfg c;
  c.mt = bm / 16;
  if (c.mt == 1 && (I / ce) % 4 == 0 && H % 64 == 0) {
    c.ksplit = 4;
    c.ni = 4;
  } else {
    c.ksplit = 1;
    c.ni = H % 256 == 0 ? 4 : 2;
  }
  c.wg_n = (4 / c.ksplit) * c.ni * 16;
  return c;
}

template <int DT, int STAGE, int MT, int NI, int KSPLIT>
static hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  const int blocks = a.n_mtiles * a.n_ntiles;
  hipLaunchKernelGGL((gemm_kernel<DT, STAGE, MT, NI, KSPLIT>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DT, int STAGE>
static hipError_t launch_dt_stage(const GemmCfg& c, const GemmArgs& a, hipStream_t st) {
  if (STAGE == 1) {
    switch (c.mt) {
      case 1: return launch_one<DT, STAGE, 1, 4, 1>(a, st);
      case 2: return launch_one<DT, STAGE, 2, 4, 1>(a, st);
      case 4: return launch_one<DT, STAGE, 4, 4, 1>(a, st);
      case 8: return launch_one<DT, STAGE, 8, 4, 1>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (c.ksplit == 4) return launch_one<DT, 2, 1, 4, 4>(a, st);
  if (c.ni == 4) {
    switch (c.mt) {
      case 1: return launch_one<DT, 2, 1, 4, 1>(a, st);
      case 2: return launch_one<DT, 2, 2, 4, 1>(a, st);
      case 4: return launch_one<DT, 2, 4, 4, 1>(a, st);
      case 8: return launch_one<DT, 2, 8, 4, 1>(a, st);
    }
  } else {
    switch (c.mt) {
      case 1: return launch_one<DT, 2, 1, 2, 1>(a, st);
      case 2: return launch_one<DT, 2, 2, 2, 1>(a, st);
      case 4: return launch_one<DT, 2, 4, 2, 1>(a, st);
      case 8: return launch_one<DT, 2, 8, 2, 1>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int dt, int stage, const GemmCfg& c, const GemmArgs& a, hipStream_t st) {
  if (dt == 0) return stage == 1 ? launch_dt_stage<0, 1>(c, a, st) : launch_dt_stage<0, 2>(c, a, st);
  return stage == 1 ? launch_dt_stage<1, 1>(c, a, st) : launch_dt_stage<1, 2>(c, a, st);
}

hipError_t launch_quant_act(const QuantArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(quant_act_kernel, dim3(a.cap), dim3(256), 0, st, a);
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
