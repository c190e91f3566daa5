// C ABI of libmoe: argument checks (before any HIP call) and kernel launches.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>

#include "../../include/moe.h"
#include "moe_launch.h"

// Scratch memory of moe_stage2_noalloc (scratch_address).
constexpr int64_t kScratchBytes = (int64_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_err[0] = 0;
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define CHECK(cond, code, ...)                  \
  do {                                          \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

bool valid_bm(int bm) { return bm == 32 || bm == 64 || bm == 128 || bm == 256; }

// ceil(2^35 / k): the kernels divide slot numbers (< 2^30) by k with a multiply.
uint64_t k_magic(int k) { return (((uint64_t)1 << 35) + k - 1) / k; }

// M-tiles per scheduling group: about 2048 rows, one expert's share at prefill.
// Row tiles per schedule group: 2048 rows, so that the tiles sharing an
// expert's weights run together; decode tiles (32 rows, about one per
// expert) run one at a time, so that the workgroups of an XCD stream
// consecutive feature tiles of one expert (contiguous weights).
int group_m(int mt) { return mt == 1 ? 1 : 2048 / (32 * mt); }

int64_t capacity(int T, int k, int E, int bm) {
  int64_t n = (int64_t)T * k + (int64_t)E * (bm - 1);
  return (n + bm - 1) / bm * bm;
}

// Checks shared by the two GEMM stages.
bool valid_dt(int dt) {
  return dt == MOE_BF16 || dt == MOE_FP8_E4M3FN || dt == MOE_MXFP8 || dt == MOE_MXFP4;
}

// Block-scaled element types: MXFP8 tokens and E8M0 weight codes per 32 values.
bool is_mx(int dt) { return dt == MOE_MXFP8 || dt == MOE_MXFP4; }

moe_status check_stage(int dt, int T, int k, int E, int H, int I, int bm) {
  CHECK(valid_dt(dt), MOE_ERR_INVALID_ARG, "dtype %d", dt);
  CHECK(T >= 0 && k >= 1 && E >= 1 && H > 0 && I > 0, MOE_ERR_INVALID_ARG,
        "sizes T=%d k=%d E=%d H=%d I=%d", T, k, E, H, I);
  CHECK(k <= E && k <= 8 && E <= 64, MOE_ERR_UNSUPPORTED, "k=%d E=%d (need k<=min(E,8), E<=64)", k,
        E);
  CHECK(valid_bm(bm), MOE_ERR_UNSUPPORTED, "block_m=%d (need 32, 64, 128 or 256)", bm);
  const int q = dt == MOE_BF16 ? 128 : 256;
  CHECK(H % q == 0 && I % q == 0, MOE_ERR_UNSUPPORTED, "H=%d I=%d must be multiples of %d", H, I,
        q);
  CHECK(!is_mx(dt) || (H <= moe::kMxMaxH && I <= moe::kMxMaxI), MOE_ERR_UNSUPPORTED,
        "MXFP8/MXFP4 need H <= %d and I <= %d (H=%d I=%d)", moe::kMxMaxH, moe::kMxMaxI, H, I);
  CHECK((int64_t)T * k <= (1 << 30) && capacity(T, k, E, bm) <= (1 << 30), MOE_ERR_UNSUPPORTED,
        "T*k too large");
  // Activation rows are addressed with 32-bit buffer offsets below 2 GiB.
  const int64_t es = dt == MOE_BF16 ? 2 : 1;
  CHECK((int64_t)T * H * es < ((int64_t)1 << 31) &&
            capacity(T, k, E, bm) * I * es < ((int64_t)1 << 31),
        MOE_ERR_UNSUPPORTED, "activations beyond 2 GiB (T=%d)", T);
  CHECK(moe::gemm_cfg_ok(dt, 1, moe::stage1_cfg(dt, T, k, E, H, I, bm), 2 * I, H) &&
            moe::gemm_cfg_ok(dt, 2, moe::stage2_cfg(dt, T, k, E, H, I, bm), H, I),
        MOE_ERR_UNSUPPORTED, "no kernel configuration for H=%d I=%d block_m=%d", H, I, bm);
  return ok();
}

moe_status stage2_run(int dt, const void* act, const float* act_amax, const void* w2,
                      const void* s2, const int32_t* sorted_slot, const int32_t* tile_expert,
                      const int32_t* total_padded, const float* topk_w, int T, int k, int E,
                      int H, int I, int block_m, void* out, char* ws, hipStream_t stream);

// Scratch memory of moe_stage2_noalloc: one file-scope device array (below,
// outside this namespace), which every GPU the library runs on holds, its own
// copy, until the process ends. In host code `scratch` only names the symbol:
// its device address comes from hipGetSymbolAddress, taken once per device
// with that device current and kept here. Nothing in it must start at zero:
// every call writes the parts it reads.
constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch[kMaxDevices];

moe_status scratch_address(char** out);

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

const char* moe_version(void) { return "moe-gfx950 0.1"; }

moe_status moe_route(const void* x, const void* w_router, const float* bias, int T, int H, int E,
                     int k, int32_t* topk_ids, float* topk_w, float* logits, void* x_q,
                     float* x_scale, hipStream_t stream) {
  CHECK(T >= 0 && H > 0, MOE_ERR_INVALID_ARG, "sizes T=%d H=%d", T, H);
  CHECK(E >= 1 && k >= 1, MOE_ERR_INVALID_ARG, "E=%d k=%d", E, k);
  CHECK(E <= 64 && k <= E && k <= 8, MOE_ERR_UNSUPPORTED, "E=%d k=%d (need E<=64, k<=min(E,8))",
        E, k);
  CHECK(H % 128 == 0 && H <= 8192, MOE_ERR_UNSUPPORTED,
        "H=%d must be a multiple of 128, at most 8192", H);
  CHECK((int64_t)T * H <= ((int64_t)1 << 40), MOE_ERR_UNSUPPORTED, "T*H too large");
  if (T == 0) return ok();
  CHECK(x && w_router && topk_ids && topk_w, MOE_ERR_INVALID_ARG, "null x/w_router/topk_ids/topk_w");
  CHECK(!x_q || x_scale, MOE_ERR_INVALID_ARG, "x_q given without x_scale");
  CHECK(aligned(x, 16) && aligned(w_router, 16) && aligned(x_q, 8), MOE_ERR_INVALID_ARG,
        "x and w_router must be 16-byte aligned, x_q 8-byte aligned");
  moe::RouteArgs a{(const uint16_t*)x, (const uint16_t*)w_router, bias, T, H, E, k, topk_ids,
                   topk_w, logits, (uint8_t*)x_q, x_scale, nullptr};
  return hip_status(moe::launch_route(a, stream), "moe_route launch");
}

moe_status moe_route_mx(const void* x, const void* w_router, const float* bias, int T, int H,
                        int E, int k, int32_t* topk_ids, float* topk_w, float* logits, void* x_q,
                        void* x_scale_e8m0, hipStream_t stream) {
  CHECK(T >= 0 && H > 0, MOE_ERR_INVALID_ARG, "sizes T=%d H=%d", T, H);
  CHECK(E >= 1 && k >= 1, MOE_ERR_INVALID_ARG, "E=%d k=%d", E, k);
  CHECK(E <= 64 && k <= E && k <= 8, MOE_ERR_UNSUPPORTED, "E=%d k=%d (need E<=64, k<=min(E,8))",
        E, k);
  CHECK(H % 128 == 0 && H <= 8192, MOE_ERR_UNSUPPORTED,
        "H=%d must be a multiple of 128, at most 8192", H);
  CHECK((int64_t)T * H <= ((int64_t)1 << 40), MOE_ERR_UNSUPPORTED, "T*H too large");
  if (T == 0) return ok();
  CHECK(x && w_router && topk_ids && topk_w && x_q && x_scale_e8m0, MOE_ERR_INVALID_ARG,
        "null x/w_router/topk_ids/topk_w/x_q/x_scale_e8m0");
  CHECK(aligned(x, 16) && aligned(w_router, 16) && aligned(x_q, 8), MOE_ERR_INVALID_ARG,
        "x and w_router must be 16-byte aligned, x_q 8-byte aligned");
  moe::RouteArgs a{(const uint16_t*)x, (const uint16_t*)w_router, bias, T, H, E, k, topk_ids,
                   topk_w, logits, (uint8_t*)x_q, nullptr, (uint8_t*)x_scale_e8m0};
  return hip_status(moe::launch_route(a, stream), "moe_route_mx launch");
}

int64_t moe_align_capacity(int T, int k, int E, int block_m) {
  if (T < 0 || k < 1 || E < 1 || !valid_bm(block_m)) return -1;
  return capacity(T, k, E, block_m);
}

moe_status moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m,
                     int32_t* sorted_slot, int32_t* tile_expert, int32_t* expert_count,
                     int32_t* expert_offset, int32_t* total_padded, hipStream_t stream) {
  CHECK(T >= 0 && k >= 1 && E >= 1, MOE_ERR_INVALID_ARG, "sizes T=%d k=%d E=%d", T, k, E);
  CHECK(E <= 64, MOE_ERR_UNSUPPORTED, "E=%d (need E<=64)", E);
  CHECK(valid_bm(block_m), MOE_ERR_UNSUPPORTED, "block_m=%d (need 32, 64, 128 or 256)", block_m);
  CHECK((int64_t)T * k <= (1 << 30), MOE_ERR_UNSUPPORTED, "T*k too large");
  if (T == 0) return ok();
  CHECK(topk_ids && sorted_slot && tile_expert && expert_count && expert_offset && total_padded,
        MOE_ERR_INVALID_ARG, "null pointer argument");
  moe::AlignArgs a{topk_ids, T * k, E, block_m, sorted_slot, tile_expert,
                   expert_count, expert_offset, total_padded};
  return hip_status(moe::launch_align(a, stream), "moe_align launch");
}

moe_status moe_route_align(const void* x, const void* w_router, const float* bias, int T, int H,
                           int E, int k, int mx, int32_t* topk_ids, float* topk_w, float* logits,
                           void* x_q, void* x_scale, int block_m, int32_t* sorted_slot,
                           int32_t* tile_expert, int32_t* expert_count, int32_t* expert_offset,
                           int32_t* total_padded, hipStream_t stream) {
  CHECK(mx == 0 || mx == 1, MOE_ERR_INVALID_ARG, "mx=%d (0 or 1)", mx);
  CHECK(T >= 0 && H > 0, MOE_ERR_INVALID_ARG, "sizes T=%d H=%d", T, H);
  CHECK(E >= 1 && k >= 1, MOE_ERR_INVALID_ARG, "E=%d k=%d", E, k);
  CHECK(E <= 64 && k <= E && k <= 8, MOE_ERR_UNSUPPORTED, "E=%d k=%d (need E<=64, k<=min(E,8))",
        E, k);
  CHECK(H % 128 == 0 && H <= 8192, MOE_ERR_UNSUPPORTED,
        "H=%d must be a multiple of 128, at most 8192", H);
  CHECK((int64_t)T * H <= ((int64_t)1 << 40), MOE_ERR_UNSUPPORTED, "T*H too large");
  CHECK(valid_bm(block_m), MOE_ERR_UNSUPPORTED, "block_m=%d (need 32, 64, 128 or 256)", block_m);
  CHECK((int64_t)T * k <= (1 << 30), MOE_ERR_UNSUPPORTED, "T*k too large");
  if (T == 0) return ok();
  CHECK(x && w_router && topk_ids && topk_w, MOE_ERR_INVALID_ARG, "null x/w_router/topk_ids/topk_w");
  CHECK(!x_q || x_scale, MOE_ERR_INVALID_ARG, "x_q given without x_scale");
  CHECK(!mx || x_q, MOE_ERR_INVALID_ARG, "mx=1 needs x_q and x_scale");
  CHECK(aligned(x, 16) && aligned(w_router, 16) && aligned(x_q, 8), MOE_ERR_INVALID_ARG,
        "x and w_router must be 16-byte aligned, x_q 8-byte aligned");
  CHECK(sorted_slot && tile_expert && expert_count && expert_offset && total_padded,
        MOE_ERR_INVALID_ARG, "null grouping pointer");
  moe::RouteArgs a{(const uint16_t*)x, (const uint16_t*)w_router, bias, T, H, E, k, topk_ids,
                   topk_w, logits, (uint8_t*)x_q, mx ? nullptr : (float*)x_scale,
                   mx ? (uint8_t*)x_scale : nullptr};
  moe::AlignArgs g{topk_ids, T * k, E, block_m, sorted_slot, tile_expert,
                   expert_count, expert_offset, total_padded};
  return hip_status(moe::launch_route_align(a, g, stream), "moe_route_align launch");
}

int64_t moe_preshuffle_bytes(moe_dtype dt, int E, int H, int I, int which) {
  if (!valid_dt(dt) || E < 1 || H < 1 || I < 1) return -1;
  const int64_t es = dt == MOE_BF16 ? 2 : 1;
  const int64_t d = dt == MOE_MXFP4 ? 2 : 1;  // E2M1: two values per byte
  if (which == 0) return 2 * (int64_t)E * I * H * es / d;
  if (which == 1) return (int64_t)E * H * I * es / d;
  if (which == 2 || which == 3) {
    if (dt == MOE_BF16) return 0;
    const int64_t rows = which == 2 ? 2 * (int64_t)E * I : (int64_t)E * H;
    if (dt == MOE_FP8_E4M3FN) return rows * 4;                // one fp32 per output row
    return rows * ((which == 2 ? H : I) / 32);                 // one E8M0 code per 32 values
  }
  return -1;
}

moe_status moe_preshuffle(moe_dtype dt, int E, int H, int I, const void* w1, const void* w3,
                          const void* w2, const void* s1, const void* s3, const void* s2,
                          void* w13_out, void* w2_out, void* s13_out, void* s2_out,
                          hipStream_t stream) {
  CHECK(valid_dt(dt), MOE_ERR_INVALID_ARG, "dtype %d", (int)dt);
  CHECK(E >= 1 && H > 0 && I > 0, MOE_ERR_INVALID_ARG, "sizes E=%d H=%d I=%d", E, H, I);
  const int q = dt == MOE_BF16 ? 128 : 256;
  CHECK(H % q == 0 && I % q == 0, MOE_ERR_UNSUPPORTED, "H=%d I=%d must be multiples of %d", H, I,
        q);
  CHECK(w1 && w3 && w2 && w13_out && w2_out, MOE_ERR_INVALID_ARG, "null weight pointer");
  CHECK(aligned(w1, 16) && aligned(w3, 16) && aligned(w2, 16) && aligned(w13_out, 16) &&
            aligned(w2_out, 16),
        MOE_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  const bool fp8 = dt == MOE_FP8_E4M3FN, mx = is_mx(dt), fp4 = dt == MOE_MXFP4;
  if (fp8 || mx)
    CHECK(s1 && s3 && s2 && s13_out && s2_out, MOE_ERR_INVALID_ARG,
          "FP8, MXFP8 and MXFP4 need all scale pointers");
  if (mx)
    CHECK(aligned(s13_out, 4) && aligned(s2_out, 4), MOE_ERR_INVALID_ARG,
          "MXFP8/MXFP4 scale outputs must be 4-byte aligned");
  // Row length in bytes of each weight matrix and the fragment order.
  const int64_t h_bytes = dt == MOE_BF16 ? 2 * (int64_t)H : fp4 ? H / 2 : H;
  const int64_t i_bytes = dt == MOE_BF16 ? 2 * (int64_t)I : fp4 ? I / 2 : I;
  const int order = fp4 ? 2 : mx ? 1 : 0;
  moe::PreshuffleArgs a13{(const uint8_t*)w1, (const uint8_t*)w3, (uint8_t*)w13_out, E, 2 * I,
                          h_bytes, order};
  hipError_t err = moe::launch_preshuffle(a13, stream);
  if (err != hipSuccess) return hip_status(err, "preshuffle W1/W3");
  moe::PreshuffleArgs a2{(const uint8_t*)w2, nullptr, (uint8_t*)w2_out, E, H, i_bytes, order};
  err = moe::launch_preshuffle(a2, stream);
  if (err != hipSuccess) return hip_status(err, "preshuffle W2");
  if (fp8) {
    const size_t row = (size_t)I * 4;
    err = hipMemcpy2DAsync(s13_out, 2 * row, s1, row, row, E, hipMemcpyDeviceToDevice, stream);
    if (err == hipSuccess)
      err = hipMemcpy2DAsync((char*)s13_out + row, 2 * row, s3, row, row, E,
                             hipMemcpyDeviceToDevice, stream);
    if (err == hipSuccess)
      err = hipMemcpyAsync(s2_out, s2, (size_t)E * H * 4, hipMemcpyDeviceToDevice, stream);
    if (err != hipSuccess) return hip_status(err, "preshuffle scales");
  }
  if (mx) {
    moe::PreshuffleArgs m13{(const uint8_t*)s1, (const uint8_t*)s3, (uint8_t*)s13_out, E, 2 * I, H,
                            1};
    err = moe::launch_preshuffle_mx_scales(m13, stream);
    if (err != hipSuccess) return hip_status(err, "preshuffle W1/W3 block scales");
    moe::PreshuffleArgs m2{(const uint8_t*)s2, nullptr, (uint8_t*)s2_out, E, H, I, 1};
    err = moe::launch_preshuffle_mx_scales(m2, stream);
    if (err != hipSuccess) return hip_status(err, "preshuffle W2 block scales");
  }
  return ok();
}

int64_t moe_stage1_amax_floats(moe_dtype dt, int T, int k, int E, int H, int I, int block_m) {
  if (check_stage(dt, T, k, E, H, I, block_m) != MOE_OK) return -1;
  if (dt != MOE_FP8_E4M3FN) return 0;
  moe::GemmCfg c = moe::stage1_cfg(dt, T, k, E, H, I, block_m);
  return capacity(T, k, E, block_m) * (2 * (int64_t)I / c.wg_n);
}

namespace {

moe_status stage1_run(moe_dtype dt, const void* x_or_xq, const void* x_scale, const void* w13,
                      const void* s13, const int32_t* sorted_slot, const int32_t* tile_expert,
                      const int32_t* total_padded, int T, int k, int E, int H, int I, int block_m,
                      void* act, float* act_amax, void* gu_out, hipStream_t stream) {
  moe_status s = check_stage(dt, T, k, E, H, I, block_m);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  const bool fp8 = dt == MOE_FP8_E4M3FN, mx = is_mx(dt);
  CHECK(x_or_xq && w13 && sorted_slot && tile_expert && total_padded && act, MOE_ERR_INVALID_ARG,
        "null pointer argument");
  CHECK(!fp8 || (x_scale && s13 && act_amax), MOE_ERR_INVALID_ARG,
        "FP8 needs x_scale, s13 and act_amax");
  CHECK(!mx || (x_scale && s13), MOE_ERR_INVALID_ARG, "MXFP8/MXFP4 need x_scale and s13");
  CHECK(aligned(x_or_xq, 16) && aligned(w13, 16) && aligned(act, 16) &&
            aligned(s13, mx ? 4 : 16) && aligned(x_scale, mx ? 8 : 4),
        MOE_ERR_INVALID_ARG,
        "x, w13 and act must be 16-byte aligned, s13 16-byte (MXFP8/MXFP4: 4), x_scale 4-byte "
        "(MXFP8/MXFP4: 8)");
  moe::GemmCfg c = moe::stage1_cfg(dt, T, k, E, H, I, block_m);
  const int64_t cap = capacity(T, k, E, block_m);
  moe::GemmArgs a{};
  a.X = (const uint8_t*)x_or_xq;
  a.W = (const uint8_t*)w13;
  if (mx) {
    a.x_mx = (const uint8_t*)x_scale;
    a.w_mx = (const uint8_t*)s13;
  } else {
    a.x_scale = (const float*)x_scale;
    a.w_scale = (const float*)s13;
  }
  a.sorted_slot = sorted_slot;
  a.tile_expert = tile_expert;
  a.total_padded = total_padded;
  a.out = act;
  a.amax_part = act_amax;
  a.T = T;
  a.k = k;
  a.N = 2 * I;
  a.I = I;
  a.cap = (int)cap;
  a.bm = block_m;
  a.K_bytes = H * (dt == MOE_BF16 ? 2 : 1);
  a.x_bytes = (int64_t)T * a.K_bytes;
  a.n_mtiles = (int)(cap / (32 * c.mt));
  a.n_ntiles = 2 * I / c.wg_n;
  a.kg = 1;
  a.group_m = group_m(c.mt);
  a.k_magic = k_magic(k);
  a.live_order = c.mt * c.nf < 16;
  a.gu_out = (uint16_t*)gu_out;
  return hip_status(moe::launch_gemm(dt, 1, c, a, stream), "moe_stage1 launch");
}

}  // namespace

moe_status moe_stage1(moe_dtype dt, const void* x_or_xq, const void* x_scale, const void* w13,
                      const void* s13, const int32_t* sorted_slot, const int32_t* tile_expert,
                      const int32_t* total_padded, int T, int k, int E, int H, int I, int block_m,
                      void* act, float* act_amax, hipStream_t stream) {
  return stage1_run(dt, x_or_xq, x_scale, w13, s13, sorted_slot, tile_expert, total_padded, T, k,
                    E, H, I, block_m, act, act_amax, nullptr, stream);
}

moe_status moe_stage1_save_preact(const void* x, const void* w13, const int32_t* sorted_slot,
                                  const int32_t* tile_expert, const int32_t* total_padded, int T,
                                  int k, int E, int H, int I, int block_m, void* act, void* gu,
                                  hipStream_t stream) {
  CHECK(gu, MOE_ERR_INVALID_ARG, "null pointer argument");
  CHECK(aligned(gu, 16), MOE_ERR_INVALID_ARG, "gu must be 16-byte aligned");
  return stage1_run(MOE_BF16, x, nullptr, w13, nullptr, sorted_slot, tile_expert, total_padded,
                    T, k, E, H, I, block_m, act, nullptr, gu, stream);
}

int64_t moe_stage2_workspace_bytes(moe_dtype dt, int T, int k, int E, int H, int I, int block_m) {
  if (check_stage(dt, T, k, E, H, I, block_m) != MOE_OK) return -1;
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  const moe::GemmCfg c = moe::stage2_cfg(dt, T, k, E, H, I, block_m);
  int64_t bytes = up((int64_t)c.kg * T * k * H * 4);  // weighted per-slot partials per split
  if (dt == MOE_FP8_E4M3FN) {
    const int64_t cap = capacity(T, k, E, block_m);
    bytes += up(cap * I) + up(cap * 4);  // requantised intermediate + row scales
  }
  if (is_mx(dt)) {
    const int64_t cap = capacity(T, k, E, block_m);
    bytes += up(cap * I) + up(cap * (I / 32));  // requantised intermediate + block codes
  }
  if (c.tail_split > 0)  // partials of the tail pieces
    bytes += up((int64_t)moe::kTailPieces * 32 * c.mt * c.wg_n * 4);
  return bytes;
}

moe_status moe_stage2(moe_dtype dt, const void* act, const float* act_amax, const void* w2,
                      const void* s2, const int32_t* sorted_slot, const int32_t* tile_expert,
                      const int32_t* total_padded, const float* topk_w, int T, int k, int E, int H,
                      int I, int block_m, void* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  moe_status s = check_stage(dt, T, k, E, H, I, block_m);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  const bool fp8 = dt == MOE_FP8_E4M3FN, mx = is_mx(dt);
  CHECK(act && w2 && sorted_slot && tile_expert && total_padded && topk_w && out && workspace,
        MOE_ERR_INVALID_ARG, "null pointer argument");
  CHECK(!fp8 || (act_amax && s2), MOE_ERR_INVALID_ARG, "FP8 needs act_amax and s2");
  CHECK(!mx || s2, MOE_ERR_INVALID_ARG, "MXFP8/MXFP4 need s2");
  CHECK(aligned(act, 16) && aligned(w2, 16) && aligned(out, 8) && aligned(workspace, 256) &&
            aligned(s2, mx ? 4 : 16),
        MOE_ERR_INVALID_ARG, "act/w2/s2 16-byte, out 8-byte, workspace 256-byte alignment");
  const int64_t need = moe_stage2_workspace_bytes(dt, T, k, E, H, I, block_m);
  CHECK((int64_t)workspace_bytes >= need, MOE_ERR_WORKSPACE, "workspace %zu bytes < %lld needed",
        workspace_bytes, (long long)need);
  return stage2_run(dt, act, act_amax, w2, s2, sorted_slot, tile_expert, total_padded, topk_w, T,
                    k, E, H, I, block_m, out, (char*)workspace, stream);
}

moe_status moe_stage2_noalloc(moe_dtype dt, const void* act, const float* act_amax,
                              const void* w2, const void* s2, const int32_t* sorted_slot,
                              const int32_t* tile_expert, const int32_t* total_padded,
                              const float* topk_w, int T, int k, int E, int H, int I,
                              int block_m, void* out, hipStream_t stream) {
  moe_status s = check_stage(dt, T, k, E, H, I, block_m);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  const bool fp8 = dt == MOE_FP8_E4M3FN, mx = is_mx(dt);
  CHECK(act && w2 && sorted_slot && tile_expert && total_padded && topk_w && out,
        MOE_ERR_INVALID_ARG, "null pointer argument");
  CHECK(!fp8 || (act_amax && s2), MOE_ERR_INVALID_ARG, "FP8 needs act_amax and s2");
  CHECK(!mx || s2, MOE_ERR_INVALID_ARG, "MXFP8/MXFP4 need s2");
  CHECK(aligned(act, 16) && aligned(w2, 16) && aligned(out, 8) && aligned(s2, mx ? 4 : 16),
        MOE_ERR_INVALID_ARG, "act/w2/s2 16-byte, out 8-byte alignment");
  const int64_t need = moe_stage2_workspace_bytes(dt, T, k, E, H, I, block_m);
  CHECK(need <= kScratchBytes, MOE_ERR_WORKSPACE,
        "moe_stage2_noalloc: this shape needs %lld bytes of scratch; the library's scratch "
        "array holds %lld (use moe_stage2 with a workspace)",
        (long long)need, (long long)kScratchBytes);
  char* sp = nullptr;
  s = scratch_address(&sp);
  if (s != MOE_OK) return s;
  return stage2_run(dt, act, act_amax, w2, s2, sorted_slot, tile_expert, total_padded, topk_w, T,
                    k, E, H, I, block_m, out, sp, stream);
}

}  // extern "C"

namespace {

// The launches of stage 2 (arguments already checked) on a workspace of
// moe_stage2_workspace_bytes(): the requantisation pass (FP8, MXFP8, MXFP4),
// the GEMM, the tail-piece sum and the combine.
moe_status stage2_run(int dt, const void* act, const float* act_amax, const void* w2,
                      const void* s2, const int32_t* sorted_slot, const int32_t* tile_expert,
                      const int32_t* total_padded, const float* topk_w, int T, int k, int E,
                      int H, int I, int block_m, void* out, char* ws, hipStream_t stream) {
  const bool fp8 = dt == MOE_FP8_E4M3FN, mx = is_mx(dt);
  const int64_t cap = capacity(T, k, E, block_m);
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  moe::GemmCfg c = moe::stage2_cfg(dt, T, k, E, H, I, block_m);
  float* part = (float*)ws;
  ws += up((int64_t)c.kg * T * k * H * 4);
  const void* x = act;
  const float* xs = nullptr;
  const uint8_t* xmx = nullptr;
  hipError_t err;
  if (fp8) {
    uint8_t* act_q = (uint8_t*)ws;
    float* act_scale = (float*)(ws + up(cap * I));
    moe::GemmCfg c1 = moe::stage1_cfg(dt, T, k, E, H, I, block_m);
    moe::QuantArgs q{(const uint16_t*)act, act_amax, 2 * I / c1.wg_n, (int)cap, I, total_padded,
                     act_q, act_scale};
    err = moe::launch_quant_act(q, stream);
    if (err != hipSuccess) return hip_status(err, "moe_stage2 requantisation");
    x = act_q;
    xs = act_scale;
    ws += up(cap * I) + up(cap * 4);
  }
  if (mx) {
    uint8_t* act_q = (uint8_t*)ws;
    uint8_t* act_mx = (uint8_t*)(ws + up(cap * I));
    moe::QuantMxArgs q{(const uint16_t*)act, (int)cap, I, total_padded, act_q, act_mx};
    err = moe::launch_quant_act_mx(q, stream);
    if (err != hipSuccess) return hip_status(err, "moe_stage2 block requantisation");
    x = act_q;
    xmx = act_mx;
    ws += up(cap * I) + up(cap * (I / 32));
  }
  moe::GemmArgs a{};
  a.X = (const uint8_t*)x;
  a.x_scale = xs;
  a.W = (const uint8_t*)w2;
  if (mx) {
    a.x_mx = xmx;
    a.w_mx = (const uint8_t*)s2;
  } else {
    a.w_scale = (const float*)s2;
  }
  a.sorted_slot = sorted_slot;
  a.tile_expert = tile_expert;
  a.total_padded = total_padded;
  a.topk_w = topk_w;
  a.out = part;
  a.T = T;
  a.k = k;
  a.N = H;
  a.I = I;
  a.cap = (int)cap;
  a.bm = block_m;
  a.K_bytes = I * (dt == MOE_BF16 ? 2 : 1);
  a.x_bytes = cap * a.K_bytes;
  a.n_mtiles = (int)(cap / (32 * c.mt));
  a.n_ntiles = H / c.wg_n;
  a.kg = c.kg;
  a.group_m = group_m(c.mt);
  a.k_magic = k_magic(k);
  a.tail_split = c.tail_split;
  a.live_order = c.mt * c.nf < 16;
  if (c.tail_split > 0) {
    a.tail_part = (float*)ws;
    a.round = c.round;
  }
  err = moe::launch_gemm(dt, 2, c, a, stream);
  if (err != hipSuccess) return hip_status(err, "moe_stage2 GEMM launch");
  if (c.tail_split > 0) {
    moe::TailReduceArgs tr{a.tail_part, sorted_slot, total_padded, part, T * k, H, 32 * c.mt,
                           c.wg_n, a.n_ntiles, a.group_m, a.round, c.tail_split,
                           a.K_bytes / c.ck};
    err = moe::launch_tail_reduce(tr, stream);
    if (err != hipSuccess) return hip_status(err, "moe_stage2 tail reduction launch");
  }
  moe::CombineArgs cb{part, total_padded, T, k, H, c.kg, (uint16_t*)out};
  return hip_status(moe::launch_combine(cb, stream), "moe_stage2 combine launch");
}

}  // namespace

extern "C" {

// --- backward pass (bf16) ---------------------------------------------------

int64_t moe_backward_preshuffle_bytes(int E, int H, int I, int which) {
  if (E < 1 || H < 1 || I < 1 || (which != 0 && which != 1)) return -1;
  return (int64_t)E * H * I * 2 * (which == 0 ? 1 : 2);
}

moe_status moe_backward_preshuffle(int E, int H, int I, const void* w1, const void* w3,
                                   const void* w2, void* w2t_out, void* w13t_out,
                                   hipStream_t stream) {
  CHECK(E >= 1 && H > 0 && I > 0, MOE_ERR_INVALID_ARG, "sizes E=%d H=%d I=%d", E, H, I);
  CHECK(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED, "H=%d I=%d must be multiples of 128",
        H, I);
  CHECK(w1 && w3 && w2 && w2t_out && w13t_out, MOE_ERR_INVALID_ARG, "null weight pointer");
  CHECK(aligned(w1, 16) && aligned(w3, 16) && aligned(w2, 16) && aligned(w2t_out, 16) &&
            aligned(w13t_out, 16),
        MOE_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  moe::PreshuffleTArgs a{(const uint16_t*)w1, (const uint16_t*)w3, (const uint16_t*)w2,
                         (uint16_t*)w2t_out, E, H, I, 0};
  hipError_t err = moe::launch_preshuffle_t(a, stream);
  if (err != hipSuccess) return hip_status(err, "backward preshuffle W2^T");
  a.dst = (uint16_t*)w13t_out;
  a.mode = 1;
  return hip_status(moe::launch_preshuffle_t(a, stream), "backward preshuffle W13^T");
}

namespace {

// Backward workspace: gu and dgu bf16 [cap][2I]; dwpart fp32 [T*k][I/wg_n];
// dl fp32 [T*k]; part fp32 [kg][T*k][H]; tail pieces (prefill sizes).
struct BwdLayout {
  moe::GemmCfg c1, cz, c3;  // recompute (stage 1), z (stage 1 over W2^T), dx (stage 2)
  int64_t gu, dgu, dwpart, dl, part, tail, rpart, xg, wdg, bytes;
};

BwdLayout bwd_layout(int T, int k, int E, int H, int I, int bm) {
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  BwdLayout L{};
  L.c1 = moe::stage1_cfg(MOE_BF16, T, k, E, H, I, bm);
  L.cz = moe::stage1_cfg(MOE_BF16, T, k, E, H, I / 2, bm);  // N = I output features
  L.c3 = moe::stage2_cfg(MOE_BF16, T, k, E, H, 2 * I, bm);  // reduction over 2I
  const int64_t cap = capacity(T, k, E, bm), S = (int64_t)T * k;
  int64_t o = 0;
  L.gu = o;
  o += up(cap * 2 * I * 2);
  L.dgu = o;
  o += up(cap * 2 * I * 2);
  L.dwpart = o;
  o += up(S * (I / L.cz.wg_n) * 4);
  L.dl = o;
  o += up(S * 4);
  L.part = o;
  o += up((int64_t)L.c3.kg * S * H * 4);
  L.tail = -1;
  if (L.c3.tail_split > 0) {
    L.tail = o;
    o += up((int64_t)moe::kTailPieces * 32 * L.c3.mt * L.c3.wg_n * 4);
  }
  L.rpart = o;
  o += up((cap / bm) * (int64_t)(H + 1) * 4);
  L.xg = o;
  o += up(cap * H * 2);
  L.wdg = o;
  o += up(cap * H * 2);
  L.bytes = o;
  return L;
}

moe_status check_backward(int T, int k, int E, int H, int I, int bm) {
  moe_status s = check_stage(MOE_BF16, T, k, E, H, I, bm);
  if (s != MOE_OK) return s;
  const BwdLayout L = bwd_layout(T, k, E, H, I, bm);
  CHECK(moe::gemm_cfg_ok(MOE_BF16, 1, L.cz, I, H) && moe::gemm_cfg_ok(MOE_BF16, 2, L.c3, H, 2 * I),
        MOE_ERR_UNSUPPORTED, "no backward kernel configuration for H=%d I=%d block_m=%d", H, I,
        bm);
  CHECK(capacity(T, k, E, bm) * 4 * I < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
        "backward intermediate beyond 2 GiB (T=%d)", T);
  return ok();
}

}  // namespace

int64_t moe_backward_workspace_bytes(int T, int k, int E, int H, int I, int block_m) {
  if (check_backward(T, k, E, H, I, block_m) != MOE_OK) return -1;
  return bwd_layout(T, k, E, H, I, block_m).bytes;
}

moe_status moe_backward(const void* x, const void* w_router, const int32_t* topk_ids,
                        const float* topk_w, const int32_t* sorted_slot,
                        const int32_t* tile_expert, const int32_t* expert_offset,
                        const int32_t* total_padded, const void* act, const void* gu_saved,
                        const void* w13, const void* w2t, const void* w13t, const void* dout,
                        int T, int k,
                        int E, int H, int I, int block_m, float* dx, float* dw1, float* dw3,
                        float* dw2, float* dw_router, float* dbias, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  moe_status s = check_backward(T, k, E, H, I, block_m);
  if (s != MOE_OK) return s;
  if (T == 0) return ok();
  CHECK(x && w_router && topk_ids && topk_w && sorted_slot && tile_expert && expert_offset &&
            total_padded && act && w13 && w2t && w13t && dout && dx && dw1 && dw3 && dw2 &&
            dw_router && workspace,
        MOE_ERR_INVALID_ARG, "null pointer argument");
  CHECK(aligned(gu_saved, 16), MOE_ERR_INVALID_ARG, "gu_saved must be 16-byte aligned");
  CHECK(aligned(x, 16) && aligned(w_router, 16) && aligned(act, 16) && aligned(w13, 16) &&
            aligned(w2t, 16) && aligned(w13t, 16) && aligned(dout, 16) && aligned(dx, 16) &&
            aligned(dw1, 16) && aligned(dw3, 16) && aligned(dw2, 16) && aligned(dw_router, 16) &&
            aligned(workspace, 256),
        MOE_ERR_INVALID_ARG, "16-byte alignment (workspace 256-byte)");
  const BwdLayout L = bwd_layout(T, k, E, H, I, block_m);
  CHECK((int64_t)workspace_bytes >= L.bytes, MOE_ERR_WORKSPACE,
        "workspace %zu bytes < %lld needed", workspace_bytes, (long long)L.bytes);
  char* ws = (char*)workspace;
  const int64_t cap = capacity(T, k, E, block_m);
  const int S = T * k;
  const uint16_t* gu = gu_saved ? (const uint16_t*)gu_saved : (const uint16_t*)(ws + L.gu);
  uint16_t* dgu = (uint16_t*)(ws + L.dgu);
  float* dwpart = (float*)(ws + L.dwpart);
  float* part = (float*)(ws + L.part);
  auto common = [&](moe::GemmArgs& a, const moe::GemmCfg& c) {
    a.sorted_slot = sorted_slot;
    a.tile_expert = tile_expert;
    a.total_padded = total_padded;
    a.topk_w = topk_w;
    a.T = T;
    a.k = k;
    a.I = I;
    a.cap = (int)cap;
    a.bm = block_m;
    a.n_mtiles = (int)(cap / (32 * c.mt));
    a.group_m = group_m(c.mt);
    a.k_magic = k_magic(k);
    a.kg = c.kg;
    a.live_order = c.mt * c.nf < 16;
  };
  // 1. g, u recomputed from x (the forward's stage 1, pre-activations out),
  //    unless the forward kept them (moe_stage1_save_preact).
  if (!gu_saved) {
    moe::GemmArgs a{};
    common(a, L.c1);
    a.X = (const uint8_t*)x;
    a.W = (const uint8_t*)w13;
    a.out = ws + L.gu;
    a.N = 2 * I;
    a.K_bytes = 2 * H;
    a.x_bytes = (int64_t)T * H * 2;
    a.n_ntiles = 2 * I / L.c1.wg_n;
    a.epi = 1;
    hipError_t err = moe::launch_gemm(MOE_BF16, 1, L.c1, a, stream);
    if (err != hipSuccess) return hip_status(err, "moe_backward recompute launch");
  }
  // 2. z = W2^T dout per row; dg, du and the partial <z, act>.
  {
    moe::GemmArgs a{};
    common(a, L.cz);
    a.X = (const uint8_t*)dout;
    a.W = (const uint8_t*)w2t;
    a.out = dgu;
    a.N = I;
    a.K_bytes = 2 * H;
    a.x_bytes = (int64_t)T * H * 2;
    a.n_ntiles = I / L.cz.wg_n;
    a.epi = 2;
    a.act_in = (const uint16_t*)act;
    a.gu = gu;
    a.dwpart = dwpart;
    hipError_t err = moe::launch_gemm(MOE_BF16, 1, L.cz, a, stream);
    if (err != hipSuccess) return hip_status(err, "moe_backward SwiGLU-gradient launch");
  }
  // 3. per slot W1^T dg + W3^T du (stage 2 over [W1^T | W3^T], weight 1).
  {
    const moe::GemmCfg& c = L.c3;
    moe::GemmArgs a{};
    common(a, c);
    a.X = (const uint8_t*)dgu;
    a.W = (const uint8_t*)w13t;
    a.out = part;
    a.N = H;
    a.I = 2 * I;
    a.K_bytes = 4 * I;
    a.x_bytes = cap * 4 * I;
    a.n_ntiles = H / c.wg_n;
    a.tail_split = c.tail_split;
    a.unit_w = 1;
    if (c.tail_split > 0) {
      a.tail_part = (float*)(ws + L.tail);
      a.round = c.round;
    }
    hipError_t err = moe::launch_gemm(MOE_BF16, 2, c, a, stream);
    if (err != hipSuccess) return hip_status(err, "moe_backward input-gradient launch");
    if (c.tail_split > 0) {
      moe::TailReduceArgs tr{a.tail_part, sorted_slot, total_padded, part, S, H, 32 * c.mt,
                             c.wg_n, a.n_ntiles, a.group_m, a.round, c.tail_split,
                             a.K_bytes / c.ck};
      err = moe::launch_tail_reduce(tr, stream);
      if (err != hipSuccess) return hip_status(err, "moe_backward tail reduction launch");
    }
  }
  // 4. router gradient, dx.
  {
    moe::BwdArgs b{T, H, k, E, I / L.cz.wg_n, L.c3.kg, dwpart, topk_w, topk_ids, part,
                   (const uint16_t*)w_router, (const uint16_t*)x, (float*)(ws + L.dl), dx,
                   dw_router, dbias, sorted_slot, expert_offset, total_padded, block_m,
                   (int)(cap / block_m), k_magic(k), (float*)(ws + L.rpart)};
    hipError_t err = moe::launch_bwd_router(b, stream);
    if (err != hipSuccess) return hip_status(err, "moe_backward router-gradient launch");
  }
  // 5. the token rows of the grouping (x and w dout), pad rows of dg, du zeroed;
  //    dW2[e] = sum over e's rows of (w dout) act^T; dW1 | dW3 = sum of [dg | du] x^T.
  {
    uint16_t* xg = (uint16_t*)(ws + L.xg);
    uint16_t* wdg = (uint16_t*)(ws + L.wdg);
    moe::GatherArgs ga{(const uint16_t*)x, (const uint16_t*)dout, topk_w, sorted_slot,
                       total_padded, H, I, S, (int)cap, k_magic(k), xg, wdg, dgu};
    hipError_t err = moe::launch_bwd_gather(ga, stream);
    if (err != hipSuccess) return hip_status(err, "moe_backward gather launch");
    moe::WgradArgs w{wdg, (const uint16_t*)act, H, I, 0, 0, cap * H * 2, cap * I * 2, H, I, E,
                     H, expert_offset, sorted_slot, topk_w, S, k_magic(k), dw2, dw2};
    err = moe::launch_wgrad(w, stream);
    if (err != hipSuccess) return hip_status(err, "moe_backward dW2 launch");
    moe::WgradArgs w13g{dgu, xg, 2 * I, H, 0, 0, cap * 4 * I, cap * H * 2, 2 * I, H, E, I,
                        expert_offset, sorted_slot, topk_w, S, k_magic(k), dw1, dw3};
    return hip_status(moe::launch_wgrad(w13g, stream), "moe_backward dW1/dW3 launch");
  }
}

}  // extern "C"

namespace {

moe_status scratch_address(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moe_stage2_noalloc: hipGetDevice");
  CHECK(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "device %d (at most %d devices)",
        dev, kMaxDevices);
  char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "moe_stage2_noalloc: hipGetSymbolAddress");
    CHECK(q, MOE_ERR_HIP, "moe_stage2_noalloc: null scratch address");
    p = (char*)q;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return ok();
}

}  // namespace
