// C ABI of libkvq: plans, argument validation, error reporting, launches.
//
// Every check runs on the host before anything is enqueued, so a failing call
// has no side effects.  Nothing here allocates device memory: the plan's sign
// vector travels to the kernels as launch arguments.
#include "../../include/kvq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "kvq_internal.hpp"

struct kvq_plan {
  int32_t D;
  int32_t G;
  int32_t bits;
  int32_t rotation;
  uint32_t options;        // KVQ_OPT_* bits
  uint64_t seed;
  uint64_t sign_bits[4];   // bit i of word i / 64 = 1 for sign -1
};

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

kvq_status fail(kvq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kvq_status ok() {
  g_last_error.clear();
  return KVQ_OK;
}

// SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): golden-ratio increment, then the 64-bit
// finaliser.
uint64_t splitmix64_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int32_t sign_count(const kvq_plan* p) {
  return p->rotation == KVQ_SRFT ? p->D / 2 : p->rotation == KVQ_SRHT ? p->D : 0;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The codec kernels form a lane's offset from its tile's first row in 32
// bits, up to 14 token strides of 2-byte elements: token strides stay below
// 2^28 elements.  The attention kernels count tokens in 32 bits: Tcap stays
// below 2^31.
constexpr int64_t kMaxTokenStride = int64_t(1) << 28;
constexpr int64_t kMaxAttnTcap = int64_t(1) << 31;

// a * b * c * d within [0, 2^62]
bool product_ok(int64_t a, int64_t b, int64_t c, int64_t d) {
  __int128 v = static_cast<__int128>(a) * b;
  if (v > (static_cast<__int128>(1) << 62)) return false;
  v *= c;
  if (v > (static_cast<__int128>(1) << 62)) return false;
  v *= d;
  return v <= (static_cast<__int128>(1) << 62);
}

// The largest element offset a strided [B, H, T, D] view reaches,
// (B-1) sb + (H-1) sh + (T-1) st + D - 1, within [0, 2^62] (non-empty view,
// non-negative strides).
bool extent_ok(int64_t B, int64_t H, int64_t T, int64_t sb, int64_t sh, int64_t st, int64_t D) {
  const __int128 e = static_cast<__int128>(B - 1) * sb + static_cast<__int128>(H - 1) * sh +
                     static_cast<__int128>(T - 1) * st + (D - 1);
  return e <= (static_cast<__int128>(1) << 62);
}

kvq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

kvq_status check_plan(const kvq_plan* p) {
  if (!p) return fail(KVQ_ERR_INVALID, "plan is NULL");
  return KVQ_OK;
}

void fill_signs(const kvq_plan* p, kvq::CodecDesc& d) {
  d.D = p->D;
  d.G = p->G;
  d.bits = p->bits;
  d.rotation = p->rotation;
  d.options = p->options;
  for (int i = 0; i < 4; ++i) d.signs[i] = p->sign_bits[i];
}

// Shared checks of the fp16 input rows of encode and rotate.
kvq_status check_x(const kvq_plan* p, const uint16_t* x, int64_t B, int64_t H, int64_t T,
                   int64_t sb, int64_t sh, int64_t st, const float* lambda, int64_t lambda_sb) {
  if (B < 0 || H < 0 || T < 0) return fail(KVQ_ERR_INVALID, "negative shape B=%lld H=%lld T=%lld",
                                           (long long)B, (long long)H, (long long)T);
  if (!x) return fail(KVQ_ERR_INVALID, "x is NULL");
  if (!lambda) return fail(KVQ_ERR_INVALID, "lambda is NULL");
  if (!aligned(x, 16)) return fail(KVQ_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned(lambda, 4)) return fail(KVQ_ERR_ALIGN, "lambda is not 4-byte aligned");
  if (sb < 0 || sh < 0 || st < 0 || lambda_sb < 0)
    return fail(KVQ_ERR_INVALID, "strides must be non-negative");
  if (sb % 8 || sh % 8 || st % 8)
    return fail(KVQ_ERR_ALIGN, "x strides must be multiples of 8 elements (16-byte rows)");
  if (st >= kMaxTokenStride) return fail(KVQ_ERR_INVALID, "x token stride %lld is not below 2^28", (long long)st);
  if (!product_ok(B, H, T, p->D)) return fail(KVQ_ERR_INVALID, "shape too large");
  if (!extent_ok(B, H, T, sb, sh, st, p->D)) return fail(KVQ_ERR_INVALID, "x strides reach too far");
  return KVQ_OK;
}

// Scales: rows of 16 bytes or more (D = 256, or groups of 16 at D = 128) are
// moved with 16-byte accesses, the others with 8-byte (encode) or 4-byte
// (decode) ones.
kvq_status check_scales_align(const kvq_plan* p, const uint16_t* scales) {
  const bool wide = (p->D == 256) || (p->D == 128 && p->G == 16);
  if (wide && !aligned(scales, 16))
    return fail(KVQ_ERR_ALIGN, "scales is not 16-byte aligned (D=%d, G=%d)", p->D, p->G);
  if (!aligned(scales, 8)) return fail(KVQ_ERR_ALIGN, "scales is not 8-byte aligned");
  return KVQ_OK;
}

std::mutex g_cu_mutex;
int g_cu_count[64] = {0};

}  // namespace

namespace kvq {

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(g_cu_mutex);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

}  // namespace kvq

extern "C" {

const char* kvq_version(void) { return "kvq 0.1 (gfx950)"; }

const char* kvq_strerror(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_ALIGN: return "misaligned pointer or stride";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

kvq_status kvq_plan_create_opt(int32_t D, int32_t G, int32_t bits, kvq_rotation rotation, uint64_t seed,
                               uint32_t options, kvq_plan** out) {
  try {
    if (!out) return fail(KVQ_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (options & ~static_cast<uint32_t>(KVQ_OPT_MFMA_ROTATION))
      return fail(KVQ_ERR_INVALID, "unknown option bits 0x%x", options);
    if ((options & KVQ_OPT_MFMA_ROTATION) && !(D == 128 && rotation == KVQ_SRFT))
      return fail(KVQ_ERR_UNSUPPORTED, "the matrix-core rotation is built for D=128 SRFT plans");
    if (kvq_status s = kvq_plan_create_ex(D, G, bits, rotation, seed, out)) return s;
    (*out)->options = options;
    return ok();
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_plan_create_ex(int32_t D, int32_t G, int32_t bits, kvq_rotation rotation, uint64_t seed,
                              kvq_plan** out) {
  try {
    if (!out) return fail(KVQ_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (rotation != KVQ_SRFT && rotation != KVQ_SRHT && rotation != KVQ_IDENTITY)
      return fail(KVQ_ERR_INVALID, "unknown rotation %d", (int)rotation);
    if (D != 128 && D != 256 && D != 80 && D != 96)
      return fail(KVQ_ERR_UNSUPPORTED, "D=%d (built: 80, 96, 128, 256)", (int)D);
    if (G != 32 && G != 16) return fail(KVQ_ERR_UNSUPPORTED, "G=%d (built: 32, 16)", (int)G);
    if (D % G) return fail(KVQ_ERR_UNSUPPORTED, "G=%d does not divide D=%d", (int)G, (int)D);
    if (bits != 4 && bits != 8) return fail(KVQ_ERR_UNSUPPORTED, "bits=%d (built: 4, 8)", (int)bits);
    if ((D == 80 || D == 96) && rotation == KVQ_SRHT)
      return fail(KVQ_ERR_UNSUPPORTED, "SRHT needs a power-of-two D (D=%d)", (int)D);
    kvq_plan* p = new (std::nothrow) kvq_plan;
    if (!p) return fail(KVQ_ERR_INVALID, "out of host memory");
    p->D = D;
    p->G = G;
    p->bits = bits;
    p->rotation = rotation;
    p->options = 0;
    p->seed = seed;
    std::memset(p->sign_bits, 0, sizeof(p->sign_bits));
    const int32_t n = sign_count(p);
    uint64_t state = seed;
    for (int32_t w = 0; w * 64 < n; ++w) {
      const uint64_t word = splitmix64_next(state);
      const int32_t nb = n - w * 64 < 64 ? n - w * 64 : 64;   // signs held by this word
      p->sign_bits[w] = nb == 64 ? word : (word & ((1ull << nb) - 1));
    }
    *out = p;
    return ok();
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_plan_create(int32_t D, int32_t G, kvq_rotation rotation, uint64_t seed, kvq_plan** out) {
  return kvq_plan_create_ex(D, G, 4, rotation, seed, out);
}

void kvq_plan_destroy(kvq_plan* plan) { delete plan; }

kvq_status kvq_plan_signs(const kvq_plan* plan, int8_t* host_signs, int64_t n) {
  if (kvq_status s = check_plan(plan)) return s;
  const int32_t want = sign_count(plan);
  if (n != want) return fail(KVQ_ERR_INVALID, "n=%lld, plan has %d signs", (long long)n, want);
  if (want > 0 && !host_signs) return fail(KVQ_ERR_INVALID, "host_signs is NULL");
  for (int32_t i = 0; i < want; ++i)
    host_signs[i] = ((plan->sign_bits[i / 64] >> (i % 64)) & 1) ? -1 : 1;
  return ok();
}

kvq_status kvq_plan_info(const kvq_plan* plan, int32_t* D, int32_t* G, int32_t* rotation) {
  return kvq_plan_info_ex(plan, D, G, nullptr, rotation);
}

kvq_status kvq_plan_options(const kvq_plan* plan, uint32_t* options) {
  if (kvq_status s = check_plan(plan)) return s;
  if (!options) return fail(KVQ_ERR_INVALID, "options is NULL");
  *options = plan->options;
  return ok();
}

kvq_status kvq_plan_info_ex(const kvq_plan* plan, int32_t* D, int32_t* G, int32_t* bits, int32_t* rotation) {
  if (kvq_status s = check_plan(plan)) return s;
  if (D) *D = plan->D;
  if (G) *G = plan->G;
  if (bits) *bits = plan->bits;
  if (rotation) *rotation = plan->rotation;
  return ok();
}

kvq_status kvq_encode(const kvq_plan* plan, const uint16_t* x, int64_t B, int64_t H, int64_t T,
                      int64_t x_sb, int64_t x_sh, int64_t x_st, const float* lambda, int64_t lambda_sb,
                      uint8_t* codes, uint16_t* scales, int64_t Tcap, int64_t t0, void* stream) {
  try {
    if (kvq_status s = check_plan(plan)) return s;
    if (B < 0 || H < 0 || T < 0 || Tcap < 0 || t0 < 0)
      return fail(KVQ_ERR_INVALID, "negative shape or offset");
    if (t0 + T > Tcap)
      return fail(KVQ_ERR_INVALID, "t0 + T = %lld exceeds Tcap = %lld", (long long)(t0 + T), (long long)Tcap);
    if (B == 0 || H == 0 || T == 0) return ok();
    if (kvq_status s = check_x(plan, x, B, H, T, x_sb, x_sh, x_st, lambda, lambda_sb)) return s;
    if (!codes || !scales) return fail(KVQ_ERR_INVALID, "codes or scales is NULL");
    if (!aligned(codes, 16)) return fail(KVQ_ERR_ALIGN, "codes is not 16-byte aligned");
    if (kvq_status s = check_scales_align(plan, scales)) return s;
    if (!product_ok(B, H, Tcap, plan->D)) return fail(KVQ_ERR_INVALID, "cache shape too large");
    kvq::CodecDesc d{};
    fill_signs(plan, d);
    d.x = x;
    d.codes = codes;
    d.scales = scales;
    d.lambda = lambda;
    d.lambda_sb = lambda_sb;
    d.B = B; d.H = H; d.T = T; d.Tcap = Tcap; d.t0 = t0;
    d.sb = x_sb; d.sh = x_sh; d.st = x_st;
    d.stream = static_cast<hipStream_t>(stream);
    return hip_status(kvq::launch_encode(d, 0), "kvq_encode launch");
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_rotate(const kvq_plan* plan, const uint16_t* x, int64_t B, int64_t H, int64_t T,
                      int64_t x_sb, int64_t x_sh, int64_t x_st, const float* lambda, int64_t lambda_sb,
                      float* w, void* stream) {
  try {
    if (kvq_status s = check_plan(plan)) return s;
    if (B < 0 || H < 0 || T < 0) return fail(KVQ_ERR_INVALID, "negative shape");
    if (B == 0 || H == 0 || T == 0) return ok();
    if (kvq_status s = check_x(plan, x, B, H, T, x_sb, x_sh, x_st, lambda, lambda_sb)) return s;
    if (!w) return fail(KVQ_ERR_INVALID, "w is NULL");
    if (!aligned(w, 16)) return fail(KVQ_ERR_ALIGN, "w is not 16-byte aligned");
    kvq::CodecDesc d{};
    fill_signs(plan, d);
    d.x = x;
    d.w = w;
    d.lambda = lambda;
    d.lambda_sb = lambda_sb;
    d.B = B; d.H = H; d.T = T; d.Tcap = T; d.t0 = 0;
    d.sb = x_sb; d.sh = x_sh; d.st = x_st;
    d.stream = static_cast<hipStream_t>(stream);
    return hip_status(kvq::launch_encode(d, 1), "kvq_rotate launch");
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_decode(const kvq_plan* plan, const uint8_t* codes, const uint16_t* scales, int64_t B, int64_t H,
                      int64_t Tcap, int64_t t0, int64_t T, const float* lambda, int64_t lambda_sb, void* y,
                      kvq_dtype y_dtype, int64_t y_sb, int64_t y_sh, int64_t y_st, void* stream) {
  try {
    if (kvq_status s = check_plan(plan)) return s;
    if (B < 0 || H < 0 || T < 0 || Tcap < 0 || t0 < 0)
      return fail(KVQ_ERR_INVALID, "negative shape or offset");
    if (t0 + T > Tcap)
      return fail(KVQ_ERR_INVALID, "t0 + T = %lld exceeds Tcap = %lld", (long long)(t0 + T), (long long)Tcap);
    if (y_dtype != KVQ_F16 && y_dtype != KVQ_F32) return fail(KVQ_ERR_INVALID, "unknown y_dtype");
    if (B == 0 || H == 0 || T == 0) return ok();
    if (!codes || !scales || !lambda || !y) return fail(KVQ_ERR_INVALID, "NULL pointer argument");
    if (!aligned(codes, 16)) return fail(KVQ_ERR_ALIGN, "codes is not 16-byte aligned");
    if (kvq_status s = check_scales_align(plan, scales)) return s;
    if (y_sb < 0 || y_sh < 0 || y_st < 0 || lambda_sb < 0)
      return fail(KVQ_ERR_INVALID, "strides must be non-negative");
    if (y_st >= kMaxTokenStride)
      return fail(KVQ_ERR_INVALID, "y token stride %lld is not below 2^28", (long long)y_st);
    if (plan->D == 128 || plan->D == 256) {
      // the decoders bring each lambda row into LDS with 16-byte direct loads
      if (!aligned(lambda, 16)) return fail(KVQ_ERR_ALIGN, "lambda is not 16-byte aligned (D=%d decode)", plan->D);
      if (lambda_sb % 4) return fail(KVQ_ERR_ALIGN, "lambda_sb must be a multiple of 4 (D=%d decode)", plan->D);
    } else if (!aligned(lambda, 4)) {
      return fail(KVQ_ERR_ALIGN, "lambda is not 4-byte aligned");
    }
    if (y_dtype == KVQ_F16) {
      if (!aligned(y, 16)) return fail(KVQ_ERR_ALIGN, "y is not 16-byte aligned");
      if (y_sb % 8 || y_sh % 8 || y_st % 8)
        return fail(KVQ_ERR_ALIGN, "fp16 y strides must be multiples of 8 elements");
    } else {
      if (!aligned(y, 8)) return fail(KVQ_ERR_ALIGN, "y is not 8-byte aligned");
      if (y_sb % 2 || y_sh % 2 || y_st % 2)
        return fail(KVQ_ERR_ALIGN, "fp32 y strides must be even");
    }
    if (!product_ok(B, H, Tcap, plan->D)) return fail(KVQ_ERR_INVALID, "shape too large");
    if (!extent_ok(B, H, T, y_sb, y_sh, y_st, plan->D)) return fail(KVQ_ERR_INVALID, "y strides reach too far");
    kvq::CodecDesc d{};
    fill_signs(plan, d);
    d.codes_in = codes;
    d.scales_in = scales;
    d.y = y;
    d.lambda = lambda;
    d.lambda_sb = lambda_sb;
    d.B = B; d.H = H; d.T = T; d.Tcap = Tcap; d.t0 = t0;
    d.sb = y_sb; d.sh = y_sh; d.st = y_st;
    d.stream = static_cast<hipStream_t>(stream);
    return hip_status(kvq::launch_decode(d, y_dtype == KVQ_F32), "kvq_decode launch");
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_attn_workspace_size(int32_t D, int64_t B, int64_t Hq, int64_t seq_len, size_t* bytes) {
  if (!bytes) return fail(KVQ_ERR_INVALID, "bytes is NULL");
  *bytes = 0;
  if (D != 128 && D != 256) return fail(KVQ_ERR_UNSUPPORTED, "D=%d", (int)D);
  if (B < 0 || Hq < 0 || seq_len < 0) return fail(KVQ_ERR_INVALID, "negative shape");
  if (!product_ok(B, Hq, seq_len > 0 ? seq_len : 1, D)) return fail(KVQ_ERR_INVALID, "shape too large");
  *bytes = kvq::attn_workspace_bytes(D, B, Hq, seq_len);
  return ok();
}

namespace {

kvq_status check_attn_common(int32_t D, const uint16_t* q, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tcap,
                             int64_t seq_len, void* out, kvq_dtype out_dtype, void* workspace,
                             size_t workspace_bytes, bool check_workspace) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || Tcap < 0) return fail(KVQ_ERR_INVALID, "bad shape");
  if (Tcap >= kMaxAttnTcap) return fail(KVQ_ERR_INVALID, "Tcap=%lld is not below 2^31", (long long)Tcap);
  if (Hq % Hkv) return fail(KVQ_ERR_INVALID, "Hq=%lld is not a multiple of Hkv=%lld", (long long)Hq, (long long)Hkv);
  if (seq_len < 1 || seq_len > Tcap)
    return fail(KVQ_ERR_INVALID, "seq_len=%lld outside [1, Tcap=%lld]", (long long)seq_len, (long long)Tcap);
  if (out_dtype != KVQ_F16 && out_dtype != KVQ_F32) return fail(KVQ_ERR_INVALID, "unknown out_dtype");
  if (!q || !out) return fail(KVQ_ERR_INVALID, "q or out is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(KVQ_ERR_ALIGN, "q and out must be 16-byte aligned");
  if (!product_ok(B, Hkv, Tcap, D)) return fail(KVQ_ERR_INVALID, "shape too large");
  if (!check_workspace) return KVQ_OK;
  const size_t need = kvq::attn_workspace_bytes(D, B, Hq, seq_len);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KVQ_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace ? workspace_bytes : 0);
  if (workspace && !aligned(workspace, 16)) return fail(KVQ_ERR_ALIGN, "workspace is not 16-byte aligned");
  return KVQ_OK;
}

kvq_status check_attn_plan(const kvq_plan* plan) {
  if (plan->D != 128 && plan->D != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "attention is built for D=128 and 256 (plan D=%d)", plan->D);
  return KVQ_OK;
}

kvq_status check_attn_cache(const uint8_t* k_codes, const uint16_t* k_scales, const float* lambda_k,
                            const uint8_t* v_codes, const uint16_t* v_scales, const float* lambda_v) {
  if (!k_codes || !k_scales || !lambda_k || !v_codes || !v_scales || !lambda_v)
    return fail(KVQ_ERR_INVALID, "NULL cache pointer");
  if (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_scales, 8) || !aligned(v_scales, 8) ||
      !aligned(lambda_k, 16) || !aligned(lambda_v, 16))
    return fail(KVQ_ERR_ALIGN, "cache codes need 16-byte, scales 8-byte, lambda 16-byte alignment");
  return KVQ_OK;
}

kvq::AttnDesc attn_desc(const kvq_plan* plan, const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                        const float* lambda_k, const uint8_t* v_codes, const uint16_t* v_scales,
                        const float* lambda_v, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tcap, int64_t seq_len,
                        float sm_scale, void* out, kvq_dtype out_dtype, void* workspace, void* stream) {
  kvq::AttnDesc d{};
  d.D = plan->D;
  d.rotation = plan->rotation;
  for (int i = 0; i < 4; ++i) d.signs[i] = plan->sign_bits[i];
  d.int4 = true;
  d.G = plan->G;
  d.bits = plan->bits;
  d.q = q;
  d.k_codes = k_codes; d.k_scales = k_scales; d.lambda_k = lambda_k;
  d.v_codes = v_codes; d.v_scales = v_scales; d.lambda_v = lambda_v;
  d.B = B; d.Hq = Hq; d.Hkv = Hkv; d.Tcap = Tcap; d.seq_len = seq_len;
  d.sm_scale = sm_scale;
  d.out = out;
  d.out_f32 = out_dtype == KVQ_F32;
  d.workspace = workspace;
  d.stream = static_cast<hipStream_t>(stream);
  return d;
}

}  // namespace

kvq_status kvq_attn_decode(const kvq_plan* plan, const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                           const float* lambda_k, const uint8_t* v_codes, const uint16_t* v_scales,
                           const float* lambda_v, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tcap, int64_t seq_len,
                           float sm_scale, void* out, kvq_dtype out_dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
  try {
    if (kvq_status s = check_plan(plan)) return s;
    if (kvq_status s = check_attn_plan(plan)) return s;
    if (kvq_status s = check_attn_common(plan->D, q, B, Hq, Hkv, Tcap, seq_len, out, out_dtype, workspace,
                                         workspace_bytes, true))
      return s;
    if (kvq_status s = check_attn_cache(k_codes, k_scales, lambda_k, v_codes, v_scales, lambda_v)) return s;
    if (B == 0 || Hq == 0) return ok();
    const kvq::AttnDesc d = attn_desc(plan, q, k_codes, k_scales, lambda_k, v_codes, v_scales, lambda_v, B, Hq,
                                      Hkv, Tcap, seq_len, sm_scale, out, out_dtype, workspace, stream);
    return hip_status(kvq::launch_attention(d), "kvq_attn_decode launch");
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_attn_decode_noalloc(const kvq_plan* plan, const uint16_t* q, const uint8_t* k_codes,
                                   const uint16_t* k_scales, const float* lambda_k, const uint8_t* v_codes,
                                   const uint16_t* v_scales, const float* lambda_v, int64_t B, int64_t Hq,
                                   int64_t Hkv, int64_t Tcap, int64_t seq_len, float sm_scale, void* out,
                                   kvq_dtype out_dtype, void* stream) {
  try {
    if (kvq_status s = check_plan(plan)) return s;
    if (kvq_status s = check_attn_plan(plan)) return s;
    // the workspace checks of the common validation are replaced by the
    // size check against the per-GPU buffer below
    if (kvq_status s = check_attn_common(plan->D, q, B, Hq, Hkv, Tcap, seq_len, out, out_dtype, nullptr, 0,
                                         /*check_workspace=*/false))
      return s;
    if (kvq_status s = check_attn_cache(k_codes, k_scales, lambda_k, v_codes, v_scales, lambda_v)) return s;
    if (B == 0 || Hq == 0) return ok();
    kvq::AttnDesc d = attn_desc(plan, q, k_codes, k_scales, lambda_k, v_codes, v_scales, lambda_v, B, Hq, Hkv,
                                Tcap, seq_len, sm_scale, out, out_dtype, nullptr, stream);
    const size_t need = kvq::attn_workspace_needed(d);
    if (need > kvq::kAttnScratchBytes)
      return fail(KVQ_ERR_WORKSPACE, "the call needs %zu bytes of split-K partials; the per-GPU buffer holds %zu",
                  need, kvq::kAttnScratchBytes);
    void* ws = nullptr;
    if (kvq_status s = hip_status(kvq::attn_scratch(&ws), "kvq_attn_decode_noalloc buffer address")) return s;
    d.workspace = ws;
    return hip_status(kvq::launch_attention(d), "kvq_attn_decode_noalloc launch");
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_attn_decode_f16(int32_t D, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                               int64_t Hq, int64_t Hkv, int64_t Tcap, int64_t seq_len, float sm_scale, void* out,
                               kvq_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (D != 128 && D != 256) return fail(KVQ_ERR_UNSUPPORTED, "attention is built for D=128 and 256 (D=%d)", (int)D);
    if (kvq_status s = check_attn_common(D, q, B, Hq, Hkv, Tcap, seq_len, out, out_dtype, workspace,
                                         workspace_bytes, true))
      return s;
    // the fp16 kernel addresses a row's tokens with 32-bit byte offsets
    if (Tcap * 2 * static_cast<int64_t>(D) > (int64_t(1) << 32))
      return fail(KVQ_ERR_INVALID, "fp16 cache rows of Tcap * 2D = %lld bytes pass 4 GiB",
                  (long long)(Tcap * 2 * static_cast<int64_t>(D)));
    if (!k || !v) return fail(KVQ_ERR_INVALID, "k or v is NULL");
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(KVQ_ERR_ALIGN, "k and v must be 16-byte aligned");
    if (B == 0 || Hq == 0) return ok();
    kvq::AttnDesc d{};
    d.D = D;
    d.rotation = KVQ_IDENTITY;
    d.int4 = false;
    d.q = q;
    d.k16 = k;
    d.v16 = v;
    d.B = B; d.Hq = Hq; d.Hkv = Hkv; d.Tcap = Tcap; d.seq_len = seq_len;
    d.sm_scale = sm_scale;
    d.out = out;
    d.out_f32 = out_dtype == KVQ_F32;
    d.workspace = workspace;
    d.stream = static_cast<hipStream_t>(stream);
    return hip_status(kvq::launch_attention(d), "kvq_attn_decode_f16 launch");
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_diag_shader_clock(uint64_t* out, int32_t iters, void* stream) {
  try {
    if (!out) return fail(KVQ_ERR_INVALID, "out is NULL");
    if (!aligned(out, 8)) return fail(KVQ_ERR_ALIGN, "out is not 8-byte aligned");
    if (iters < 1 || iters > (1 << 24)) return fail(KVQ_ERR_INVALID, "iters must be in [1, 2^24] (got %d)", iters);
    return hip_status(kvq::launch_shader_clock(out, iters, static_cast<hipStream_t>(stream)),
                      "kvq_diag_shader_clock launch");
  } catch (...) {
    return fail(KVQ_ERR_INVALID, "internal error");
  }
}

kvq_status kvq_diag_wall_clock_khz(int32_t* khz) {
  if (!khz) return fail(KVQ_ERR_INVALID, "khz is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  int rate = 0;
  e = hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return hip_status(e, "hipDeviceGetAttribute(WallClockRate)");
  *khz = rate;
  return ok();
}

}  // extern "C"
