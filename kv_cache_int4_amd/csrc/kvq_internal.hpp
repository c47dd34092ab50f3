// Internal interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

enum { KVQ_ROT_SRFT = 0, KVQ_ROT_SRHT = 1, KVQ_ROT_ID = 2 };

// Plan options (kvq_plan_create_opt): the SRFT's DFT of the D = 128 encoder
// on the matrix cores.
constexpr uint32_t kOptMfmaRotation = 1u;

// A validated codec call (encode, rotate or decode).
struct CodecDesc {
  int D;
  int G;                      // group size: 32 or 16
  int bits;                   // code width: 4 or 8
  int rotation;
  uint32_t options;           // plan options (kOptMfmaRotation)
  uint64_t signs[4];          // sign bits, bit i of word i / 64
  const uint16_t* x;          // encode / rotate input
  const uint8_t* codes_in;    // decode input
  const uint16_t* scales_in;
  uint8_t* codes;             // encode output
  uint16_t* scales;
  float* w;                   // rotate output
  void* y;                    // decode output
  const float* lambda;
  int64_t lambda_sb;
  int64_t B, H, T, Tcap, t0;
  int64_t sb, sh, st;
  hipStream_t stream;
};

// A validated decode-step attention call.
struct AttnDesc {
  int D;
  int rotation;
  uint64_t signs[4];
  bool int4;                  // quantized cache (true) or fp16 cache (false)
  int G;                      // quantized cache: group size (32 or 16)
  int bits;                   // quantized cache: code width (4 or 8)
  const uint16_t* q;
  const uint8_t* k_codes;
  const uint16_t* k_scales;
  const float* lambda_k;
  const uint8_t* v_codes;
  const uint16_t* v_scales;
  const float* lambda_v;
  const uint16_t* k16;
  const uint16_t* v16;
  int64_t B, Hq, Hkv, Tcap, seq_len;
  float sm_scale;
  void* out;
  bool out_f32;
  void* workspace;
  hipStream_t stream;
};

// Compute units of the current device (cached per device).
int device_cu_count();

// mode 0 = encode (codes + scales), mode 1 = rotate (fp32 w)
hipError_t launch_encode(const CodecDesc& d, int mode);
hipError_t launch_decode(const CodecDesc& d, bool f32);
// D = 80 and 96 (SRFT over the mixed-radix DFT, or no rotation)
hipError_t launch_encode_mixed(const CodecDesc& d, int mode);
hipError_t launch_decode_mixed(const CodecDesc& d, bool f32);

// Split-K geometry of the attention kernels.
// Workspace bytes any call with this seq_len may need (the caller-owned
// workspace is sized by this), and bytes this call needs on the current
// device (no more than the former).
size_t attn_workspace_bytes(int D, int64_t B, int64_t Hq, int64_t seq_len);
size_t attn_workspace_needed(const AttnDesc& d);
hipError_t launch_attention(const AttnDesc& d);

// Size of the per-GPU buffer that stands in for the workspace of
// kvq_attn_decode_noalloc, and its device address on the current device
// (looked up once per device).
constexpr size_t kAttnScratchBytes = static_cast<size_t>(16) << 20;
hipError_t attn_scratch(void** ptr);

// Measurement aid: one wave records shader-clock and wall-clock ticks over
// a dependent chain of iters FMAs into out[0], out[1] (out[2]: scratch).
hipError_t launch_shader_clock(uint64_t* out, int iters, hipStream_t stream);

}  // namespace kvq
