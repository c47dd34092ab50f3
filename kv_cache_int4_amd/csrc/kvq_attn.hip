// Decode-step attention over the int4 cache (and the fp16-cache comparator).
//
// Head sizes D = 128 and 256: a head vector is NH = D / 128 halves of 128
// channels, and everything below runs once per half where it touches
// channels (loads, QK, PV, the query records), with the halves of a D = 256
// vector paired in the rotations exactly as the codec pairs them.
//
// Two launches per step on the caller's stream:
//   1. split:   one wave per (b, kv head, group of <= 4 query heads, context
//               split).  While its first block of the cache streams in, the
//               wave forms q~ = sm_scale * log2(e) * (R q) / lambda_K for
//               its heads (one lane per channel pair and half, the codec's
//               transform across lanes).  Scores can then be taken directly
//               against the stored codes: the cache holds lambda * R k, and
//               q . k^ = (R q) . (R k^).  For the int4 cache q~ is held as
//               three int8 limbs per 32-channel group,
//               q~ ~= s (Q1 + Q2/256 + Q3/65536) with s = max|q~| / 127
//               (about 23 bits), staged through a small LDS record; for the
//               fp16 cache as fp16 hi + lo halves.  Then the wave
//               streams its slice of the cache 32 tokens at a time:
//                 QK (int4): v_mfma_i32_16x16x64_i8, rows = 16 tokens,
//                   columns = (channel group, head) pairs, so every lane
//                   holds useful scores.  The codes enter as signed bytes
//                   16 q (each nibble moved to the top of its byte, top bit
//                   flipped: a shift and one bit operation per word), and
//                   the group scale multiplies the exact integer result.
//                 QK (fp16): v_mfma_f32_16x16x32_f16 on the fp16 keys.
//                 softmax: online, base 2, exact running maximum.
//                 PV: v_mfma_f32_16x16x32_f16.  For the int4 cache the rows
//                   are again (channel group, head) pairs: a row's weights
//                   p * scale_V carry the value scale of one group and the
//                   codes enter as exact small fp16 integers (n - 8, built
//                   from the nibble with a biased exponent).  The weights are
//                   split into fp16 hi + lo halves (two MFMAs), which keeps
//                   ~22 bits: one fp16 rounding of p costs up to ~5e-3
//                   relative error through cancellation across tokens.
//               It writes the partial (max, sum, D weighted values) of
//               every head to the workspace.
//   2. combine: merges the splits (log-sum-exp), divides by lambda_V and
//               applies the inverse rotation across the 64 lanes of a wave
//               (radix-2 steps with cross-lane shuffles; for D = 256 one
//               more radix-2 step between a lane's two halves).
//
// Method: the read side of the paper's fused quantizer ("When Quantization
// Is Free", abstract; gist.science explainer, "Methodik" 1-2) fused into the
// attention read that the paper times end to end (the abstract's decode
// latencies on Gemma-3 1B, head size 256, and Qwen2.5-1.5B, head size 128).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_attn_kernels.hpp"

namespace kvq {

namespace {

// Split count: one round of the waves a CU holds at once (waves_per_cu),
// at least 256 tokens per split.
void split_geometry(int64_t B, int64_t Hq, int64_t Hkv, int64_t seq_len, int64_t& S, int64_t& chunk,
                    int64_t& n_hchunks, int cus, int waves_per_cu) {
  const int64_t rep = Hq / Hkv;
  n_hchunks = (rep + kHeadsPerWave - 1) / kHeadsPerWave;
  const int64_t units = B * Hkv * n_hchunks;
  const int64_t target = static_cast<int64_t>(cus) * waves_per_cu;
  int64_t s = units > 0 ? (target + units - 1) / units : 1;
  const int64_t max_s = (seq_len + 255) / 256;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  chunk = (seq_len + s - 1) / s;
  chunk = (chunk + kBlk - 1) / kBlk * kBlk;
  S = (seq_len + chunk - 1) / chunk;
}

template <int ROT, int NH>
hipError_t run_attention(const AttnDesc& d, AttnArgs& a) {
  const int int4 = d.int4 ? 1 : 0;
  const unsigned nsplit = static_cast<unsigned>(d.B * d.Hkv * a.n_hchunks * a.S);
  const int fmt = (d.bits == 8 ? 2 : 0) + (d.G == 16 ? 1 : 0);
  if (!d.int4) {
    const hipError_t e = launch_attn_split_f16(a, NH, nsplit, d.stream);
    if (e != hipSuccess) return e;
  } else if (fmt == 1) {
    hipLaunchKernelGGL((attn_split_kernel<true, ROT, 1, NH>), dim3(nsplit), dim3(64), 0, d.stream, a);
  } else if (fmt == 2) {
    hipLaunchKernelGGL((attn_split_kernel<true, ROT, 2, NH>), dim3(nsplit), dim3(64), 0, d.stream, a);
  } else if (fmt == 3) {
    hipLaunchKernelGGL((attn_split_kernel<true, ROT, 3, NH>), dim3(nsplit), dim3(64), 0, d.stream, a);
  } else {
    hipLaunchKernelGGL((attn_split_kernel<true, ROT, 0, NH>), dim3(nsplit), dim3(64), 0, d.stream, a);
  }
  const unsigned nc = static_cast<unsigned>(d.B * d.Hq);
  if (d.out_f32) {
    hipLaunchKernelGGL((attn_combine_kernel<ROT, 1, NH>), dim3(nc), dim3(64), 0, d.stream, a, int4);
  } else {
    hipLaunchKernelGGL((attn_combine_kernel<ROT, 0, NH>), dim3(nc), dim3(64), 0, d.stream, a, int4);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int64_t max_splits(int64_t seq_len) { return (seq_len + 255) / 256 > 0 ? (seq_len + 255) / 256 : 1; }

// Workspace layout for S splits (256-aligned sections): (max, sum)
// [B*Hq][S][2] f32, then the partial sums [B*Hq][S][D] f32.
size_t workspace_for(int D, int64_t B, int64_t Hq, int64_t S) {
  const size_t rows = static_cast<size_t>(B * Hq);
  return align256(rows * S * 2 * 4) + align256(rows * S * D * 4);
}

// Split geometry of a call on the current device.
void geometry_of(const AttnDesc& d, AttnArgs& a) {
  const int wpc = d.D == 128 ? (d.int4 ? waves_per_cu<true, 1>() : waves_per_cu<false, 1>())
                             : (d.int4 ? waves_per_cu<true, 2>() : waves_per_cu<false, 2>());
  split_geometry(d.B, d.Hq, d.Hkv, d.seq_len, a.S, a.chunk, a.n_hchunks, device_cu_count(), wpc);
}

}  // namespace

// The workspace any call with this seq_len may need: the layout above for
// the largest split count a shape with this seq_len can use.
size_t attn_workspace_bytes(int D, int64_t B, int64_t Hq, int64_t seq_len) {
  return workspace_for(D, B, Hq, max_splits(seq_len));
}

// The workspace this call needs on the current device (its actual split
// count): at most attn_workspace_bytes.
size_t attn_workspace_needed(const AttnDesc& d) {
  AttnArgs a{};
  geometry_of(d, a);
  return workspace_for(d.D, d.B, d.Hq, a.S);
}

hipError_t launch_attention(const AttnDesc& d) {
  AttnArgs a{};
  a.q = d.q;
  a.k_codes = d.k_codes;
  a.k_scales = d.k_scales;
  a.lambda_k = d.lambda_k;
  a.v_codes = d.v_codes;
  a.v_scales = d.v_scales;
  a.lambda_v = d.lambda_v;
  a.k16 = d.k16;
  a.v16 = d.v16;
  a.out = d.out;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.Tcap = d.Tcap;
  a.seq_len = d.seq_len;
  a.sm_scale = d.sm_scale;
  for (int i = 0; i < 4; ++i) a.signs[i] = d.signs[i];
  geometry_of(d, a);
  if (a.S > max_splits(d.seq_len)) return hipErrorInvalidValue;
  const size_t rows = static_cast<size_t>(d.B * d.Hq);
  uint8_t* ws = static_cast<uint8_t*>(d.workspace);
  a.part_ml = reinterpret_cast<float*>(ws);
  a.part_acc = reinterpret_cast<float*>(ws + align256(rows * a.S * 2 * 4));
  if (d.D == 256) {
    switch (d.int4 ? d.rotation : KVQ_ROT_ID) {
      case KVQ_ROT_SRFT: return run_attention<KVQ_ROT_SRFT, 2>(d, a);
      case KVQ_ROT_SRHT: return run_attention<KVQ_ROT_SRHT, 2>(d, a);
      default: return run_attention<KVQ_ROT_ID, 2>(d, a);
    }
  }
  switch (d.int4 ? d.rotation : KVQ_ROT_ID) {
    case KVQ_ROT_SRFT: return run_attention<KVQ_ROT_SRFT, 1>(d, a);
    case KVQ_ROT_SRHT: return run_attention<KVQ_ROT_SRHT, 1>(d, a);
    default: return run_attention<KVQ_ROT_ID, 1>(d, a);
  }
}

}  // namespace kvq
