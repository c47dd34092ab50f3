// Decode-step attention over the int4 cache (and the fp16-cache comparator).
//
// Three launches per step on the caller's stream:
//   1. qrot:    q~ = sm_scale * log2(e) * (R q) / lambda_K for every (b, h):
//               scores can then be taken directly against the rotated,
//               lambda-scaled cache, since q . k^ = (R q) . (R k^) and the
//               cache stores lambda * R k (one lane per query vector, the
//               same in-register FFT as the codec).
//   2. split:   one wave per (b, kv head, group of <= 4 query heads, context
//               split) streams its slice of the cache 16 tokens at a time:
//                 QK: v_mfma_f32_16x16x32_f16 with the 16 tokens as rows and
//                     the query heads as columns, one MFMA per 32-channel
//                     group (the group's fp16 scale is applied to the MFMA
//                     result); q~ is split into fp16 hi + lo halves so the
//                     product keeps ~22 bits;
//                 softmax: online, base 2, with the running maximum moved
//                     only when a score exceeds it by more than 2^8 (the
//                     common rescale factor cancels in the final division);
//                 PV: v_mfma_f32_16x16x16f16 with rows = (channel group,
//                     head) pairs, so each row's weights p * scale_V carry
//                     the value scale of one group and the int4 values enter
//                     the MFMA exactly as small integers.
//               It writes the partial (max, sum, 128 weighted values) of
//               every head to the workspace.
//   3. combine: merges the splits (log-sum-exp), divides by lambda_V and
//               applies the inverse rotation once per output vector.
//
// Method: the read side of the paper's fused quantizer ("When Quantization
// Is Free", abstract; gist.science explainer, "Methodik" 1-2) fused into the
// attention read that the paper times end to end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kHeadsPerWave = 4;
constexpr int kTok = 16;              // tokens per inner step

struct AttnArgs {
  const uint16_t* q;
  const uint8_t* k_codes;
  const uint16_t* k_scales;
  const float* lambda_k;
  const uint8_t* v_codes;
  const uint16_t* v_scales;
  const float* lambda_v;
  const uint16_t* k16;
  const uint16_t* v16;
  float* qt;          // [B*Hq][128] rotated, scaled queries
  float* part_acc;    // [B*Hq][S][128]
  float* part_ml;     // [B*Hq][S][2]
  void* out;
  int64_t B, Hq, Hkv, Tcap, seq_len;
  int64_t S, chunk;   // splits and tokens per split
  int64_t n_hchunks;  // ceil(rep / 4)
  float sm_scale;
  uint64_t signs[4];
};

// ---------------------------------------------------------------------------
// 1. query rotation
// ---------------------------------------------------------------------------
template <int ROT>
__global__ void __launch_bounds__(64) attn_qrot_kernel(AttnArgs a, int int4) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
  if (idx >= a.B * a.Hq) return;
  const int64_t h = idx % a.Hq;
  const int64_t g = h / (a.Hq / a.Hkv);
  const uint16_t* qr = a.q + idx * 128;
  float v[128];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint4 w = *reinterpret_cast<const uint4*>(qr + 8 * j);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * j + e;   // pair index
      uint32_t m = 0;
      if (int4 && ROT == KVQ_ROT_SRFT) {
        m = ((a.signs[k >> 6] >> (k & 63)) & 1) ? 0x80008000u : 0u;
      } else if (int4 && ROT == KVQ_ROT_SRHT) {
        const int i0 = 2 * k, i1 = 2 * k + 1;
        m = (static_cast<uint32_t>((a.signs[i0 >> 6] >> (i0 & 63)) & 1) << 15) |
            (static_cast<uint32_t>((a.signs[i1 >> 6] >> (i1 & 63)) & 1) << 31);
      }
      const uint32_t x = ws[e] ^ m;
      v[2 * k] = f16_bits_to_f32(x & 0xFFFFu);
      v[2 * k + 1] = f16_bits_to_f32(x >> 16);
    }
  }
  float* out = a.qt + idx * 128;
  if (!int4) {
    const float s = a.sm_scale * kLog2e;
#pragma unroll
    for (int j = 0; j < 128; j += 4)
      *reinterpret_cast<float4*>(out + j) = make_float4(v[j] * s, v[j + 1] * s, v[j + 2] * s, v[j + 3] * s);
    return;
  }
  float c = 1.f;
  if (ROT == KVQ_ROT_SRFT) {
    fft64<false>(v);
    c = 0.125f;
  } else if (ROT == KVQ_ROT_SRHT) {
    wht128(v);
    c = 0.0883883476483184405f;
  }
  const float s = a.sm_scale * kLog2e * c;
  const float* lk = a.lambda_k + g * 128;
#pragma unroll
  for (int j = 0; j < 128; j += 4) {
    float4 o;
    o.x = v[chan_reg<ROT>(j)] * s / lk[j];
    o.y = v[chan_reg<ROT>(j + 1)] * s / lk[j + 1];
    o.z = v[chan_reg<ROT>(j + 2)] * s / lk[j + 2];
    o.w = v[chan_reg<ROT>(j + 3)] * s / lk[j + 3];
    *reinterpret_cast<float4*>(out + j) = o;
  }
}

// ---------------------------------------------------------------------------
// 2. split-K streaming kernel
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// fp16 pair (lo, hi) = (q_a - 8, q_b - 8) from two offset nibbles sitting in
// bits 0..3 and 16..19 of x (the other bits zero): 0x6400 | n is the fp16
// value 1024 + n, exactly.
__device__ __forceinline__ uint32_t nib_pair_to_f16x2(uint32_t x) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = __builtin_bit_cast(h2, x | 0x64006400u);
  const h2 r = v - (h2){(_Float16)1032.0f, (_Float16)1032.0f};
  return __builtin_bit_cast(uint32_t, r);
}

template <bool INT4>
__global__ void __launch_bounds__(64, 2) attn_split_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int n16 = lane & 15;
  const int kq = lane >> 4;
  const int64_t rep = a.Hq / a.Hkv;

  int64_t blk = blockIdx.x;
  const int64_t s = blk % a.S;
  blk /= a.S;
  const int64_t hc = blk % a.n_hchunks;
  const int64_t bg = blk / a.n_hchunks;
  const int64_t b = bg / a.Hkv;
  const int64_t g = bg - b * a.Hkv;
  const int64_t hq0 = g * rep + hc * kHeadsPerWave;
  const int nh = static_cast<int>(rep - hc * kHeadsPerWave < kHeadsPerWave ? rep - hc * kHeadsPerWave
                                                                          : kHeadsPerWave);
  const int64_t t_begin = s * a.chunk;
  int64_t t_end = t_begin + a.chunk;
  if (t_end > a.seq_len) t_end = a.seq_len;

  // QK right operand: q~ of head n16 (zero for padding columns), channels
  // 32 grp + 8 kq + {0, 4, 1, 5, 2, 6, 3, 7} in the eight k slots -- the
  // order in which the key nibbles are unpacked below.
  half8_t qb_hi[4], qb_lo[4];
  {
    const float* qrow = a.qt + (b * a.Hq + hq0 + (n16 < nh ? n16 : 0)) * 128;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ch = 32 * grp + 8 * kq + p + 4 * e;
          const float x = (n16 < nh) ? qrow[ch] : 0.f;
          const _Float16 hi = static_cast<_Float16>(x);
          const _Float16 lo = static_cast<_Float16>(x - static_cast<float>(hi));
          qb_hi[grp][2 * p + e] = hi;
          qb_lo[grp][2 * p + e] = lo;
        }
      }
    }
  }

  float4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max of head n16 (same in its 4 lanes)
  float l_part = 0.f;        // this lane's share of the running sum

  const int64_t row_kv = b * a.Hkv + g;
  // useful PV rows: int4 rows are (channel group, head) = (n16 / 4, n16 % 4);
  // fp16 rows are heads.
  const int pv_head = INT4 ? (n16 & 3) : n16;

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTok) {
    // ---- keys: A operand (token n16, k slice kq of each group) ----
    const int64_t tk = t0 + n16;
    const bool kvalid = tk < t_end;
    half8_t ka[4];
    if (INT4) {
      const uint32_t* krow = reinterpret_cast<const uint32_t*>(a.k_codes + (row_kv * a.Tcap + tk) * 64);
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const uint32_t w = kvalid ? krow[4 * grp + kq] : 0x88888888u;
        // slots (2p, 2p+1) = nibbles (p, p + 4)
        uint32_t h2[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) h2[p] = nib_pair_to_f16x2((w >> (4 * p)) & 0x000F000Fu);
        ka[grp] = __builtin_bit_cast(half8_t, make_uint4(h2[0], h2[1], h2[2], h2[3]));
      }
    } else {
      const uint16_t* krow = a.k16 + (row_kv * a.Tcap + tk) * 128;
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        uint4 w = kvalid ? *reinterpret_cast<const uint4*>(krow + 32 * grp + 8 * kq) : make_uint4(0, 0, 0, 0);
        // reorder the 8 channels to slots {0, 4, 1, 5, 2, 6, 3, 7}
        const uint32_t c01 = w.x, c23 = w.y, c45 = w.z, c67 = w.w;
        const uint32_t s0 = __builtin_amdgcn_perm(c45, c01, 0x05040100u);  // (c0, c4)
        const uint32_t s1 = __builtin_amdgcn_perm(c45, c01, 0x07060302u);  // (c1, c5)
        const uint32_t s2 = __builtin_amdgcn_perm(c67, c23, 0x05040100u);  // (c2, c6)
        const uint32_t s3 = __builtin_amdgcn_perm(c67, c23, 0x07060302u);  // (c3, c7)
        ka[grp] = __builtin_bit_cast(half8_t, make_uint4(s0, s1, s2, s3));
      }
    }

    // ---- scores: C[token 4 kq + i][head n16] ----
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
    if (INT4) {
      // key scales of this lane's four output tokens
      uint2 ks[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 4 * kq + i;
        ks[i] = (t < t_end) ? *reinterpret_cast<const uint2*>(a.k_scales + (row_kv * a.Tcap + t) * 4)
                            : make_uint2(0, 0);
      }
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        float4_t c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[grp], qb_hi[grp], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[grp], qb_lo[grp], c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t sw = (grp < 2 ? ks[i].x : ks[i].y) >> (16 * (grp & 1));
          sc[i] = fmaf(f16_bits_to_f32(sw & 0xFFFFu), c[i], sc[i]);
        }
      }
    } else {
      float4_t c = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[grp], qb_hi[grp], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[grp], qb_lo[grp], c, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = c[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (t0 + 4 * kq + i >= t_end) sc[i] = -INFINITY;

    // ---- online softmax (base 2) ----
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = fmaxf(bm, shfl_xor(bm, 16));
    bm = fmaxf(bm, shfl_xor(bm, 32));
    const bool grow = bm > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_run, bm);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      l_part *= alpha;
      m_run = m_new;
      // rescale the PV accumulator rows of every head
      float al[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) al[h] = __shfl(alpha, h, 64);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[c][i] *= INT4 ? al[i] : (kq == 0 ? al[i] : 1.f);
      }
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2f(sc[i] - m_run);
      l_part += p[i];
    }

    // ---- PV left operand: rows (group, head) for int4, heads for fp16 ----
    half4_t pa;
    if (INT4) {
      const int src = (lane & ~15) | pv_head;     // lane holding head pv_head
      const int grp = n16 >> 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pi = __shfl(p[i], src, 64);
        const int64_t t = t0 + 4 * kq + i;
        float sv = 0.f;
        if (t < t_end) sv = f16_bits_to_f32(a.v_scales[(row_kv * a.Tcap + t) * 4 + grp]);
        pa[i] = static_cast<_Float16>(pi * sv);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = static_cast<_Float16>(p[i]);
    }

    // ---- values: lane (n16, kq) reads 8 channels 8 n16 .. 8 n16 + 7 of
    // tokens 4 kq .. 4 kq + 3; MFMA c takes channel 8 n16 + c ----
    if (INT4) {
      uint32_t vw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 4 * kq + i;
        vw[i] = (t < t_end) ? reinterpret_cast<const uint32_t*>(a.v_codes + (row_kv * a.Tcap + t) * 64)[n16]
                            : 0x88888888u;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int by = c >> 1;
        const uint32_t sel = 0x0c000c00u | (static_cast<uint32_t>(4 + by) << 16) | static_cast<uint32_t>(by);
        uint32_t x01 = __builtin_amdgcn_perm(vw[1], vw[0], sel);
        uint32_t x23 = __builtin_amdgcn_perm(vw[3], vw[2], sel);
        if (c & 1) { x01 >>= 4; x23 >>= 4; }
        const uint32_t h01 = nib_pair_to_f16x2(x01 & 0x000F000Fu);
        const uint32_t h23 = nib_pair_to_f16x2(x23 & 0x000F000Fu);
        const half4_t vb = __builtin_bit_cast(half4_t, make_uint2(h01, h23));
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, acc[c], 0, 0, 0);
      }
    } else {
      uint4 vr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 4 * kq + i;
        vr[i] = (t < t_end) ? *reinterpret_cast<const uint4*>(a.v16 + (row_kv * a.Tcap + t) * 128 + 8 * n16)
                            : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t w0 = (&vr[0].x)[c >> 1], w1 = (&vr[1].x)[c >> 1];
        const uint32_t w2 = (&vr[2].x)[c >> 1], w3 = (&vr[3].x)[c >> 1];
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t h01 = __builtin_amdgcn_perm(w1, w0, sel);
        const uint32_t h23 = __builtin_amdgcn_perm(w3, w2, sel);
        const half4_t vb = __builtin_bit_cast(half4_t, make_uint2(h01, h23));
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, acc[c], 0, 0, 0);
      }
    }
  }

  // ---- partial results ----
  l_part += shfl_xor(l_part, 16);
  l_part += shfl_xor(l_part, 32);
  const int64_t ws_base = (b * a.Hq + hq0);
  if (kq == 0 && n16 < nh) {
    float* ml = a.part_ml + ((ws_base + n16) * a.S + s) * 2;
    ml[0] = m_run;
    ml[1] = l_part;
  }
  // acc[c][i]: row (int4: group kq, head i; fp16: head 4 kq + i), channel 8 n16 + c
  const bool useful = INT4 ? (kq == (n16 >> 2)) : (kq == 0);
  if (useful) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nh) {
        float* dst = a.part_acc + ((ws_base + i) * a.S + s) * 128 + 8 * n16;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. combine splits, inverse rotation
// ---------------------------------------------------------------------------
template <int ROT, int OUT_F32>
__global__ void __launch_bounds__(64) attn_combine_kernel(AttnArgs a, int int4) {
  __shared__ float sh[128];
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t h = bh % a.Hq;
  const int64_t g = h / (a.Hq / a.Hkv);
  const float* ml = a.part_ml + bh * a.S * 2;
  float m = -INFINITY;
  for (int64_t s = 0; s < a.S; ++s) m = fmaxf(m, ml[2 * s]);
  float l = 0.f, x0 = 0.f, x1 = 0.f;
  for (int64_t s = 0; s < a.S; ++s) {
    const float ms = ml[2 * s];
    if (ms == -INFINITY) continue;
    const float wgt = exp2f(ms - m);
    l = fmaf(wgt, ml[2 * s + 1], l);
    const float2 v = *reinterpret_cast<const float2*>(a.part_acc + (bh * a.S + s) * 128 + 2 * lane);
    x0 = fmaf(wgt, v.x, x0);
    x1 = fmaf(wgt, v.y, x1);
  }
  const float inv = 1.f / l;
  sh[2 * lane] = x0 * inv;
  sh[2 * lane + 1] = x1 * inv;
  __syncthreads();
  if (lane != 0) return;

  float v[128];
  if (int4) {
    float c = 1.f;
    if (ROT == KVQ_ROT_SRFT) c = 0.125f;
    else if (ROT == KVQ_ROT_SRHT) c = 0.0883883476483184405f;
    const float* lv = a.lambda_v + g * 128;
#pragma unroll
    for (int j = 0; j < 128; ++j) v[j] = sh[j] * c / lv[j];
    if (ROT == KVQ_ROT_SRFT) fft64<true>(v);
    else if (ROT == KVQ_ROT_SRHT) wht128(v);
  } else {
#pragma unroll
    for (int j = 0; j < 128; ++j) v[j] = sh[j];
  }
#pragma unroll
  for (int k = 0; k < 64; ++k) {
    const int p = (int4 && ROT == KVQ_ROT_SRFT) ? rev4(k) : k;
    float lo = v[2 * p], hi = v[2 * p + 1];
    if (int4 && ROT == KVQ_ROT_SRFT) {
      if ((a.signs[k >> 6] >> (k & 63)) & 1) { lo = -lo; hi = -hi; }
    } else if (int4 && ROT == KVQ_ROT_SRHT) {
      const int i0 = 2 * k, i1 = 2 * k + 1;
      if ((a.signs[i0 >> 6] >> (i0 & 63)) & 1) lo = -lo;
      if ((a.signs[i1 >> 6] >> (i1 & 63)) & 1) hi = -hi;
    }
    if (OUT_F32) {
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + bh * 128 + 2 * k) = make_float2(lo, hi);
    } else {
      static_cast<uint32_t*>(a.out)[bh * 64 + k] = pack_f16x2(lo, hi);
    }
  }
}

// Split count: about two waves per CU slot across the whole grid, at least
// 256 tokens per split.
void split_geometry(int64_t B, int64_t Hq, int64_t Hkv, int64_t seq_len, int64_t& S, int64_t& chunk,
                    int64_t& n_hchunks, int cus) {
  const int64_t rep = Hq / Hkv;
  n_hchunks = (rep + kHeadsPerWave - 1) / kHeadsPerWave;
  const int64_t units = B * Hkv * n_hchunks;
  const int64_t target = static_cast<int64_t>(cus) * 16;
  int64_t s = units > 0 ? (target + units - 1) / units : 1;
  const int64_t max_s = (seq_len + 255) / 256;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  chunk = (seq_len + s - 1) / s;
  chunk = (chunk + kTok - 1) / kTok * kTok;
  S = (seq_len + chunk - 1) / chunk;
}

template <int ROT>
hipError_t run_attention(const AttnDesc& d, AttnArgs& a) {
  const int int4 = d.int4 ? 1 : 0;
  const unsigned nq = static_cast<unsigned>((d.B * d.Hq + 63) / 64);
  hipLaunchKernelGGL((attn_qrot_kernel<ROT>), dim3(nq), dim3(64), 0, d.stream, a, int4);
  const unsigned nsplit = static_cast<unsigned>(d.B * d.Hkv * a.n_hchunks * a.S);
  if (d.int4) {
    hipLaunchKernelGGL((attn_split_kernel<true>), dim3(nsplit), dim3(64), 0, d.stream, a);
  } else {
    hipLaunchKernelGGL((attn_split_kernel<false>), dim3(nsplit), dim3(64), 0, d.stream, a);
  }
  const unsigned nc = static_cast<unsigned>(d.B * d.Hq);
  if (d.out_f32) {
    hipLaunchKernelGGL((attn_combine_kernel<ROT, 1>), dim3(nc), dim3(64), 0, d.stream, a, int4);
  } else {
    hipLaunchKernelGGL((attn_combine_kernel<ROT, 0>), dim3(nc), dim3(64), 0, d.stream, a, int4);
  }
  return hipGetLastError();
}

// Workspace layout (bytes, 256-aligned sections): qt [B*Hq*128] f32,
// part_ml [B*Hq*S*2] f32, part_acc [B*Hq*S*128] f32.
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

int64_t attn_num_splits(int64_t B, int64_t Hkv, int64_t seq_len) {
  int64_t S, chunk, nh;
  split_geometry(B, Hkv * 4, Hkv, seq_len, S, chunk, nh, device_cu_count());
  return S;
}

size_t attn_workspace_bytes(int D, int64_t B, int64_t Hq, int64_t seq_len) {
  (void)D;
  // sized for the largest split count any Hkv could produce (Hkv = 1)
  const int64_t S = (seq_len + 255) / 256 > 0 ? (seq_len + 255) / 256 : 1;
  const size_t rows = static_cast<size_t>(B * Hq);
  return align256(rows * 128 * 4) + align256(rows * S * 2 * 4) + align256(rows * S * 128 * 4);
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
  split_geometry(d.B, d.Hq, d.Hkv, d.seq_len, a.S, a.chunk, a.n_hchunks, device_cu_count());
  const int64_t max_s = (d.seq_len + 255) / 256 > 0 ? (d.seq_len + 255) / 256 : 1;
  if (a.S > max_s) return hipErrorInvalidValue;
  const size_t rows = static_cast<size_t>(d.B * d.Hq);
  uint8_t* ws = static_cast<uint8_t*>(d.workspace);
  a.qt = reinterpret_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + align256(rows * 128 * 4));
  a.part_acc = reinterpret_cast<float*>(ws + align256(rows * 128 * 4) + align256(rows * max_s * 2 * 4));
  switch (d.int4 ? d.rotation : KVQ_ROT_ID) {
    case KVQ_ROT_SRFT: return run_attention<KVQ_ROT_SRFT>(d, a);
    case KVQ_ROT_SRHT: return run_attention<KVQ_ROT_SRHT>(d, a);
    default: return run_attention<KVQ_ROT_ID>(d, a);
  }
}

}  // namespace kvq
