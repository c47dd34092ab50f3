// Decode-step attention over the int4 cache (and the fp16-cache comparator).
//
// Two launches per step on the caller's stream:
//   1. split:   one wave per (b, kv head, group of <= 4 query heads, context
//               split).  While its first block of the cache streams in, the
//               wave forms q~ = sm_scale * log2(e) * (R q) / lambda_K for
//               its heads (one lane per channel pair, the codec's transform
//               across lanes).  Scores can then be taken directly against
//               the stored codes: the cache holds lambda * R k, and
//               q . k^ = (R q) . (R k^).  For the int4 cache q~ is held as
//               three int8 limbs per 32-channel group,
//               q~ ~= s (Q1 + Q2/256 + Q3/65536) with s = max|q~| / 127
//               (about 23 bits), staged through a small LDS record; for the
//               fp16 cache as fp16 hi + lo halves.  Then the wave
//               streams its slice of the cache 32 tokens at a time:
//                 QK (int4): v_mfma_i32_16x16x64_i8, rows = 16 tokens,
//                   columns = (channel group, head) pairs, so every lane
//                   holds useful scores.  The codes enter as unsigned
//                   nibbles (n = q + 8, one AND and one shift per word); the
//                   -8 offset is the accumulator's initial value, and the
//                   group scale multiplies the exact integer result.
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
//               It writes the partial (max, sum, 128 weighted values) of
//               every head to the workspace.
//   2. combine: merges the splits (log-sum-exp), divides by lambda_V and
//               applies the inverse rotation across the 64 lanes of a wave
//               (radix-2 steps with cross-lane shuffles).
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

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kHeadsPerWave = 4;
constexpr int kBlk = 32;              // tokens per inner step
// Record layout (quantized cache; 448 bytes, 544 with the sums per 16
// channels): three int8 limbs per channel,
// q~ ~= s (Q1 + Q2 / 256 + Q3 / 65536): [0,128) Q1, [128,256) Q2,
// [256,384) Q3, [384,400) s[4] f32, [400,448) sums of Q1, Q2, Q3 per group
// (i32[3][4]).
constexpr int kRecS = 384;
constexpr int kRecSum = 400;
constexpr int kRecSum16 = 448;        // groups of 16: sums per 16 channels, i32[3][8]

__constant__ TwTable kTw64Const = make_twiddles(64);

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
  float* part_acc;    // [B*Hq][S][128]
  float* part_ml;     // [B*Hq][S][2]
  void* out;
  int64_t B, Hq, Hkv, Tcap, seq_len;
  int64_t S, chunk;   // splits and tokens per split
  int64_t n_hchunks;  // ceil(rep / 4)
  float sm_scale;
  uint64_t signs[4];
};

__device__ __forceinline__ uint32_t sign_bit(const uint64_t (&s)[4], int i) {
  const uint64_t w = i < 64 ? s[0] : i < 128 ? s[1] : i < 192 ? s[2] : s[3];
  return static_cast<uint32_t>(w >> (i & 63)) & 1u;
}

// ---------------------------------------------------------------------------
// Query rotation (the start of the split kernel)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Maximum of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows):
// v_permlane16_swap / v_permlane32_swap exchange rows inside the VALU, so
// each step leaves the pair (x[l], x[l ^ 16]) (then ^ 32) in its two
// registers.  Written as assembly: the compiler folds the max of the two
// results of its swap intrinsics down to one of them.  The s_nop covers the
// VALU write of the operands just before the swap.
__device__ __forceinline__ float max_over_rows(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  x = fmaxf(a, b);
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

__device__ __forceinline__ int bitrev6(int x) {
  return static_cast<int>(__builtin_bitreverse32(static_cast<uint32_t>(x)) >> 26);
}

// Loads of the query rotation (int4 cache): the lane's pair word of each of
// the wave's heads, its two lambda_K entries and the twiddles of its six
// butterfly stages.  They are issued before the first cache block, so that
// waiting for them does not wait for the block.
struct QueryIn {
  uint32_t w[4];      // head hh: fp16 pair bitrev(lane) (SRFT) or lane
  float l0, l1;       // lambda_K of channels 2 lane, 2 lane + 1
  float cw[6], sw[6]; // SRFT stage twiddles
};

template <int ROT>
__device__ __forceinline__ void query_loads(const AttnArgs& a, const uint16_t* q0, int nh, const float* lk, int lane,
                                            QueryIn& in) {
  const int k = ROT == KVQ_ROT_SRFT ? bitrev6(lane) : lane;
#pragma unroll
  for (int hh = 0; hh < kHeadsPerWave; ++hh)
    in.w[hh] = hh < nh ? reinterpret_cast<const uint32_t*>(q0 + hh * 128)[k] : 0u;
  in.l0 = lk[2 * lane];
  in.l1 = lk[2 * lane + 1];
  if (ROT == KVQ_ROT_SRFT) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int hh = 1 << i;
      const int e = (lane & (hh - 1)) * (32 / hh);
      in.cw[i] = kTw64Const.c[e];
      in.sw[i] = kTw64Const.s[e];
    }
  }
}

// Rotated query records of the wave's four heads (int4 cache), computed by
// one wave from the pair words in.w: lane l owns channels 2l, 2l+1 of every
// head.  The heads advance together through each cross-lane step (four
// independent shuffles per wait); the records go to LDS at rec + head * REC
// (with the per-16-channel limb sums when SUM16).
template <int ROT, int REC, bool SUM16>
__device__ __forceinline__ void query_records(const AttnArgs& a, const QueryIn& in, int lane, uint8_t* rec) {
  constexpr int NH = kHeadsPerWave;
  float y0[NH], y1[NH];   // rotated channels 2 lane, 2 lane + 1 (unnormalized)
  float c = 1.f;
  if (ROT == KVQ_ROT_SRFT) {
    // forward 64-point DFT across lanes, radix-2 decimation in time: lane l
    // starts with pair bitrev(l) (signed) and ends with frequency l
    const uint32_t m = sign_bit(a.signs, bitrev6(lane)) ? 0x80008000u : 0u;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const uint32_t w = in.w[h] ^ m;
      y0[h] = f16_bits_to_f32(w & 0xFFFFu);
      y1[h] = f16_bits_to_f32(w >> 16);
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int hh = 1 << i;
      const bool upper = lane & hh;
      const float cw = in.cw[i], sw = in.sw[i];
      float pr[NH], pi[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        pr[h] = shfl_xor(y0[h], hh);
        pi[h] = shfl_xor(y1[h], hh);
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        // t = W^j * (the upper element), W = exp(-2 pi i / (2 hh))
        const float ur = upper ? y0[h] : pr[h], ui = upper ? y1[h] : pi[h];
        const float tr = ur * cw + ui * sw, ti = ui * cw - ur * sw;
        const float br = upper ? pr[h] : y0[h], bi = upper ? pi[h] : y1[h];
        y0[h] = upper ? br - tr : br + tr;
        y1[h] = upper ? bi - ti : bi + ti;
      }
    }
    c = 0.125f;
  } else {
    uint32_t m = 0;
    if (ROT == KVQ_ROT_SRHT) m = (sign_bit(a.signs, 2 * lane) << 15) | (sign_bit(a.signs, 2 * lane + 1) << 31);
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      y0[h] = f16_bits_to_f32((in.w[h] ^ m) & 0xFFFFu);
      y1[h] = f16_bits_to_f32((in.w[h] ^ m) >> 16);
    }
    if (ROT == KVQ_ROT_SRHT) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const float t0 = y0[h] + y1[h], t1 = y0[h] - y1[h];
        y0[h] = t0;
        y1[h] = t1;
      }
#pragma unroll
      for (int hh = 1; hh <= 32; hh <<= 1) {
        float p0[NH], p1[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          p0[h] = shfl_xor(y0[h], hh);
          p1[h] = shfl_xor(y1[h], hh);
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          if (lane & hh) { y0[h] = p0[h] - y0[h]; y1[h] = p1[h] - y1[h]; }
          else { y0[h] += p0[h]; y1[h] += p1[h]; }
        }
      }
      c = 0.0883883476483184405f;
    }
  }
  const float sc = a.sm_scale * kLog2e * c;
  const float r0 = sc / in.l0, r1 = sc / in.l1;
  float q0[NH], q1[NH], amax[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    q0[h] = y0[h] * r0;
    q1[h] = y1[h] * r1;
    amax[h] = fmaxf(fabsf(q0[h]), fabsf(q1[h]));
  }
  // group = 16 lanes: abs max, three int8 limbs
#pragma unroll
  for (int m = 1; m <= 8; m <<= 1) {
    float o[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) o[h] = shfl_xor(amax[h], m);
#pragma unroll
    for (int h = 0; h < NH; ++h) amax[h] = fmaxf(amax[h], o[h]);
  }
  int li[NH][3][2];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const float inv = amax[h] > 0.f ? 127.f / amax[h] : 0.f;
    const float t[2] = {q0[h] * inv, q1[h] * inv};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      // |t| <= 127; each residual is at most half a unit of its limb
      float r1 = rintf(t[e]);
      const float u = (t[e] - r1) * 256.f;
      float r2 = rintf(u);
      const float r3 = fminf(fmaxf(rintf((u - r2) * 256.f), -128.f), 127.f);
      if (r2 > 127.f) {          // +128 is no int8: carry into the first limb
        r2 -= 256.f;
        r1 += 1.f;
      }
      li[h][0][e] = static_cast<int>(r1);
      li[h][1][e] = static_cast<int>(r2);
      li[h][2][e] = static_cast<int>(r3);
    }
  }
  float sum[NH][3];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int limb = 0; limb < 3; ++limb) sum[h][limb] = static_cast<float>(li[h][limb][0] + li[h][limb][1]);
  float sum16[NH][3];      // after the steps over 8 lanes: sums per 16 channels
#pragma unroll
  for (int m = 1; m <= 8; m <<= 1) {
    if (m == 8) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int limb = 0; limb < 3; ++limb) sum16[h][limb] = sum[h][limb];
    }
    float o[NH][3];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int limb = 0; limb < 3; ++limb) o[h][limb] = shfl_xor(sum[h][limb], m);
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int limb = 0; limb < 3; ++limb) sum[h][limb] += o[h][limb];
  }
  const int grp = lane >> 4;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    uint8_t* r = rec + h * REC;
#pragma unroll
    for (int limb = 0; limb < 3; ++limb) {
      reinterpret_cast<uint16_t*>(r + 128 * limb)[lane] =
          static_cast<uint16_t>((li[h][limb][0] & 0xFF) | ((li[h][limb][1] & 0xFF) << 8));
      if ((lane & 15) == 0) reinterpret_cast<int*>(r + kRecSum)[4 * limb + grp] = static_cast<int>(sum[h][limb]);
      if (SUM16 && (lane & 7) == 0)
        reinterpret_cast<int*>(r + kRecSum16)[8 * limb + (lane >> 3)] = static_cast<int>(sum16[h][limb]);
    }
    if ((lane & 15) == 0) reinterpret_cast<float*>(r + kRecS)[grp] = amax[h] > 0.f ? amax[h] / 127.f : 0.f;
  }
}

// ---------------------------------------------------------------------------
// 1. split-K streaming kernel
// ---------------------------------------------------------------------------
// x + (x of lane (l + n) mod 16 within the row): DPP row_ror
template <int N>
__device__ __forceinline__ float add_row_ror(float x) {
  const float r = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF, true));
  return x + r;
}

// Cache loads of one 32-token block (sub-blocks sb = 0, 1 of 16 tokens).
template <bool INT4>
struct Blk {
  uint4 k[2];            // int4: 16 code bytes of token 16 sb + n16, group kq
  uint4 kf[2][4];        // fp16: 8 channels of each group for that token
  uint32_t v[2][4];      // int4: code dword n16 of token 16 sb + 4 kq + i
  uint4 vf[2][4];        // fp16: channels 8 n16 .. 8 n16 + 7 of that token
  uint16_t ks[2][4];     // int4: key scale of token 16 sb + 4 kq + i, group n16 / 4
  uint16_t vs[2][4];     // int4: value scale of the same token, group n16 / 4
};

// Row-relative bases of one (batch, kv head): every offset below is 32-bit.
struct Rows {
  const uint8_t* kc;     // int4 codes of token 0
  const uint16_t* ksc;
  const uint8_t* vc;
  const uint16_t* vsc;
  const uint16_t* k16;   // fp16 cache
  const uint16_t* v16;
};

// Token index actually read: in the last (tail) block of a split the
// positions past the end re-read its last token; their scores are masked.
template <bool TAIL>
__device__ __forceinline__ uint32_t tok(uint32_t t, uint32_t t_last) {
  return TAIL ? min(t, t_last) : t;
}

// Loads at a wave-uniform base plus an unsigned 32-bit lane offset (the
// SGPR-base form of the global load instructions).
template <typename T>
__device__ __forceinline__ T ld(const void* base, uint32_t off) {
  return *reinterpret_cast<const T*>(static_cast<const uint8_t*>(base) + off);
}

template <bool INT4, bool TAIL>
__device__ __forceinline__ void load_blk(const Rows& r, uint32_t t0, uint32_t t_last, uint32_t n16, uint32_t kq,
                                         Blk<INT4>& o) {
  const uint32_t grp = n16 >> 2;
#pragma unroll
  for (uint32_t sb = 0; sb < 2; ++sb) {
    const uint32_t tk = tok<TAIL>(t0 + 16 * sb + n16, t_last);
    if (INT4) {
      o.k[sb] = ld<uint4>(r.kc, (tk << 6) + (kq << 4));
    } else {
#pragma unroll
      for (uint32_t gq = 0; gq < 4; ++gq) o.kf[sb][gq] = ld<uint4>(r.k16, (tk << 8) + 64 * gq + 16 * kq);
    }
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
      const uint32_t t = tok<TAIL>(t0 + 16 * sb + 4 * kq + i, t_last);
      if (INT4) {
        o.v[sb][i] = ld<uint32_t>(r.vc, (t << 6) + (n16 << 2));
        o.ks[sb][i] = ld<uint16_t>(r.ksc, (t << 3) + (grp << 1));
        o.vs[sb][i] = ld<uint16_t>(r.vsc, (t << 3) + (grp << 1));
      } else {
        o.vf[sb][i] = ld<uint4>(r.v16, (t << 8) + (n16 << 4));
      }
    }
  }
}

// Per-wave streaming state.
template <bool INT4>
struct State {
  int4_t qb[3][2];           // int4 QK right operand: [limb][k-step]
  int4_t corr[3];            // int4 accumulator start: -8 * sum(Q) per limb
  int4_t corr1[3];           // int4 in groups of 16: the same for k-step 1
  float sfac;                // int4: s / 256 of column (group, head)
  half8_t qh[4], ql[4];      // fp16 QK right operand: hi / lo
  float4_t acc[8];           // PV accumulators, MFMA c <-> channel 8 n16 + c
  float m_run;               // running max of this lane's head
  float l_part;              // this lane's share of the running sum
};

template <bool INT4, bool TAIL>
__device__ __forceinline__ void process_blk(State<INT4>& st, const Blk<INT4>& cur, uint32_t t0, uint32_t t_end,
                                            uint32_t kq) {
  // ---- scores: lane holds tokens t0 + 16 sb + 4 kq + i of its head ----
  float sc[2][4];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    if (INT4) {
      const uint4 w = cur.k[sb];
      // unsigned nibbles as int8: k-step 0 = even channels, 1 = odd channels
      const int4_t a0 = (int4_t){static_cast<int>(w.x & 0x0F0F0F0Fu), static_cast<int>(w.y & 0x0F0F0F0Fu),
                                 static_cast<int>(w.z & 0x0F0F0F0Fu), static_cast<int>(w.w & 0x0F0F0F0Fu)};
      const int4_t a1 = (int4_t){static_cast<int>((w.x >> 4) & 0x0F0F0F0Fu),
                                 static_cast<int>((w.y >> 4) & 0x0F0F0F0Fu),
                                 static_cast<int>((w.z >> 4) & 0x0F0F0F0Fu),
                                 static_cast<int>((w.w >> 4) & 0x0F0F0F0Fu)};
      int4_t c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[0][0], st.corr[0], 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[0][1], c1, 0, 0, 0);
      int4_t c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[1][0], st.corr[1], 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[1][1], c2, 0, 0, 0);
      int4_t c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[2][0], st.corr[2], 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[2][1], c3, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // 256 c1 + c2 is exact in int32; the third limb joins in fp32
        const float f = fmaf(static_cast<float>(c1[i] * 256 + c2[i]), 256.f, static_cast<float>(c3[i])) * st.sfac;
        float x = f * f16_bits_to_f32(cur.ks[sb][i]);
        x = add_row_ror<8>(x);     // + group (g + 2) mod 4
        x = add_row_ror<4>(x);     // + groups (g + 1), (g + 3)
        sc[sb][i] = x;
      }
    } else {
      float4_t c = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const half8_t ka = __builtin_bit_cast(half8_t, cur.kf[sb][grp]);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, st.qh[grp], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, st.ql[grp], c, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[sb][i] = c[i];
    }
    if (TAIL) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + 16 * sb + 4 * kq + i >= t_end) sc[sb][i] = -INFINITY;
    }
  }

  // ---- online softmax (base 2, exact running max) ----
  float bm = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                   fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
  bm = max_over_rows(bm);
  if (__builtin_amdgcn_ballot_w64(bm > st.m_run) != 0) {
    const float m_new = fmaxf(st.m_run, bm);
    const float alpha = (st.m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.l_part *= alpha;
    st.m_run = m_new;
    // PV rows (block kq, head i) scale by the factor of head i (lane i)
    float al[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      al[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[c][i] *= al[i];
    }
  }

  // ---- PV left operand: p (times the value scale of group n16 / 4) ----
  half8_t pa_hi, pa_lo;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(sc[sb][i] - st.m_run);
      st.l_part += p;
      const float w = INT4 ? p * f16_bits_to_f32(cur.vs[sb][i]) : p;
      const _Float16 hi = static_cast<_Float16>(w);
      pa_hi[4 * sb + i] = hi;
      pa_lo[4 * sb + i] = static_cast<_Float16>(w - static_cast<float>(hi));
    }
  }

  // ---- PV: MFMA c takes channel 8 n16 + c; k slot 4 sb + i <-> token.
  // A nibble masked under the exponent of 1024 is the fp16 number 1024 + n
  // (low nibble) or 1024 + 16 n (high nibble); one packed subtraction makes
  // it n - 8 or 16 (n - 8), exact normal fp16 values.  (Products of two fp16
  // subnormals, which a nibble masked in place would be, do not keep their
  // full value in the matrix unit's fp32 sums.) ----
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t hv[4];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        if (INT4) {
          const int by = c >> 1;
          const uint32_t sel = 0x0c000c00u | (static_cast<uint32_t>(4 + by) << 16) | static_cast<uint32_t>(by);
          const uint32_t x = __builtin_amdgcn_perm(cur.v[sb][2 * pr + 1], cur.v[sb][2 * pr], sel);
          const uint32_t biased = (x & ((c & 1) ? 0x00F000F0u : 0x000F000Fu)) | 0x64006400u;
          const half2_t off = (c & 1) ? (half2_t){static_cast<_Float16>(-1152.f), static_cast<_Float16>(-1152.f)}
                                         : (half2_t){static_cast<_Float16>(-1032.f), static_cast<_Float16>(-1032.f)};
          hv[2 * sb + pr] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, biased) + off);
        } else {
          const uint32_t w0 = (&cur.vf[sb][2 * pr].x)[c >> 1];
          const uint32_t w1 = (&cur.vf[sb][2 * pr + 1].x)[c >> 1];
          hv[2 * sb + pr] = __builtin_amdgcn_perm(w1, w0, (c & 1) ? 0x07060302u : 0x05040100u);
        }
      }
    }
    const half8_t vb = __builtin_bit_cast(half8_t, make_uint4(hv[0], hv[1], hv[2], hv[3]));
    st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_hi, vb, st.acc[c], 0, 0, 0);
    st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_lo, vb, st.acc[c], 0, 0, 0);
  }
}

// ---- quantized cache: block loads at wave-uniform bases ----
// Code format FMT = 2 * (bits == 8) + (G == 16), as in the codec; D = 128.
template <int FMT>
struct QF {
  static constexpr int BITS = (FMT & 2) ? 8 : 4;
  static constexpr bool G16 = (FMT & 1) != 0;
  static constexpr int W = BITS / 4;            // K uint4s per lane and sub-block, V dwords per token
  static constexpr int CBT = 16 * BITS;         // code bytes per token (64 or 128)
  static constexpr int SBT = G16 ? 16 : 8;      // scale bytes per token
  static constexpr int REC = G16 ? 544 : 448;   // query record bytes
};

// Lane (n16, kq), n16 = 4 g + h: QK column (32-channel slice g, head h); its
// scores are those of tokens 16 sb + 4 kq + i (i < 4).
template <int FMT>
struct Blk4 {
  uint4 k[2][QF<FMT>::W];        // code bytes of token 16 sb + n16, channels 32 kq .. 32 kq + 31
  uint32_t v[2][4][QF<FMT>::W];  // codes of channels 8 n16 .. 8 n16 + 7 of token 16 sb + 4 kq + i
  uint32_t ks[2];                // key scale (fp16) of token 16 sb + 4 kq + h for group g (G = 32), or
                                 // of groups 2 g and 2 g + 1 (G = 16: low and high half)
  uint32_t vs[2];                // value scale(s) of the same token and group(s)
};

// Lane byte offsets of a full block's loads, from the block's first token.
struct Off4 {
  uint32_t k, v, s;
};

template <int FMT>
__device__ __forceinline__ Off4 lane_offsets4(uint32_t n16, uint32_t kq) {
  using F = QF<FMT>;
  Off4 o;
  o.k = n16 * F::CBT + kq * 16 * F::W;
  o.v = kq * 4 * F::CBT + n16 * 4 * F::W;
  o.s = (4 * kq + (n16 & 3)) * F::SBT + (n16 >> 2) * (F::G16 ? 4 : 2);
  return o;
}

// *(T*)(base + off + imm): base wave-uniform, off a 32-bit lane offset, imm a
// constant the load instruction carries.
template <typename T>
__device__ __forceinline__ T ldi(const uint8_t* base, uint32_t off, int imm) {
  return *reinterpret_cast<const T*>(base + off + imm);
}

// Loads of the block starting at token t0.  In a tail block the positions
// past t_last re-read token t_last (their scores are masked).
template <int FMT, bool TAIL>
__device__ __forceinline__ void load4(const Rows& r, uint32_t t0, uint32_t t_last, const Off4& o, uint32_t n16,
                                      uint32_t kq, Blk4<FMT>& b) {
  using F = QF<FMT>;
  const uint8_t* kc = r.kc + static_cast<size_t>(t0) * F::CBT;
  const uint8_t* vc = r.vc + static_cast<size_t>(t0) * F::CBT;
  const uint8_t* ksc = reinterpret_cast<const uint8_t*>(r.ksc) + static_cast<size_t>(t0) * F::SBT;
  const uint8_t* vsc = reinterpret_cast<const uint8_t*>(r.vsc) + static_cast<size_t>(t0) * F::SBT;
  auto load_v = [&](uint32_t* dst, uint32_t off, int imm) {
    if (F::W == 1) {
      dst[0] = ldi<uint32_t>(vc, off, imm);
    } else {
      const uint2 x = ldi<uint2>(vc, off, imm);
      dst[0] = x.x;
      dst[F::W - 1] = x.y;
    }
  };
  auto load_s = [&](uint32_t& ks, uint32_t& vs, uint32_t off, int imm) {
    if (F::G16) {
      ks = ldi<uint32_t>(ksc, off, imm);
      vs = ldi<uint32_t>(vsc, off, imm);
    } else {
      ks = ldi<uint16_t>(ksc, off, imm);
      vs = ldi<uint16_t>(vsc, off, imm);
    }
  };
  if (!TAIL) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int w = 0; w < F::W; ++w) b.k[sb][w] = ldi<uint4>(kc, o.k, 16 * F::CBT * sb + 16 * w);
#pragma unroll
      for (int i = 0; i < 4; ++i) load_v(b.v[sb][i], o.v, F::CBT * (16 * sb + i));
      load_s(b.ks[sb], b.vs[sb], o.s, 16 * F::SBT * sb);
    }
  } else {
    const uint32_t last = t_last - t0;
#pragma unroll
    for (uint32_t sb = 0; sb < 2; ++sb) {
      const uint32_t tk = min(16 * sb + n16, last);
#pragma unroll
      for (int w = 0; w < F::W; ++w) b.k[sb][w] = ldi<uint4>(kc, tk * F::CBT + kq * 16 * F::W, 16 * w);
#pragma unroll
      for (uint32_t i = 0; i < 4; ++i) {
        const uint32_t t = min(16 * sb + 4 * kq + i, last);
        load_v(b.v[sb][i], t * F::CBT + n16 * 4 * F::W, 0);
      }
      const uint32_t ts = min(16 * sb + 4 * kq + (n16 & 3), last);
      load_s(b.ks[sb], b.vs[sb], ts * F::SBT + (n16 >> 2) * (F::G16 ? 4 : 2), 0);
    }
  }
}

// x of lane 4 (l / 4) + I: the value of quad position I, to every lane of
// the quad (DPP quad_perm [I, I, I, I]).
template <int I>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), I * 0x55, 0xF, 0xF, true));
}

// Combined QK score of one column from its three limb accumulators: 256 c1
// + c2 is exact in int32; the third limb joins in fp32.
__device__ __forceinline__ float limb_score(const int4_t& c1, const int4_t& c2, const int4_t& c3, int i) {
  return fmaf(static_cast<float>(c1[i] * 256 + c2[i]), 256.f, static_cast<float>(c3[i]));
}

// Low / high nibbles of the four bytes of a word as int8 lanes.
__device__ __forceinline__ int lo_nib(uint32_t x) { return static_cast<int>(x & 0x0F0F0F0Fu); }
__device__ __forceinline__ int hi_nib(uint32_t x) { return static_cast<int>((x >> 4) & 0x0F0F0F0Fu); }

template <int FMT, bool TAIL>
__device__ __forceinline__ void process4(State<true>& st, const Blk4<FMT>& cur, uint32_t t0, uint32_t t_end,
                                         uint32_t kq, uint32_t n16, uint32_t mag_lo, uint32_t mag_hi) {
  using F = QF<FMT>;
  // ---- scores ----
  float sc[2][4];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    float xs[4];
    // key scale of token i: loaded by quad position i (same group, head i)
    const float ksf = f16_bits_to_f32(cur.ks[sb] & 0xFFFFu);
    const float ks4[4] = {quad_bcast<0>(ksf), quad_bcast<1>(ksf), quad_bcast<2>(ksf), quad_bcast<3>(ksf)};
    if (FMT == 0) {
      const uint4 w = cur.k[sb][0];
      // unsigned nibbles as int8: k-step 0 = even channels, 1 = odd channels
      const int4_t a0 = (int4_t){lo_nib(w.x), lo_nib(w.y), lo_nib(w.z), lo_nib(w.w)};
      const int4_t a1 = (int4_t){hi_nib(w.x), hi_nib(w.y), hi_nib(w.z), hi_nib(w.w)};
      int4_t c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[0][0], st.corr[0], 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[0][1], c1, 0, 0, 0);
      int4_t c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[1][0], st.corr[1], 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[1][1], c2, 0, 0, 0);
      int4_t c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[2][0], st.corr[2], 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[2][1], c3, 0, 0, 0);
      // sfac is this column's query scale
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[i] = limb_score(c1, c2, c3, i) * st.sfac * ks4[i];
    } else {
      // k-step s covers channels 32 kq + 16 s .. + 15 (int4: as low / high
      // nibble words; int8: the signed code bytes in order)
      int4_t av[2];
      if (F::BITS == 4) {
        const uint4 w = cur.k[sb][0];
        av[0] = (int4_t){lo_nib(w.x), hi_nib(w.x), lo_nib(w.y), hi_nib(w.y)};
        av[1] = (int4_t){lo_nib(w.z), hi_nib(w.z), lo_nib(w.w), hi_nib(w.w)};
      } else {
        av[0] = __builtin_bit_cast(int4_t, cur.k[sb][0]);
        av[1] = __builtin_bit_cast(int4_t, cur.k[sb][F::W - 1]);
      }
      if (!F::G16) {
        // one group per 32-channel slice: both k-steps into one sum
        int4_t c[3];
#pragma unroll
        for (int limb = 0; limb < 3; ++limb) {
          c[limb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[0], st.qb[limb][0], st.corr[limb], 0, 0, 0);
          c[limb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[1], st.qb[limb][1], c[limb], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[i] = limb_score(c[0], c[1], c[2], i) * st.sfac * ks4[i];
      } else {
        // groups of 16: each k-step is one group with its own key scale
        int4_t c0[3], c1[3];
#pragma unroll
        for (int limb = 0; limb < 3; ++limb) {
          c0[limb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[0], st.qb[limb][0], st.corr[limb], 0, 0, 0);
          c1[limb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[1], st.qb[limb][1], st.corr1[limb], 0, 0, 0);
        }
        const float kgf = f16_bits_to_f32(cur.ks[sb] >> 16);
        const float kg4[4] = {quad_bcast<0>(kgf), quad_bcast<1>(kgf), quad_bcast<2>(kgf), quad_bcast<3>(kgf)};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xs[i] = fmaf(limb_score(c0[0], c0[1], c0[2], i), ks4[i], limb_score(c1[0], c1[1], c1[2], i) * kg4[i]) *
                  st.sfac;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = add_row_ror<8>(xs[i]);   // + slice (g + 2) mod 4
      x = add_row_ror<4>(x);             // + slices (g + 1), (g + 3)
      sc[sb][i] = x;
    }
    if (TAIL) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + 16 * sb + 4 * kq + i >= t_end) sc[sb][i] = -INFINITY;
    }
  }

  // ---- online softmax (base 2, exact running max) ----
  float bm = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                   fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
  bm = max_over_rows(bm);
  if (__builtin_amdgcn_ballot_w64(bm > st.m_run) != 0) {
    const float m_new = fmaxf(st.m_run, bm);
    const float alpha = (st.m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.l_part *= alpha;
    st.m_run = m_new;
    // PV rows (value group kq, head i) scale by the factor of head i (lane i)
    float al[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      al[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[c][i] *= al[i];
    }
  }

  // ---- PV left operand: p times the value scale of the row's group, hi +
  // lo (groups of 16: a second operand pb for the odd group of the slice) ----
  half8_t pa_hi, pa_lo, pb_hi, pb_lo;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const float vsf = f16_bits_to_f32(cur.vs[sb] & 0xFFFFu);
    const float vs4[4] = {quad_bcast<0>(vsf), quad_bcast<1>(vsf), quad_bcast<2>(vsf), quad_bcast<3>(vsf)};
    float vg4[4] = {0.f, 0.f, 0.f, 0.f};
    if (F::G16) {
      const float vgf = f16_bits_to_f32(cur.vs[sb] >> 16);
      vg4[0] = quad_bcast<0>(vgf); vg4[1] = quad_bcast<1>(vgf); vg4[2] = quad_bcast<2>(vgf); vg4[3] = quad_bcast<3>(vgf);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(sc[sb][i] - st.m_run);
      st.l_part += p;
      const float w = p * vs4[i];
      const _Float16 hi = static_cast<_Float16>(w);
      pa_hi[4 * sb + i] = hi;
      pa_lo[4 * sb + i] = static_cast<_Float16>(w - static_cast<float>(hi));
      if (F::G16) {
        const float w1 = p * vg4[i];
        const _Float16 h1 = static_cast<_Float16>(w1);
        pb_hi[4 * sb + i] = h1;
        pb_lo[4 * sb + i] = static_cast<_Float16>(w1 - static_cast<float>(h1));
      }
    }
  }

  // ---- PV: MFMA c takes channel 8 n16 + c; k slot 4 sb + i <-> token.
  // Codes enter as exact normal fp16 integers under a biased exponent: an
  // int4 low nibble under 1024 (unit in bit 0) gives 1024 + n, a high nibble
  // under 64 (unit in bit 4) gives 64 + n, an int8 byte with its top bit
  // flipped under 1024 gives 1024 + q + 128; one packed subtraction leaves
  // the code.  (Products of two fp16 subnormals, which a nibble masked in
  // place would be, do not keep their full value in the matrix unit's fp32
  // sums.)  Groups of 16: the columns of the slice's odd group take the pb
  // rows, those of its even group the pa rows; the other operand's columns
  // are zero, so both passes accumulate into the same registers.
  const half2_t off_lo = {static_cast<_Float16>(-1032.f), static_cast<_Float16>(-1032.f)};
  const half2_t off_hi = {static_cast<_Float16>(-72.f), static_cast<_Float16>(-72.f)};
  const half2_t off_8 = {static_cast<_Float16>(-1152.f), static_cast<_Float16>(-1152.f)};
  const bool odd_group = ((n16 >> 1) & 1) != 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t hv[4];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        if (F::BITS == 4) {
          const int by = c >> 1;
          const uint32_t sel = 0x0c000c00u | (static_cast<uint32_t>(4 + by) << 16) | static_cast<uint32_t>(by);
          const uint32_t x = __builtin_amdgcn_perm(cur.v[sb][2 * pr + 1][0], cur.v[sb][2 * pr][0], sel);
          const uint32_t biased = (c & 1) ? ((x & 0x00F000F0u) | mag_hi) : ((x & 0x000F000Fu) | mag_lo);
          hv[2 * sb + pr] =
              __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, biased) + ((c & 1) ? off_hi : off_lo));
        } else {
          const int wi = (c >> 2) % F::W, by = c & 3;
          const uint32_t sel = 0x0c000c00u | (static_cast<uint32_t>(4 + by) << 16) | static_cast<uint32_t>(by);
          const uint32_t x = __builtin_amdgcn_perm(cur.v[sb][2 * pr + 1][wi], cur.v[sb][2 * pr][wi], sel);
          const uint32_t biased = (x ^ 0x00800080u) | mag_lo;
          hv[2 * sb + pr] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, biased) + off_8);
        }
      }
    }
    if (!F::G16) {
      const half8_t vb = __builtin_bit_cast(half8_t, make_uint4(hv[0], hv[1], hv[2], hv[3]));
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_hi, vb, st.acc[c], 0, 0, 0);
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_lo, vb, st.acc[c], 0, 0, 0);
    } else {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      const uint4 h4 = make_uint4(hv[0], hv[1], hv[2], hv[3]);
      const half8_t v0 = __builtin_bit_cast(half8_t, odd_group ? z : h4);
      const half8_t v1 = __builtin_bit_cast(half8_t, odd_group ? h4 : z);
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_hi, v0, st.acc[c], 0, 0, 0);
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_lo, v0, st.acc[c], 0, 0, 0);
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb_hi, v1, st.acc[c], 0, 0, 0);
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb_lo, v1, st.acc[c], 0, 0, 0);
    }
  }
}

// Waves per CU the split geometry targets.  The int4 kernel holds two waves
// per SIMD (up to 256 registers), so eight per CU run at once: one round of
// waves, each with a longer slice, measured faster than two rounds (fewer
// query rotations and partials to combine).  The fp16 kernel holds four per
// SIMD.
constexpr int kWavesPerCuInt4 = 8;
constexpr int kWavesPerCuF16 = 16;

template <bool INT4, int ROT, int FMT>
__global__ void __launch_bounds__(64, 2) attn_split_kernel(AttnArgs a) {
  using F = QF<FMT>;
  // rotated query records of the wave's heads (quantized cache)
  __shared__ __attribute__((aligned(16))) uint8_t qrec[kHeadsPerWave * F::REC];
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
  const uint32_t t_begin = static_cast<uint32_t>(s * a.chunk);
  const uint32_t t_end = static_cast<uint32_t>(min(s * a.chunk + a.chunk, a.seq_len));
  const int64_t cell0 = (b * a.Hkv + g) * a.Tcap;
  Rows rows;
  rows.kc = a.k_codes + cell0 * F::CBT;
  rows.ksc = a.k_scales + cell0 * (F::SBT / 2);
  rows.vc = a.v_codes + cell0 * F::CBT;
  rows.vsc = a.v_scales + cell0 * (F::SBT / 2);
  rows.k16 = a.k16 + cell0 * 128;
  rows.v16 = a.v16 + cell0 * 128;

  // The head whose scores this lane holds: int4 columns are (group, head)
  // pairs with head = n16 & 3; fp16 columns are heads.
  const int my_head = INT4 ? (n16 & 3) : n16;
  const bool head_ok = my_head < nh;
  const int64_t qrow0 = b * a.Hq + hq0;

  State<INT4> st;
  // int4 cache: rotate and quantize the wave's query heads into LDS records,
  // then gather this lane's MFMA operand.  Runs once the first block's loads
  // are in flight.
  QueryIn qin;
  auto init_query = [&]() {
    // all four records (heads past nh hold a zero word and are never read)
    query_records<ROT, F::REC, F::G16 && F::BITS == 4>(a, qin, lane, qrec);
    // one wave: its LDS writes are visible once its LDS counter drains
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const uint8_t* rec = qrec + (head_ok ? my_head : 0) * F::REC;
    const int grp = n16 >> 2;
    const bool live = head_ok && grp == kq;
#pragma unroll
    for (int limb = 0; limb < 3; ++limb) {
      uint32_t d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        d[e] = live ? reinterpret_cast<const uint32_t*>(rec + 128 * limb + 32 * kq)[e] : 0u;
      if (FMT == 0) {
        // k slot j of k-step ks <-> channel 32 kq + 2 j + ks
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint32_t sel = ks ? 0x07050301u : 0x06040200u;
          st.qb[limb][ks] = (int4_t){static_cast<int>(__builtin_amdgcn_perm(d[1], d[0], sel)),
                                     static_cast<int>(__builtin_amdgcn_perm(d[3], d[2], sel)),
                                     static_cast<int>(__builtin_amdgcn_perm(d[5], d[4], sel)),
                                     static_cast<int>(__builtin_amdgcn_perm(d[7], d[6], sel))};
        }
      } else if (F::BITS == 4) {
        // k-step ks covers channels 32 kq + 16 ks + (0, 2, 4, 6, 1, 3, 5, 7,
        // 8, 10, 12, 14, 9, 11, 13, 15): the order the nibbles of four code
        // bytes enter as low, high, low, high words
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          st.qb[limb][ks] = (int4_t){static_cast<int>(__builtin_amdgcn_perm(d[4 * ks + 1], d[4 * ks], 0x06040200u)),
                                     static_cast<int>(__builtin_amdgcn_perm(d[4 * ks + 1], d[4 * ks], 0x07050301u)),
                                     static_cast<int>(__builtin_amdgcn_perm(d[4 * ks + 3], d[4 * ks + 2], 0x06040200u)),
                                     static_cast<int>(__builtin_amdgcn_perm(d[4 * ks + 3], d[4 * ks + 2], 0x07050301u))};
      } else {
        // int8 codes in channel order: k-step ks covers channels 32 kq + 16 ks ..
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          st.qb[limb][ks] = (int4_t){static_cast<int>(d[4 * ks]), static_cast<int>(d[4 * ks + 1]),
                                     static_cast<int>(d[4 * ks + 2]), static_cast<int>(d[4 * ks + 3])};
      }
      // unsigned int4 nibbles (n = q + 8): the accumulators start at -8 sum(Q)
      // over the channels they cover; int8 codes are signed
      int c0 = 0, c1 = 0;
      if (F::BITS == 4 && !F::G16) {
        c0 = -8 * (head_ok ? reinterpret_cast<const int*>(rec + kRecSum)[4 * limb + grp] : 0);
      } else if (F::BITS == 4) {
        c0 = -8 * (head_ok ? reinterpret_cast<const int*>(rec + kRecSum16)[8 * limb + 2 * grp] : 0);
        c1 = -8 * (head_ok ? reinterpret_cast<const int*>(rec + kRecSum16)[8 * limb + 2 * grp + 1] : 0);
      }
      st.corr[limb] = (int4_t){c0, c0, c0, c0};
      st.corr1[limb] = (int4_t){c1, c1, c1, c1};
    }
    st.sfac = head_ok ? reinterpret_cast<const float*>(rec + kRecS)[grp] * (1.f / 65536.f) : 0.f;
  };
  if (!INT4) {
    // fp16 cache: q * sm_scale * log2(e) as fp16 hi + lo halves, channels
    // 32 grp + 8 kq .. + 7 of head n16
    const float sc = a.sm_scale * kLog2e;
    const uint16_t* qr = a.q + (qrow0 + (head_ok ? my_head : 0)) * 128;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const uint4 w = head_ok ? *reinterpret_cast<const uint4*>(qr + 32 * grp + 8 * kq) : make_uint4(0, 0, 0, 0);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = f16_bits_to_f32(ws[e] & 0xFFFFu) * sc, x1 = f16_bits_to_f32(ws[e] >> 16) * sc;
        hw[e] = pack_f16x2(x0, x1);
        lw[e] = pack_f16x2(x0 - f16_bits_to_f32(hw[e] & 0xFFFFu), x1 - f16_bits_to_f32(hw[e] >> 16));
      }
      st.qh[grp] = __builtin_bit_cast(half8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      st.ql[grp] = __builtin_bit_cast(half8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) st.acc[c] = (float4_t){0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.f;

  // 32-token blocks; the block that reaches t_end is a tail
  const uint32_t t_last = t_end - 1;
  const int n_full = static_cast<int>((t_end - t_begin) / kBlk);   // blocks entirely inside
  uint32_t t0 = t_begin;
  if (INT4) {
    // Split s takes the row's 32-token blocks s, s + S, s + 2 S, ...: the
    // splits of a row running side by side then read neighbouring blocks,
    // so each array streams from a contiguous window of memory.  The row's
    // last block is partial when seq_len is not a multiple of 32; it is the
    // tail of the split it falls to.  Ping-pong without copies: the next
    // block streams in while this one is processed; bases are wave-uniform,
    // lane offsets fixed.
    uint32_t mag_lo, mag_hi;     // fp16 pairs (1024, 1024), (64, 64) as v_and_or operands
    asm("v_mov_b32 %0, 0x64006400" : "=v"(mag_lo));
    asm("v_mov_b32 %0, 0x54005400" : "=v"(mag_hi));
    const Off4 o4 = lane_offsets4<FMT>(n16, kq);
    const uint32_t seq = static_cast<uint32_t>(a.seq_len);
    const uint32_t nbr = (seq + kBlk - 1) / kBlk;                    // blocks of the row
    const uint32_t S = static_cast<uint32_t>(a.S);
    const uint32_t sp = static_cast<uint32_t>(s);
    const uint32_t cnt = nbr > sp ? (nbr - 1 - sp) / S + 1 : 0;      // blocks of this split
    const bool has_tail = (seq % kBlk) != 0 && (nbr - 1) % S == sp;
    const int n_full = static_cast<int>(cnt) - (has_tail ? 1 : 0);
    const uint32_t step = kBlk * S;
    const uint32_t t_end = seq, t_last = seq - 1;
    uint32_t t0 = kBlk * sp;
    State<true>& s4 = reinterpret_cast<State<true>&>(st);
    query_loads<ROT>(a, a.q + qrow0 * 128, nh, a.lambda_k + g * 128, lane, qin);
    Blk4<FMT> b0, b1;
    if (n_full == 0) {
      if (has_tail) load4<FMT, true>(rows, t0, t_last, o4, n16, kq, b0);
      init_query();
      if (has_tail) process4<FMT, true>(s4, b0, t0, t_end, kq, n16, mag_lo, mag_hi);
    } else {
      load4<FMT, false>(rows, t0, t_last, o4, n16, kq, b0);
      init_query();
      // b0 holds block i at the top; blocks i + 1 and i + 2 are full
      int i = 0;
      for (; i + 2 < n_full; i += 2) {
        load4<FMT, false>(rows, t0 + step, t_last, o4, n16, kq, b1);
        process4<FMT, false>(s4, b0, t0, t_end, kq, n16, mag_lo, mag_hi);
        t0 += step;
        load4<FMT, false>(rows, t0 + step, t_last, o4, n16, kq, b0);
        process4<FMT, false>(s4, b1, t0, t_end, kq, n16, mag_lo, mag_hi);
        t0 += step;
      }
      // one or two full blocks left, then maybe the tail
      if (n_full - i == 2) {
        load4<FMT, false>(rows, t0 + step, t_last, o4, n16, kq, b1);
        process4<FMT, false>(s4, b0, t0, t_end, kq, n16, mag_lo, mag_hi);
        t0 += step;
        if (has_tail) load4<FMT, true>(rows, t0 + step, t_last, o4, n16, kq, b0);
        process4<FMT, false>(s4, b1, t0, t_end, kq, n16, mag_lo, mag_hi);
        t0 += step;
        if (has_tail) process4<FMT, true>(s4, b0, t0, t_end, kq, n16, mag_lo, mag_hi);
      } else {
        if (has_tail) load4<FMT, true>(rows, t0 + step, t_last, o4, n16, kq, b1);
        process4<FMT, false>(s4, b0, t0, t_end, kq, n16, mag_lo, mag_hi);
        t0 += step;
        if (has_tail) process4<FMT, true>(s4, b1, t0, t_end, kq, n16, mag_lo, mag_hi);
      }
    }
  } else {
    // the fp16 tile is four times larger: one buffer, occupancy hides latency
    for (int i = 0; i < n_full; ++i, t0 += kBlk) {
      Blk<INT4> bb;
      load_blk<INT4, false>(rows, t0, t_last, n16, kq, bb);
      process_blk<INT4, false>(st, bb, t0, t_end, kq);
    }
    if (t0 < t_end) {
      Blk<INT4> bb;
      load_blk<INT4, true>(rows, t0, t_last, n16, kq, bb);
      process_blk<INT4, true>(st, bb, t0, t_end, kq);
    }
  }

  // ---- partial results ----
  float l_part = st.l_part;
  l_part += shfl_xor(l_part, 16);
  l_part += shfl_xor(l_part, 32);
  const int64_t ws_base = b * a.Hq + hq0;
  if (kq == 0 && n16 < nh) {      // lane n16 = head (group 0 column for int4)
    float* ml = a.part_ml + ((ws_base + n16) * a.S + s) * 2;
    ml[0] = st.m_run;
    ml[1] = l_part;
  }
  // acc[c][i]: row block kq (int4: value group kq; fp16: heads 4 kq ..),
  // head i, channel 8 n16 + c
  const bool useful = INT4 ? (kq == (n16 >> 2)) : (kq == 0);
  if (useful) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nh) {
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          v[c] = st.acc[c][i];
        }
        float* dst = a.part_acc + ((ws_base + i) * a.S + s) * 128 + 8 * n16;
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2. combine splits, inverse rotation across the wave
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += shfl_xor(x, m);
  return x;
}

template <int ROT, int OUT_F32>
__global__ void __launch_bounds__(64) attn_combine_kernel(AttnArgs a, int int4) {
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t h = bh % a.Hq;
  const int64_t g = h / (a.Hq / a.Hkv);
  const float* ml = a.part_ml + bh * a.S * 2;
  const float* acc = a.part_acc + bh * a.S * 128 + 2 * lane;

  // lambda_V of the lane's channels, loaded with the partials
  float lv0 = 1.f, lv1 = 1.f;
  if (int4) {
    lv0 = a.lambda_v[g * 128 + 2 * lane];
    lv1 = a.lambda_v[g * 128 + 2 * lane + 1];
  }
  float l = 0.f, x0 = 0.f, x1 = 0.f;
  float m = -INFINITY;
  if (a.S <= 16) {
    // one pass with every load issued up front: the split maxima and sums
    // (one split per lane) and the lane's two channels of every split
    const int S = static_cast<int>(a.S);
    const float2 msl = lane < S ? *reinterpret_cast<const float2*>(ml + 2 * lane) : make_float2(-INFINITY, 0.f);
    float2 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = u < S ? *reinterpret_cast<const float2*>(acc + u * 128) : make_float2(0.f, 0.f);
    m = wave_max(msl.x);
    const float w = msl.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(msl.x - m);
    l = w * msl.y;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
      x0 = fmaf(wu, v[u].x, x0);
      x1 = fmaf(wu, v[u].y, x1);
    }
  } else {
    // split maxima and sums, 64 splits per pass (one per lane)
    for (int64_t s0 = 0; s0 < a.S; s0 += 64)
      if (s0 + lane < a.S) m = fmaxf(m, ml[2 * (s0 + lane)]);
    m = wave_max(m);
    for (int64_t s0 = 0; s0 < a.S; s0 += 64) {
      const int64_t sl = s0 + lane;
      const float ms = sl < a.S ? ml[2 * sl] : -INFINITY;
      const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - m);
      if (sl < a.S) l = fmaf(w, ml[2 * sl + 1], l);
      const int n = static_cast<int>(a.S - s0 < 64 ? a.S - s0 : 64);
      int j = 0;
      for (; j + 8 <= n; j += 8) {
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float2*>(acc + (s0 + j + u) * 128);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j + u));
          x0 = fmaf(wu, v[u].x, x0);
          x1 = fmaf(wu, v[u].y, x1);
        }
      }
      for (; j < n; ++j) {
        const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
        const float2 v = *reinterpret_cast<const float2*>(acc + (s0 + j) * 128);
        x0 = fmaf(wu, v.x, x0);
        x1 = fmaf(wu, v.y, x1);
      }
    }
  }
  l = wave_sum(l);
  const float inv = 1.f / l;
  x0 *= inv;
  x1 *= inv;

  int k = lane;              // pair index this lane writes
  uint32_t neg0 = 0, neg1 = 0;
  if (int4) {
    if (ROT == KVQ_ROT_SRFT) {
      // Z_lane = (x0 + i x1) / lambda, unitary inverse 64-point DFT across
      // lanes: radix-2 decimation in frequency, output bit-reversed
      float re = x0 * (0.125f / lv0);
      float im = x1 * (0.125f / lv1);
#pragma unroll
      for (int hh = 32; hh >= 1; hh >>= 1) {
        const float pr = shfl_xor(re, hh), pi = shfl_xor(im, hh);
        if (lane & hh) {
          const float dr = pr - re, di = pi - im;
          const int e = (lane & (hh - 1)) * (32 / hh);   // exp(+2 pi i e / 64)
          const float cw = kTw64Const.c[e], sw = kTw64Const.s[e];
          re = dr * cw - di * sw;
          im = dr * sw + di * cw;
        } else {
          re += pr;
          im += pi;
        }
      }
      k = bitrev6(lane);
      x0 = re;
      x1 = im;
      neg0 = neg1 = sign_bit(a.signs, k);
    } else if (ROT == KVQ_ROT_SRHT) {
      // H_128 on channels 2 lane + e: the stride-1 step inside the lane,
      // strides 2 .. 64 across lanes
      float y0 = x0 * (0.0883883476483184405f / lv0);
      float y1 = x1 * (0.0883883476483184405f / lv1);
      const float t0 = y0 + y1, t1 = y0 - y1;
      y0 = t0;
      y1 = t1;
#pragma unroll
      for (int hh = 1; hh <= 32; hh <<= 1) {
        const float p0 = shfl_xor(y0, hh), p1 = shfl_xor(y1, hh);
        if (lane & hh) { y0 = p0 - y0; y1 = p1 - y1; }
        else { y0 += p0; y1 += p1; }
      }
      x0 = y0;
      x1 = y1;
      neg0 = sign_bit(a.signs, 2 * lane);
      neg1 = sign_bit(a.signs, 2 * lane + 1);
    } else {
      x0 /= lv0;
      x1 /= lv1;
    }
  }
  if (neg0) x0 = -x0;
  if (neg1) x1 = -x1;
  if (OUT_F32) {
    *reinterpret_cast<float2*>(static_cast<float*>(a.out) + bh * 128 + 2 * k) = make_float2(x0, x1);
  } else {
    static_cast<uint32_t*>(a.out)[bh * 64 + k] = pack_f16x2(x0, x1);
  }
}

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

template <int ROT>
hipError_t run_attention(const AttnDesc& d, AttnArgs& a) {
  const int int4 = d.int4 ? 1 : 0;
  const unsigned nsplit = static_cast<unsigned>(d.B * d.Hkv * a.n_hchunks * a.S);
  const int fmt = (d.bits == 8 ? 2 : 0) + (d.G == 16 ? 1 : 0);
  if (!d.int4) {
    hipLaunchKernelGGL((attn_split_kernel<false, KVQ_ROT_ID, 0>), dim3(nsplit), dim3(64), 0, d.stream, a);
  } else if (fmt == 1) {
    hipLaunchKernelGGL((attn_split_kernel<true, ROT, 1>), dim3(nsplit), dim3(64), 0, d.stream, a);
  } else if (fmt == 2) {
    hipLaunchKernelGGL((attn_split_kernel<true, ROT, 2>), dim3(nsplit), dim3(64), 0, d.stream, a);
  } else if (fmt == 3) {
    hipLaunchKernelGGL((attn_split_kernel<true, ROT, 3>), dim3(nsplit), dim3(64), 0, d.stream, a);
  } else {
    hipLaunchKernelGGL((attn_split_kernel<true, ROT, 0>), dim3(nsplit), dim3(64), 0, d.stream, a);
  }
  const unsigned nc = static_cast<unsigned>(d.B * d.Hq);
  if (d.out_f32) {
    hipLaunchKernelGGL((attn_combine_kernel<ROT, 1>), dim3(nc), dim3(64), 0, d.stream, a, int4);
  } else {
    hipLaunchKernelGGL((attn_combine_kernel<ROT, 0>), dim3(nc), dim3(64), 0, d.stream, a, int4);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int64_t max_splits(int64_t seq_len) { return (seq_len + 255) / 256 > 0 ? (seq_len + 255) / 256 : 1; }

}  // namespace

int64_t attn_num_splits(int64_t B, int64_t Hkv, int64_t seq_len) {
  int64_t S, chunk, nh;
  split_geometry(B, Hkv * 4, Hkv, seq_len, S, chunk, nh, device_cu_count(), kWavesPerCuInt4);
  return S;
}

// Workspace layout (256-aligned sections): (max, sum) [B*Hq][S][2] f32,
// partial sums [B*Hq][S][128] f32, sized for the largest split count any
// shape with this seq_len can use.
size_t attn_workspace_bytes(int D, int64_t B, int64_t Hq, int64_t seq_len) {
  (void)D;
  const int64_t S = max_splits(seq_len);
  const size_t rows = static_cast<size_t>(B * Hq);
  return align256(rows * S * 2 * 4) + align256(rows * S * 128 * 4);
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
  split_geometry(d.B, d.Hq, d.Hkv, d.seq_len, a.S, a.chunk, a.n_hchunks, device_cu_count(),
                 d.int4 ? kWavesPerCuInt4 : kWavesPerCuF16);
  const int64_t ms = max_splits(d.seq_len);
  if (a.S > ms) return hipErrorInvalidValue;
  const size_t rows = static_cast<size_t>(d.B * d.Hq);
  uint8_t* ws = static_cast<uint8_t*>(d.workspace);
  a.part_ml = reinterpret_cast<float*>(ws);
  a.part_acc = reinterpret_cast<float*>(ws + align256(rows * ms * 2 * 4));
  switch (d.int4 ? d.rotation : KVQ_ROT_ID) {
    case KVQ_ROT_SRFT: return run_attention<KVQ_ROT_SRFT>(d, a);
    case KVQ_ROT_SRHT: return run_attention<KVQ_ROT_SRHT>(d, a);
    default: return run_attention<KVQ_ROT_ID>(d, a);
  }
}

}  // namespace kvq
