// Device code of the decode-step attention kernels: the split kernel
// (query rotation, block stream, online softmax, weighted sum) and the
// combine kernel.  The operation and the design are described at the top of
// kvq_attn.hip; kvq_attn_f16.hip instantiates the fp16-cache comparator.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {

// Arguments of the split and combine kernels (one struct, passed by value).
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
  float* part_acc;    // [B*Hq][S][D]
  float* part_ml;     // [B*Hq][S][2]
  void* out;
  int64_t B, Hq, Hkv, Tcap, seq_len;
  int64_t S, chunk;   // splits and tokens per split
  int64_t n_hchunks;  // ceil(rep / 4)
  float sm_scale;
  uint64_t signs[4];
};

// The fp16-cache comparator's split kernel, launched from its own
// translation unit (built without the attention source's register option).
hipError_t launch_attn_split_f16(const AttnArgs& a, int nh, unsigned nsplit, hipStream_t stream);

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kHeadsPerWave = 4;
constexpr int kBlk = 32;              // tokens per inner step

// Query record of one head (quantized cache), NH halves: three int8 limbs
// per channel, q~ ~= s (Q1 + Q2 / 256 + Q3 / 65536):
//   [0, 384 NH)        limbs Q1, Q2, Q3, 128 NH bytes each, channel order
//   [384 NH, 400 NH)   s[4 NH] f32, one per 32-channel group
template <int NH>
struct Rec {
  static constexpr int S = 384 * NH;
  static constexpr int BYTES = 400 * NH;
};

__constant__ TwTable kTw64Const = make_twiddles(64);
__constant__ TwTable kTw128Const = make_twiddles(128);

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

// Channel pair a lane loads for half hf of a query: SRFT with D = 128
// starts the across-lane decimation in time from pair bitrev(lane); with
// D = 256 from pairs 2 bitrev(lane) + hf (the even and the odd pairs, whose
// 64-point transforms one more radix-2 step joins); SRHT and no rotation
// from pair 64 hf + lane.
template <int ROT, int NH>
__device__ __forceinline__ int query_pair(int lane, int hf) {
  if (ROT == KVQ_ROT_SRFT) return NH == 1 ? bitrev6(lane) : 2 * bitrev6(lane) + hf;
  return 64 * hf + lane;
}

// Loads of the query rotation (int4 cache): the lane's pair word of each of
// the wave's heads and halves, its lambda_K entries and the twiddles of its
// butterfly stages.  They are issued before the first cache block, so that
// waiting for them does not wait for the block.
struct QueryIn {
  uint32_t w[2][4];   // [half][head]: fp16 pair query_pair(lane, half)
  float l[2][2];      // lambda_K of channels 128 hf + 2 lane, + 1
  float cw[6], sw[6]; // SRFT stage twiddles
  float c128, s128;   // SRFT, D = 256: cos, sin (2 pi lane / 128)
};

template <int ROT, int NH>
__device__ __forceinline__ void query_loads(const AttnArgs& a, const uint16_t* q0, int nh, const float* lk, int lane,
                                            QueryIn& in) {
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    const int k = query_pair<ROT, NH>(lane, hf);
#pragma unroll
    for (int hh = 0; hh < kHeadsPerWave; ++hh)
      in.w[hf][hh] = hh < nh ? reinterpret_cast<const uint32_t*>(q0 + hh * 128 * NH)[k] : 0u;
    in.l[hf][0] = lk[128 * hf + 2 * lane];
    in.l[hf][1] = lk[128 * hf + 2 * lane + 1];
  }
  if (ROT == KVQ_ROT_SRFT) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int hh = 1 << i;
      const int e = (lane & (hh - 1)) * (32 / hh);
      in.cw[i] = kTw64Const.c[e];
      in.sw[i] = kTw64Const.s[e];
    }
    if (NH == 2) {
      in.c128 = kTw128Const.c[lane];
      in.s128 = kTw128Const.s[lane];
    }
  }
}

// Rotated query records of the wave's four heads (int4 cache), computed by
// one wave from the pair words in.w: lane l owns channels 128 hf + 2 l,
// 128 hf + 2 l + 1 of every head and half.  The heads advance together
// through each cross-lane step (independent shuffles per wait); the records
// go to LDS at rec + head * Rec<NH>::BYTES.
template <int ROT, int NH>
__device__ __forceinline__ void query_records(const AttnArgs& a, const QueryIn& in, int lane, uint8_t* rec) {
  constexpr int NHD = kHeadsPerWave;
  using RL = Rec<NH>;
  float y0[NH][NHD], y1[NH][NHD];   // rotated channels 128 hf + 2 lane, + 1 (unnormalized)
  float c = 1.f;
  if (ROT == KVQ_ROT_SRFT) {
    // forward 64-point DFT across lanes, radix-2 decimation in time: lane l
    // starts with pair bitrev(l) (D = 128) or pairs 2 bitrev(l) + hf (D =
    // 256: the even and the odd pairs), signed, and ends with frequency l
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const uint32_t m = sign_bit(a.signs, query_pair<ROT, NH>(lane, hf)) ? 0x80008000u : 0u;
#pragma unroll
      for (int h = 0; h < NHD; ++h) {
        const uint32_t w = in.w[hf][h] ^ m;
        y0[hf][h] = f16_bits_to_f32(w & 0xFFFFu);
        y1[hf][h] = f16_bits_to_f32(w >> 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int hh = 1 << i;
      const bool upper = lane & hh;
      const float cw = in.cw[i], sw = in.sw[i];
      float pr[NH][NHD], pi[NH][NHD];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
#pragma unroll
        for (int h = 0; h < NHD; ++h) {
          pr[hf][h] = shfl_xor(y0[hf][h], hh);
          pi[hf][h] = shfl_xor(y1[hf][h], hh);
        }
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
#pragma unroll
        for (int h = 0; h < NHD; ++h) {
          // t = W^j * (the upper element), W = exp(-2 pi i / (2 hh))
          const float ur = upper ? y0[hf][h] : pr[hf][h], ui = upper ? y1[hf][h] : pi[hf][h];
          const float tr = ur * cw + ui * sw, ti = ui * cw - ur * sw;
          const float br = upper ? pr[hf][h] : y0[hf][h], bi = upper ? pi[hf][h] : y1[hf][h];
          y0[hf][h] = upper ? br - tr : br + tr;
          y1[hf][h] = upper ? bi - ti : bi + ti;
        }
    }
    if (NH == 2) {
      // Z_l = E_l + W^l O_l, Z_{l+64} = E_l - W^l O_l, W = exp(-2 pi i / 128)
#pragma unroll
      for (int h = 0; h < NHD; ++h) {
        const float er = y0[0][h], ei = y1[0][h], orr = y0[NH - 1][h], oi = y1[NH - 1][h];
        const float tr = orr * in.c128 + oi * in.s128, ti = oi * in.c128 - orr * in.s128;
        y0[0][h] = er + tr;
        y1[0][h] = ei + ti;
        y0[NH - 1][h] = er - tr;
        y1[NH - 1][h] = ei - ti;
      }
    }
    c = NH == 1 ? 0.125f : 0.0883883476483184405f;
  } else {
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      uint32_t m = 0;
      if (ROT == KVQ_ROT_SRHT)
        m = (sign_bit(a.signs, 128 * hf + 2 * lane) << 15) | (sign_bit(a.signs, 128 * hf + 2 * lane + 1) << 31);
#pragma unroll
      for (int h = 0; h < NHD; ++h) {
        y0[hf][h] = f16_bits_to_f32((in.w[hf][h] ^ m) & 0xFFFFu);
        y1[hf][h] = f16_bits_to_f32((in.w[hf][h] ^ m) >> 16);
      }
    }
    if (ROT == KVQ_ROT_SRHT) {
      if (NH == 2) {
        // H_256 [u; v] = [H_128 (u + v); H_128 (u - v)]
#pragma unroll
        for (int h = 0; h < NHD; ++h) {
          const float a0 = y0[0][h], a1 = y1[0][h], b0 = y0[NH - 1][h], b1 = y1[NH - 1][h];
          y0[0][h] = a0 + b0;
          y1[0][h] = a1 + b1;
          y0[NH - 1][h] = a0 - b0;
          y1[NH - 1][h] = a1 - b1;
        }
      }
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
#pragma unroll
        for (int h = 0; h < NHD; ++h) {
          const float t0 = y0[hf][h] + y1[hf][h], t1 = y0[hf][h] - y1[hf][h];
          y0[hf][h] = t0;
          y1[hf][h] = t1;
        }
#pragma unroll
      for (int hh = 1; hh <= 32; hh <<= 1) {
        float p0[NH][NHD], p1[NH][NHD];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf)
#pragma unroll
          for (int h = 0; h < NHD; ++h) {
            p0[hf][h] = shfl_xor(y0[hf][h], hh);
            p1[hf][h] = shfl_xor(y1[hf][h], hh);
          }
#pragma unroll
        for (int hf = 0; hf < NH; ++hf)
#pragma unroll
          for (int h = 0; h < NHD; ++h) {
            if (lane & hh) { y0[hf][h] = p0[hf][h] - y0[hf][h]; y1[hf][h] = p1[hf][h] - y1[hf][h]; }
            else { y0[hf][h] += p0[hf][h]; y1[hf][h] += p1[hf][h]; }
          }
      }
      c = NH == 1 ? 0.0883883476483184405f : 0.0625f;
    }
  }
  const float sc = a.sm_scale * kLog2e * c;
  const int grp = lane >> 4;
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    const float r0 = sc / in.l[hf][0], r1 = sc / in.l[hf][1];
    float q0[NHD], q1[NHD], amax[NHD];
#pragma unroll
    for (int h = 0; h < NHD; ++h) {
      q0[h] = y0[hf][h] * r0;
      q1[h] = y1[hf][h] * r1;
      amax[h] = fmaxf(fabsf(q0[h]), fabsf(q1[h]));
    }
    // group = 16 lanes: abs max, three int8 limbs
#pragma unroll
    for (int m = 1; m <= 8; m <<= 1) {
      float o[NHD];
#pragma unroll
      for (int h = 0; h < NHD; ++h) o[h] = shfl_xor(amax[h], m);
#pragma unroll
      for (int h = 0; h < NHD; ++h) amax[h] = fmaxf(amax[h], o[h]);
    }
    int li[NHD][3][2];
#pragma unroll
    for (int h = 0; h < NHD; ++h) {
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
    const int gi = 4 * hf + grp;            // 32-channel group of the head vector
#pragma unroll
    for (int h = 0; h < NHD; ++h) {
      uint8_t* r = rec + h * RL::BYTES;
#pragma unroll
      for (int limb = 0; limb < 3; ++limb) {
        reinterpret_cast<uint16_t*>(r + 128 * NH * limb + 128 * hf)[lane] =
            static_cast<uint16_t>((li[h][limb][0] & 0xFF) | ((li[h][limb][1] & 0xFF) << 8));
      }
      if ((lane & 15) == 0) reinterpret_cast<float*>(r + RL::S)[gi] = amax[h] > 0.f ? amax[h] / 127.f : 0.f;
    }
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

// Row-relative bases of one (batch, kv head): every offset below is 32-bit.
struct Rows {
  const uint8_t* kc;     // int4 codes of token 0
  const uint16_t* ksc;
  const uint8_t* vc;
  const uint16_t* vsc;
  const uint16_t* k16;   // fp16 cache
  const uint16_t* v16;
};

// Loads at a wave-uniform base plus an unsigned 32-bit lane offset (the
// SGPR-base form of the global load instructions).
template <typename T>
__device__ __forceinline__ T ld(const void* base, uint32_t off) {
  return *reinterpret_cast<const T*>(static_cast<const uint8_t*>(base) + off);
}

// ---- fp16 cache (the comparator): one 32-token block per step ----
// Loads of one block (sub-blocks sb = 0, 1 of 16 tokens).
template <int NH>
struct BlkF {
  uint4 kf[2][4 * NH];   // 8 channels 32 gq + 8 kq .. of token 16 sb + n16, 32-channel slice gq
  uint4 vf[2][4][NH];    // channels 128 hf + 8 n16 .. + 7 of token 16 sb + 4 kq + i
};

// Token index actually read: in the last (tail) block of a split the
// positions past the end re-read its last token; their scores are masked.
template <bool TAIL>
__device__ __forceinline__ uint32_t tok(uint32_t t, uint32_t t_last) {
  return TAIL ? min(t, t_last) : t;
}

template <bool TAIL, int NH>
__device__ __forceinline__ void load_blkf(const Rows& r, uint32_t t0, uint32_t t_last, uint32_t n16, uint32_t kq,
                                          BlkF<NH>& o) {
  constexpr uint32_t kRow = 256 * NH;     // bytes per token
#pragma unroll
  for (uint32_t sb = 0; sb < 2; ++sb) {
    const uint32_t tk = tok<TAIL>(t0 + 16 * sb + n16, t_last);
#pragma unroll
    for (uint32_t gq = 0; gq < 4 * NH; ++gq) o.kf[sb][gq] = ld<uint4>(r.k16, tk * kRow + 64 * gq + 16 * kq);
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
      const uint32_t t = tok<TAIL>(t0 + 16 * sb + 4 * kq + i, t_last);
#pragma unroll
      for (uint32_t hf = 0; hf < NH; ++hf) o.vf[sb][i][hf] = ld<uint4>(r.v16, t * kRow + 256 * hf + (n16 << 4));
    }
  }
}

// Per-wave streaming state of the fp16 cache.
template <int NH>
struct StateF {
  half8_t qh[4 * NH], ql[4 * NH];   // QK right operand: hi / lo
  float4_t acc[NH][8];              // PV accumulators, MFMA c <-> channel 128 hf + 8 n16 + c
  float m_run;                      // running max of this lane's head
  float l_part;                     // this lane's share of the running sum
};

template <bool TAIL, int NH>
__device__ __forceinline__ void process_blkf(StateF<NH>& st, const BlkF<NH>& cur, uint32_t t0, uint32_t t_end,
                                             uint32_t kq) {
  // ---- scores: lane holds tokens t0 + 16 sb + 4 kq + i of its head ----
  float sc[2][4];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    float4_t c = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int grp = 0; grp < 4 * NH; ++grp) {
      const half8_t ka = __builtin_bit_cast(half8_t, cur.kf[sb][grp]);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, st.qh[grp], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, st.ql[grp], c, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[sb][i] = c[i];
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
    // PV rows (heads 4 kq + i) scale by the factor of head i (lane i)
    float al[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      al[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) st.acc[hf][c][i] *= al[i];
  }

  // ---- PV left operand: p as fp16 hi + lo ----
  half8_t pa_hi, pa_lo;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(sc[sb][i] - st.m_run);
      st.l_part += p;
      const _Float16 hi = static_cast<_Float16>(p);
      pa_hi[4 * sb + i] = hi;
      pa_lo[4 * sb + i] = static_cast<_Float16>(p - static_cast<float>(hi));
    }
  }

  // ---- PV: MFMA c takes channel 128 hf + 8 n16 + c; k slot 4 sb + i <-> token ----
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t hv[4];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const uint32_t w0 = (&cur.vf[sb][2 * pr][hf].x)[c >> 1];
          const uint32_t w1 = (&cur.vf[sb][2 * pr + 1][hf].x)[c >> 1];
          hv[2 * sb + pr] = __builtin_amdgcn_perm(w1, w0, (c & 1) ? 0x07060302u : 0x05040100u);
        }
      }
      const half8_t vb = __builtin_bit_cast(half8_t, make_uint4(hv[0], hv[1], hv[2], hv[3]));
      st.acc[hf][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_hi, vb, st.acc[hf][c], 0, 0, 0);
      st.acc[hf][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_lo, vb, st.acc[hf][c], 0, 0, 0);
    }
  }
}

// ---- quantized cache: block loads at wave-uniform bases ----
// Code format FMT = 2 * (bits == 8) + (G == 16), as in the codec; NH halves
// of 128 channels.
template <int FMT, int NH>
struct QF {
  static constexpr int BITS = (FMT & 2) ? 8 : 4;
  static constexpr bool G16 = (FMT & 1) != 0;
  static constexpr int W = BITS / 4;            // K uint4s per lane and sub-block, V dwords per token
  static constexpr int HB = 16 * BITS;          // code bytes per token and half (64 or 128)
  static constexpr int CBT = NH * HB;           // code bytes per token
  static constexpr int HS = G16 ? 16 : 8;       // scale bytes per token and half
  static constexpr int SBT = NH * HS;           // scale bytes per token
};

// Lane (n16, kq), n16 = 4 g + h: QK column (32-channel slice g of each half,
// head h); its scores are those of tokens 16 sb + 4 kq + i (i < 4).
template <int FMT, int NH>
struct Blk4 {
  uint4 k[2][NH][QF<FMT, NH>::W];        // code bytes of token 16 sb + n16, channels 128 hf + 32 kq .. + 31
  uint32_t v[2][4][NH][QF<FMT, NH>::W];  // codes of channels 128 hf + 8 n16 .. + 7 of token 16 sb + 4 kq + i
  uint32_t ks[2][NH];                    // key scale (fp16) of token 16 sb + 4 kq + h for group 4 hf + g
                                         // (G = 32), or of groups 2 g, 2 g + 1 of half hf (G = 16)
  uint32_t vs[2][NH];                    // value scale(s) of the same token and group(s)
};

// Lane byte offsets of a full block's loads, from the block's first token
// (the half's offset is an instruction immediate).
struct Off4 {
  uint32_t k, v, s;
};

template <int FMT, int NH>
__device__ __forceinline__ Off4 lane_offsets4(uint32_t n16, uint32_t kq) {
  using F = QF<FMT, NH>;
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
template <int FMT, bool TAIL, int NH>
__device__ __forceinline__ void load4(const Rows& r, uint32_t t0, uint32_t t_last, const Off4& o, uint32_t n16,
                                      uint32_t kq, Blk4<FMT, NH>& b) {
  using F = QF<FMT, NH>;
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
      for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
        for (int w = 0; w < F::W; ++w)
          b.k[sb][hf][w] = ldi<uint4>(kc, o.k, 16 * F::CBT * sb + F::HB * hf + 16 * w);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_v(b.v[sb][i][hf], o.v, F::CBT * (16 * sb + i) + F::HB * hf);
        load_s(b.ks[sb][hf], b.vs[sb][hf], o.s, 16 * F::SBT * sb + F::HS * hf);
      }
    }
  } else {
    const uint32_t last = t_last - t0;
#pragma unroll
    for (uint32_t sb = 0; sb < 2; ++sb) {
      const uint32_t tk = min(16 * sb + n16, last);
      const uint32_t ts = min(16 * sb + 4 * kq + (n16 & 3), last);
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
        for (int w = 0; w < F::W; ++w)
          b.k[sb][hf][w] = ldi<uint4>(kc, tk * F::CBT + kq * 16 * F::W, F::HB * hf + 16 * w);
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i) {
          const uint32_t t = min(16 * sb + 4 * kq + i, last);
          load_v(b.v[sb][i][hf], t * F::CBT + n16 * 4 * F::W, F::HB * hf);
        }
        load_s(b.ks[sb][hf], b.vs[sb][hf], ts * F::SBT + (n16 >> 2) * (F::G16 ? 4 : 2), F::HS * hf);
      }
    }
  }
}

// Per-wave streaming state of the quantized cache.
template <int NH>
struct StateQ {
  int4_t qb[NH][3][2];       // QK right operand: [half][limb][k-step]
  float sfac[NH];            // s / 256 of column (group, head) in each half
  float4_t acc[NH][8];       // PV accumulators, MFMA c <-> channel 128 hf + 8 n16 + c
  float m_run;               // running max of this lane's head
  float l_part;              // this lane's share of the running sum
};

// x of lane 4 (l / 4) + I: the value of quad position I, to every lane of
// the quad (DPP quad_perm [I, I, I, I]).
template <int I>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), I * 0x55, 0xF, 0xF, true));
}

// Combined QK score of one column from its three limb accumulators: 256 c1
// + c2 is exact in int32; the third limb joins in fp32.  BITS = 4: the codes
// entered as 16 q, every sum is a multiple of 16, and the result is 16 times
// the score (the shift by 4 is exact, so is 256 c1 + c2 as a float).
template <int BITS>
__device__ __forceinline__ float limb_score(const int4_t& c1, const int4_t& c2, const int4_t& c3, int i) {
  if (BITS == 4) return fmaf(static_cast<float>((c1[i] * 256 + c2[i]) >> 4), 4096.f, static_cast<float>(c3[i]));
  return fmaf(static_cast<float>(c1[i] * 256 + c2[i]), 256.f, static_cast<float>(c3[i]));
}

// The int4 codes q = n - 8 of the low / high nibbles n of the four bytes of
// a word, as int8 lanes holding 16 q: the nibble placed in the top half of
// its byte with its top bit flipped is 16 q in two's complement.
__device__ __forceinline__ int lo_q16(uint32_t x) { return static_cast<int>(((x << 4) & 0xF0F0F0F0u) ^ 0x80808080u); }
__device__ __forceinline__ int hi_q16(uint32_t x) { return static_cast<int>((x & 0xF0F0F0F0u) ^ 0x80808080u); }

// QK of one half: this lane's column scores xs[i] (tokens 16 sb + 4 kq + i)
// before the sum over the four groups of the half, added into xs.
template <int FMT, int NH>
__device__ __forceinline__ void qk_half(const StateQ<NH>& st, const Blk4<FMT, NH>& cur, int sb, int hf,
                                        float (&xs)[4]) {
  using F = QF<FMT, NH>;
  // key scale of token i: loaded by quad position i (same group, head i)
  const float ksf = f16_bits_to_f32(cur.ks[sb][hf] & 0xFFFFu);
  const float ks4[4] = {quad_bcast<0>(ksf), quad_bcast<1>(ksf), quad_bcast<2>(ksf), quad_bcast<3>(ksf)};
  if (FMT == 0) {
    const uint4 w = cur.k[sb][hf][0];
    // codes as int8 16 q: k-step 0 = even channels, 1 = odd channels
    const int4_t a0 = (int4_t){lo_q16(w.x), lo_q16(w.y), lo_q16(w.z), lo_q16(w.w)};
    const int4_t a1 = (int4_t){hi_q16(w.x), hi_q16(w.y), hi_q16(w.z), hi_q16(w.w)};
    const int4_t z = (int4_t){0, 0, 0, 0};
    int4_t c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[hf][0][0], z, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[hf][0][1], c1, 0, 0, 0);
    int4_t c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[hf][1][0], z, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[hf][1][1], c2, 0, 0, 0);
    int4_t c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.qb[hf][2][0], z, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.qb[hf][2][1], c3, 0, 0, 0);
    // sfac is this column's query scale (over 16)
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[i] = fmaf(limb_score<4>(c1, c2, c3, i) * st.sfac[hf], ks4[i], xs[i]);
  } else {
    // k-step s covers channels 32 kq + 16 s .. + 15 (int4: as low / high
    // nibble words; int8: the signed code bytes in order)
    int4_t av[2];
    if (F::BITS == 4) {
      const uint4 w = cur.k[sb][hf][0];
      av[0] = (int4_t){lo_q16(w.x), hi_q16(w.x), lo_q16(w.y), hi_q16(w.y)};
      av[1] = (int4_t){lo_q16(w.z), hi_q16(w.z), lo_q16(w.w), hi_q16(w.w)};
    } else {
      av[0] = __builtin_bit_cast(int4_t, cur.k[sb][hf][0]);
      av[1] = __builtin_bit_cast(int4_t, cur.k[sb][hf][F::W - 1]);
    }
    const int4_t z = (int4_t){0, 0, 0, 0};
    if (!F::G16) {
      // one group per 32-channel slice: both k-steps into one sum
      int4_t c[3];
#pragma unroll
      for (int limb = 0; limb < 3; ++limb) {
        c[limb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[0], st.qb[hf][limb][0], z, 0, 0, 0);
        c[limb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[1], st.qb[hf][limb][1], c[limb], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xs[i] = fmaf(limb_score<F::BITS>(c[0], c[1], c[2], i) * st.sfac[hf], ks4[i], xs[i]);
    } else {
      // groups of 16: each k-step is one group with its own key scale
      int4_t c0[3], c1[3];
#pragma unroll
      for (int limb = 0; limb < 3; ++limb) {
        c0[limb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[0], st.qb[hf][limb][0], z, 0, 0, 0);
        c1[limb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[1], st.qb[hf][limb][1], z, 0, 0, 0);
      }
      const float kgf = f16_bits_to_f32(cur.ks[sb][hf] >> 16);
      const float kg4[4] = {quad_bcast<0>(kgf), quad_bcast<1>(kgf), quad_bcast<2>(kgf), quad_bcast<3>(kgf)};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xs[i] = fmaf(fmaf(limb_score<F::BITS>(c0[0], c0[1], c0[2], i), ks4[i],
                          limb_score<F::BITS>(c1[0], c1[1], c1[2], i) * kg4[i]),
                     st.sfac[hf], xs[i]);
    }
  }
}

template <int FMT, bool TAIL, int NH>
__device__ __forceinline__ void process4(StateQ<NH>& st, const Blk4<FMT, NH>& cur, uint32_t t0, uint32_t t_end,
                                         uint32_t kq, uint32_t n16, uint32_t mag_lo, uint32_t mag_hi) {
  using F = QF<FMT, NH>;
  // ---- scores ----
  float sc[2][4];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    float xs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) qk_half<FMT, NH>(st, cur, sb, hf, xs);
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
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) st.acc[hf][c][i] *= al[i];
  }

  float p[2][4];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[sb][i] = __builtin_amdgcn_exp2f(sc[sb][i] - st.m_run);
      st.l_part += p[sb][i];
    }

  const half2_t off_lo = {static_cast<_Float16>(-1032.f), static_cast<_Float16>(-1032.f)};
  const half2_t off_hi = {static_cast<_Float16>(-72.f), static_cast<_Float16>(-72.f)};
  const half2_t off_8 = {static_cast<_Float16>(-1152.f), static_cast<_Float16>(-1152.f)};
  const bool odd_group = ((n16 >> 1) & 1) != 0;
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    // ---- PV left operand: p times the value scale of the row's group, hi +
    // lo (groups of 16: a second operand pb for the odd group of the slice) ----
    half8_t pa_hi, pa_lo, pb_hi, pb_lo;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const float vsf = f16_bits_to_f32(cur.vs[sb][hf] & 0xFFFFu);
      const float vs4[4] = {quad_bcast<0>(vsf), quad_bcast<1>(vsf), quad_bcast<2>(vsf), quad_bcast<3>(vsf)};
      float vg4[4] = {0.f, 0.f, 0.f, 0.f};
      if (F::G16) {
        const float vgf = f16_bits_to_f32(cur.vs[sb][hf] >> 16);
        vg4[0] = quad_bcast<0>(vgf); vg4[1] = quad_bcast<1>(vgf); vg4[2] = quad_bcast<2>(vgf); vg4[3] = quad_bcast<3>(vgf);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w = p[sb][i] * vs4[i];
        const _Float16 hi = static_cast<_Float16>(w);
        pa_hi[4 * sb + i] = hi;
        pa_lo[4 * sb + i] = static_cast<_Float16>(w - static_cast<float>(hi));
        if (F::G16) {
          const float w1 = p[sb][i] * vg4[i];
          const _Float16 h1 = static_cast<_Float16>(w1);
          pb_hi[4 * sb + i] = h1;
          pb_lo[4 * sb + i] = static_cast<_Float16>(w1 - static_cast<float>(h1));
        }
      }
    }

    // ---- PV: MFMA c takes channel 128 hf + 8 n16 + c; k slot 4 sb + i <->
    // token.  Codes enter as exact normal fp16 integers under a biased
    // exponent: an int4 low nibble under 1024 (unit in bit 0) gives 1024 + n,
    // a high nibble under 64 (unit in bit 4) gives 64 + n, an int8 byte with
    // its top bit flipped under 1024 gives 1024 + q + 128; one packed
    // subtraction leaves the code.  (Products of two fp16 subnormals, which a
    // nibble masked in place would be, do not keep their full value in the
    // matrix unit's fp32 sums.)  Groups of 16: the columns of the slice's odd
    // group take the pb rows, those of its even group the pa rows; the other
    // operand's columns are zero, so both passes accumulate into the same
    // registers. ----
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
            const uint32_t x = __builtin_amdgcn_perm(cur.v[sb][2 * pr + 1][hf][0], cur.v[sb][2 * pr][hf][0], sel);
            const uint32_t biased = (c & 1) ? ((x & 0x00F000F0u) | mag_hi) : ((x & 0x000F000Fu) | mag_lo);
            hv[2 * sb + pr] =
                __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, biased) + ((c & 1) ? off_hi : off_lo));
          } else {
            const int wi = (c >> 2) % F::W, by = c & 3;
            const uint32_t sel = 0x0c000c00u | (static_cast<uint32_t>(4 + by) << 16) | static_cast<uint32_t>(by);
            const uint32_t x = __builtin_amdgcn_perm(cur.v[sb][2 * pr + 1][hf][wi], cur.v[sb][2 * pr][hf][wi], sel);
            const uint32_t biased = (x ^ 0x00800080u) | mag_lo;
            hv[2 * sb + pr] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, biased) + off_8);
          }
        }
      }
      if (!F::G16) {
        const half8_t vb = __builtin_bit_cast(half8_t, make_uint4(hv[0], hv[1], hv[2], hv[3]));
        st.acc[hf][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_hi, vb, st.acc[hf][c], 0, 0, 0);
        st.acc[hf][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_lo, vb, st.acc[hf][c], 0, 0, 0);
      } else {
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        const uint4 h4 = make_uint4(hv[0], hv[1], hv[2], hv[3]);
        const half8_t v0 = __builtin_bit_cast(half8_t, odd_group ? z : h4);
        const half8_t v1 = __builtin_bit_cast(half8_t, odd_group ? h4 : z);
        st.acc[hf][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_hi, v0, st.acc[hf][c], 0, 0, 0);
        st.acc[hf][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa_lo, v0, st.acc[hf][c], 0, 0, 0);
        st.acc[hf][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb_hi, v1, st.acc[hf][c], 0, 0, 0);
        st.acc[hf][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb_lo, v1, st.acc[hf][c], 0, 0, 0);
      }
    }
  }
}

// Waves per CU the split geometry targets.  The int4 kernel at D = 128 holds
// two waves per SIMD (up to 256 registers), so eight per CU run at once: one
// round of waves, each with a longer slice, measured faster than two rounds
// (fewer query rotations and partials to combine).  At D = 256 its state and
// blocks are twice as large: one wave per SIMD (up to 512 registers), each
// with twice the bytes in flight.  The fp16 kernel holds four per SIMD at
// D = 128, one at D = 256.
template <bool INT4, int NH>
constexpr int waves_per_cu() {
  return INT4 ? (NH == 1 ? 8 : 4) : (NH == 1 ? 16 : 4);
}

template <bool INT4, int ROT, int FMT, int NH>
__global__ void __launch_bounds__(64, NH == 1 ? 2 : 1) attn_split_kernel(AttnArgs a) {
  using F = QF<FMT, NH>;
  constexpr int D = 128 * NH;
  // rotated query records of the wave's heads (quantized cache)
  __shared__ __attribute__((aligned(16))) uint8_t qrec[INT4 ? kHeadsPerWave * Rec<NH>::BYTES : 16];
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
  const int64_t cell0 = (b * a.Hkv + g) * a.Tcap;
  Rows rows;
  rows.kc = a.k_codes + cell0 * F::CBT;
  rows.ksc = a.k_scales + cell0 * (F::SBT / 2);
  rows.vc = a.v_codes + cell0 * F::CBT;
  rows.vsc = a.v_scales + cell0 * (F::SBT / 2);
  rows.k16 = a.k16 + cell0 * D;
  rows.v16 = a.v16 + cell0 * D;

  // The head whose scores this lane holds: int4 columns are (group, head)
  // pairs with head = n16 & 3; fp16 columns are heads.
  const int my_head = INT4 ? (n16 & 3) : n16;
  const bool head_ok = my_head < nh;
  const int64_t qrow0 = b * a.Hq + hq0;
  const int64_t ws_base = b * a.Hq + hq0;

  if constexpr (INT4) {
    StateQ<NH> st;
    QueryIn qin;
    // int4 cache: rotate and quantize the wave's query heads into LDS
    // records, then gather this lane's MFMA operand.  Runs once the first
    // block's loads are in flight.
    auto init_query = [&]() {
      // all four records (heads past nh hold a zero word and are never read)
      query_records<ROT, NH>(a, qin, lane, qrec);
      // one wave: its LDS writes are visible once its LDS counter drains
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const uint8_t* rec = qrec + (head_ok ? my_head : 0) * Rec<NH>::BYTES;
      const int grp = n16 >> 2;
      const bool live = head_ok && grp == kq;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
        for (int limb = 0; limb < 3; ++limb) {
          uint32_t d[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            d[e] = live ? reinterpret_cast<const uint32_t*>(rec + 128 * NH * limb + 128 * hf + 32 * kq)[e] : 0u;
          if (FMT == 0) {
            // k slot j of k-step ks <-> channel 32 kq + 2 j + ks
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const uint32_t sel = ks ? 0x07050301u : 0x06040200u;
              st.qb[hf][limb][ks] = (int4_t){static_cast<int>(__builtin_amdgcn_perm(d[1], d[0], sel)),
                                             static_cast<int>(__builtin_amdgcn_perm(d[3], d[2], sel)),
                                             static_cast<int>(__builtin_amdgcn_perm(d[5], d[4], sel)),
                                             static_cast<int>(__builtin_amdgcn_perm(d[7], d[6], sel))};
            }
          } else if (F::BITS == 4) {
            // k-step ks covers channels 32 kq + 16 ks + (0, 2, 4, 6, 1, 3, 5,
            // 7, 8, 10, 12, 14, 9, 11, 13, 15): the order the nibbles of four
            // code bytes enter as low, high, low, high words
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
              st.qb[hf][limb][ks] =
                  (int4_t){static_cast<int>(__builtin_amdgcn_perm(d[4 * ks + 1], d[4 * ks], 0x06040200u)),
                           static_cast<int>(__builtin_amdgcn_perm(d[4 * ks + 1], d[4 * ks], 0x07050301u)),
                           static_cast<int>(__builtin_amdgcn_perm(d[4 * ks + 3], d[4 * ks + 2], 0x06040200u)),
                           static_cast<int>(__builtin_amdgcn_perm(d[4 * ks + 3], d[4 * ks + 2], 0x07050301u))};
          } else {
            // int8 codes in channel order: k-step ks covers channels 32 kq + 16 ks ..
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
              st.qb[hf][limb][ks] = (int4_t){static_cast<int>(d[4 * ks]), static_cast<int>(d[4 * ks + 1]),
                                             static_cast<int>(d[4 * ks + 2]), static_cast<int>(d[4 * ks + 3])};
          }
        }
        // s / 2^16 for the limbs; int4 scores come out 16 times too large
        constexpr float kSf = F::BITS == 4 ? 1.f / 1048576.f : 1.f / 65536.f;
        st.sfac[hf] = head_ok ? reinterpret_cast<const float*>(rec + Rec<NH>::S)[4 * hf + grp] * kSf : 0.f;
      }
    };
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[hf][c] = (float4_t){0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_part = 0.f;

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
    const Off4 o4 = lane_offsets4<FMT, NH>(n16, kq);
    const uint32_t seq = static_cast<uint32_t>(a.seq_len);
    const uint32_t nbr = (seq + kBlk - 1) / kBlk;                    // blocks of the row
    const uint32_t S = static_cast<uint32_t>(a.S);
    const uint32_t sp = static_cast<uint32_t>(s);
    const uint32_t cnt = nbr > sp ? (nbr - 1 - sp) / S + 1 : 0;      // blocks of this split
    const bool has_tail = (seq % kBlk) != 0 && (nbr - 1) % S == sp;
    const int n_full = static_cast<int>(cnt) - (has_tail ? 1 : 0);
    const uint32_t step = kBlk * S;
    const uint32_t t_end = seq, t_last = seq - 1;
    // The split's full blocks in a rotated order: block i at position
    // (i + rot) mod n_full, rot = this unit's index.  At any moment the
    // units then read different stretches of their rows, not the same
    // offset of every row (rows lie a fixed stride apart, so equal offsets
    // fall on few memory channels when the stride aliases the channel
    // interleave; measured up to 10% on some cache placements).  The tail,
    // if any, stays last.
    const uint32_t t_first = kBlk * sp;
    const uint32_t rot = n_full > 0 ? (static_cast<uint32_t>(blockIdx.x) / S) % static_cast<uint32_t>(n_full) : 0u;
    auto t_blk = [&](int i) {
      uint32_t j = static_cast<uint32_t>(i) + rot;
      if (j >= static_cast<uint32_t>(n_full)) j -= static_cast<uint32_t>(n_full);
      return t_first + j * step;
    };
    const uint32_t t_tail = t_first + static_cast<uint32_t>(n_full) * step;
    query_loads<ROT, NH>(a, a.q + qrow0 * D, nh, a.lambda_k + g * D, lane, qin);
    Blk4<FMT, NH> b0, b1;
    if (n_full == 0) {
      if (has_tail) load4<FMT, true, NH>(rows, t_tail, t_last, o4, n16, kq, b0);
      init_query();
      if (has_tail) process4<FMT, true, NH>(st, b0, t_tail, t_end, kq, n16, mag_lo, mag_hi);
    } else {
      load4<FMT, false, NH>(rows, t_blk(0), t_last, o4, n16, kq, b0);
      init_query();
      // b0 holds block i at the top; blocks i + 1 and i + 2 are full
      int i = 0;
      for (; i + 2 < n_full; i += 2) {
        load4<FMT, false, NH>(rows, t_blk(i + 1), t_last, o4, n16, kq, b1);
        process4<FMT, false, NH>(st, b0, 0, t_end, kq, n16, mag_lo, mag_hi);
        load4<FMT, false, NH>(rows, t_blk(i + 2), t_last, o4, n16, kq, b0);
        process4<FMT, false, NH>(st, b1, 0, t_end, kq, n16, mag_lo, mag_hi);
      }
      // one or two full blocks left, then maybe the tail
      if (n_full - i == 2) {
        load4<FMT, false, NH>(rows, t_blk(i + 1), t_last, o4, n16, kq, b1);
        process4<FMT, false, NH>(st, b0, 0, t_end, kq, n16, mag_lo, mag_hi);
        if (has_tail) load4<FMT, true, NH>(rows, t_tail, t_last, o4, n16, kq, b0);
        process4<FMT, false, NH>(st, b1, 0, t_end, kq, n16, mag_lo, mag_hi);
        if (has_tail) process4<FMT, true, NH>(st, b0, t_tail, t_end, kq, n16, mag_lo, mag_hi);
      } else {
        if (has_tail) load4<FMT, true, NH>(rows, t_tail, t_last, o4, n16, kq, b1);
        process4<FMT, false, NH>(st, b0, 0, t_end, kq, n16, mag_lo, mag_hi);
        if (has_tail) process4<FMT, true, NH>(st, b1, t_tail, t_end, kq, n16, mag_lo, mag_hi);
      }
    }

    // ---- partial results ----
    float l_part = st.l_part;
    l_part += shfl_xor(l_part, 16);
    l_part += shfl_xor(l_part, 32);
    if (kq == 0 && n16 < nh) {      // lane n16 = head (group 0 column)
      float* ml = a.part_ml + ((ws_base + n16) * a.S + s) * 2;
      ml[0] = st.m_run;
      ml[1] = l_part;
    }
    // acc[hf][c][i]: row block kq (value group kq of the half), head i,
    // channel 128 hf + 8 n16 + c
    if (kq == (n16 >> 2)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nh) {
          float* dst = a.part_acc + ((ws_base + i) * a.S + s) * D + 8 * n16;
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) {
            *reinterpret_cast<float4*>(dst + 128 * hf) =
                make_float4(st.acc[hf][0][i], st.acc[hf][1][i], st.acc[hf][2][i], st.acc[hf][3][i]);
            *reinterpret_cast<float4*>(dst + 128 * hf + 4) =
                make_float4(st.acc[hf][4][i], st.acc[hf][5][i], st.acc[hf][6][i], st.acc[hf][7][i]);
          }
        }
      }
    }
  } else {
    StateF<NH> st;
    const uint32_t t_begin = static_cast<uint32_t>(s * a.chunk);
    const uint32_t t_end = static_cast<uint32_t>(min(s * a.chunk + a.chunk, a.seq_len));
    // fp16 cache: q * sm_scale * log2(e) as fp16 hi + lo halves, channels
    // 32 grp + 8 kq .. + 7 of head n16
    const float scl = a.sm_scale * kLog2e;
    const uint16_t* qr = a.q + (qrow0 + (head_ok ? my_head : 0)) * D;
#pragma unroll
    for (int grp = 0; grp < 4 * NH; ++grp) {
      const uint4 w = head_ok ? *reinterpret_cast<const uint4*>(qr + 32 * grp + 8 * kq) : make_uint4(0, 0, 0, 0);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = f16_bits_to_f32(ws[e] & 0xFFFFu) * scl, x1 = f16_bits_to_f32(ws[e] >> 16) * scl;
        hw[e] = pack_f16x2(x0, x1);
        lw[e] = pack_f16x2(x0 - f16_bits_to_f32(hw[e] & 0xFFFFu), x1 - f16_bits_to_f32(hw[e] >> 16));
      }
      st.qh[grp] = __builtin_bit_cast(half8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      st.ql[grp] = __builtin_bit_cast(half8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[hf][c] = (float4_t){0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_part = 0.f;
    // 32-token blocks; the block that reaches t_end is a tail.  The fp16
    // tile is four times larger: one buffer, occupancy hides latency.
    const uint32_t t_last = t_end - 1;
    const int n_full = static_cast<int>((t_end - t_begin) / kBlk);   // blocks entirely inside
    // full blocks from a rotated start, as the quantized cache's stream
    // (rows a fixed stride apart would otherwise be read at equal offsets
    // at the same time); the tail stays last
    const uint32_t rotf =
        n_full > 0 ? (static_cast<uint32_t>(blockIdx.x) / static_cast<uint32_t>(a.S)) % static_cast<uint32_t>(n_full) : 0u;
    for (int i = 0; i < n_full; ++i) {
      uint32_t jj = static_cast<uint32_t>(i) + rotf;
      if (jj >= static_cast<uint32_t>(n_full)) jj -= static_cast<uint32_t>(n_full);
      const uint32_t tb = t_begin + jj * kBlk;
      BlkF<NH> bb;
      load_blkf<false, NH>(rows, tb, t_last, n16, kq, bb);
      process_blkf<false, NH>(st, bb, tb, t_end, kq);
    }
    const uint32_t t0 = t_begin + static_cast<uint32_t>(n_full) * kBlk;
    if (t0 < t_end) {
      BlkF<NH> bb;
      load_blkf<true, NH>(rows, t0, t_last, n16, kq, bb);
      process_blkf<true, NH>(st, bb, t0, t_end, kq);
    }

    // ---- partial results ----
    float l_part = st.l_part;
    l_part += shfl_xor(l_part, 16);
    l_part += shfl_xor(l_part, 32);
    if (kq == 0 && n16 < nh) {      // lane n16 = head
      float* ml = a.part_ml + ((ws_base + n16) * a.S + s) * 2;
      ml[0] = st.m_run;
      ml[1] = l_part;
    }
    // acc[hf][c][i]: heads 4 kq + i (only kq = 0 holds real heads), channel
    // 128 hf + 8 n16 + c
    if (kq == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nh) {
          float* dst = a.part_acc + ((ws_base + i) * a.S + s) * D + 8 * n16;
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) {
            *reinterpret_cast<float4*>(dst + 128 * hf) =
                make_float4(st.acc[hf][0][i], st.acc[hf][1][i], st.acc[hf][2][i], st.acc[hf][3][i]);
            *reinterpret_cast<float4*>(dst + 128 * hf + 4) =
                make_float4(st.acc[hf][4][i], st.acc[hf][5][i], st.acc[hf][6][i], st.acc[hf][7][i]);
          }
        }
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

// Unitary inverse 64-point DFT across the wave, in place on (re, im) of
// every entry of the arrays: lane l holds frequency l, radix-2 decimation in
// frequency (kernel exp(+2 pi i / 64) without the scale), and ends with time
// index bitrev(l).
template <int N>
__device__ __forceinline__ void idft64_lanes(float (&re)[N], float (&im)[N], int lane) {
#pragma unroll
  for (int hh = 32; hh >= 1; hh >>= 1) {
    const int e = (lane & (hh - 1)) * (32 / hh);   // exp(+2 pi i e / 64)
    const float cw = kTw64Const.c[e], sw = kTw64Const.s[e];
    float pr[N], pi[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      pr[n] = shfl_xor(re[n], hh);
      pi[n] = shfl_xor(im[n], hh);
    }
#pragma unroll
    for (int n = 0; n < N; ++n) {
      if (lane & hh) {
        const float dr = pr[n] - re[n], di = pi[n] - im[n];
        re[n] = dr * cw - di * sw;
        im[n] = dr * sw + di * cw;
      } else {
        re[n] += pr[n];
        im[n] += pi[n];
      }
    }
  }
}

// Walsh-Hadamard transform of 128 channels across the wave, in place on
// every entry: lane l holds channels 2 l (y0) and 2 l + 1 (y1).
template <int N>
__device__ __forceinline__ void wht128_lanes(float (&y0)[N], float (&y1)[N], int lane) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float t0 = y0[n] + y1[n], t1 = y0[n] - y1[n];
    y0[n] = t0;
    y1[n] = t1;
  }
#pragma unroll
  for (int hh = 1; hh <= 32; hh <<= 1) {
    float p0[N], p1[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      p0[n] = shfl_xor(y0[n], hh);
      p1[n] = shfl_xor(y1[n], hh);
    }
#pragma unroll
    for (int n = 0; n < N; ++n) {
      if (lane & hh) { y0[n] = p0[n] - y0[n]; y1[n] = p1[n] - y1[n]; }
      else { y0[n] += p0[n]; y1[n] += p1[n]; }
    }
  }
}

template <int ROT, int OUT_F32, int NH>
__global__ void __launch_bounds__(64) attn_combine_kernel(AttnArgs a, int int4) {
  constexpr int D = 128 * NH;
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t h = bh % a.Hq;
  const int64_t g = h / (a.Hq / a.Hkv);
  const float* ml = a.part_ml + bh * a.S * 2;
  const float* acc = a.part_acc + bh * a.S * D + 2 * lane;

  // lambda_V of the lane's channels 128 hf + 2 lane, + 1, loaded with the
  // partials
  float lv[NH][2];
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    lv[hf][0] = int4 ? a.lambda_v[g * D + 128 * hf + 2 * lane] : 1.f;
    lv[hf][1] = int4 ? a.lambda_v[g * D + 128 * hf + 2 * lane + 1] : 1.f;
  }
  float l = 0.f;
  float x[NH][2] = {};
  float m = -INFINITY;
  if (a.S <= 16) {
    // one pass with every load issued up front: the split maxima and sums
    // (one split per lane) and the lane's channels of every split
    const int S = static_cast<int>(a.S);
    const float2 msl = lane < S ? *reinterpret_cast<const float2*>(ml + 2 * lane) : make_float2(-INFINITY, 0.f);
    float2 v[16][NH];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
        v[u][hf] = u < S ? *reinterpret_cast<const float2*>(acc + u * D + 128 * hf) : make_float2(0.f, 0.f);
    m = wave_max(msl.x);
    const float w = msl.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(msl.x - m);
    l = w * msl.y;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        x[hf][0] = fmaf(wu, v[u][hf].x, x[hf][0]);
        x[hf][1] = fmaf(wu, v[u][hf].y, x[hf][1]);
      }
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
        float2 v[8][NH];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int hf = 0; hf < NH; ++hf)
            v[u][hf] = *reinterpret_cast<const float2*>(acc + (s0 + j + u) * D + 128 * hf);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j + u));
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) {
            x[hf][0] = fmaf(wu, v[u][hf].x, x[hf][0]);
            x[hf][1] = fmaf(wu, v[u][hf].y, x[hf][1]);
          }
        }
      }
      for (; j < n; ++j) {
        const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
          const float2 v = *reinterpret_cast<const float2*>(acc + (s0 + j) * D + 128 * hf);
          x[hf][0] = fmaf(wu, v.x, x[hf][0]);
          x[hf][1] = fmaf(wu, v.y, x[hf][1]);
        }
      }
    }
  }
  l = wave_sum(l);
  const float inv = 1.f / l;
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    x[hf][0] *= inv;
    x[hf][1] *= inv;
  }

  // ch[n]: first channel of the pair x[n] (n = hf) is written to, and its
  // sign bits
  int ch[NH];
  uint32_t neg[NH][2] = {};
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) ch[hf] = 128 * hf + 2 * lane;
  if (int4) {
    if (ROT == KVQ_ROT_SRFT) {
      // Z = x / lambda (unitary scale folded in); unitary inverse DFT
      constexpr float c = NH == 1 ? 0.125f : 0.0883883476483184405f;
      float re[NH], im[NH];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        re[hf] = x[hf][0] * (c / lv[hf][0]);
        im[hf] = x[hf][1] * (c / lv[hf][1]);
      }
      if (NH == 2) {
        // lane l holds Z_l and Z_{l+64}: A_l = Z_l + Z_{l+64} feeds the even
        // outputs z_{2k}, B_l = (Z_l - Z_{l+64}) exp(+2 pi i l / 128) the odd
        // ones z_{2k+1}
        const float cw = kTw128Const.c[lane], sw = kTw128Const.s[lane];
        const float ar = re[0] + re[NH - 1], ai = im[0] + im[NH - 1];
        const float dr = re[0] - re[NH - 1], di = im[0] - im[NH - 1];
        re[0] = ar;
        im[0] = ai;
        re[NH - 1] = dr * cw - di * sw;
        im[NH - 1] = dr * sw + di * cw;
      }
      idft64_lanes<NH>(re, im, lane);
      const int k = bitrev6(lane);
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        const int pair = NH == 1 ? k : 2 * k + hf;    // complex pair this entry holds
        ch[hf] = 2 * pair;
        x[hf][0] = re[hf];
        x[hf][1] = im[hf];
        neg[hf][0] = neg[hf][1] = sign_bit(a.signs, pair);
      }
    } else if (ROT == KVQ_ROT_SRHT) {
      constexpr float c = NH == 1 ? 0.0883883476483184405f : 0.0625f;
      float y0[NH], y1[NH];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        y0[hf] = x[hf][0] * (c / lv[hf][0]);
        y1[hf] = x[hf][1] * (c / lv[hf][1]);
      }
      if (NH == 2) {
        // H_256 [u; v] = [H_128 (u + v); H_128 (u - v)]
        const float a0 = y0[0], a1 = y1[0], b0 = y0[NH - 1], b1 = y1[NH - 1];
        y0[0] = a0 + b0;
        y1[0] = a1 + b1;
        y0[NH - 1] = a0 - b0;
        y1[NH - 1] = a1 - b1;
      }
      wht128_lanes<NH>(y0, y1, lane);
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        x[hf][0] = y0[hf];
        x[hf][1] = y1[hf];
        neg[hf][0] = sign_bit(a.signs, ch[hf]);
        neg[hf][1] = sign_bit(a.signs, ch[hf] + 1);
      }
    } else {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        x[hf][0] /= lv[hf][0];
        x[hf][1] /= lv[hf][1];
      }
    }
  }
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    const float o0 = neg[hf][0] ? -x[hf][0] : x[hf][0];
    const float o1 = neg[hf][1] ? -x[hf][1] : x[hf][1];
    if (OUT_F32) {
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + bh * D + ch[hf]) = make_float2(o0, o1);
    } else {
      static_cast<uint32_t*>(a.out)[(bh * D + ch[hf]) / 2] = pack_f16x2(o0, o1);
    }
  }
}

}  // namespace

}  // namespace kvq
