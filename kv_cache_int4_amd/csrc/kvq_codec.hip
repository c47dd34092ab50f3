// Encode / rotate / decode kernels of the int4 KV-cache codec (gfx950).
//
// Work decomposition.  A wave owns a tile of 16 KiB of fp16 input: 64 head
// vectors of D=128 (one per lane) or 32 vectors of D=256 (a lane pair each).
// Tiles never cross a (batch, head) row, so the lambda row is wave-uniform.
// The grid has one wave per tile, up to 32 waves per CU; larger calls have
// the waves walk the tiles with a stride of the grid, loading the next tile
// while computing the current one.  Two waves share every SIMD, so one
// streams its tile in while the other computes.
//
// Hot kernels (encode128/256, decode128/256): the next tile's input goes
// straight from HBM into LDS with direct (global -> LDS) loads while the
// current tile computes in registers; each lane then reads its own vector
// (or half vector) from a bank-swizzled LDS block, runs the fp32 transform,
// lambda, group abs-max and int4 packing (or the reverse), and the results
// leave through coalesced 16-byte stores.  Random signs are applied as XOR
// masks on fp16 words where each lane's masks are fixed for the kernel.
//
// The encoders also write the rotated fp32 values (rotate mode, for
// checking the transform); decode_f32_kernel (fp32 output) stages rows
// through registers and LDS with ordinary loads.
//
// Method (gist.science explainer of "When Quantization Is Free",
// "Methodik" 1-2): sign -> FFT over the D/2 complex pairs -> pack ->
// lambda -> per-group abs-max -> int4 -> two nibbles per byte.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"

namespace kvq {

namespace {

// One plan-independent description of a codec launch.
struct CodecArgs {
  const uint16_t* x;          // encode / rotate input, fp16
  const uint8_t* codes_in;    // decode input
  const uint16_t* scales_in;
  uint8_t* codes;             // encode output
  uint16_t* scales;
  void* y;                    // decode output (fp16 or fp32)
  float* w;                   // rotate output
  const float* lambda;
  int64_t H, T, Tcap, t0;
  int64_t sb, sh, st;         // strides of x (encode, rotate) or y (decode)
  int64_t lambda_sb;
  int64_t tiles_per_row, n_tiles;
  FastDiv div_tpr, div_h;     // by tiles_per_row and by H
  uint64_t signs[4];
};

template <int D>
struct Geo {
  static constexpr int L = D / 128;            // lanes per vector
  static constexpr int VPT = 64 / L;           // vectors per tile
  static constexpr int CPR = D / 8;            // 16-byte chunks per fp16 row
  static constexpr int RPI = 64 / CPR;         // rows per 64-lane load
  static constexpr int NLD = VPT * CPR / 64;   // loads per lane per tile (16)
};

// Unitary scale of the rotation, folded into per-group constants.
template <int D, int ROT>
__host__ __device__ constexpr float rot_scale() {
  return ROT == KVQ_ROT_SRFT ? (D == 128 ? 0.125f : 0.0883883476483184405f)
       : ROT == KVQ_ROT_SRHT ? (D == 128 ? 0.0883883476483184405f : 0.0625f)
       : 1.0f;
}

__host__ __device__ __forceinline__ uint32_t sign_bit(const uint64_t (&s)[4], int i) {
  const uint64_t w = i < 64 ? s[0] : i < 128 ? s[1] : i < 192 ? s[2] : s[3];
  return static_cast<uint32_t>(w >> (i & 63)) & 1u;
}

// XOR mask for fp16 pair word k (channels 2k, 2k+1) of a row: the random
// signs, plus a negation of the data the second lane of a D=256 vector owns
// (it lets the cross-lane radix-2 step use one fused multiply-add).
template <int D, int ROT>
__host__ __device__ __forceinline__ uint32_t word_mask(const uint64_t (&s)[4], int k) {
  uint32_t m = 0;
  if (ROT == KVQ_ROT_SRFT) {
    m = sign_bit(s, k) ? 0x80008000u : 0u;
    if (D == 256 && (k & 1)) m ^= 0x80008000u;
  } else if (ROT == KVQ_ROT_SRHT) {
    m = (sign_bit(s, 2 * k) << 15) | (sign_bit(s, 2 * k + 1) << 31);
    if (D == 256 && k >= 64) m ^= 0x80008000u;
  }
  return m;
}

// LDS byte offset of 16-byte chunk j of the 256-byte block owned by lane
// `blk`: the chunk index is XOR-swizzled with the block so that a lane-
// parallel read of chunk j by 16 consecutive lanes hits 16 distinct bank
// groups.
__device__ __forceinline__ uint32_t blk_off(int blk, int j) {
  return static_cast<uint32_t>(blk * 256 + ((j ^ (blk & 15)) << 4));
}

// LDS byte offset of 16-byte chunk q of the 64-byte code row of lane r.
__device__ __forceinline__ uint32_t code_off(int r, int q) {
  return static_cast<uint32_t>(r * 64 + ((q ^ ((r >> 2) & 3)) << 4));
}

struct Tile {
  int64_t row;      // b * H + h
  int64_t b, h;
  int64_t t_start;
  int nv;           // valid vectors in the tile
};

template <int D>
__device__ __forceinline__ Tile tile_info(const CodecArgs& a, int64_t tile) {
  Tile t;
  t.row = static_cast<int64_t>(fdiv(static_cast<uint64_t>(tile), a.div_tpr));
  t.t_start = (tile - t.row * a.tiles_per_row) * Geo<D>::VPT;
  t.b = static_cast<int64_t>(fdiv(static_cast<uint64_t>(t.row), a.div_h));
  t.h = t.row - t.b * a.H;
  const int64_t left = a.T - t.t_start;
  t.nv = static_cast<int>(left < Geo<D>::VPT ? left : Geo<D>::VPT);
  return t;
}

// ---------------------------------------------------------------------------
// D = 128 encode: one vector per lane, tiles of 64 vectors (16 KiB) brought
// into LDS by direct global->LDS loads, one tile ahead of the compute.
// ---------------------------------------------------------------------------

// fp16 + fp16 -> fp32 (or -) with both conversions folded into one
// v_fma_mix_f32: (+-b_half) * 1.0 + a_half.  SELA / SELB pick the low (0)
// or high (1) half of each packed word.
#define KVQ_MIX(NAME, SELA, SELB, NEG)                                                     \
  __device__ __forceinline__ float NAME(uint32_t a, uint32_t b) {                          \
    float r;                                                                               \
    asm("v_fma_mix_f32 %0, " NEG "%1, 1.0, %2 op_sel:[" #SELB ",0," #SELA "] op_sel_hi:[1,0,1]" \
        : "=v"(r) : "v"(b), "v"(a));                                                       \
    return r;                                                                              \
  }
KVQ_MIX(mix_add_ll, 0, 0, "")
KVQ_MIX(mix_sub_ll, 0, 0, "-")
KVQ_MIX(mix_add_hh, 1, 1, "")
KVQ_MIX(mix_sub_hh, 1, 1, "-")
KVQ_MIX(mix_add_lh, 0, 1, "")
KVQ_MIX(mix_sub_lh, 0, 1, "-")
#undef KVQ_MIX

// Cache policy of the D=128 encoder's tile loads: non-temporal (the fp16
// input is read once).  Measured in one process against plain loads: int8
// encode 4-6% faster, int4 within 1%; the same hint on the decoders' code
// loads made them 6-15% slower and on the D=256 encoder changed nothing,
// so only these loads carry it.
constexpr int kNonTemporal = 2;

// Slot i*64 + lane of the LDS tile (16 bytes) receives row 4i + lane/16,
// chunk (lane%16) ^ (row%16): exactly where blk_off puts it, so the per-lane
// row reads below are free of bank conflicts.  The lane's byte offset inside
// a group of four rows depends only on i % 4 (off4, fixed per call); the rest
// of the address is wave-uniform, so the loads take the scalar-base form.
// Rows past the tile's end are not loaded (their lanes compute on stale data
// and store nothing).
__device__ __forceinline__ void dma_tile128(const CodecArgs& a, const Tile& t, uint8_t* lds, int lane,
                                            const uint32_t (&off4)[4]) {
  const char* base = reinterpret_cast<const char*>(a.x + t.b * a.sb + t.h * a.sh + t.t_start * a.st);
  const int64_t step = 8 * a.st;        // bytes of four rows
  if (t.nv == 64) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_global_load_lds(base + i * step + off4[i & 3], lds + 1024 * i, 16, 0, kNonTemporal);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (4 * i + (lane >> 4) < t.nv)
        __builtin_amdgcn_global_load_lds(base + i * step + off4[i & 3], lds + 1024 * i, 16, 0, kNonTemporal);
  }
}

// First radix-4 DIF stage of the 64-point transform, straight from the
// packed fp16 pairs p[k] = (re, im) of z_k.
__device__ __forceinline__ void dif4_first_packed(const uint32_t (&p)[64], float (&v)[128]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t a = p[j], b = p[j + 16], c = p[j + 32], d = p[j + 48];
    const float t0r = mix_add_ll(a, c), t0i = mix_add_hh(a, c);
    const float t1r = mix_sub_ll(a, c), t1i = mix_sub_hh(a, c);
    const float t2r = mix_add_ll(b, d), t2i = mix_add_hh(b, d);
    const float t3r = mix_sub_ll(b, d), t3i = mix_sub_hh(b, d);
    const int i0 = j, i1 = j + 16, i2 = j + 32, i3 = j + 48;
    v[2 * i0] = t0r + t2r;
    v[2 * i0 + 1] = t0i + t2i;
    v[2 * i2] = t0r - t2r;
    v[2 * i2 + 1] = t0i - t2i;
    v[2 * i1] = t1r + t3i;
    v[2 * i1 + 1] = t1i - t3r;
    v[2 * i3] = t1r - t3i;
    v[2 * i3 + 1] = t1i + t3r;
    twiddle<64, false>(v[2 * i1], v[2 * i1 + 1], j);
    twiddle<64, false>(v[2 * i2], v[2 * i2 + 1], 2 * j);
    twiddle<64, false>(v[2 * i3], v[2 * i3 + 1], 3 * j);
  }
}

// Forward rotation of one packed fp16 vector (signs already applied):
// result in v with channel j at chan_reg<ROT>(j), unnormalized.
template <int ROT>
__device__ __forceinline__ void rotate_packed(const uint32_t (&p)[64], float (&v)[128]) {
  if (ROT == KVQ_ROT_SRFT) {
    dif4_first_packed(p, v);
    dif4_stage<16, false>(v);
    dif4_stage<4, false>(v);
  } else if (ROT == KVQ_ROT_SRHT) {
    // stride-1 butterflies inside each packed word, then the rest
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      v[2 * k] = mix_add_lh(p[k], p[k]);
      v[2 * k + 1] = mix_sub_lh(p[k], p[k]);
    }
#pragma unroll
    for (int h = 2; h < 128; h *= 2) {
#pragma unroll
      for (int i = 0; i < 128; i += 2 * h) {
#pragma unroll
        for (int j = i; j < i + h; ++j) {
          const float x0 = v[j], x1 = v[j + h];
          v[j] = x0 + x1;
          v[j + h] = x0 - x1;
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      v[2 * k] = f16_bits_to_f32(p[k] & 0xFFFFu);
      v[2 * k + 1] = f16_bits_to_f32(p[k] >> 16);
    }
  }
}

// Code format of a plan: FMT = 2 * (bits == 8) + (G == 16).  A lane owns 128
// channels (a D=128 vector or half a D=256 vector); these are its sizes.
template <int FMT>
struct Fmt {
  static constexpr int BITS = (FMT & 2) ? 8 : 4;
  static constexpr int G = (FMT & 1) ? 16 : 32;
  static constexpr int NG = 128 / G;            // groups per lane
  static constexpr int CW = 128 * BITS / 32;    // code words per lane (16 or 32)
  static constexpr int CB = 4 * CW;             // code bytes per lane (64 or 128)
  static constexpr int SB = 2 * NG;             // scale bytes per lane (8 or 16)
  static constexpr int IQMAX = BITS == 4 ? 7 : 127;
};

// Codes of group g (G channels) from w and r = 1 / scale: int4 as pair
// bytes (G / 8 words), int8 as two's-complement channel bytes (G / 4 words),
// written to cw[0 ..].  Without CLAMP the magic-number rounding alone gives
// the code: with a normal fp16 scale |w r| <= qmax (1 + 2^-11) (1 + 2^-23) <
// qmax + 1/2.
template <int ROT, bool CLAMP, int FMT>
__device__ __forceinline__ void quant_group(const float (&v)[128], int g, float r, uint32_t* cw) {
  using F = Fmt<FMT>;
  if (F::BITS == 4) {
#pragma unroll
    for (int q = 0; q < F::G / 8; ++q) {
      uint32_t by[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = F::G * g + 8 * q + 2 * e;
        uint32_t lo, hi;
        if (CLAMP) {
          lo = quant_bits(v[chan_reg<ROT>(j)], r);
          hi = quant_bits(v[chan_reg<ROT>(j + 1)], r);
        } else {
          lo = __builtin_bit_cast(uint32_t, fmaf(v[chan_reg<ROT>(j)], r, kMagic));
          hi = __builtin_bit_cast(uint32_t, fmaf(v[chan_reg<ROT>(j + 1)], r, kMagic));
        }
        by[e] = pair_byte(lo, hi);
      }
      cw[q] = pack4(by[0], by[1], by[2], by[3]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < F::G / 4; ++q) {
      uint32_t by[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = F::G * g + 4 * q + e;
        by[e] = CLAMP ? quant_bits8(v[chan_reg<ROT>(j)], r)
                      : __builtin_bit_cast(uint32_t, fmaf(v[chan_reg<ROT>(j)], r, kMagic8));
      }
      // offset bytes q + 128 -> two's complement
      cw[q] = pack4(by[0], by[1], by[2], by[3]) ^ 0x80808080u;
    }
  }
}

constexpr int kLdsTile = 16384;              // LDS tile of the D=128 encoder

// LDS memory as the direct-load builtins take it.
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Read-only data for scalar loads (the constant address space).
typedef __attribute__((address_space(4))) const float cfloat;

// Sign mask of complex pair k (one fp16 word pair) of a D=128 vector.
template <int ROT>
__device__ __forceinline__ uint32_t pair_mask128(const CodecArgs& a, int k) {
  if (ROT == KVQ_ROT_SRFT) return ((a.signs[0] >> k) & 1u) ? 0x80008000u : 0u;
  if (ROT == KVQ_ROT_SRHT) {
    const uint64_t w = k < 32 ? a.signs[0] : a.signs[1];
    const int i = (2 * k) & 63;
    return (static_cast<uint32_t>((w >> i) & 1u) << 15) | (static_cast<uint32_t>((w >> (i + 1)) & 1u) << 31);
  }
  return 0u;
}

// One lane's codes (F::CB bytes) and scales (F::SB bytes) at byte offsets
// lane * CB and lane * SB of wave-uniform bases.
template <typename F>
__device__ __forceinline__ void store_lane_codes(char* cbase, char* sbase, int lane, const uint4 (&c)[F::CB / 16],
                                                 const uint32_t (&sw)[F::NG / 2]) {
  if (F::NG == 4) {
    *reinterpret_cast<uint2*>(sbase + static_cast<uint32_t>(lane * F::SB)) = make_uint2(sw[0], sw[1]);
  } else {
    *reinterpret_cast<uint4*>(sbase + static_cast<uint32_t>(lane * F::SB)) =
        make_uint4(sw[0], sw[1 % (F::NG / 2)], sw[2 % (F::NG / 2)], sw[3 % (F::NG / 2)]);
  }
#pragma unroll
  for (int q = 0; q < F::CB / 16; ++q)
    *reinterpret_cast<uint4*>(cbase + static_cast<uint32_t>(lane * F::CB + 16 * q)) = c[q];
}

// The same stores with the code rows turned around in LDS first (lds: at
// least 64 * CB free bytes), so that every store instruction writes 1 KiB of
// consecutive rows: row r goes to LDS row r with its NC = CB / 16 chunks
// XOR-swizzled by (r NC / 16) mod NC (16 consecutive lanes then hit 16
// distinct four-bank groups, both when a lane writes its row and when lanes
// read chunk L mod NC of row L / NC); lane L stores chunk L mod NC of row
// 64 i / NC + L / NC with instruction i.  Rows at or past nv are not stored.
// One wave: its LDS reads follow its LDS writes in order.  The lane index
// is laundered so that the addresses are formed here, not hoisted out of
// the tile loop (where they would hold registers across the transform).
// NT: the 1 KiB row stores as non-temporal stores.
template <typename F, bool NT>
__device__ __forceinline__ void store_codes_staged(char* cbase, char* sbase, int lane, int nv, uint8_t* lds,
                                                   const uint4 (&c)[F::CB / 16], const uint32_t (&sw)[F::NG / 2]) {
  constexpr int NC = F::CB / 16;
  asm volatile("" : "+v"(lane));
  const int sw_w = (lane * NC / 16) % NC;
#pragma unroll
  for (int q = 0; q < NC; ++q) *reinterpret_cast<uint4*>(lds + lane * F::CB + 16 * (q ^ sw_w)) = c[q];
  if (lane < nv) {
    if (F::NG == 4) {
      *reinterpret_cast<uint2*>(sbase + static_cast<uint32_t>(lane * F::SB)) = make_uint2(sw[0], sw[1]);
    } else {
      *reinterpret_cast<uint4*>(sbase + static_cast<uint32_t>(lane * F::SB)) =
          make_uint4(sw[0], sw[1 % (F::NG / 2)], sw[2 % (F::NG / 2)], sw[3 % (F::NG / 2)]);
    }
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int row = 64 / NC * i + lane / NC;
    const int q = lane % NC;
    const uint4 w = *reinterpret_cast<const uint4*>(lds + row * F::CB + 16 * (q ^ ((row * NC / 16) % NC)));
    if (row < nv) {
      char* dst = cbase + static_cast<uint32_t>(1024 * i + 16 * lane);
      if (NT) st_stream16(dst, w);
      else *reinterpret_cast<uint4*>(dst) = w;
    }
  }
}

// ONE: the grid has a wave per tile (no prefetch; the codes leave through
// the free tile buffer).
template <int ROT, int MODE, int FMT, bool ONE>
__global__ void __launch_bounds__(64, 2) encode128_kernel(CodecArgs a) {
  using F = Fmt<FMT>;
  // separate LDS objects, so that reads of the masks and of lambda need not
  // wait for the direct loads into the tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsTile];
  __shared__ __attribute__((aligned(16))) uint32_t mask_lds[64];
  __shared__ __attribute__((aligned(16))) float lam_lds[128];
  const int lane = threadIdx.x;
  constexpr float kScale = rot_scale<128, ROT>();

  mask_lds[lane] = pair_mask128<ROT>(a, lane);
  uint32_t off4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + (lane >> 4);
    off4[i] = static_cast<uint32_t>((lane >> 4) * 2 * a.st + 16 * ((lane & 15) ^ (r & 15)));
  }
  // lambda of a tile: lane l holds channels l and l + 64 in registers from
  // loads issued right after the tile's direct loads (so the one wait at the
  // top of the loop covers both), and writes them to LDS there
  float lam_r0 = 0.f, lam_r1 = 0.f;
  int64_t tile = blockIdx.x;
  if (tile < a.n_tiles) {
    const Tile t = tile_info<128>(a, tile);
    dma_tile128(a, t, lds, lane, off4);
    const float* lr = a.lambda + t.b * a.lambda_sb + t.h * 128;
    lam_r0 = lr[lane];
    lam_r1 = lr[lane + 64];
  }
  __syncthreads();
  // codes and scales of the previous tile, stored only after the next tile's
  // loads are on their way (so that the wait for those loads at the top of
  // the loop never waits on fresh stores)
  uint4 pend_c[F::CB / 16] = {};
  uint32_t pend_s[F::NG / 2] = {};
  bool pend_valid = false;
  char* pend_cbase = nullptr;
  char* pend_sbase = nullptr;
  for (; tile < a.n_tiles; tile += gridDim.x) {
    const Tile t = tile_info<128>(a, tile);
    // the tile's direct loads have landed in LDS (everything issued after
    // them is a store of the tile before, a transform ago)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lam_lds[lane] = lam_r0;
    lam_lds[lane + 64] = lam_r1;
    const uint4* masks = reinterpret_cast<const uint4*>(mask_lds);
    uint32_t p[64];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 w = *reinterpret_cast<const uint4*>(lds + blk_off(lane, j));
      const uint4 m = masks[j];
      p[4 * j] = w.x ^ m.x;
      p[4 * j + 1] = w.y ^ m.y;
      p[4 * j + 2] = w.z ^ m.z;
      p[4 * j + 3] = w.w ^ m.w;
    }
    // the tile is in registers: the buffer takes the next one
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t nxt = tile + gridDim.x;
    if (!ONE && nxt < a.n_tiles) {
      const Tile tn = tile_info<128>(a, nxt);
      dma_tile128(a, tn, lds, lane, off4);
      const float* lr = a.lambda + tn.b * a.lambda_sb + tn.h * 128;
      lam_r0 = lr[lane];
      lam_r1 = lr[lane + 64];
    }
    if (MODE == 0 && !ONE && pend_valid) store_lane_codes<F>(pend_cbase, pend_sbase, lane, pend_c, pend_s);

    float v[128];
    rotate_packed<ROT>(p, v);
    // keep the lambda reads below the transform (hoisted they would hold
    // registers across it)
    asm volatile("" ::: "memory");
    const float4* lam4 = reinterpret_cast<const float4*>(lam_lds);
    const bool valid = lane < t.nv;

    if (MODE == 1) {
      float* wr = a.w + ((t.row * a.T) + t.t_start + lane) * 128;
      if (valid) {
#pragma unroll
        for (int j = 0; j < 128; j += 4) {
          float4 o;
          const float4 l4 = lam4[j / 4];
          o.x = v[chan_reg<ROT>(j)] * l4.x * kScale;
          o.y = v[chan_reg<ROT>(j + 1)] * l4.y * kScale;
          o.z = v[chan_reg<ROT>(j + 2)] * l4.z * kScale;
          o.w = v[chan_reg<ROT>(j + 3)] * l4.w * kScale;
          *reinterpret_cast<float4*>(wr + j) = o;
        }
      }
    } else {
      float r[F::NG];
      uint32_t sc[F::NG];
      bool tiny = false;
#pragma unroll
      for (int g = 0; g < F::NG; ++g) {
        asm volatile("" ::: "memory");    // one group's lambda reads at a time
        float amax = 0.f;
#pragma unroll
        for (int jj = 0; jj < F::G; jj += 4) {
          const int j = F::G * g + jj;
          const float4 l4 = lam4[j / 4];
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float wv = v[chan_reg<ROT>(j + e)] * lv[e];
            v[chan_reg<ROT>(j + e)] = wv;
            amax = fmaxf(amax, fabsf(wv));
          }
        }
        // scale = fp16(fp32(absmax / qmax)) with the IEEE fp32 quotient
        // (div_by: three instructions per group); amax * kScale is the
        // unitary abs-max, exact where kScale is a power of two
        sc[g] = f32_to_f16_bits(div_by<F::IQMAX>(amax * kScale));
        const float sf = f16_bits_to_f32(sc[g]);
        r[g] = sf > 0.f ? kScale * __builtin_amdgcn_rcpf(sf) : 0.f;
        tiny |= (sc[g] != 0u) && (sc[g] < 0x0400u);    // fp16-subnormal scale
      }
      uint32_t cw[F::CW];
      constexpr int kWordsPerGroup = F::CW / F::NG;
      if (__builtin_amdgcn_ballot_w64(tiny && valid) == 0) {
#pragma unroll
        for (int g = 0; g < F::NG; ++g) quant_group<ROT, false, FMT>(v, g, r[g], cw + kWordsPerGroup * g);
      } else {
#pragma unroll
        for (int g = 0; g < F::NG; ++g) quant_group<ROT, true, FMT>(v, g, r[g], cw + kWordsPerGroup * g);
      }
      const int64_t cell0 = t.row * a.Tcap + a.t0 + t.t_start;   // wave-uniform
      pend_sbase = reinterpret_cast<char*>(a.scales + cell0 * F::NG);
      pend_cbase = reinterpret_cast<char*>(a.codes + cell0 * F::CB);
#pragma unroll
      for (int i = 0; i < F::NG / 2; ++i) pend_s[i] = sc[2 * i] | (sc[2 * i + 1] << 16);
#pragma unroll
      for (int q = 0; q < F::CB / 16; ++q)
        pend_c[q] = make_uint4(cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]);
      pend_valid = valid;
      if (ONE) {
        // the input tile is in registers and its LDS buffer is free: the
        // code rows leave through it as 1 KiB non-temporal stores (int8
        // rows of 128 bytes: 11-13% faster than per-lane stores; with the
        // non-temporal hint int4 2.4-4.1% and int8 a further 1.4-2.1%
        // faster; int4 rows as normal 1 KiB stores gained nothing)
        store_codes_staged<F, true>(pend_cbase, pend_sbase, lane, t.nv, lds, pend_c, pend_s);
        pend_valid = false;
      }
    }
  }
  if (MODE == 0 && !ONE && pend_valid) store_lane_codes<F>(pend_cbase, pend_sbase, lane, pend_c, pend_s);
}

// ---------------------------------------------------------------------------
// D = 128 SRFT encode with the DFT on the matrix cores (a plan option).
//
// The 64-point DFT of pairs z_k, k = 8a + b, to frequencies m = c + 8d
// factors as Z_{c+8d} = sum_b W_64^{b(c+8d)} sum_a W_8^{ac} z_{8a+b}:
//   stage 1: for each b, an 8-point DFT over a: Y_b[c] = sum_a W_8^{ac}
//            z_{8a+b}, one v_mfma_f32_16x16x32_f16 per b over 16 vectors:
//            A = [F_hi | F_lo] (the real 16x16 form of the DFT, split into
//            fp16 halves), B = the exact fp16 pairs twice, so F z is exact
//            to about 2^-22;
//   stage 2: for each c, Z_{c+8d} = sum_b G_c[d][b] Y_b[c] with G_c =
//            W_64^{b(c+8d)} (twiddles and the 8-point DFT over b in one
//            matrix), four v_mfma_f32_16x16x4_f32 per c on the fp32 Y.
// Columns are 16 vectors; lane (v, r) = lane v + 16 r.  After stage 1 the
// lane holds Y_b[c] for c in {2r, 2r+1}; stage 2 needs, for each c, the
// values of every b, so Y passes through LDS (into the rows of the tile the
// group has just read) in two halves of c.  After stage 2 lane (v, r) holds
// Z_m for m = 16 r .. 16 r + 15 of vector v: output channels 32 r .. 32 r +
// 31, exactly one group of 32 (two of 16), so lambda, the abs-max, the scale
// and the codes are the lane's own work, and the lane's 16 code bytes are
// chunk r of row v: a group of 16 vectors stores 1 KiB of codes with one
// coalesced instruction.
// ---------------------------------------------------------------------------
typedef _Float16 mf_half8 __attribute__((ext_vector_type(8)));
typedef float mf_float4 __attribute__((ext_vector_type(4)));

// fp16 bits of a double below 65504 in magnitude, rounded to nearest even,
// subnormals kept (compile time).
constexpr uint32_t mf_f16_bits(double x) {
  if (x == 0.0) return 0u;
  const uint32_t sgn = x < 0 ? 0x8000u : 0u;
  double m = x < 0 ? -x : x;
  int e = 0;
  while (m >= 2.0) { m /= 2.0; ++e; }
  while (m < 1.0) { m *= 2.0; --e; }
  if (e < -14) {                           // subnormal: multiples of 2^-24
    double f = x < 0 ? -x : x;
    for (int i = 0; i < 24; ++i) f *= 2.0;
    uint32_t q = static_cast<uint32_t>(f);
    const double rem = f - q;
    if (rem > 0.5 || (rem == 0.5 && (q & 1u))) ++q;
    return sgn | q;                        // q = 1024 is the smallest normal
  }
  // m in [1, 2): 10 fraction bits, round half to even
  double f = (m - 1.0) * 1024.0;
  uint32_t q = static_cast<uint32_t>(f);
  const double rem = f - q;
  if (rem > 0.5 || (rem == 0.5 && (q & 1u))) ++q;
  if (q == 1024u) { q = 0; ++e; }
  return sgn | (static_cast<uint32_t>(e + 15) << 10) | q;
}

constexpr double mf_f16_value(uint32_t h) {
  if ((h & 0x7FFFu) == 0) return 0.0;
  if (((h >> 10) & 31u) == 0) {            // subnormal
    double v = (h & 1023u);
    for (int i = 0; i < 24; ++i) v /= 2.0;
    return (h & 0x8000u) ? -v : v;
  }
  const int e = static_cast<int>((h >> 10) & 31u) - 15;
  double v = 1.0 + (h & 1023u) / 1024.0;
  for (int i = 0; i < e; ++i) v *= 2.0;
  for (int i = 0; i > e; --i) v /= 2.0;
  return (h & 0x8000u) ? -v : v;
}

// Per-lane matrix operands of the two stages (lane l: row l % 16, k-slice
// l / 16), without the plan's signs: stage 1 as fp16 pairs, stage 2 as fp32.
struct MfTables {
  uint32_t a1[64][4];
  float a2[64][32];      // [c * 4 + kc]
};

constexpr MfTables make_mf_tables() {
  MfTables t{};
  // cos, sin (2 pi e / 64) rounded once to float, quarter turns exact
  constexpr TwTable tw = make_twiddles(64);
  for (int l = 0; l < 64; ++l) {
    const int rr = l & 15, r = l >> 4, eo = rr & 1, c = rr >> 1;
    // stage 1, row rr = 2 c + eo, k = 2 a + ei: [[cos, sin], [-sin, cos]]
    // of theta = 2 pi a c / 8; hi (r < 2) or lo (r >= 2) fp16 half
    for (int u = 0; u < 4; ++u) {
      uint32_t w = 0;
      for (int h = 0; h < 2; ++h) {
        const int k = 8 * (r & 1) + 2 * u + h, aa = k >> 1, ei = k & 1;
        // the table's fp32 value split into fp16 hi + lo: W_8^{ac} to about
        // 2^-22 (the fp32 rounding of the entry, 2^-24, is the larger error)
        const int e = 8 * ((aa * c) & 7);
        const double cs = tw.c[e], sn = tw.s[e];
        const double f = eo == 0 ? (ei == 0 ? cs : sn) : (ei == 0 ? -sn : cs);
        const uint32_t hi = mf_f16_bits(f);
        const uint32_t bits = r < 2 ? hi : mf_f16_bits(f - mf_f16_value(hi));
        w |= bits << (16 * h);
      }
      t.a1[l][u] = w;
    }
    // stage 2 for c, k = 4 kc + r <-> (b = 2 kc + r / 2, ei = r % 2), row
    // rr = 2 d + eo: W_64^{b (c + 8 d)} in real form
    for (int cc = 0; cc < 8; ++cc)
      for (int kc = 0; kc < 4; ++kc) {
        const int d = rr >> 1, b = 2 * kc + (r >> 1), ei = r & 1;
        const int e = (b * (cc + 8 * d)) & 63;
        const float cs = tw.c[e], sn = tw.s[e];
        t.a2[l][4 * cc + kc] = eo == 0 ? (ei == 0 ? cs : sn) : (ei == 0 ? -sn : cs);
      }
  }
  return t;
}

__constant__ MfTables kMfTab = make_mf_tables();

// LDS byte offset of 16-byte slot q (0..15) of the 256-byte staging row of
// vector v16 (one of the 16 vectors of a group), inside the group's 4 KiB:
// the slot index is XOR-swizzled with the row.
__device__ __forceinline__ uint32_t mf_slot(int v16, int q) {
  return static_cast<uint32_t>(v16 * 256 + ((q ^ v16) << 4));
}


// Quantize the lane's 32 channels w (one group of 32 or two of 16) with the
// reciprocal scales rr into code words cw (16 bytes int4, 32 bytes int8).
template <int FMT, bool CLAMP>
__device__ __forceinline__ void mf_quant(const float (&w)[32], const float (&rr)[2], uint32_t* cw) {
  using F = Fmt<FMT>;
#pragma unroll
  for (int q = 0; q < F::BITS; ++q) {
    uint32_t by[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (F::BITS == 4) {
        const int j = 8 * q + 2 * e;
        const float rg = rr[j / F::G];
        const uint32_t lo = CLAMP ? quant_bits(w[j], rg) : __builtin_bit_cast(uint32_t, fmaf(w[j], rg, kMagic));
        const uint32_t hi =
            CLAMP ? quant_bits(w[j + 1], rg) : __builtin_bit_cast(uint32_t, fmaf(w[j + 1], rg, kMagic));
        by[e] = pair_byte(lo, hi);
      } else {
        const int j = 4 * q + e;
        const float rg = rr[j / F::G];
        by[e] = CLAMP ? quant_bits8(w[j], rg) : __builtin_bit_cast(uint32_t, fmaf(w[j], rg, kMagic8));
      }
    }
    cw[q] = pack4(by[0], by[1], by[2], by[3]) ^ (F::BITS == 8 ? 0x80808080u : 0u);
  }
}

// The lambda row of a tile (512 bytes) by one direct load of 16 bytes per
// lane, into the LDS the caller passes (a plain pointer, as for the tile:
// the waits for both are explicit).
__device__ __forceinline__ void mf_dma_lambda(const CodecArgs& a, const Tile& t, uint8_t* lds, int lane) {
  const float* gl = a.lambda + t.b * a.lambda_sb + t.h * 128 + 4 * lane;
  if (lane < 32) __builtin_amdgcn_global_load_lds(gl, lds, 16, 0, 0);
}

// Eight 16-byte LDS reads of the lambda row (channels 32 r ..), issued and
// waited for in one assembly block: written as plain loads, the compiler
// would wait for every direct load in flight (it tracks the direct load that
// filled the row, not the group's own wait).
struct MfLam {
  float4 v[8];
};

__device__ __forceinline__ MfLam mf_read_lambda_blk(const float* lam_lds, int r) {
  typedef __attribute__((address_space(3))) const float lds_f;
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_f*)lam_lds)) + 128u * r;
  MfLam o;
  typedef float f4v __attribute__((ext_vector_type(4)));
  f4v x0, x1, x2, x3, x4, x5, x6, x7;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:16\n\t"
      "ds_read_b128 %2, %8 offset:32\n\t"
      "ds_read_b128 %3, %8 offset:48\n\t"
      "ds_read_b128 %4, %8 offset:64\n\t"
      "ds_read_b128 %5, %8 offset:80\n\t"
      "ds_read_b128 %6, %8 offset:96\n\t"
      "ds_read_b128 %7, %8 offset:112\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3), "=v"(x4), "=v"(x5), "=v"(x6), "=v"(x7)
      : "v"(addr)
      : "memory");
  const f4v xs[8] = {x0, x1, x2, x3, x4, x5, x6, x7};
#pragma unroll
  for (int i = 0; i < 8; ++i) o.v[i] = make_float4(xs[i][0], xs[i][1], xs[i][2], xs[i][3]);
  return o;
}

template <int MODE, int FMT>
__global__ void __launch_bounds__(64, 2) encode128_mfma_kernel(CodecArgs a) {
  using F = Fmt<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsTile];
  __shared__ __attribute__((aligned(16))) float lam_lds[128];
  const int lane = threadIdx.x;
  const int v16 = lane & 15;               // column: vector of the group
  const int r = lane >> 4;                 // row group / k-slice
  const int a0 = 4 * (r & 1);              // stage 1 reads pairs 8 a + b, a = a0 .. a0 + 3
  constexpr float kScale = 0.125f;         // 1 / sqrt(64): the transforms are unnormalized

  // stage 1 matrices, one per b: the table's halves with the sign of pair
  // 8 a + b (exact); this lane's a = a0 + u for dword u
  uint4 a1s;
  {
    const uint4* t1 = reinterpret_cast<const uint4*>(kMfTab.a1[lane]);
    a1s = *t1;
  }
  const uint32_t sw = static_cast<uint32_t>(a.signs[0] >> (32 * (r & 1)));   // bits 8 u + b
  mf_half8 A1[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    uint32_t d[4] = {a1s.x, a1s.y, a1s.z, a1s.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) d[u] ^= ((sw >> (8 * u + b)) & 1u) * 0x80008000u;
    A1[b] = __builtin_bit_cast(mf_half8, make_uint4(d[0], d[1], d[2], d[3]));
  }
  float A2[32];
  {
    const float4* t2 = reinterpret_cast<const float4*>(kMfTab.a2[lane]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 x = t2[i];
      A2[4 * i] = x.x; A2[4 * i + 1] = x.y; A2[4 * i + 2] = x.z; A2[4 * i + 3] = x.w;
    }
  }
  uint32_t off4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rw = 4 * i + (lane >> 4);
    off4[i] = static_cast<uint32_t>((lane >> 4) * 2 * a.st + 16 * ((lane & 15) ^ (rw & 15)));
  }

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const Tile t = tile_info<128>(a, tile);
    // lambda first, then the tile's rows: loads complete in issue order, so
    // group g (rows 16 g .., loads 4 g .. 4 g + 3) can start once all but the
    // 12 - 4 g youngest loads are back, while later groups still stream in.
    // Codes and scales are stored after the last group, so that no store
    // sits among the loads (a partial tile, whose loads are predicated, and
    // the rotate mode wait for everything instead).
    mf_dma_lambda(a, t, reinterpret_cast<uint8_t*>(lam_lds), lane);
    dma_tile128(a, t, lds, lane, off4);
    const bool staged = MODE == 0 && t.nv == 64;
    const int64_t cell0 = t.row * a.Tcap + a.t0 + t.t_start;   // wave-uniform
    uint4 out_c[4][F::BITS / 4];
    uint32_t out_s[4];

#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (16 * g >= t.nv) break;                      // wave-uniform
      asm volatile("" ::: "memory");                  // one group at a time
      if (!staged) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else if (g == 0) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      else if (g == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (g == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int v = 16 * g + v16;                     // vector of the tile
      uint8_t* stage = lds + 4096 * g;                // this group's rows, free after stage 1

      // ---- stage 1: 8-point DFTs over a, one MFMA per b; operand dword u
      // is pair 8 (a0 + u) + b of row v ----
      float Y[8][4];                                  // [b][(c = 2r re, im, c = 2r+1 re, im)]
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = 8 * (a0 + u) + b;
          w[u] = *reinterpret_cast<const uint32_t*>(lds + blk_off(v, k >> 2) + 4 * (k & 3));
        }
        const mf_half8 B1 = __builtin_bit_cast(mf_half8, make_uint4(w[0], w[1], w[2], w[3]));
        const mf_float4 y =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[b], B1, (mf_float4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Y[b][e] = y[e];
      }

      // ---- exchange: stage 2 for c needs Y_b[c] of every b, held by row
      // group c / 2.  Two halves of c (row groups 0-1, then 2-3) pass
      // through the group's 4 KiB (its rows, read above; a wave's LDS
      // operations run in order): row v16, 16-byte slot ((c / 2) % 2) * 8 + b
      // (XOR v16) holds Y_b[c], Y_b[c + 1] of the c pair ----
      float Z[8][4];                                  // [c][(d = 2r re, im, d = 2r+1 re, im)]
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if ((r >> 1) == h) {
#pragma unroll
          for (int b = 0; b < 8; ++b)
            *reinterpret_cast<float4*>(stage + mf_slot(v16, 8 * (r & 1) + b)) =
                make_float4(Y[b][0], Y[b][1], Y[b][2], Y[b][3]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // B of stage 2 for c, k-chunk kc: Y_b[c] component e, b = 2 kc + r / 2, e = r % 2
#pragma unroll
        for (int cl = 0; cl < 4; ++cl) {
          const int c = 4 * h + cl;
          float bq[4];
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) {
            const int b = 2 * kc + (r >> 1);
            bq[kc] = *reinterpret_cast<const float*>(stage + mf_slot(v16, 8 * (cl >> 1) + b) + 8 * (cl & 1) +
                                                     4 * (r & 1));
          }
          mf_float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A2[4 * c + kc], bq[kc], acc, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) Z[c][e] = acc[e];
        }
        // the next half's writes follow these reads in LDS order
      }

      // Z[c][2 dd + e] = Z_m, m = c + 8 (2 r + dd): output channel
      // j = 2 m + e = 32 r + 16 dd + 2 c + e; local index jl = j - 32 r
      const bool valid = v < t.nv;
      float w[32];
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int e = 0; e < 2; ++e) w[16 * dd + 2 * c + e] = Z[c][2 * dd + e];
      {
        // lambda of channels 32 r .. 32 r + 31, read in one block that waits
        // for its own reads (the direct load that filled the row has landed:
        // the group's wait above covers it)
        const MfLam l4 = mf_read_lambda_blk(lam_lds, r);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          w[4 * q] *= l4.v[q].x; w[4 * q + 1] *= l4.v[q].y; w[4 * q + 2] *= l4.v[q].z; w[4 * q + 3] *= l4.v[q].w;
        }
      }
      if (MODE == 1) {
        float* wr = a.w + ((t.row * a.T) + t.t_start + v) * 128 + 32 * r;
        if (valid) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            *reinterpret_cast<float4*>(wr + 4 * q) =
                make_float4(w[4 * q] * kScale, w[4 * q + 1] * kScale, w[4 * q + 2] * kScale, w[4 * q + 3] * kScale);
        }
        continue;
      }
      // ---- scale(s) and codes of the lane's 32 channels ----
      constexpr int NGL = 32 / F::G;                  // groups per lane: 1 or 2
      float rr[2] = {0.f, 0.f};
      uint32_t sc[2] = {0u, 0u};
      bool tiny = false;
#pragma unroll
      for (int gg = 0; gg < NGL; ++gg) {
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < F::G; ++j) amax = fmaxf(amax, fabsf(w[F::G * gg + j]));
        sc[gg] = f32_to_f16_bits(div_by<F::IQMAX>(amax * kScale));
        const float sf = f16_bits_to_f32(sc[gg]);
        rr[gg] = sf > 0.f ? kScale * __builtin_amdgcn_rcpf(sf) : 0.f;
        tiny |= (sc[gg] != 0u) && (sc[gg] < 0x0400u);
      }
      uint32_t cw[F::BITS];                           // 16 (int4) or 32 (int8) code bytes
      if (__builtin_amdgcn_ballot_w64(tiny && valid) == 0) mf_quant<FMT, false>(w, rr, cw);
      else mf_quant<FMT, true>(w, rr, cw);
#pragma unroll
      for (int q = 0; q < F::BITS / 4; ++q)
        out_c[g][q] = make_uint4(cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]);
      out_s[g] = sc[0] | (sc[1] << 16);
    }
    if (MODE == 0) {
      // codes: row v, bytes r * CB / 4 .. (1 KiB per group of 16 vectors, as
      // non-temporal stores: 2.5-4.5% faster than normal ones); scales:
      // entries v * NG + r * NGL ..
      constexpr int NGL = 32 / F::G;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int v = 16 * g + v16;
        if (v < t.nv) {
          char* cb = reinterpret_cast<char*>(a.codes + (cell0 + v) * F::CB) + r * (F::CB / 4);
#pragma unroll
          for (int q = 0; q < F::BITS / 4; ++q) st_stream16(cb + 16 * q, out_c[g][q]);
          uint16_t* sp = a.scales + (cell0 + v) * F::NG + r * NGL;
          if (NGL == 1) *sp = static_cast<uint16_t>(out_s[g]);
          else *reinterpret_cast<uint32_t*>(sp) = out_s[g];
        }
      }
    }
    // the tile's rows served as staging: every LDS access of this tile is
    // done before the next tile's direct loads write them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// ---------------------------------------------------------------------------
// D = 256 encode: a lane pair per vector, 32 vectors (16 KiB) per tile in the
// D = 128 tile layout with rows = half vectors (row 2v + h = channels
// 128h .. 128h + 127 of vector v).  SRFT by decimation in time: lane 2v + h
// takes the complex pairs 2k + h (k < 64), transforms them with the 64-point
// FFT, the odd lane multiplies by W_128^m (by -W_128^m for m >= 33, a
// rotation within pi/2, done by shears in place), and one butterfly across
// the pair leaves Z_m on lane 0 and Z_{m+64} on lane 1.  SRHT (Sylvester H_256 =
// H_2 (x) H_128 on the top index bit): the butterfly across the pair comes
// first (x_lo + x_hi, x_lo - x_hi), then H_128 in each lane.  Either way a
// lane ends with a contiguous half of the output channels and quantizes it
// like a D = 128 vector.  The butterfly computes own + sign * partner (the
// sign negated on the pairs whose twiddle took the opposite angle), which
// on the odd lane is the negated value except on those pairs; the sign is
// folded into that lane's half of the lambda table.
// ---------------------------------------------------------------------------
// Chunk swizzle of row r of a D=256 tile.  The SRFT lanes read one row per
// lane pair (rows 2v + R of every v at once): the swizzle by bits 1-4 of the
// row spreads those 32 rows over all 16 chunk columns, so each half-wave's
// dword reads hit distinct banks.  The SRHT and unrotated lanes read
// consecutive rows, which the swizzle by bits 0-3 spreads.
template <int ROT>
__device__ __forceinline__ int swz256(int r) {
  return ROT == KVQ_ROT_SRFT ? (r >> 1) & 15 : r & 15;
}

// Slot i * 64 + lane of the LDS tile receives row r = 4 i + lane / 16
// (vector r / 2, half r % 2), chunk (lane % 16) ^ swz256(r).  The lane's
// source offsets repeat every eight loads; they are recomputed per call from
// a laundered lane index (held across the transform they would spill).
template <int ROT>
__device__ __forceinline__ void dma_tile256(const CodecArgs& a, const Tile& t, lds_u8* lds, int lane) {
  asm volatile("" : "+v"(lane));
  uint32_t off8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    off8[i] = static_cast<uint32_t>((lane >> 5) * 2 * a.st + ((lane >> 4) & 1) * 256 +
                                    16 * ((lane & 15) ^ swz256<ROT>(r)));
  }
  const char* base = reinterpret_cast<const char*>(a.x + t.b * a.sb + t.h * a.sh + t.t_start * a.st);
  const int64_t step = 4 * a.st;        // bytes of two vectors (four rows)
  if (t.nv == 32) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_global_load_lds(base + i * step + off8[i & 7], lds + 1024 * i, 16, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (2 * i + (lane >> 5) < t.nv)
        __builtin_amdgcn_global_load_lds(base + i * step + off8[i & 7], lds + 1024 * i, 16, 0, 0);
  }
}

// Sign mask of local pair k of lane half h: SRFT pair 2k + h (decimation in
// time), SRHT channels 128h + 2k, 128h + 2k + 1.
template <int ROT>
__device__ __forceinline__ uint32_t pair_mask256(const CodecArgs& a, int h, int k) {
  if (ROT == KVQ_ROT_SRFT) {
    const int P = 2 * k + h;
    return ((a.signs[P >> 6] >> (P & 63)) & 1u) ? 0x80008000u : 0u;
  }
  if (ROT == KVQ_ROT_SRHT) {
    const int c = 128 * h + 2 * k;
    const uint64_t w = a.signs[c >> 6];
    const int i = c & 63;
    return (static_cast<uint32_t>((w >> i) & 1u) << 15) | (static_cast<uint32_t>((w >> (i + 1)) & 1u) << 31);
  }
  return 0u;
}

// Sign folded into lambda of channel c: the pair step leaves the odd lane's
// half (channels 128 ..) negated, except, with SRFT, the pairs of
// frequencies m + 64, m >= 33 (channels 194 ..), whose twiddles took the
// opposite angle.
template <int ROT>
__host__ __device__ constexpr float lam_sign256(int c) {
  if (ROT == KVQ_ROT_ID || c < 128) return 1.f;
  return (ROT == KVQ_ROT_SRFT && c >= 128 + 2 * 33) ? 1.f : -1.f;
}

// Word offsets of the second half's sign masks and lambda row in LDS: one
// 16-byte chunk past a whole number of bank rows.
constexpr int kMaskH256 = 64 + 4;
constexpr int kLamH256 = 128 + 4;

// MODE 0 writes codes and scales; MODE 1 writes the rotated values w =
// lambda * R x in fp32 (the transform of this kernel, for checking).
template <int ROT, int MODE, int FMT, bool ONE>
__global__ void __launch_bounds__(64, 2) encode256_kernel(CodecArgs a) {
  using F = Fmt<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsTile];
  // [h][k] and [h][local channel] (sign folded); half 1 starts kMaskH256 /
  // kLamH256 words in, so the two halves' 16-byte reads at the same
  // position fall on different banks
  __shared__ __attribute__((aligned(16))) uint32_t mask_lds[kMaskH256 + 64];
  __shared__ __attribute__((aligned(16))) float lam_lds[kLamH256 + 128];
  const int lane = threadIdx.x;
  const int hh = lane & 1;                  // half of the vector
  constexpr float kScale = rot_scale<256, ROT>();
  const float sgn = hh ? -1.f : 1.f;
  // the butterfly across the pair leaves the odd lane's half negated
  // (rotations only); its lambda half carries the sign back
  constexpr bool kPair = ROT != KVQ_ROT_ID;

  mask_lds[lane] = pair_mask256<ROT>(a, 0, lane);
  mask_lds[kMaskH256 + lane] = pair_mask256<ROT>(a, 1, lane);
  // lambda of a tile: lane l holds channels l, l + 64, l + 128, l + 192
  float lam_r[4] = {0.f, 0.f, 0.f, 0.f};
  int64_t tile = blockIdx.x;
  if (tile < a.n_tiles) {
    const Tile t = tile_info<256>(a, tile);
    dma_tile256<ROT>(a, t, (lds_u8*)lds, lane);
    const float* lr = a.lambda + t.b * a.lambda_sb + t.h * 256;
#pragma unroll
    for (int q = 0; q < 4; ++q) lam_r[q] = lr[lane + 64 * q];
  }
  __syncthreads();
  uint4 pend_c[F::CB / 16] = {};
  uint32_t pend_s[F::NG / 2] = {};
  bool pend_valid = false;
  char* pend_cbase = nullptr;
  char* pend_sbase = nullptr;
  for (; tile < a.n_tiles; tile += gridDim.x) {
    const Tile t = tile_info<256>(a, tile);
    // the tile's direct loads have landed in LDS (everything issued after
    // them is a store of the tile before, a transform ago)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int q = 0; q < 4; ++q)
      lam_lds[lane + 64 * q + (q >= 2 ? kLamH256 - 128 : 0)] = lam_sign256<ROT>(lane + 64 * q) * lam_r[q];
    uint32_t p[64];
    const uint4* masks = reinterpret_cast<const uint4*>(mask_lds + kMaskH256 * hh);   // [j]
    if (ROT == KVQ_ROT_SRFT) {
      // pairs 2k + hh: rows 2v (k < 32) and 2v + 1, two dwords per 16-byte chunk
      const int v2 = lane & ~1;
#pragma unroll
      for (int R = 0; R < 2; ++R) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const int r = v2 + R;
          const uint32_t w0 = ((r * 256 + ((c ^ swz256<ROT>(r)) << 4)) >> 2) + hh;
          p[32 * R + 2 * c] = reinterpret_cast<const uint32_t*>(lds)[w0];
          p[32 * R + 2 * c + 1] = reinterpret_cast<const uint32_t*>(lds)[w0 + 2];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint4 w = *reinterpret_cast<const uint4*>(lds + blk_off(lane, j));
        p[4 * j] = w.x; p[4 * j + 1] = w.y; p[4 * j + 2] = w.z; p[4 * j + 3] = w.w;
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 m = masks[j];
      p[4 * j] ^= m.x; p[4 * j + 1] ^= m.y; p[4 * j + 2] ^= m.z; p[4 * j + 3] ^= m.w;
    }
    // the tile is in registers: the buffer takes the next one
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t nxt = tile + gridDim.x;
    if (!ONE && nxt < a.n_tiles) {
      const Tile tn = tile_info<256>(a, nxt);
      dma_tile256<ROT>(a, tn, (lds_u8*)lds, lane);
      const float* lr = a.lambda + tn.b * a.lambda_sb + tn.h * 256;
#pragma unroll
      for (int q = 0; q < 4; ++q) lam_r[q] = lr[lane + 64 * q];
    }
    if (MODE == 0 && !ONE && pend_valid) store_lane_codes<F>(pend_cbase, pend_sbase, lane, pend_c, pend_s);

    float v[128];
    if (ROT == KVQ_ROT_SRFT) {
      rotate_packed<KVQ_ROT_SRFT>(p, v);
      if (hh) pair_twiddles_srft<false>(v);
      pair_fma_all_srft(v, sgn);
    } else {
#pragma unroll
      for (int k = 0; k < 64; ++k) {
        v[2 * k] = f16_bits_to_f32(p[k] & 0xFFFFu);
        v[2 * k + 1] = f16_bits_to_f32(p[k] >> 16);
      }
      if (kPair) {
        pair_fma_all(v, sgn);
      }
      if (ROT == KVQ_ROT_SRHT) wht128(v);
    }
    // keep the lambda reads below the transform
    asm volatile("" ::: "memory");
    const float4* lam4 = reinterpret_cast<const float4*>(lam_lds + kLamH256 * hh);   // [j / 4]
    const bool valid = (lane >> 1) < t.nv;

    if (MODE == 1) {
      // lane 2v + h: channels 128 h .. 128 h + 127 of vector v
      float* wr = a.w + ((t.row * a.T) + t.t_start + (lane >> 1)) * 256 + 128 * hh;
      if (valid) {
#pragma unroll
        for (int j = 0; j < 128; j += 4) {
          const float4 l4 = lam4[j / 4];
          float4 o;
          o.x = v[chan_reg<ROT>(j)] * l4.x * kScale;
          o.y = v[chan_reg<ROT>(j + 1)] * l4.y * kScale;
          o.z = v[chan_reg<ROT>(j + 2)] * l4.z * kScale;
          o.w = v[chan_reg<ROT>(j + 3)] * l4.w * kScale;
          *reinterpret_cast<float4*>(wr + j) = o;
        }
      }
      continue;
    }

    float r[F::NG];
    uint32_t sc[F::NG];
    bool tiny = false;
#pragma unroll
    for (int g = 0; g < F::NG; ++g) {
      asm volatile("" ::: "memory");
      float amax = 0.f;
#pragma unroll
      for (int jj = 0; jj < F::G; jj += 4) {
        const int j = F::G * g + jj;
        const float4 l4 = lam4[j / 4];
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float wv = v[chan_reg<ROT>(j + e)] * lv[e];
          v[chan_reg<ROT>(j + e)] = wv;
          amax = fmaxf(amax, fabsf(wv));
        }
      }
      sc[g] = f32_to_f16_bits(div_by<F::IQMAX>(amax * kScale));
      const float sf = f16_bits_to_f32(sc[g]);
      r[g] = sf > 0.f ? kScale * __builtin_amdgcn_rcpf(sf) : 0.f;
      tiny |= (sc[g] != 0u) && (sc[g] < 0x0400u);
    }
    uint32_t cw[F::CW];
    constexpr int kWordsPerGroup = F::CW / F::NG;
    if (__builtin_amdgcn_ballot_w64(tiny && valid) == 0) {
#pragma unroll
      for (int g = 0; g < F::NG; ++g) quant_group<ROT, false, FMT>(v, g, r[g], cw + kWordsPerGroup * g);
    } else {
#pragma unroll
      for (int g = 0; g < F::NG; ++g) quant_group<ROT, true, FMT>(v, g, r[g], cw + kWordsPerGroup * g);
    }
    // lane 2v + h: the code and scale bytes of half h of vector v, i.e. CB
    // and SB contiguous bytes at lane * CB, lane * SB
    const int64_t cell0 = t.row * a.Tcap + a.t0 + t.t_start;   // wave-uniform
    pend_sbase = reinterpret_cast<char*>(a.scales + cell0 * 2 * F::NG);
    pend_cbase = reinterpret_cast<char*>(a.codes + cell0 * 2 * F::CB);
#pragma unroll
    for (int i = 0; i < F::NG / 2; ++i) pend_s[i] = sc[2 * i] | (sc[2 * i + 1] << 16);
#pragma unroll
    for (int q = 0; q < F::CB / 16; ++q)
      pend_c[q] = make_uint4(cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]);
    pend_valid = valid;
    if (ONE) {
      // the half-vector code rows (row = lane) leave through the free tile
      // buffer as 1 KiB non-temporal stores (against per-lane int4 rows and
      // normal staged int8 rows: SRFT / SRHT encode 4.5%, int8 5.9%, groups
      // of 16 14% faster, codes bit-identical)
      store_codes_staged<F, true>(pend_cbase, pend_sbase, lane, 2 * t.nv, lds, pend_c, pend_s);
      pend_valid = false;
    }
  }
  if (MODE == 0 && !ONE && pend_valid) store_lane_codes<F>(pend_cbase, pend_sbase, lane, pend_c, pend_s);
}

// ---------------------------------------------------------------------------
// D = 128 decode to fp16: codes, scales and the lambda row of the next tile
// arrive in LDS by direct loads while the current tile computes; the fp16
// rows leave through a 9 KiB LDS stage, one half-row (64 channels) at a time.
// ---------------------------------------------------------------------------
// Direct-load targets (one LDS object): 64 code rows of F::CB bytes
// (swizzled), their scales (F::SB each) and the lambda row ...
template <typename F>
struct DecIn {
  static constexpr int kCodes = 0;
  static constexpr int kScales = 64 * F::CB;
  static constexpr int kLam = kScales + 64 * F::SB;
  static constexpr int kBytes = kLam + 512;
};
// ... and the LDS the compute phase uses (another object, so that its reads
// need not wait for the direct loads in flight)
constexpr int kDecRl = 0;                // 512 B: unitary scale / lambda
constexpr int kDecOut = 512;             // 9 KiB: half rows of 128 B at a 144 B pitch
constexpr int kDecPitch = 144;           // 16 B of padding: conflict-free both ways
constexpr int kLdsDecWork = kDecOut + 64 * kDecPitch;

// LDS byte offset of 16-byte chunk q of the code row of lane r: rows of 4
// chunks (int4) or 8 chunks (int8), the chunk index XOR-swizzled with the
// row so that a lane-parallel read of one chunk spreads over the banks.
template <typename F>
__device__ __forceinline__ uint32_t code_off_f(int r, int q) {
  if (F::CB == 64) return code_off(r, q);
  return static_cast<uint32_t>(r * 128 + (((q ^ r) & 7) << 4));
}

template <typename F>
__device__ __forceinline__ void dma_codes128(const CodecArgs& a, const Tile& t, lds_u8* lds, int lane) {
  using L = DecIn<F>;
  const int64_t cell0 = t.row * a.Tcap + a.t0 + t.t_start;
  const char* cb = reinterpret_cast<const char*>(a.codes_in + cell0 * F::CB);
  const char* sb = reinterpret_cast<const char*>(a.scales_in + cell0 * F::NG);
  constexpr int kRowsPerLoad = 1024 / F::CB;       // code rows per 64-lane load
  constexpr int kChunks = F::CB / 16;
  // (every pointer goes through a local first: inside a template the
  // direct-load builtin rejects value-dependent pointer expressions)
  // slot 64 i + lane holds chunk q of vector v, at code_off_f(v, q)
#pragma unroll
  for (int i = 0; i < 64 / kRowsPerLoad; ++i) {
    const int v = kRowsPerLoad * i + lane / kChunks;
    const int p = lane % kChunks;                  // position in the LDS row
    const int q = F::CB == 64 ? p ^ ((v >> 2) & 3) : (p ^ v) & 7;
    const char* g = cb + static_cast<uint32_t>(F::CB * v + 16 * q);
    lds_u8* l = lds + L::kCodes + 1024 * i;
    if (v < t.nv) __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
  }
  if (F::SB == 8) {
    // scales: one dword (two scales) per lane and instruction
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const char* g = sb + static_cast<uint32_t>(256 * i + 4 * lane);
      lds_u8* l = lds + L::kScales + 256 * i;
      if (32 * i + (lane >> 1) < t.nv) __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
    }
  } else {
    // 16 bytes of scales per vector, one vector per lane
    const char* g = sb + static_cast<uint32_t>(16 * lane);
    lds_u8* l = lds + L::kScales;
    if (lane < t.nv) __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
  }
  const float* gl = a.lambda + t.b * a.lambda_sb + t.h * 128 + 4 * lane;
  lds_u8* ll = lds + L::kLam;
  if (lane < 32) __builtin_amdgcn_global_load_lds(gl, ll, 16, 0, 0);
}

// The kernels of this file run one wave per workgroup, and a wave's LDS
// operations complete in order: lanes see each other's LDS writes once the
// wave's own LDS counter drains.  (A workgroup barrier would also wait for
// the vector-memory counter, i.e. for the next tile's direct loads.)
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// code * scale * rl for the lane's 128 channels.  cw holds the lane's code
// words, whose channels are v[8d ..] (int4: byte b of word d holds v[8d+2b]
// low and v[8d+2b+1] high; the word is unpacked as channel pairs (0,4),
// (1,5), (2,6), (3,7)) or v[4d ..] (int8: byte e of word d is v[4d+e]); runs
// of DPG consecutive words share one scale, s16[d / DPG]; rl4 (LDS) holds the
// per-channel factor (unitary scale / lambda) of v[j] at float j.
//   int4: (n - 8) * scale exactly: the nibble under the exponent of 1024 is
//         the fp16 number 1024 + n (low nibble of a byte) or 1024 + 16 n
//         (high nibble); one fma_mix removes the bias.
//   int8: the byte with its top bit flipped is q + 128 (v_cvt_f32_ubyte),
//         one fma removes the bias.
template <typename F, int DPG, typename Words>
__device__ __forceinline__ void dequant_lane(const Words& cw, const uint32_t* s16, const float4* rl4,
                                             uint32_t magic, float (&v)[128]) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int g = 0; g < F::CW / DPG; ++g) {
    // one group's rl reads at a time (hoisted, they would hold 128 registers)
    asm volatile("" ::: "memory");
    const float sg = f16_bits_to_f32(s16[g]);
    if (F::BITS == 4) {
      const float m_lo = -1032.f * sg;
      const float sg16 = sg * 0.0625f;
      const float m_hi = -72.f * sg;       // -1152 * sg / 16
#pragma unroll
      for (int k = 0; k < DPG; ++k) {
        const int d = DPG * g + k;
        const uint32_t x = cw[d], y = x >> 8;
        const h2_t h0 = __builtin_bit_cast(h2_t, (x & 0x000F000Fu) | magic);   // channels 0, 4
        const h2_t h1 = __builtin_bit_cast(h2_t, (x & 0x00F000F0u) | magic);   // channels 1, 5
        const h2_t h2 = __builtin_bit_cast(h2_t, (y & 0x000F000Fu) | magic);   // channels 2, 6
        const h2_t h3 = __builtin_bit_cast(h2_t, (y & 0x00F000F0u) | magic);   // channels 3, 7
        const int j = 8 * d;
        const float4 ra = rl4[2 * d], rb = rl4[2 * d + 1];
        v[j] = fmaf(static_cast<float>(h0[0]), sg, m_lo) * ra.x;
        v[j + 1] = fmaf(static_cast<float>(h1[0]), sg16, m_hi) * ra.y;
        v[j + 2] = fmaf(static_cast<float>(h2[0]), sg, m_lo) * ra.z;
        v[j + 3] = fmaf(static_cast<float>(h3[0]), sg16, m_hi) * ra.w;
        v[j + 4] = fmaf(static_cast<float>(h0[1]), sg, m_lo) * rb.x;
        v[j + 5] = fmaf(static_cast<float>(h1[1]), sg16, m_hi) * rb.y;
        v[j + 6] = fmaf(static_cast<float>(h2[1]), sg, m_lo) * rb.z;
        v[j + 7] = fmaf(static_cast<float>(h3[1]), sg16, m_hi) * rb.w;
      }
    } else {
      const float m = -128.f * sg;
#pragma unroll
      for (int k = 0; k < DPG; ++k) {
        const int d = DPG * g + k;
        const uint32_t x = cw[d] ^ 0x80808080u;
        const float4 ra = rl4[d];
        v[4 * d] = fmaf(static_cast<float>(x & 0xFFu), sg, m) * ra.x;
        v[4 * d + 1] = fmaf(static_cast<float>((x >> 8) & 0xFFu), sg, m) * ra.y;
        v[4 * d + 2] = fmaf(static_cast<float>((x >> 16) & 0xFFu), sg, m) * ra.z;
        v[4 * d + 3] = fmaf(static_cast<float>(x >> 24), sg, m) * ra.w;
      }
    }
  }
}

// A lane's code words, read from the tile's LDS rows as they are used (the
// decoders with a wave per tile: the buffer takes no next tile, and the
// words need not all be held in registers at once).
template <typename F>
struct LdsWords {
  const uint8_t* base;
  int lane;
  __device__ __forceinline__ uint32_t operator[](int d) const {
    const uint4 w = *reinterpret_cast<const uint4*>(base + code_off_f<F>(lane, d / 4));
    return (d % 4) == 0 ? w.x : (d % 4) == 1 ? w.y : (d % 4) == 2 ? w.z : w.w;
  }
};

// ONE: the grid has a wave per tile (no prefetch; codes read from LDS as
// the dequantization uses them).
template <int ROT, int FMT, bool ONE>
__global__ void __launch_bounds__(64, 2) decode128_kernel(CodecArgs a) {
  using F = Fmt<FMT>;
  using L = DecIn<F>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t work[kLdsDecWork];
  const int lane = threadIdx.x;
  constexpr float kScale = rot_scale<128, ROT>();
  uint32_t magic;   // fp16 pair (1024, 1024): a register operand for v_and_or
  asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  const uint32_t out_lane = static_cast<uint32_t>((lane >> 3) * 2 * a.st + 16 * (lane & 7));
  const int64_t out_step = 16 * a.st;     // bytes of eight rows

  int64_t tile = blockIdx.x;
  if (tile < a.n_tiles) dma_codes128<F>(a, tile_info<128>(a, tile), (lds_u8*)lds, lane);
  __syncthreads();
  for (; tile < a.n_tiles; tile += gridDim.x) {
    const Tile t = tile_info<128>(a, tile);
    uint32_t cw[ONE ? 1 : F::CW];
    if (!ONE) {
#pragma unroll
      for (int q = 0; q < F::CB / 16; ++q) {
        const uint4 w = *reinterpret_cast<const uint4*>(lds + L::kCodes + code_off_f<F>(lane, q));
        cw[4 * q] = w.x; cw[4 * q + 1] = w.y; cw[4 * q + 2] = w.z; cw[4 * q + 3] = w.w;
      }
    }
    uint32_t s16[F::NG];
    if (F::SB == 8) {
      const uint2 s2 = *reinterpret_cast<const uint2*>(lds + L::kScales + 8 * lane);
      const uint32_t sw[2] = {s2.x, s2.y};
#pragma unroll
      for (int i = 0; i < F::NG; ++i) s16[i] = (sw[(i / 2) % 2] >> (16 * (i % 2))) & 0xFFFFu;
    } else {
      const uint4 s4 = *reinterpret_cast<const uint4*>(lds + L::kScales + 16 * lane);
      const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int i = 0; i < F::NG; ++i) s16[i] = (sw[(i / 2) % 4] >> (16 * (i % 2))) & 0xFFFFu;
    }
    const float l0 = reinterpret_cast<const float*>(lds + L::kLam)[lane];
    const float l1 = reinterpret_cast<const float*>(lds + L::kLam)[lane + 64];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t nxt = tile + gridDim.x;
    if (!ONE && nxt < a.n_tiles) dma_codes128<F>(a, tile_info<128>(a, nxt), (lds_u8*)lds, lane);
    reinterpret_cast<float*>(work + kDecRl)[lane] = kScale * __builtin_amdgcn_rcpf(l0);
    reinterpret_cast<float*>(work + kDecRl)[lane + 64] = kScale * __builtin_amdgcn_rcpf(l1);
    lds_sync();

    float v[128];
    if (ONE) {
      const LdsWords<F> words{lds + L::kCodes, lane};
      dequant_lane<F, F::CW / F::NG>(words, s16, reinterpret_cast<const float4*>(work + kDecRl), magic, v);
    } else {
      dequant_lane<F, F::CW / F::NG>(cw, s16, reinterpret_cast<const float4*>(work + kDecRl), magic, v);
    }

    if (ROT == KVQ_ROT_SRFT) fft64<true>(v);
    else if (ROT == KVQ_ROT_SRHT) wht128(v);
    // the next tile's direct loads (the only vector-memory operations issued
    // since the last stores) have had the dequantization and the transform
    // to land; waiting here rather than at the top of the loop keeps this
    // tile's stores out of the wait
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const char* ybase = reinterpret_cast<const char*>(static_cast<uint16_t*>(a.y) + t.b * a.sb + t.h * a.sh +
                                                      t.t_start * a.st);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // the lane's 32 pairs of this half: chunk c (pairs 4c..4c+3) of row
      // `lane` at lane * 144 + 16 c
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 32 * hf + 4 * c + e;
          const int pp = ROT == KVQ_ROT_SRFT ? rev4(k) : k;
          wv[e] = pack_f16x2(v[2 * pp], v[2 * pp + 1]);
        }
        *reinterpret_cast<uint4*>(work + kDecOut + lane * kDecPitch + 16 * c) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
      lds_sync();
      // signs of the 16-byte chunk this lane stores (pairs 32 hf + 4 (lane % 8) ..)
      const int k0 = 32 * hf + 4 * (lane & 7);
      const uint4 mk = make_uint4(pair_mask128<ROT>(a, k0), pair_mask128<ROT>(a, k0 + 1),
                                  pair_mask128<ROT>(a, k0 + 2), pair_mask128<ROT>(a, k0 + 3));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * i + (lane >> 3), c = lane & 7;
        uint4 w = *reinterpret_cast<const uint4*>(work + kDecOut + r * kDecPitch + 16 * c);
        w.x ^= mk.x; w.y ^= mk.y; w.z ^= mk.z; w.w ^= mk.w;
        if (r < t.nv) st_stream16(const_cast<char*>(ybase) + i * out_step + hf * 128 + out_lane, w);
      }
      lds_sync();
    }
  }
}

// ---------------------------------------------------------------------------
// D = 256 decode to fp16: a lane pair per vector, 32 vectors per tile, the
// same direct-load / staging scheme as D = 128 with rows = half vectors.
// SRFT by decimation in time: lane 2v + h gathers the code bytes of the odd
// or even frequencies (Z_{2m+h}, one byte perm per two code dwords), runs the
// inverse 64-point FFT, the odd lane multiplies by conj(W_128^k), and one
// butterfly across the pair leaves z_k on lane 0 and z_{k+64} on lane 1: a
// contiguous half of the output row per lane.  SRHT: the butterfly across
// the pair comes first, then H_128 in each lane (H_256 = H_2 (x) H_128).  The
// butterfly computes own + sign * partner; the odd lane's half of the
// 1 / lambda table is negated so that both lanes end with the plain result.
// ---------------------------------------------------------------------------
// Direct-load targets: 32 code rows of 2 F::CB bytes (R = F::CB / 8 chunks
// of 16 bytes; chunk q of vector v at LDS byte 2 CB v + 16 ((q ^ v) % R), so
// that a lane-parallel read of one chunk of consecutive rows spans the
// banks), their scales (2 F::SB bytes each) and the 1 KiB lambda row; the
// compute side's 1/lambda table and output stage.
template <typename F>
struct DecIn256 {
  static constexpr int kCodes = 0;
  static constexpr int kScales = 64 * F::CB;
  static constexpr int kLam = kScales + 64 * F::SB;
  static constexpr int kBytes = kLam + 1024;
};
constexpr int kDec2Rl = 0;               // 1 KiB: [h][local channel] unitary scale / lambda
constexpr int kDec2Out = 1024;           // 9 KiB staging, rows = half vectors
constexpr int kLdsDec2Work = kDec2Out + 64 * kDecPitch;

template <typename F>
__device__ __forceinline__ void dma_codes256(const CodecArgs& a, const Tile& t, lds_u8* lds, int lane_in) {
  using L = DecIn256<F>;
  // the lane's offsets are recomputed per call (a few integer operations):
  // hoisted out of the tile loop they would hold registers the transform
  // needs, and their spill reloads would wait on the loads just issued
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int64_t cell0 = t.row * a.Tcap + a.t0 + t.t_start;
  const char* cb = reinterpret_cast<const char*>(a.codes_in + cell0 * 2 * F::CB);
  const char* sb = reinterpret_cast<const char*>(a.scales_in + cell0 * 2 * F::NG);
  const uint32_t off16 = static_cast<uint32_t>(16 * lane);
  // (every pointer goes through a local first: inside a template the
  // direct-load builtin rejects value-dependent pointer expressions)
  lds_u8* l = lds + L::kCodes;
  if (F::CB == 64) {
    // slot 64 i + lane: row 8 i + lane / 8, LDS position lane % 8; the lane's
    // global offset is the same for every i, and the instruction offset
    // (1 KiB per slot row) advances the global and the LDS address alike
    const uint32_t off = static_cast<uint32_t>(128 * (lane >> 3) + 16 * ((lane & 7) ^ ((lane >> 3) & 7)));
    const char* g = cb + off;
    if (t.nv == 32) {
      __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(g, l, 16, 1024, 0);
      __builtin_amdgcn_global_load_lds(g, l, 16, 2048, 0);
      __builtin_amdgcn_global_load_lds(g, l, 16, 3072, 0);
    } else {
      // vector 8 i + lane / 8: one lane value against a wave-uniform bound
      const int r = lane >> 3;
      if (r < t.nv) __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
      if (r < t.nv - 8) __builtin_amdgcn_global_load_lds(g, l, 16, 1024, 0);
      if (r < t.nv - 16) __builtin_amdgcn_global_load_lds(g, l, 16, 2048, 0);
      if (r < t.nv - 24) __builtin_amdgcn_global_load_lds(g, l, 16, 3072, 0);
    }
  } else {
    // 256-byte rows: slot 64 i + lane is row 4 i + lane / 16, LDS position
    // lane % 16, global chunk (lane % 16) ^ row (mod 16)
    const int vr = lane >> 4, p = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = static_cast<uint32_t>(256 * vr + 16 * ((p ^ (4 * i + vr)) & 15));
      const char* g = cb + 1024 * i + off;
      lds_u8* li = l + 1024 * i;
      if (vr < t.nv - 4 * i) __builtin_amdgcn_global_load_lds(g, li, 16, 0, 0);
    }
  }
  // 2 F::SB bytes of scales per vector: 16 per lane
  const char* gs = sb + off16;
  lds_u8* ls = lds + L::kScales;
  if (lane < t.nv * (2 * F::SB / 16)) __builtin_amdgcn_global_load_lds(gs, ls, 16, 0, 0);
  const char* gl = reinterpret_cast<const char*>(a.lambda + t.b * a.lambda_sb + t.h * 256) + off16;
  lds_u8* ll = lds + L::kLam;
  __builtin_amdgcn_global_load_lds(gl, ll, 16, 0, 0);
}

__device__ __forceinline__ uint64_t sign_word(const CodecArgs& a, int i) {
  return i == 0 ? a.signs[0] : i == 1 ? a.signs[1] : i == 2 ? a.signs[2] : a.signs[3];
}

// Sign mask of output pair kg (channels 2 kg, 2 kg + 1) of a D = 256 vector.
template <int ROT>
__device__ __forceinline__ uint32_t out_mask256(const CodecArgs& a, int kg) {
  if (ROT == KVQ_ROT_SRFT) {
    // the odd lane's pairs 64 + k, k >= 33, leave the pair step negated
    const uint32_t flip = kg >= 64 + 33 ? 0x80008000u : 0u;
    return (((sign_word(a, kg >> 6) >> (kg & 63)) & 1u) ? 0x80008000u : 0u) ^ flip;
  }
  if (ROT == KVQ_ROT_SRHT) {
    const uint64_t w = sign_word(a, kg >> 5);
    const int i = (2 * kg) & 63;
    return (static_cast<uint32_t>((w >> i) & 1u) << 15) | (static_cast<uint32_t>((w >> (i + 1)) & 1u) << 31);
  }
  return 0u;
}

template <int ROT, int FMT>
__global__ void __launch_bounds__(64, 2) decode256_kernel(CodecArgs a) {
  using F = Fmt<FMT>;
  using L = DecIn256<F>;
  constexpr int R = F::CB / 8;              // 16-byte chunks per code row
  // SRFT lanes see every scale of their vector, through code words of DPG
  // words per group (int4: 4 frequencies = 8 channels in 4 code bytes per
  // word; int8: 2 frequencies per word); the others their half's scales
  constexpr int DPG = ROT == KVQ_ROT_SRFT ? F::G * F::BITS / 64 : F::CW / F::NG;
  constexpr int NS = F::CW / DPG;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t work[kLdsDec2Work];
  const int lane = threadIdx.x;
  const int hh = lane & 1;                  // half of the vector
  const int vec = lane >> 1;
  constexpr float kScale = rot_scale<256, ROT>();
  constexpr bool kPair = ROT != KVQ_ROT_ID;
  const float sgn = hh ? 1.f : -1.f;
  uint32_t magic;   // fp16 pair (1024, 1024): a register operand for v_and_or
  asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));
  // int4: bytes h, h + 2 of two code dwords (frequencies 2m + h); int8:
  // half-word h of two code dwords (both bytes of frequency 2m + h)
  const uint32_t sel = F::BITS == 4 ? 0x06040200u + 0x01010101u * static_cast<uint32_t>(hh)
                                    : 0x05040100u + 0x02020202u * static_cast<uint32_t>(hh);

  // where this lane's lambda entries c = lane + 64 q go in the 1 / lambda
  // table, and their sign (negated on the odd half)
  uint32_t rl_dst[4];
  float rl_mul[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = lane + 64 * q;
    int h, j;
    if (ROT == KVQ_ROT_SRFT) { h = (c >> 1) & 1; j = 2 * (c >> 2) + (c & 1); }
    else { h = c >> 7; j = c & 127; }
    rl_dst[q] = static_cast<uint32_t>(4 * (128 * h + j));
    rl_mul[q] = (kPair && h) ? -kScale : kScale;
  }

  // rows 8 i + lane / 8 of a half-row pass: vector 4 i + lane / 16, half
  // (lane / 8) % 2, 16-byte chunk lane % 8
  const uint32_t out_lane = static_cast<uint32_t>((lane >> 4) * 2 * a.st + ((lane >> 3) & 1) * 256 + 16 * (lane & 7));
  const int64_t out_step = 8 * a.st;      // bytes of four vectors

  int64_t tile = blockIdx.x;
  if (tile < a.n_tiles) dma_codes256<F>(a, tile_info<256>(a, tile), (lds_u8*)lds, lane);
  __syncthreads();
  for (; tile < a.n_tiles; tile += gridDim.x) {
    const Tile t = tile_info<256>(a, tile);
    uint32_t cw[F::CW];
    uint32_t s16[NS];
    const uint8_t* crow = lds + L::kCodes + 2 * F::CB * vec;
    const uint8_t* srow = lds + L::kScales + 2 * F::SB * vec;
    if (ROT == KVQ_ROT_SRFT) {
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const uint4 w = *reinterpret_cast<const uint4*>(crow + 16 * ((q ^ vec) & (R - 1)));
        cw[2 * q] = __builtin_amdgcn_perm(w.y, w.x, sel);
        cw[2 * q + 1] = __builtin_amdgcn_perm(w.w, w.z, sel);
      }
      // every scale of the vector
#pragma unroll
      for (int i = 0; i < NS / 8; ++i) {
        const uint4 s4 = *reinterpret_cast<const uint4*>(srow + 16 * i);
        const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) { s16[8 * i + 2 * e] = sw[e] & 0xFFFFu; s16[8 * i + 2 * e + 1] = sw[e] >> 16; }
      }
    } else {
#pragma unroll
      for (int q = 0; q < R / 2; ++q) {
        const uint4 w = *reinterpret_cast<const uint4*>(crow + 16 * (((R / 2) * hh + q ^ vec) & (R - 1)));
        cw[4 * q] = w.x; cw[4 * q + 1] = w.y; cw[4 * q + 2] = w.z; cw[4 * q + 3] = w.w;
      }
      // this half's scales
      if (F::SB == 8) {
        const uint2 s2 = *reinterpret_cast<const uint2*>(srow + 8 * hh);
        const uint32_t sw[2] = {s2.x, s2.y};
#pragma unroll
        for (int i = 0; i < NS; ++i) s16[i] = (sw[(i / 2) % 2] >> (16 * (i % 2))) & 0xFFFFu;
      } else {
        const uint4 s4 = *reinterpret_cast<const uint4*>(srow + 16 * hh);
        const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int i = 0; i < NS; ++i) s16[i] = (sw[(i / 2) % 4] >> (16 * (i % 2))) & 0xFFFFu;
      }
    }
    float lq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) lq[q] = reinterpret_cast<const float*>(lds + L::kLam)[lane + 64 * q];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t nxt = tile + gridDim.x;
    if (nxt < a.n_tiles) dma_codes256<F>(a, tile_info<256>(a, nxt), (lds_u8*)lds, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float*>(work + kDec2Rl + rl_dst[q]) = rl_mul[q] * __builtin_amdgcn_rcpf(lq[q]);
    lds_sync();

    float v[128];
    dequant_lane<F, DPG>(cw, s16, reinterpret_cast<const float4*>(work + kDec2Rl) + 32 * hh, magic, v);

    if (ROT == KVQ_ROT_SRFT) {
      fft64<true>(v);
      if (hh) pair_twiddles_srft<true>(v);
      pair_fma_all_srft(v, sgn);
    } else if (ROT == KVQ_ROT_SRHT) {
      pair_fma_all(v, sgn);
      wht128(v);
    }
    // the next tile's direct loads have had the transform to land
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const char* ybase = reinterpret_cast<const char*>(static_cast<uint16_t*>(a.y) + t.b * a.sb + t.h * a.sh +
                                                      t.t_start * a.st);
    const int ho = (lane >> 3) & 1;         // half of the rows this lane stores
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 32 * hf + 4 * c + e;
          const int pp = ROT == KVQ_ROT_SRFT ? rev4(k) : k;
          wv[e] = pack_f16x2(v[2 * pp], v[2 * pp + 1]);
        }
        *reinterpret_cast<uint4*>(work + kDec2Out + lane * kDecPitch + 16 * c) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
      lds_sync();
      const int k0 = 64 * ho + 32 * hf + 4 * (lane & 7);
      const uint4 mk = make_uint4(out_mask256<ROT>(a, k0), out_mask256<ROT>(a, k0 + 1),
                                  out_mask256<ROT>(a, k0 + 2), out_mask256<ROT>(a, k0 + 3));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * i + (lane >> 3), c = lane & 7;
        uint4 w = *reinterpret_cast<const uint4*>(work + kDec2Out + r * kDecPitch + 16 * c);
        w.x ^= mk.x; w.y ^= mk.y; w.z ^= mk.z; w.w ^= mk.w;
        // vector 4 i + lane / 16: one lane value against a wave-uniform bound
        if ((lane >> 4) < t.nv - 4 * i) st_stream16(const_cast<char*>(ybase) + i * out_step + hf * 128 + out_lane, w);
      }
      lds_sync();
    }
  }
}

// ---------------------------------------------------------------------------
// Decode to fp32 (exact transform output, for checking): each lane writes its
// own channels
// ---------------------------------------------------------------------------
template <int D, int ROT, int FMT>
__global__ void __launch_bounds__(64, 2) decode_f32_kernel(CodecArgs a) {
  using G = Geo<D>;
  using F = Fmt<FMT>;
  constexpr int NSLOT = F::CB / 16;         // 16-byte code chunks per lane
  __shared__ __attribute__((aligned(16))) uint8_t lds[16384];
  const int lane = threadIdx.x;
  constexpr float kScale = rot_scale<D, ROT>();

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const Tile t = tile_info<D>(a, tile);
    // a lane's codes (its vector, or its half of a D=256 vector) are the
    // F::CB contiguous bytes at lane * CB from the tile's first cell
    const int64_t cell = t.row * a.Tcap + a.t0 + t.t_start;
    const uint8_t* cbase = a.codes_in + cell * (D * F::BITS / 8);
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
      const int s = i * 64 + lane;
      const int r = s / NSLOT;               // lane row
      const uint4 w = (r / G::L < t.nv) ? ld_stream16(cbase + s * 16) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(lds + code_off_f<F>(r, s % NSLOT)) = w;
    }
    uint32_t s16[F::NG];
    {
      const uint16_t* sp = a.scales_in + cell * (D / F::G) + lane * F::NG;
      if (lane / G::L < t.nv) {
#pragma unroll
        for (int i = 0; i < F::NG; ++i) s16[i] = sp[i];
      } else {
#pragma unroll
        for (int i = 0; i < F::NG; ++i) s16[i] = 0u;
      }
    }
    __syncthreads();
    uint32_t cw[F::CW];
#pragma unroll
    for (int q = 0; q < NSLOT; ++q) {
      const uint4 w = *reinterpret_cast<const uint4*>(lds + code_off_f<F>(lane, q));
      cw[4 * q] = w.x; cw[4 * q + 1] = w.y; cw[4 * q + 2] = w.z; cw[4 * q + 3] = w.w;
    }
    __syncthreads();

    const int half = (D == 256) ? (lane & 1) : 0;
    const float* lam = a.lambda + t.b * a.lambda_sb + t.h * D + half * 128;
    float v[128];
#pragma unroll
    for (int g = 0; g < F::NG; ++g) {
      const float sg = f16_bits_to_f32(s16[g]);
#pragma unroll
      for (int jj = 0; jj < F::G; ++jj) {
        const int j = F::G * g + jj;
        int code;
        if (F::BITS == 4) code = static_cast<int>((cw[j >> 3] >> (4 * (j & 7))) & 15u) - 8;
        else code = static_cast<int>(static_cast<int8_t>((cw[j >> 2] >> (8 * (j & 3))) & 0xFFu));
        // q * scale exactly, then divide by lambda (times the unitary scale
        // of the inverse rotation)
        v[j] = static_cast<float>(code) * sg * (kScale * __builtin_amdgcn_rcpf(lam[j]));
      }
    }

    // inverse rotation
    if (ROT == KVQ_ROT_SRFT) {
      if (D == 256) {
        // lane 2v: A_m = Z_m + Z_{m+64}; lane 2v+1: -(Z_m - Z_{m+64}) W^-m
        const float sgn = (lane & 1) ? -1.f : 1.f;
        pair_fma_all(v, sgn);
        if (lane & 1) {
#pragma unroll
          for (int m = 0; m < 64; ++m) twiddle_mul<128, true>(v[2 * m], v[2 * m + 1], m);
        }
      }
      fft64<true>(v);
    } else if (ROT == KVQ_ROT_SRHT) {
      if (D == 256) {
        const float sgn = (lane & 1) ? -1.f : 1.f;
        pair_fma_all(v, sgn);
      }
      wht128(v);
    }

    const int vec = lane / G::L;
    if (vec < t.nv) {
      // each lane writes its own channels
      float* yr = static_cast<float*>(a.y) + t.b * a.sb + t.h * a.sh + (t.t_start + vec) * a.st;
#pragma unroll
      for (int k = 0; k < 64; ++k) {
        const int p = ROT == KVQ_ROT_SRFT ? rev4(k) : k;
        int kg, ch;   // global pair index and its first channel
        if (D == 128) { kg = k; ch = 2 * k; }
        else if (ROT == KVQ_ROT_SRFT) { kg = 2 * k + (lane & 1); ch = 2 * kg; }
        else { kg = 64 * (lane & 1) + k; ch = 2 * kg; }
        const uint32_t m = word_mask<D, ROT>(a.signs, kg);
        const float lo = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[2 * p]) ^ ((m & 0x8000u) << 16));
        const float hi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[2 * p + 1]) ^ (m & 0x80000000u));
        *reinterpret_cast<float2*>(yr + ch) = make_float2(lo, hi);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Small calls: one wave per vector, its transform spread over the 64 lanes.
// A call of a few thousand vectors (the append of one token per sequence of
// a decode step, a short prompt) is bound by latency, not bandwidth: the tile
// kernels run a vector's whole transform in one lane (about 1.7k dependent
// instructions).  Here lane l holds complex pair l (and pair l + 64 at
// D = 256), the transform runs as radix-2 steps across the lanes (a
// cross-lane read and a few operations per step), the group abs-max is a
// cross-lane reduction, and each lane quantizes and stores its own channels.
// Same arithmetic contract as the tile kernels: fp32 transform, sigma =
// fp16 of the fp32 quotient, magic-number rounding with the clamp.
// ---------------------------------------------------------------------------
__constant__ TwTable kSmTw = make_twiddles(128);

__device__ __forceinline__ float xlane(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Bit reversal of a 6-bit index.
__device__ __forceinline__ int brev6(int l) { return static_cast<int>(__builtin_bitreverse32(l) >> 26); }

// N complex values per lane: the unnormalized 64-point DFT across the lanes,
// as radix-2 steps over the lane index.  Forward (kernel exp(-2 pi i / 64)):
// decimation in frequency, lane l starts with element l and ends with
// frequency bitrev(l).  INV: the steps in the opposite order with conjugate
// twiddles, each the inverse of the forward step times 2, so frequency
// bitrev(l) in lane l goes to 64 times element l of the inverse transform,
// i.e. the conjugate-kernel DFT in natural order.
template <bool INV, int N>
__device__ __forceinline__ void dft64_lanes(float (&re)[N], float (&im)[N], int lane) {
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int h = INV ? (1 << st) : (32 >> st);
    const bool bot = (lane & h) != 0;
    const int e = (lane & (h - 1)) * (32 / h);        // W_64^e on the pair's upper element
    const float sgn = bot ? -1.f : 1.f;
    const float c = bot ? kSmTw.c[2 * e] : 1.f;
    const float sn = bot ? (INV ? -kSmTw.s[2 * e] : kSmTw.s[2 * e]) : 0.f;
    if (INV) {
#pragma unroll
      for (int n = 0; n < N; ++n) {            // (re + i im)(c + i s) on the upper lane
        const float r2 = fmaf(re[n], c, im[n] * sn);
        const float i2 = fmaf(im[n], c, -(re[n] * sn));
        re[n] = r2;
        im[n] = i2;
      }
    }
    float pr[N], pi[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      pr[n] = xlane(re[n], h);
      pi[n] = xlane(im[n], h);
    }
#pragma unroll
    for (int n = 0; n < N; ++n) {                // lower lane x + p, upper lane p - x
      re[n] = fmaf(re[n], sgn, pr[n]);
      im[n] = fmaf(im[n], sgn, pi[n]);
    }
    if (!INV) {
#pragma unroll
      for (int n = 0; n < N; ++n) {            // (re + i im)(c - i s) on the upper lane
        const float r2 = fmaf(re[n], c, im[n] * sn);
        const float i2 = fmaf(im[n], c, -(re[n] * sn));
        re[n] = r2;
        im[n] = i2;
      }
    }
  }
}

// Sylvester Walsh-Hadamard steps over the lane bits (channel bits 1..6 when
// lane l holds channels 2l, 2l+1): the lower lane keeps x + p, the upper p - x.
template <int N>
__device__ __forceinline__ void wht_lanes(float (&v)[N], int lane) {
#pragma unroll
  for (int h = 1; h < 64; h *= 2) {
    const float sgn = (lane & h) ? -1.f : 1.f;
    float p[N];
#pragma unroll
    for (int n = 0; n < N; ++n) p[n] = xlane(v[n], h);
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = fmaf(v[n], sgn, p[n]);
  }
}

// Where a lane's NC = D / 64 values live after the forward transform.
// SRFT: lane l holds Z_m, m = bitrev(l) (D = 128: channels 2m, 2m+1;
// D = 256: Z_2m, Z_2m+1, channels 4m .. 4m+3), all in one group; the lanes
// of a group share the low log2(D / G) lane bits.  SRHT and no rotation:
// channels 2l, 2l+1 (and 128 + 2l, 129 + 2l), in one group per half; the
// lanes of a group share the high lane bits.
template <int D, int ROT, int G>
struct SmallLayout {
  static constexpr int NC = D / 64;
  static constexpr bool FREQ = ROT == KVQ_ROT_SRFT;
  static constexpr int SLOTS = FREQ ? 1 : D / 128;      // groups per lane
  static constexpr int PER_SLOT = NC / SLOTS;
  __device__ static int chan(int lane, int j) {
    if (FREQ) return NC * brev6(lane) + j;
    return 128 * (j / 2) + 2 * lane + (j & 1);
  }
  // the smallest and largest lane-index XOR that stays in the group
  static constexpr int MASK_LO = FREQ ? D / G : 1;
  static constexpr int MASK_HI = FREQ ? 32 : G / 4;
  // a lane of each group, the one that stores the scale
  __device__ static bool rep(int lane) { return FREQ ? lane < D / G : (lane % (G / 2)) == 0; }
};

template <int D, int ROT>
__device__ __forceinline__ uint32_t small_pair_mask(const uint64_t (&s)[4], int k) {
  if (ROT == KVQ_ROT_SRFT) return sign_bit(s, k) ? 0x80008000u : 0u;
  if (ROT == KVQ_ROT_SRHT) return (sign_bit(s, 2 * k) << 15) | (sign_bit(s, 2 * k + 1) << 31);
  return 0u;
}

// Forward transform of one vector: lane l loads pair words l (and l + 64),
// applies the signs and leaves its NC values in SmallLayout order,
// unnormalized.
template <int D, int ROT>
__device__ __forceinline__ void small_forward(const CodecArgs& a, const uint16_t* xr, int lane, float (&v)[D / 64]) {
  constexpr int NP = D / 128;
  float re[NP], im[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int k = lane + 64 * j;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(xr + 2 * k) ^ small_pair_mask<D, ROT>(a.signs, k);
    re[j] = f16_bits_to_f32(w & 0xFFFFu);
    im[j] = f16_bits_to_f32(w >> 16);
  }
  if (ROT == KVQ_ROT_SRFT) {
    if (D == 256) {
      // first radix-2 step of the 128-point DIF, inside the lane: u = A + B,
      // w = (A - B) W_128^l; the 64-point transforms of u and w are the even
      // and the odd frequencies
      const float c = kSmTw.c[lane], sn = kSmTw.s[lane];
      const float ur = re[0] + re[NP - 1], ui = im[0] + im[NP - 1];
      const float dr = re[0] - re[NP - 1], di = im[0] - im[NP - 1];
      re[0] = ur;
      im[0] = ui;
      re[NP - 1] = fmaf(dr, c, di * sn);
      im[NP - 1] = fmaf(di, c, -(dr * sn));
    }
    dft64_lanes<false, NP>(re, im, lane);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      v[2 * j] = re[j];
      v[2 * j + 1] = im[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      v[2 * j] = re[j];
      v[2 * j + 1] = im[j];
    }
    if (ROT == KVQ_ROT_SRHT) {
      if (D == 256) {                       // channel bit 7: the two halves
        const float a0 = v[0], a1 = v[1];
        v[0] = a0 + v[2];
        v[1] = a1 + v[3];
        v[2] = a0 - v[2];
        v[3] = a1 - v[3];
      }
#pragma unroll
      for (int j = 0; j < D / 64; j += 2) { // channel bit 0, inside the lane
        const float a0 = v[j];
        v[j] = a0 + v[j + 1];
        v[j + 1] = a0 - v[j + 1];
      }
      wht_lanes<D / 64>(v, lane);
    }
  }
}

template <int D, int ROT, int FMT, int MODE>
__global__ void __launch_bounds__(64) encode_small_kernel(CodecArgs a) {
  using F = Fmt<FMT>;
  using Lay = SmallLayout<D, ROT, F::G>;
  constexpr int NC = Lay::NC;
  constexpr float kScale = rot_scale<D, ROT>();
  constexpr int CBV = D * F::BITS / 8;           // code bytes per vector
  constexpr int NGV = D / F::G;                  // groups per vector
  const int lane = threadIdx.x;
  const int64_t vi = blockIdx.x;
  const int64_t t = vi % a.T;
  const int64_t bh = vi / a.T;
  const int64_t h = bh % a.H;
  const int64_t b = bh / a.H;
  const uint16_t* xr = a.x + b * a.sb + h * a.sh + t * a.st;
  const float* lr = a.lambda + b * a.lambda_sb + h * D;

  float v[NC];
  small_forward<D, ROT>(a, xr, lane, v);
  float wv[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) wv[j] = v[j] * lr[Lay::chan(lane, j)];
  if (MODE == 1) {
    float* wr = a.w + ((b * a.H + h) * a.T + t) * D;
#pragma unroll
    for (int j = 0; j < NC; ++j) wr[Lay::chan(lane, j)] = wv[j] * kScale;
    return;
  }
  const int64_t cell = (b * a.H + h) * a.Tcap + a.t0 + t;
  uint8_t* cr = a.codes + cell * CBV;
  uint16_t* sr = a.scales + cell * NGV;
  uint32_t byte[NC];
#pragma unroll
  for (int sl = 0; sl < Lay::SLOTS; ++sl) {
    float amax = 0.f;
#pragma unroll
    for (int j = sl * Lay::PER_SLOT; j < (sl + 1) * Lay::PER_SLOT; ++j) amax = fmaxf(amax, fabsf(wv[j]));
#pragma unroll
    for (int m = Lay::MASK_LO; m <= Lay::MASK_HI; m *= 2) amax = fmaxf(amax, xlane(amax, m));
    const uint32_t sc = f32_to_f16_bits(div_by<F::IQMAX>(amax * kScale));
    const float sf = f16_bits_to_f32(sc);
    const float r = sf > 0.f ? kScale * __builtin_amdgcn_rcpf(sf) : 0.f;
    const int j0 = sl * Lay::PER_SLOT;
    if (Lay::rep(lane)) sr[Lay::chan(lane, j0) / F::G] = static_cast<uint16_t>(sc);
#pragma unroll
    for (int j = j0; j < j0 + Lay::PER_SLOT; ++j)
      byte[j] = F::BITS == 4 ? quant_bits(wv[j], r) : ((quant_bits8(wv[j], r) & 0xFFu) ^ 0x80u);
  }
  // the lane's channels are consecutive in runs of two (four for SRFT at
  // D = 256): int4 one byte per two channels, int8 one per channel
#pragma unroll
  for (int j = 0; j < NC; j += (Lay::FREQ ? NC : 2)) {
    const int ch = Lay::chan(lane, j);
    if (F::BITS == 4) {
      if (Lay::FREQ && NC == 4) {
        const uint32_t lo = pair_byte(byte[0], byte[1]) & 0xFFu, hi = pair_byte(byte[2], byte[3]) & 0xFFu;
        *reinterpret_cast<uint16_t*>(cr + ch / 2) = static_cast<uint16_t>(lo | (hi << 8));
      } else {
        cr[ch / 2] = static_cast<uint8_t>(pair_byte(byte[j], byte[j + 1]) & 0xFFu);
      }
    } else {
      if (Lay::FREQ && NC == 4) {
        *reinterpret_cast<uint32_t*>(cr + ch) = byte[0] | (byte[1] << 8) | (byte[2] << 16) | (byte[3] << 24);
      } else {
        *reinterpret_cast<uint16_t*>(cr + ch) = static_cast<uint16_t>(byte[j] | (byte[j + 1] << 8));
      }
    }
  }
}

template <int D, int ROT, int FMT, bool F32>
__global__ void __launch_bounds__(64) decode_small_kernel(CodecArgs a) {
  using F = Fmt<FMT>;
  using Lay = SmallLayout<D, ROT, F::G>;
  constexpr int NC = Lay::NC;
  constexpr int NP = D / 128;
  constexpr float kScale = rot_scale<D, ROT>();
  constexpr int CBV = D * F::BITS / 8;
  constexpr int NGV = D / F::G;
  const int lane = threadIdx.x;
  const int64_t vi = blockIdx.x;
  const int64_t t = vi % a.T;
  const int64_t bh = vi / a.T;
  const int64_t h = bh % a.H;
  const int64_t b = bh / a.H;
  const float* lr = a.lambda + b * a.lambda_sb + h * D;
  const int64_t cell = (b * a.H + h) * a.Tcap + a.t0 + t;
  const uint8_t* cr = a.codes_in + cell * CBV;
  const uint16_t* sr = a.scales_in + cell * NGV;

  // codes of the lane's channels, as signed integers
  int q[NC];
#pragma unroll
  for (int j = 0; j < NC; j += (Lay::FREQ ? NC : 2)) {
    const int ch = Lay::chan(lane, j);
    const int run = Lay::FREQ ? NC : 2;
    if (F::BITS == 4) {
      uint32_t bytes = run == 4 ? *reinterpret_cast<const uint16_t*>(cr + ch / 2) : cr[ch / 2];
#pragma unroll
      for (int u = 0; u < run; ++u) q[j + u] = static_cast<int>((bytes >> (4 * u)) & 0xFu) - 8;
    } else {
      const uint32_t bytes = run == 4 ? *reinterpret_cast<const uint32_t*>(cr + ch)
                                      : *reinterpret_cast<const uint16_t*>(cr + ch);
#pragma unroll
      for (int u = 0; u < run; ++u) q[j + u] = static_cast<int>(static_cast<int8_t>((bytes >> (8 * u)) & 0xFFu));
    }
  }
  float v[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int ch = Lay::chan(lane, j);
    const float sg = f16_bits_to_f32(sr[ch / F::G]);
    v[j] = static_cast<float>(q[j]) * sg * (kScale * __builtin_amdgcn_rcpf(lr[ch]));
  }
  // inverse transform: lane l ends with channels 2l, 2l+1 (and 128 + 2l,
  // 129 + 2l)
  float o[NC];
  if (ROT == KVQ_ROT_SRFT) {
    float re[NP], im[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      re[j] = v[2 * j];
      im[j] = v[2 * j + 1];
    }
    dft64_lanes<true, NP>(re, im, lane);
    if (D == 256) {
      // the inverse of the first radix-2 step: A = U + W V, B = U - W V,
      // W = conj(W_128^l)
      const float c = kSmTw.c[lane], sn = -kSmTw.s[lane];
      const float wr = fmaf(re[NP - 1], c, im[NP - 1] * sn), wi = fmaf(im[NP - 1], c, -(re[NP - 1] * sn));
      const float ur = re[0], ui = im[0];
      re[0] = ur + wr;
      im[0] = ui + wi;
      re[NP - 1] = ur - wr;
      im[NP - 1] = ui - wi;
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      o[2 * j] = re[j];
      o[2 * j + 1] = im[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < NC; ++j) o[j] = v[j];
    if (ROT == KVQ_ROT_SRHT) {
      if (D == 256) {
        const float a0 = o[0], a1 = o[1];
        o[0] = a0 + o[2];
        o[1] = a1 + o[3];
        o[2] = a0 - o[2];
        o[3] = a1 - o[3];
      }
#pragma unroll
      for (int j = 0; j < NC; j += 2) {
        const float a0 = o[j];
        o[j] = a0 + o[j + 1];
        o[j + 1] = a0 - o[j + 1];
      }
      wht_lanes<NC>(o, lane);
    }
  }
  // signs, then the row: pair k = lane + 64 j at element 2 k
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int k = lane + 64 * j;
    const uint32_t m = small_pair_mask<D, ROT>(a.signs, k);
    const float y0 = (m & 0x8000u) ? -o[2 * j] : o[2 * j];
    const float y1 = (m & 0x80000000u) ? -o[2 * j + 1] : o[2 * j + 1];
    if (F32) {
      float* yr = static_cast<float*>(a.y) + b * a.sb + h * a.sh + t * a.st;
      *reinterpret_cast<float2*>(yr + 2 * k) = make_float2(y0, y1);
    } else {
      uint16_t* yr = static_cast<uint16_t*>(a.y) + b * a.sb + h * a.sh + t * a.st;
      *reinterpret_cast<uint32_t*>(yr + 2 * k) = pack_f16x2(y0, y1);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

// One wave per tile: the dispatcher starts each wave as a slot frees up, so
// the resident waves drift out of phase and their loads, arithmetic and
// stores overlap better than those of a persistent grid walking the tiles
// in lockstep (measured 5-14% faster at the prefix sizes).  Past a cap the
// waves take several tiles each, with a stride of the grid, loading the next
// tile while computing one: 32 waves per CU (four times what fits at once)
// for the decoders.  The encoders keep one wave per tile up to 64 per CU
// (at 2 tiles per wave a 1M-vector encode measured 7% slower than at one)
// and take 32 per CU beyond (at 8 tiles per wave a 4M-vector call is as
// fast as or faster than at one).
int64_t launch_grid(int64_t n_tiles, bool encoder) {
  const int64_t cus = device_cu_count();
  if (encoder && n_tiles <= cus * 64) return n_tiles;
  const int64_t cap = cus * 32;
  return n_tiles < cap ? n_tiles : cap;
}

template <int D>
void fill_common(CodecArgs& a, const CodecDesc& d) {
  a.H = d.H;
  a.T = d.T;
  a.Tcap = d.Tcap;
  a.t0 = d.t0;
  a.sb = d.sb;
  a.sh = d.sh;
  a.st = d.st;
  a.lambda = d.lambda;
  a.lambda_sb = d.lambda_sb;
  a.tiles_per_row = (d.T + Geo<D>::VPT - 1) / Geo<D>::VPT;
  a.n_tiles = d.B * d.H * a.tiles_per_row;
  a.div_tpr = make_fastdiv(static_cast<uint64_t>(a.tiles_per_row));
  a.div_h = make_fastdiv(static_cast<uint64_t>(d.H));
  for (int i = 0; i < 4; ++i) a.signs[i] = d.signs[i];
}

// Format index of a call: 2 * (bits == 8) + (G == 16).
int format_of(const CodecDesc& d) { return (d.bits == 8 ? 2 : 0) + (d.G == 16 ? 1 : 0); }

// Calls of at most this many vectors take the one-wave-per-vector kernels
// (measured from graph replays on an MI355X: at 256-2048 vectors they take
// 3-4 us where the tile kernels take 6-7.5, and they stop winning near 6k
// vectors at D = 128, 8k at D = 256).
template <int D>
constexpr int64_t small_limit() {
  return D == 128 ? 4096 : 8192;
}

template <int D, int ROT, int FMT>
hipError_t encode_dispatch(const CodecDesc& d, int mode) {
  CodecArgs a{};
  fill_common<D>(a, d);
  a.x = d.x;
  a.codes = d.codes;
  a.scales = d.scales;
  a.w = d.w;
  if (a.n_tiles == 0) return hipSuccess;
  const int64_t n_vec = d.B * d.H * d.T;
  if (d.options == 0 && n_vec <= small_limit<D>()) {
    if (mode == 1) {
      hipLaunchKernelGGL((encode_small_kernel<D, ROT, 0, 1>), dim3(static_cast<unsigned>(n_vec)), dim3(64), 0,
                         d.stream, a);
    } else {
      hipLaunchKernelGGL((encode_small_kernel<D, ROT, FMT, 0>), dim3(static_cast<unsigned>(n_vec)), dim3(64), 0,
                         d.stream, a);
    }
    return hipGetLastError();
  }
  if (a.n_tiles >= (int64_t(1) << 32)) return hipErrorInvalidValue;   // index math is 32-bit exact
  const dim3 grid(static_cast<unsigned>(launch_grid(a.n_tiles, true)));
  if (D == 128 && ROT == KVQ_ROT_SRFT && (d.options & kOptMfmaRotation)) {
    if (mode == 1) {
      hipLaunchKernelGGL((encode128_mfma_kernel<1, 0>), grid, dim3(64), 0, d.stream, a);
    } else {
      hipLaunchKernelGGL((encode128_mfma_kernel<0, FMT>), grid, dim3(64), 0, d.stream, a);
    }
    return hipGetLastError();
  }
  const bool one = grid.x >= a.n_tiles;   // a wave per tile
  if (mode == 1) {
    // rotate only: the quantizer format plays no part
    if (D == 128) {
      hipLaunchKernelGGL((encode128_kernel<ROT, 1, 0, false>), grid, dim3(64), 0, d.stream, a);
    } else {
      hipLaunchKernelGGL((encode256_kernel<ROT, 1, 0, false>), grid, dim3(64), 0, d.stream, a);
    }
  } else if (D == 128) {
    if (one) {
      hipLaunchKernelGGL((encode128_kernel<ROT, 0, FMT, true>), grid, dim3(64), 0, d.stream, a);
    } else {
      hipLaunchKernelGGL((encode128_kernel<ROT, 0, FMT, false>), grid, dim3(64), 0, d.stream, a);
    }
  } else {
    if (one) {
      hipLaunchKernelGGL((encode256_kernel<ROT, 0, FMT, true>), grid, dim3(64), 0, d.stream, a);
    } else {
      hipLaunchKernelGGL((encode256_kernel<ROT, 0, FMT, false>), grid, dim3(64), 0, d.stream, a);
    }
  }
  return hipGetLastError();
}

template <int D, int ROT, int FMT>
hipError_t decode_dispatch(const CodecDesc& d, bool f32) {
  CodecArgs a{};
  fill_common<D>(a, d);
  a.codes_in = d.codes_in;
  a.scales_in = d.scales_in;
  a.y = d.y;
  if (a.n_tiles == 0) return hipSuccess;
  const int64_t n_vec = d.B * d.H * d.T;
  if (n_vec <= small_limit<D>()) {
    if (f32) {
      hipLaunchKernelGGL((decode_small_kernel<D, ROT, FMT, true>), dim3(static_cast<unsigned>(n_vec)), dim3(64), 0,
                         d.stream, a);
    } else {
      hipLaunchKernelGGL((decode_small_kernel<D, ROT, FMT, false>), dim3(static_cast<unsigned>(n_vec)), dim3(64),
                         0, d.stream, a);
    }
    return hipGetLastError();
  }
  if (a.n_tiles >= (int64_t(1) << 32)) return hipErrorInvalidValue;   // index math is 32-bit exact
  const dim3 grid(static_cast<unsigned>(launch_grid(a.n_tiles, false)));
  if (f32) {
    hipLaunchKernelGGL((decode_f32_kernel<D, ROT, FMT>), grid, dim3(64), 0, d.stream, a);
  } else if (D == 128) {
    if (grid.x >= a.n_tiles) {   // a wave per tile
      hipLaunchKernelGGL((decode128_kernel<ROT, FMT, true>), grid, dim3(64), 0, d.stream, a);
    } else {
      hipLaunchKernelGGL((decode128_kernel<ROT, FMT, false>), grid, dim3(64), 0, d.stream, a);
    }
  } else {
    hipLaunchKernelGGL((decode256_kernel<ROT, FMT>), grid, dim3(64), 0, d.stream, a);
  }
  return hipGetLastError();
}

template <int D, int ROT>
hipError_t encode_fmt(const CodecDesc& d, int mode) {
  switch (format_of(d)) {
    case 1: return encode_dispatch<D, ROT, 1>(d, mode);
    case 2: return encode_dispatch<D, ROT, 2>(d, mode);
    case 3: return encode_dispatch<D, ROT, 3>(d, mode);
    default: return encode_dispatch<D, ROT, 0>(d, mode);
  }
}

template <int D, int ROT>
hipError_t decode_fmt(const CodecDesc& d, bool f32) {
  switch (format_of(d)) {
    case 1: return decode_dispatch<D, ROT, 1>(d, f32);
    case 2: return decode_dispatch<D, ROT, 2>(d, f32);
    case 3: return decode_dispatch<D, ROT, 3>(d, f32);
    default: return decode_dispatch<D, ROT, 0>(d, f32);
  }
}

template <int D>
hipError_t encode_rot(const CodecDesc& d, int mode) {
  switch (d.rotation) {
    case KVQ_ROT_SRFT: return encode_fmt<D, KVQ_ROT_SRFT>(d, mode);
    case KVQ_ROT_SRHT: return encode_fmt<D, KVQ_ROT_SRHT>(d, mode);
    default: return encode_fmt<D, KVQ_ROT_ID>(d, mode);
  }
}

template <int D>
hipError_t decode_rot(const CodecDesc& d, bool f32) {
  switch (d.rotation) {
    case KVQ_ROT_SRFT: return decode_fmt<D, KVQ_ROT_SRFT>(d, f32);
    case KVQ_ROT_SRHT: return decode_fmt<D, KVQ_ROT_SRHT>(d, f32);
    default: return decode_fmt<D, KVQ_ROT_ID>(d, f32);
  }
}

}  // namespace

hipError_t launch_encode(const CodecDesc& d, int mode) {
  if (d.D == 128) return encode_rot<128>(d, mode);
  if (d.D == 256) return encode_rot<256>(d, mode);
  return launch_encode_mixed(d, mode);
}

hipError_t launch_decode(const CodecDesc& d, bool f32) {
  if (d.D == 128) return decode_rot<128>(d, f32);
  if (d.D == 256) return decode_rot<256>(d, f32);
  return launch_decode_mixed(d, f32);
}

}  // namespace kvq
