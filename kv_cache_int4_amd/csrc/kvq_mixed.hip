// Encode / rotate / decode kernels for head dimensions that are not powers of
// two: D = 80 (M = 40 complex pairs) and D = 96 (M = 48), with the SRFT over
// the mixed-radix M-point DFT of kvq_mixfft.hpp, or no rotation.
//
// The pages prefer the SRFT to the Walsh-Hadamard rotation because the DFT
// exists at every length (paper abstract); the encoder is the same chain as
// at D = 128 (gist.science explainer of "When Quantization Is Free",
// "Methodik" 1-2): signs on the D/2 complex pairs -> unitary DFT -> unpair
// -> lambda -> per-group abs-max -> codes.  Groups must divide D: D = 80
// takes G = 16 only (five groups), D = 96 takes G = 32 or 16.
//
// Work decomposition.  A wave owns a tile of 64 consecutive vectors of one
// (batch, head) row, one vector per lane; the grid has one wave per tile up
// to 32 waves per CU (larger calls have the waves walk the tiles with a
// stride of the grid, the next tile's input streaming in while the current
// one computes).  Tile
// input moves from HBM straight into LDS with direct (global -> LDS) 16-byte
// loads and is computed in registers:
//   encode: the fp16 rows (D / 8 chunks of 16 bytes each) land in a
//           row-major LDS tile whose chunks are XOR-swizzled per row, so that
//           each lane's read of its own row is free of bank conflicts; the
//           loads themselves take 64 consecutive chunks of the tile each.
//   decode: the tile's code bytes (one contiguous block of 64 * CB bytes)
//           land in LDS the same way; the fp16 output goes back through a
//           swizzled LDS tile and leaves in row-major 16-byte stores.
// Group scales and lambda travel in registers, loaded with the next tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.hpp"
#include "kvq_internal.hpp"
#include "kvq_mixfft.hpp"

namespace kvq {

namespace {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

struct MixArgs {
  const uint16_t* x;          // encode / rotate input, fp16
  const uint8_t* codes_in;    // decode input
  const uint16_t* scales_in;
  uint8_t* codes;             // encode output
  uint16_t* scales;
  void* y;                    // decode output (fp16 or fp32)
  float* w;                   // rotate output
  const float* lambda;
  int64_t H, T, Tcap, t0;
  int64_t sb, sh, st;         // strides of x (encode, rotate) or y (decode), elements
  int64_t lambda_sb;
  int64_t tiles_per_row, n_tiles;
  FastDiv div_tpr, div_h;
  uint64_t signs;             // SRFT: bit k = sign of complex pair k (M <= 64)
};

// Geometry of a D-channel vector (D = 80 or 96) in 16-byte fp16 chunks.
template <int D>
struct MGeo {
  static constexpr int M = D / 2;                       // complex pairs
  static constexpr int C = D / 8;                       // fp16 chunks per row (10, 12)
  // per-row chunk swizzle: chunk j of row r sits at column j ^ swz(r)
  static constexpr int SWZ_SHIFT = C == 12 ? 2 : 3;
  static constexpr int SWZ_MASK = C == 12 ? 3 : 1;
  // the chunk loads repeat their lane pattern every PER loads (RPP rows)
  static constexpr int PER = C == 12 ? 3 : 5;
  static constexpr int RPP = 64 * PER / C;              // 16, 32
  static constexpr int kTileBytes = 64 * C * 16;
};

template <int D>
__device__ __forceinline__ int swz(int r) {
  return (r >> MGeo<D>::SWZ_SHIFT) & MGeo<D>::SWZ_MASK;
}

// Code format: FMT = 2 * (bits == 8) + (G == 16), as for D = 128.
template <int D, int FMT>
struct MFmt {
  static constexpr int BITS = (FMT & 2) ? 8 : 4;
  static constexpr int G = (FMT & 1) ? 16 : 32;
  static constexpr int NG = D / G;                      // groups per vector
  static constexpr int CB = D * BITS / 8;               // code bytes per vector
  static constexpr int CW = CB / 4;                     // code words
  static constexpr int SB = 2 * NG;                     // scale bytes
  static constexpr int WPG = CW / NG;                   // code words per group
  static constexpr int IQMAX = BITS == 4 ? 7 : 127;
  // direct loads of a tile's codes: 16-byte slots where CB allows, else
  // dwords (CB = 40); NU slots per vector, as many loads per lane
  static constexpr int CU = CB % 16 == 0 ? 16 : 4;
  static constexpr int NU = CB / CU;
  static_assert(D % G == 0, "groups must divide D");
};

// LDS slot (in CU units) of slot q of vector r's codes: 16-byte slots of a
// six-slot row are swizzled by bit 3 of the row (conflict-free lane reads).
template <typename F>
__device__ __forceinline__ int code_slot(int r, int q) {
  return r * F::NU + (F::CU == 16 && F::NU == 6 ? (q ^ ((r >> 3) & 1)) : q);
}

template <int ROT, int D>
__host__ __device__ constexpr float mix_scale() {
  return ROT == KVQ_ROT_SRFT ? static_cast<float>(const_rsqrt(D / 2)) : 1.0f;
}

// Register of output channel j after the forward transform.
template <int ROT, int D>
__host__ __device__ constexpr int mreg(int j) {
  return ROT == KVQ_ROT_SRFT ? 2 * mr_pos<D / 2>(j >> 1) + (j & 1) : j;
}

struct MTile {
  int64_t row, b, h, t_start;
  int nv;
};

__device__ __forceinline__ MTile mtile(const MixArgs& a, int64_t tile) {
  MTile t;
  t.row = static_cast<int64_t>(fdiv(static_cast<uint64_t>(tile), a.div_tpr));
  t.t_start = (tile - t.row * a.tiles_per_row) * 64;
  t.b = static_cast<int64_t>(fdiv(static_cast<uint64_t>(t.row), a.div_h));
  t.h = t.row - t.b * a.H;
  const int64_t left = a.T - t.t_start;
  t.nv = static_cast<int>(left < 64 ? left : 64);
  return t;
}

// Per-lane offsets of the row-major 16-byte chunk slots of a tile: slot
// s = 64 i + lane is row r = s / C, column c = s % C, holding chunk
// c ^ swz(r) of that row (the LDS tile is the slots in order).  The pattern
// repeats every PER loads, RPP rows further on; rb[b] and ob[b] are the row
// and the byte offset (for a row stride of st elements) of load b < PER.
template <int D>
__device__ __forceinline__ void slot_offsets(int lane, int64_t st, int (&rb)[MGeo<D>::PER],
                                             int64_t (&ob)[MGeo<D>::PER]) {
  using G = MGeo<D>;
#pragma unroll
  for (int b = 0; b < G::PER; ++b) {
    const int s = 64 * b + lane;
    const int r = s / G::C;
    const int c = s % G::C;
    rb[b] = r;
    ob[b] = static_cast<int64_t>(r) * 2 * st + 16 * (c ^ swz<D>(r));
  }
}

__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Direct loads of the fp16 rows of a tile into the swizzled LDS tile.
template <int D>
__device__ __forceinline__ void dma_rows(const MixArgs& a, const MTile& t, lds_u8* lds,
                                         const int (&rb)[MGeo<D>::PER], const int64_t (&ob)[MGeo<D>::PER]) {
  using G = MGeo<D>;
  const char* base = reinterpret_cast<const char*>(a.x + t.b * a.sb + t.h * a.sh + t.t_start * a.st);
  const int64_t per_step = static_cast<int64_t>(G::RPP) * 2 * a.st;
#pragma unroll
  for (int i = 0; i < G::C; ++i) {
    const int pi = i / G::PER, b = i % G::PER;
    const char* src = base + pi * per_step + ob[b];
    lds_u8* dst = lds + 1024 * i;
    if (rb[b] < t.nv - pi * G::RPP) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
  }
}

// Sign mask of complex pair k (one word of two fp16).
template <int ROT>
__device__ __forceinline__ uint32_t mix_mask(uint64_t signs, int k) {
  return (ROT == KVQ_ROT_SRFT && ((signs >> k) & 1u)) ? 0x80008000u : 0u;
}

// Codes of group g of the lane's vector from the lambda-scaled values w
// (channel j in register mreg(j)) and r = 1 / scale.
template <int ROT, int D, int FMT, bool CLAMP>
__device__ __forceinline__ void mquant_group(const float (&v)[D], int g, float r, uint32_t* cw) {
  using F = MFmt<D, FMT>;
#pragma unroll
  for (int q = 0; q < F::WPG; ++q) {
    uint32_t by[4];
    if (F::BITS == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = F::G * g + 8 * q + 2 * e;
        uint32_t lo, hi;
        if (CLAMP) {
          lo = quant_bits(v[mreg<ROT, D>(j)], r);
          hi = quant_bits(v[mreg<ROT, D>(j + 1)], r);
        } else {
          lo = __builtin_bit_cast(uint32_t, fmaf(v[mreg<ROT, D>(j)], r, kMagic));
          hi = __builtin_bit_cast(uint32_t, fmaf(v[mreg<ROT, D>(j + 1)], r, kMagic));
        }
        by[e] = pair_byte(lo, hi);
      }
      cw[q] = pack4(by[0], by[1], by[2], by[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = F::G * g + 4 * q + e;
        by[e] = CLAMP ? quant_bits8(v[mreg<ROT, D>(j)], r)
                      : __builtin_bit_cast(uint32_t, fmaf(v[mreg<ROT, D>(j)], r, kMagic8));
      }
      cw[q] = pack4(by[0], by[1], by[2], by[3]) ^ 0x80808080u;
    }
  }
}

typedef uint32_t mx_u32x2 __attribute__((ext_vector_type(2)));

// The tile's code rows, dense in memory from cbase (nb bytes), from the
// staging buffer stg (row = lane, CB bytes each) as non-temporal stores of
// 16 bytes (CB a multiple of 16) or 8 bytes per lane and instruction.
// Against each lane storing its own row: encode 4-7% faster (int4) and 21%
// (int8), codes bit-identical.
template <typename F>
__device__ __forceinline__ void store_staged_rows(uint8_t* cbase, int nb, const uint8_t* stg, int lane) {
  constexpr int U = F::CU == 16 ? 16 : 8;
  constexpr int kInst = (64 * F::CB / U + 63) / 64;
#pragma unroll
  for (int i = 0; i < kInst; ++i) {
    const int off = U * (64 * i + lane);
    if (off < nb) {
      if (U == 16) {
        st_stream16(cbase + off, *reinterpret_cast<const uint4*>(stg + off));
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(stg + off);
        const mx_u32x2 v = {w.x, w.y};
        __builtin_nontemporal_store(v, reinterpret_cast<mx_u32x2*>(cbase + off));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Encode (MODE 0: codes + scales) and rotate (MODE 1: fp32 w = lambda R x)
// ---------------------------------------------------------------------------
template <int D, int ROT, int FMT, int MODE>
__global__ void __launch_bounds__(64, 2) mix_encode_kernel(MixArgs a) {
  using G = MGeo<D>;
  using F = MFmt<D, FMT>;
  constexpr int M = G::M;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) float lam_lds[D];
  // code rows of the previous tile (row = lane), stored with the next
  // tile's loads out
  __shared__ __attribute__((aligned(16))) uint8_t stg[MODE == 0 ? 64 * F::CB : 16];
  const int lane = threadIdx.x;
  constexpr float kScale = mix_scale<ROT, D>();

  int rb[G::PER];
  int64_t ob[G::PER];
  slot_offsets<D>(lane, a.st, rb, ob);

  // lambda of a tile: lane l holds channels l and l + 64 (if < D), loaded
  // with the tile's rows and written to LDS once they have landed
  float lam_r0 = 0.f, lam_r1 = 0.f;
  int64_t tile = blockIdx.x;
  if (tile < a.n_tiles) {
    const MTile t = mtile(a, tile);
    dma_rows<D>(a, t, (lds_u8*)lds, rb, ob);
    const float* lr = a.lambda + t.b * a.lambda_sb + t.h * D;
    lam_r0 = lr[lane];
    if (lane + 64 < D) lam_r1 = lr[lane + 64];
  }
  // codes and scales of the previous tile, stored once the next tile's
  // loads are on their way
  uint32_t pend_s[F::NG] = {};
  bool pend_valid = false;
  uint16_t* pend_sp = nullptr;
  uint8_t* pend_cb = nullptr;     // the staged tile's first code byte
  int pend_nb = 0;                // and its code bytes
  for (; tile < a.n_tiles; tile += gridDim.x) {
    const MTile t = mtile(a, tile);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lam_lds[lane] = lam_r0;
    if (lane + 64 < D) lam_lds[lane + 64] = lam_r1;
    uint32_t p[M];
#pragma unroll
    for (int j = 0; j < G::C; ++j) {
      const uint4 w = *reinterpret_cast<const uint4*>(lds + 16 * (lane * G::C + (j ^ swz<D>(lane))));
      p[4 * j] = w.x ^ mix_mask<ROT>(a.signs, 4 * j);
      p[4 * j + 1] = w.y ^ mix_mask<ROT>(a.signs, 4 * j + 1);
      p[4 * j + 2] = w.z ^ mix_mask<ROT>(a.signs, 4 * j + 2);
      p[4 * j + 3] = w.w ^ mix_mask<ROT>(a.signs, 4 * j + 3);
    }
    // the tile is in registers: the LDS tile takes the next one
    lds_sync();
    const int64_t nxt = tile + gridDim.x;
    if (nxt < a.n_tiles) {
      const MTile tn = mtile(a, nxt);
      dma_rows<D>(a, tn, (lds_u8*)lds, rb, ob);
      const float* lr = a.lambda + tn.b * a.lambda_sb + tn.h * D;
      lam_r0 = lr[lane];
      if (lane + 64 < D) lam_r1 = lr[lane + 64];
    }
    if (MODE == 0 && pend_nb > 0) {
      store_staged_rows<F>(pend_cb, pend_nb, stg, lane);
      if (pend_valid) {
#pragma unroll
        for (int g = 0; g < F::NG; ++g) pend_sp[g] = static_cast<uint16_t>(pend_s[g]);
      }
    }

    float v[D];
#pragma unroll
    for (int k = 0; k < M; ++k) {
      v[2 * k] = f16_bits_to_f32(p[k] & 0xFFFFu);
      v[2 * k + 1] = f16_bits_to_f32(p[k] >> 16);
    }
    if (ROT == KVQ_ROT_SRFT) mr_fft<M, false>(v);
    asm volatile("" ::: "memory");
    const bool valid = lane < t.nv;

    if (MODE == 1) {
      float* wr = a.w + ((t.row * a.T) + t.t_start + lane) * D;
      if (valid) {
#pragma unroll
        for (int j = 0; j < D; j += 4) {
          const float4 l4 = *reinterpret_cast<const float4*>(lam_lds + j);
          float4 o;
          o.x = v[mreg<ROT, D>(j)] * l4.x * kScale;
          o.y = v[mreg<ROT, D>(j + 1)] * l4.y * kScale;
          o.z = v[mreg<ROT, D>(j + 2)] * l4.z * kScale;
          o.w = v[mreg<ROT, D>(j + 3)] * l4.w * kScale;
          *reinterpret_cast<float4*>(wr + j) = o;
        }
      }
    } else {
      float r[F::NG];
      uint32_t sc[F::NG];
      bool tiny = false;
#pragma unroll
      for (int g = 0; g < F::NG; ++g) {
        float amax = 0.f;
#pragma unroll
        for (int jj = 0; jj < F::G; jj += 4) {
          const int j = F::G * g + jj;
          const float4 l4 = *reinterpret_cast<const float4*>(lam_lds + j);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float wv = v[mreg<ROT, D>(j + e)] * lv[e];
            v[mreg<ROT, D>(j + e)] = wv;
            amax = fmaxf(amax, fabsf(wv));
          }
        }
        // scale = fp16(fp32(absmax / qmax)) of the unitary values kScale *
        // wv, with the IEEE fp32 quotient
        sc[g] = f32_to_f16_bits(div_by<F::IQMAX>(amax * kScale));
        const float sf = f16_bits_to_f32(sc[g]);
        r[g] = sf > 0.f ? kScale * __builtin_amdgcn_rcpf(sf) : 0.f;
        tiny |= (sc[g] != 0u) && (sc[g] < 0x0400u);     // fp16-subnormal scale
      }
      uint32_t cw[F::CW];
      if (__builtin_amdgcn_ballot_w64(tiny && valid) == 0) {
#pragma unroll
        for (int g = 0; g < F::NG; ++g) mquant_group<ROT, D, FMT, false>(v, g, r[g], cw + F::WPG * g);
      } else {
#pragma unroll
        for (int g = 0; g < F::NG; ++g) mquant_group<ROT, D, FMT, true>(v, g, r[g], cw + F::WPG * g);
      }
      const int64_t cell = t.row * a.Tcap + a.t0 + t.t_start + lane;
      pend_sp = a.scales + cell * F::NG;
      // the lane's code row into the staging buffer (the staged rows of the
      // tile before were stored above, a transform ago)
      if (F::CU == 16) {
#pragma unroll
        for (int q = 0; q < F::CB / 16; ++q)
          *reinterpret_cast<uint4*>(stg + lane * F::CB + 16 * q) =
              make_uint4(cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]);
      } else {
#pragma unroll
        for (int q = 0; q < F::CB / 8; ++q)
          *reinterpret_cast<uint2*>(stg + lane * F::CB + 8 * q) = make_uint2(cw[2 * q], cw[2 * q + 1]);
      }
      pend_cb = a.codes + (t.row * a.Tcap + a.t0 + t.t_start) * F::CB;
      pend_nb = t.nv * F::CB;
#pragma unroll
      for (int g = 0; g < F::NG; ++g) pend_s[g] = sc[g];
      pend_valid = valid;
    }
  }
  if (MODE == 0 && pend_nb > 0) {
    store_staged_rows<F>(pend_cb, pend_nb, stg, lane);
    if (pend_valid) {
#pragma unroll
      for (int g = 0; g < F::NG; ++g) pend_sp[g] = static_cast<uint16_t>(pend_s[g]);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode: unpack, rescale, divide by lambda, inverse rotation; fp16 output
// through a swizzled LDS tile and row-major stores, or fp32 output (exact
// transform output, for checking) stored by each lane
// ---------------------------------------------------------------------------

// Direct loads of a tile's code block (64 * CB contiguous bytes from the
// tile's first cell) into LDS slots code_slot(r, q).
template <typename F>
__device__ __forceinline__ void dma_codes(const uint8_t* cbase, int nv, lds_u8* lds, const int (&src)[F::NU],
                                          const int (&row)[F::NU]) {
#pragma unroll
  for (int i = 0; i < F::NU; ++i) {
    const char* s = reinterpret_cast<const char*>(cbase) + src[i];
    lds_u8* dst = lds + 64 * F::CU * i;
    if (row[i] < nv) {
      if constexpr (F::CU == 16) __builtin_amdgcn_global_load_lds(s, dst, 16, 0, 0);
      else __builtin_amdgcn_global_load_lds(s, dst, 4, 0, 0);
    }
  }
}

template <int D, int ROT, int FMT, bool F32>
__global__ void __launch_bounds__(64, 2) mix_decode_kernel(MixArgs a) {
  using G = MGeo<D>;
  using F = MFmt<D, FMT>;
  constexpr int M = G::M;
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[64 * F::CB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_out[F32 ? 16 : G::kTileBytes];
  __shared__ __attribute__((aligned(16))) float rl_lds[D];
  const int lane = threadIdx.x;
  constexpr float kScale = mix_scale<ROT, D>();
  constexpr float kOff = F::BITS == 4 ? 8.f : 128.f;

  // direct-load slot i of this lane: LDS slot 64 i + lane is slot q of row
  // r, whose source is byte CU * (r * NU + q) of the tile's code block
  int csrc[F::NU], crow[F::NU];
#pragma unroll
  for (int i = 0; i < F::NU; ++i) {
    const int s = 64 * i + lane;
    const int r = s / F::NU, c = s % F::NU;
    const int q = (F::CU == 16 && F::NU == 6) ? (c ^ ((r >> 3) & 1)) : c;
    csrc[i] = F::CU * (r * F::NU + q);
    crow[i] = r;
  }
  int rb[G::PER];
  int64_t ob[G::PER];
  slot_offsets<D>(lane, a.st, rb, ob);

  float lam_r0 = 1.f, lam_r1 = 1.f;
  uint32_t s_r[F::NG];
#pragma unroll
  for (int g = 0; g < F::NG; ++g) s_r[g] = 0u;
  auto issue = [&](int64_t tl) {
    const MTile t = mtile(a, tl);
    const int64_t cell0 = t.row * a.Tcap + a.t0 + t.t_start;
    dma_codes<F>(a.codes_in + cell0 * F::CB, t.nv, (lds_u8*)lds_codes, csrc, crow);
    if (lane < t.nv) {
      const uint16_t* sp = a.scales_in + (cell0 + lane) * F::NG;
#pragma unroll
      for (int g = 0; g < F::NG; ++g) s_r[g] = sp[g];
    }
    const float* lr = a.lambda + t.b * a.lambda_sb + t.h * D;
    lam_r0 = lr[lane];
    if (lane + 64 < D) lam_r1 = lr[lane + 64];
  };

  int64_t tile = blockIdx.x;
  if (tile < a.n_tiles) issue(tile);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (; tile < a.n_tiles; tile += gridDim.x) {
    const MTile t = mtile(a, tile);
    uint32_t cw[F::CW];
    if (F::CU == 16) {
#pragma unroll
      for (int q = 0; q < F::NU; ++q) {
        const uint4 w = *reinterpret_cast<const uint4*>(lds_codes + 16 * code_slot<F>(lane, q));
        cw[4 * q] = w.x; cw[4 * q + 1] = w.y; cw[4 * q + 2] = w.z; cw[4 * q + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < F::CB / 8; ++q) {
        const uint2 w = *reinterpret_cast<const uint2*>(lds_codes + lane * F::CB + 8 * q);
        cw[2 * q] = w.x; cw[2 * q + 1] = w.y;
      }
    }
    uint32_t s16[F::NG];
#pragma unroll
    for (int g = 0; g < F::NG; ++g) s16[g] = s_r[g];
    rl_lds[lane] = kScale * __builtin_amdgcn_rcpf(lam_r0);
    if (lane + 64 < D) rl_lds[lane + 64] = kScale * __builtin_amdgcn_rcpf(lam_r1);
    lds_sync();
    const int64_t nxt = tile + gridDim.x;
    if (nxt < a.n_tiles) issue(nxt);

    // code * scale exactly (fma(n, s, -off s) with n = code + off), then
    // times kScale / lambda
    float v[D];
#pragma unroll
    for (int g = 0; g < F::NG; ++g) {
      const float sg = f16_bits_to_f32(s16[g]);
      const float nsg = -kOff * sg;
#pragma unroll
      for (int jj = 0; jj < F::G; jj += 4) {
        const int j = F::G * g + jj;
        const float4 r4 = *reinterpret_cast<const float4*>(rl_lds + j);
        const float rv[4] = {r4.x, r4.y, r4.z, r4.w};
        uint32_t n[4];
        if (F::BITS == 4) {
          // channels j .. j+3 are nibbles 0..3 of word j / 8 when j % 8 == 0,
          // else nibbles 4..7
          const uint32_t wd = cw[j >> 3] >> (4 * (j & 7));
          n[0] = wd & 15u; n[1] = (wd >> 4) & 15u; n[2] = (wd >> 8) & 15u; n[3] = (wd >> 12) & 15u;
        } else {
          const uint32_t wd = cw[j >> 2] ^ 0x80808080u;
          n[0] = wd & 255u; n[1] = (wd >> 8) & 255u; n[2] = (wd >> 16) & 255u; n[3] = wd >> 24;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j + e] = fmaf(static_cast<float>(n[e]), sg, nsg) * rv[e];
      }
    }
    if (ROT == KVQ_ROT_SRFT) mr_fft<M, true>(v);
    const bool valid = lane < t.nv;

    if (F32) {
      if (valid) {
        float* yr = static_cast<float*>(a.y) + t.b * a.sb + t.h * a.sh + (t.t_start + lane) * a.st;
#pragma unroll
        for (int k = 0; k < M; ++k) {
          const int pp = ROT == KVQ_ROT_SRFT ? mr_pos<M>(k) : k;
          const uint32_t m = mix_mask<ROT>(a.signs, k) << 16;
          const float lo = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[2 * pp]) ^ m);
          const float hi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[2 * pp + 1]) ^ m);
          *reinterpret_cast<float2*>(yr + 2 * k) = make_float2(lo, hi);
        }
      }
      // the next tile's loads must land before the loop reads them
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      // the lane's row into the swizzled output tile, signs applied
#pragma unroll
      for (int c = 0; c < G::C; ++c) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * c + e;
          const int pp = ROT == KVQ_ROT_SRFT ? mr_pos<M>(k) : k;
          wv[e] = pack_f16x2(v[2 * pp], v[2 * pp + 1]) ^ mix_mask<ROT>(a.signs, k);
        }
        *reinterpret_cast<uint4*>(lds_out + 16 * (lane * G::C + (c ^ swz<D>(lane)))) =
            make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
      // the next tile's direct loads (the only vector-memory operations
      // since the last stores) have had the dequantization and transform to
      // land; waiting here keeps this tile's stores out of the wait
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_sync();
      char* ybase = reinterpret_cast<char*>(static_cast<uint16_t*>(a.y) + t.b * a.sb + t.h * a.sh +
                                            t.t_start * a.st);
      const int64_t per_step = static_cast<int64_t>(G::RPP) * 2 * a.st;
#pragma unroll
      for (int i = 0; i < G::C; ++i) {
        const int pi = i / G::PER, b = i % G::PER;
        const uint4 w = *reinterpret_cast<const uint4*>(lds_out + 1024 * i + 16 * lane);
        if (rb[b] < t.nv - pi * G::RPP) st_stream16(ybase + pi * per_step + ob[b], w);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// One wave per tile up to 32 waves per CU; larger calls have the waves walk
// the tiles with a stride of the grid, as for D = 128 and 256.
int64_t mix_grid(int64_t n_tiles) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 32;
  return n_tiles < cap ? n_tiles : cap;
}

void fill_mix(MixArgs& a, const CodecDesc& d) {
  a.H = d.H;
  a.T = d.T;
  a.Tcap = d.Tcap;
  a.t0 = d.t0;
  a.sb = d.sb;
  a.sh = d.sh;
  a.st = d.st;
  a.lambda = d.lambda;
  a.lambda_sb = d.lambda_sb;
  a.tiles_per_row = (d.T + 63) / 64;
  a.n_tiles = d.B * d.H * a.tiles_per_row;
  a.div_tpr = make_fastdiv(static_cast<uint64_t>(a.tiles_per_row));
  a.div_h = make_fastdiv(static_cast<uint64_t>(d.H));
  a.signs = d.signs[0];
}

template <int D, int ROT, int FMT>
hipError_t mix_encode_fmt(const CodecDesc& d, int mode) {
  MixArgs a{};
  fill_mix(a, d);
  a.x = d.x;
  a.codes = d.codes;
  a.scales = d.scales;
  a.w = d.w;
  if (a.n_tiles == 0) return hipSuccess;
  if (a.n_tiles >= (int64_t(1) << 32)) return hipErrorInvalidValue;   // index math is 32-bit exact
  const dim3 grid(static_cast<unsigned>(mix_grid(a.n_tiles)));
  if (mode == 1) {
    hipLaunchKernelGGL((mix_encode_kernel<D, ROT, FMT, 1>), grid, dim3(64), 0, d.stream, a);
  } else {
    hipLaunchKernelGGL((mix_encode_kernel<D, ROT, FMT, 0>), grid, dim3(64), 0, d.stream, a);
  }
  return hipGetLastError();
}

template <int D, int ROT, int FMT>
hipError_t mix_decode_fmt(const CodecDesc& d, bool f32) {
  MixArgs a{};
  fill_mix(a, d);
  a.codes_in = d.codes_in;
  a.scales_in = d.scales_in;
  a.y = d.y;
  if (a.n_tiles == 0) return hipSuccess;
  if (a.n_tiles >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(mix_grid(a.n_tiles)));
  if (f32) {
    hipLaunchKernelGGL((mix_decode_kernel<D, ROT, FMT, true>), grid, dim3(64), 0, d.stream, a);
  } else {
    hipLaunchKernelGGL((mix_decode_kernel<D, ROT, FMT, false>), grid, dim3(64), 0, d.stream, a);
  }
  return hipGetLastError();
}

// Format index 2 * (bits == 8) + (G == 16); D = 80 has only the G = 16 ones.
template <int D, int ROT>
hipError_t mix_encode_rot(const CodecDesc& d, int mode) {
  const int fmt = (d.bits == 8 ? 2 : 0) + (d.G == 16 ? 1 : 0);
  if (D == 80 && !(fmt & 1)) return hipErrorInvalidValue;
  switch (fmt) {
    case 1: return mix_encode_fmt<D, ROT, 1>(d, mode);
    case 3: return mix_encode_fmt<D, ROT, 3>(d, mode);
    case 2: return mix_encode_fmt<D, ROT, D == 80 ? 3 : 2>(d, mode);
    default: return mix_encode_fmt<D, ROT, D == 80 ? 1 : 0>(d, mode);
  }
}

template <int D, int ROT>
hipError_t mix_decode_rot(const CodecDesc& d, bool f32) {
  const int fmt = (d.bits == 8 ? 2 : 0) + (d.G == 16 ? 1 : 0);
  if (D == 80 && !(fmt & 1)) return hipErrorInvalidValue;
  switch (fmt) {
    case 1: return mix_decode_fmt<D, ROT, 1>(d, f32);
    case 3: return mix_decode_fmt<D, ROT, 3>(d, f32);
    case 2: return mix_decode_fmt<D, ROT, D == 80 ? 3 : 2>(d, f32);
    default: return mix_decode_fmt<D, ROT, D == 80 ? 1 : 0>(d, f32);
  }
}

template <int D>
hipError_t mix_encode_d(const CodecDesc& d, int mode) {
  if (d.rotation == KVQ_ROT_SRFT) return mix_encode_rot<D, KVQ_ROT_SRFT>(d, mode);
  if (d.rotation == KVQ_ROT_ID) return mix_encode_rot<D, KVQ_ROT_ID>(d, mode);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t mix_decode_d(const CodecDesc& d, bool f32) {
  if (d.rotation == KVQ_ROT_SRFT) return mix_decode_rot<D, KVQ_ROT_SRFT>(d, f32);
  if (d.rotation == KVQ_ROT_ID) return mix_decode_rot<D, KVQ_ROT_ID>(d, f32);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode_mixed(const CodecDesc& d, int mode) {
  if (d.D == 80) return mix_encode_d<80>(d, mode);
  if (d.D == 96) return mix_encode_d<96>(d, mode);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mixed(const CodecDesc& d, bool f32) {
  if (d.D == 80) return mix_decode_d<80>(d, f32);
  if (d.D == 96) return mix_decode_d<96>(d, f32);
  return hipErrorInvalidValue;
}

}  // namespace kvq
