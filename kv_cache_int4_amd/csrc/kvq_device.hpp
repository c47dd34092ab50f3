// Device primitives of the int4 KV-cache codec for CDNA4 (gfx950).
//
// One lane owns 128 real values: a whole D=128 head vector, or one half of a
// D=256 vector (the two halves live in adjacent lanes 2v and 2v+1).  The
// transforms run entirely in VGPRs with compile-time indices, so every
// twiddle factor is an instruction literal and nothing touches scratch.
//
// Method (paper "When Quantization Is Free", gist.science explainer,
// "Methodik" 1-2): SRFT(x) = pack(F diag(s) x) with F the unitary DFT over
// the D/2 complex pairs; the fused kernel then applies the per-channel
// lambda, the per-group abs-max and int4 rounding, and packs two codes per
// byte.  The explainer's kernel runs log2(d/2) radix-2 Stockham passes; here
// the 64-point transform is three radix-4 decimation-in-frequency stages held
// in registers (the data never leaves the lane between stages), and the
// 128-point one adds a radix-2 step across a lane pair.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// ---------------------------------------------------------------------------
// Compile-time twiddle tables: c[e] = cos(2 pi e / N), s[e] = sin(2 pi e / N)
// evaluated in double by a Taylor series on [-pi, pi] and rounded once to
// float; quarter turns are exact.
// ---------------------------------------------------------------------------
struct TwTable {
  float c[128];
  float s[128];
};

constexpr double kPi = 3.14159265358979323846264338327950288;

constexpr double taylor_sin(double x) {
  double t = x, s = x;
  for (int n = 1; n < 30; ++n) {
    t *= -x * x / ((2.0 * n) * (2.0 * n + 1.0));
    s += t;
  }
  return s;
}

constexpr double taylor_cos(double x) {
  double t = 1.0, s = 1.0;
  for (int n = 1; n < 30; ++n) {
    t *= -x * x / ((2.0 * n - 1.0) * (2.0 * n));
    s += t;
  }
  return s;
}

constexpr TwTable make_twiddles(int N) {
  TwTable t{};
  for (int e = 0; e < N; ++e) {
    double x = 2.0 * kPi * e / N;
    if (x > kPi) x -= 2.0 * kPi;
    t.c[e] = static_cast<float>(taylor_cos(x));
    t.s[e] = static_cast<float>(taylor_sin(x));
    if ((4 * e) % N == 0) {
      const int q = (4 * e) / N;
      t.c[e] = q == 0 ? 1.f : (q == 2 ? -1.f : 0.f);
      t.s[e] = q == 1 ? 1.f : (q == 3 ? -1.f : 0.f);
    }
  }
  return t;
}

constexpr TwTable kTw128 = make_twiddles(128);

// Rotation by shears (Paeth): multiplying x + i y by exp(i phi) is the
// product of three shears, x -= tan(phi/2) y, y += sin(phi) x,
// x -= tan(phi/2) y, so a twiddle costs three in-place FMAs instead of two
// products and two FMAs into new registers.  With |phi| <= pi/2 the shear
// factors are at most 1 and the result is as accurate as the direct
// product (within two ulps of the exact rotation).  Factors of the angles
// phi = 2 pi r / 128, |r| <= 32, rounded once to float; r = 0 and the
// quarter turns are exact.
struct ShearTable {
  float t[65];   // tan(phi / 2) at index r + 32
  float s[65];   // sin(phi)
};

constexpr ShearTable make_shears() {
  ShearTable h{};
  for (int r = -32; r <= 32; ++r) {
    const double x = 2.0 * kPi * r / 128.0;
    const double sn = taylor_sin(x), cs = taylor_cos(x);
    h.t[r + 32] = static_cast<float>(sn / (1.0 + cs));
    h.s[r + 32] = static_cast<float>(sn);
  }
  h.t[32] = 0.f; h.s[32] = 0.f;
  h.t[0] = -1.f; h.s[0] = -1.f;
  h.t[64] = 1.f; h.s[64] = 1.f;
  return h;
}

constexpr ShearTable kShear = make_shears();

// (re + i im) *= exp(2 pi i r / 128) in place, |r| <= 32 (r a compile-time
// constant): three FMAs on the operands' own registers, so the step can run
// under a lane mask with no copies where the masked and unmasked values
// meet.
__device__ __forceinline__ void rot_shear(float& re, float& im, int r) {
  if (r == 0) return;
  const float t = kShear.t[r + 32], s = kShear.s[r + 32];
  re = fmaf(-t, im, re);
  im = fmaf(s, re, im);
  re = fmaf(-t, im, re);
}

// (re + i im) *= exp(-+ 2 pi i e / N): INV = false takes the forward kernel
// exp(-2 pi i e / N), INV = true its conjugate.  N divides 128.  The angle
// splits into the nearest quarter turn, applied by renaming the registers
// and flipping signs (folded into the adds that use the result), and a
// rest of at most pi/4, applied by three shears.
template <int N, bool INV>
__device__ __forceinline__ void twiddle(float& re, float& im, int e) {
  e %= N;
  const int A = (INV ? e : (N - e) % N) * (128 / N);   // angle 2 pi A / 128
  const int Q = (A + 16) / 32;                         // nearest quarter turn
  const int r = A - 32 * Q;                            // -16 <= r < 16
  rot_shear(re, im, r);
  const float x = re, y = im;
  switch (Q & 3) {
    case 1: re = -y; im = x; break;     // times i
    case 2: re = -x; im = -y; break;    // times -1
    case 3: re = y; im = -x; break;     // times -i
    default: break;
  }
}

// The same product formed directly (two products, two FMAs into new
// registers): for a twiddle step under a lane mask whose angles exceed the
// range of rot_shear.
template <int N, bool INV>
__device__ __forceinline__ void twiddle_mul(float& re, float& im, int e) {
  e %= N;
  if (e == 0) return;
  const float c = kTw128.c[e * (128 / N)];
  const float s = INV ? -kTw128.s[e * (128 / N)] : kTw128.s[e * (128 / N)];
  // (re + i im)(c - i s) = (re c + im s) + i (im c - re s)
  const float r2 = fmaf(re, c, im * s);
  const float i2 = fmaf(im, c, -(re * s));
  re = r2;
  im = i2;
}

// Base-4 digit reversal of a 64-point index: where the decimation-in-
// frequency transform leaves frequency m.
__host__ __device__ constexpr int rev4(int m) {
  return 16 * (m & 3) + 4 * ((m >> 2) & 3) + (m >> 4);
}

// One radix-4 DIF stage over sub-transforms of length L (v holds 64 complex
// values as v[2p] + i v[2p+1]).
template <int L, bool INV>
__device__ __forceinline__ void dif4_stage(float (&v)[128]) {
  constexpr int Q = L / 4;
#pragma unroll
  for (int base = 0; base < 64; base += L) {
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      const int i0 = base + j, i1 = i0 + Q, i2 = i0 + 2 * Q, i3 = i0 + 3 * Q;
      const float t0r = v[2 * i0] + v[2 * i2], t0i = v[2 * i0 + 1] + v[2 * i2 + 1];
      const float t1r = v[2 * i0] - v[2 * i2], t1i = v[2 * i0 + 1] - v[2 * i2 + 1];
      const float t2r = v[2 * i1] + v[2 * i3], t2i = v[2 * i1 + 1] + v[2 * i3 + 1];
      const float t3r = v[2 * i1] - v[2 * i3], t3i = v[2 * i1 + 1] - v[2 * i3 + 1];
      v[2 * i0] = t0r + t2r;
      v[2 * i0 + 1] = t0i + t2i;
      v[2 * i2] = t0r - t2r;
      v[2 * i2 + 1] = t0i - t2i;
      if (!INV) {  // y1 = t1 - i t3, y3 = t1 + i t3
        v[2 * i1] = t1r + t3i;
        v[2 * i1 + 1] = t1i - t3r;
        v[2 * i3] = t1r - t3i;
        v[2 * i3 + 1] = t1i + t3r;
      } else {     // y1 = t1 + i t3, y3 = t1 - i t3
        v[2 * i1] = t1r - t3i;
        v[2 * i1 + 1] = t1i + t3r;
        v[2 * i3] = t1r + t3i;
        v[2 * i3 + 1] = t1i - t3r;
      }
      twiddle<L, INV>(v[2 * i1], v[2 * i1 + 1], j);
      twiddle<L, INV>(v[2 * i2], v[2 * i2 + 1], 2 * j);
      twiddle<L, INV>(v[2 * i3], v[2 * i3 + 1], 3 * j);
    }
  }
}

// Unnormalized 64-point DFT in registers: input in natural order, output
// frequency m at position rev4(m).  INV selects the conjugate kernel.
template <bool INV>
__device__ __forceinline__ void fft64(float (&v)[128]) {
  dif4_stage<64, INV>(v);
  dif4_stage<16, INV>(v);
  dif4_stage<4, INV>(v);
}

// Unnormalized Walsh-Hadamard transform of 128 reals in Sylvester (natural)
// order: H_2n = [[H_n, H_n], [H_n, -H_n]] applied as log2(128) butterfly
// sweeps.
__device__ __forceinline__ void wht128(float (&v)[128]) {
#pragma unroll
  for (int h = 1; h < 128; h *= 2) {
#pragma unroll
    for (int i = 0; i < 128; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// Register holding local channel j (0..127) after the forward transform.
template <int ROT>
__host__ __device__ constexpr int chan_reg(int j) {
  return ROT == 0 ? 2 * rev4(j >> 1) + (j & 1) : j;
}

// v += sign * (the same register of the partner lane l ^ 1), for every
// register: the radix-2 step between the two halves of a D=256 vector.
__device__ __forceinline__ float pair_fma(float own, float sign) {
  // quad_perm [1,0,3,2]: read the partner lane of each pair
  const float other = __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, own), 0xB1, 0xF, 0xF, false));
  return fmaf(other, sign, own);
}

// The same step on eight registers, the partner read fused into the FMA as
// its DPP operand (v_fmac_f32_dpp: v += sign * v[l ^ 1]), which the
// compiler does not form by itself when the DPP source is the accumulator.
// A DPP read of a register a VALU wrote in the two instructions before
// needs two wait states: the s_nop covers the instructions ahead of the
// block; inside it every instruction reads a register no earlier one of
// the block writes.  Same single rounding as fmaf.
__device__ __forceinline__ void pair_fma8(float* v, float sign) {
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
      : "v"(sign));
}

// pair_fma on all 128 registers of a lane's half vector.
__device__ __forceinline__ void pair_fma_all(float (&v)[128], float sign) {
#pragma unroll
  for (int i = 0; i < 128; i += 8) pair_fma8(v + i, sign);
}

// The radix-2 step between the halves of a D=256 SRFT vector where the odd
// lane's twiddles of frequencies m >= 33 were applied as rotations by the
// opposite angle (a factor -1, which keeps every shear angle within pi/2):
// their register pairs rev4(m) take -sign.  Same form as pair_fma8, one
// sign operand per register.
__device__ __forceinline__ void pair_fma8s(float* v, const float (&sg)[8]) {
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %9 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %10 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %11 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %12 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %13 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %14 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %15 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
      : "v"(sg[0]), "v"(sg[1]), "v"(sg[2]), "v"(sg[3]), "v"(sg[4]), "v"(sg[5]), "v"(sg[6]), "v"(sg[7]));
}

// Whether register j of a lane's 64-point transform output (frequency
// rev4(j / 2)) is one of those rotated by the opposite angle.
__host__ __device__ constexpr bool srft_flipped(int j) { return rev4(j >> 1) >= 33; }

__device__ __forceinline__ void pair_fma_all_srft(float (&v)[128], float sign) {
  const float neg = -sign;
#pragma unroll
  for (int i = 0; i < 128; i += 8) {
    float sg[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sg[k] = srft_flipped(i + k) ? neg : sign;
    pair_fma8s(v + i, sg);
  }
}

// The odd lane's twiddles of the D=256 SRFT step, W_128^(-+m) on frequency
// m (held in register pair rev4(m)): m <= 32 as the rotation itself, m >= 33
// as the rotation by the opposite angle (the factor -1 goes to the pair
// step and to the sign of that lane's output channels).
template <bool INV>
__device__ __forceinline__ void pair_twiddles_srft(float (&v)[128]) {
#pragma unroll
  for (int m = 1; m < 64; ++m) {
    const int r = m <= 32 ? (INV ? m : -m) : (INV ? m - 64 : 64 - m);
    rot_shear(v[2 * rev4(m)], v[2 * rev4(m) + 1], r);
  }
}

// Streaming 16-byte global load / store (touched once: nontemporal hint).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void st_stream16(void* p, const uint4& w) {
  const u32x4_t v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, static_cast<u32x4_t*>(p));
}

// ---------------------------------------------------------------------------
// Index arithmetic
// ---------------------------------------------------------------------------

// Division by a call constant d (1 <= d < 2^32) of n < 2^32 (tile and row
// indices): with M = floor((2^64 - 1) / d) + 1 = ceil(2^64 / d), n * M / 2^64
// exceeds n / d by less than n / 2^64 < 2^-32, while n / d is at least 1/d
// below the next integer, so the high 64 bits of n * M are floor(n / d).
// d = 1 uses M = 0 and returns n.
struct FastDiv {
  uint64_t magic;
  uint64_t d;
};

inline __host__ FastDiv make_fastdiv(uint64_t d) {
  FastDiv f;
  f.d = d;
  f.magic = d <= 1 ? 0 : (~0ull / d) + 1;
  return f;
}

__device__ __forceinline__ uint64_t fdiv(uint64_t n, const FastDiv& f) {
  return f.magic == 0 ? n : __umul64hi(n, f.magic);
}

// ---------------------------------------------------------------------------
// Quantizer helpers
// ---------------------------------------------------------------------------

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default
// rounding mode).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// Two fp32 -> one word of two fp16 (round to nearest even), low half first
// (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 h = __builtin_convertvector((f2){lo, hi}, h2);
  return __builtin_bit_cast(uint32_t, h);
}

// a / Q in fp32, rounded to nearest even (Q = 7 or 127, the code range of
// int4 or int8): the product with fp32(1/Q), then one fused correction by
// the exact residual a - Q * q1.  Three instructions where a division takes
// about ten; the result equals the IEEE quotient for every fp32 a (checked
// on the host over every value of the subnormal range and of whole binades,
// and the method scales exactly between binades).  The quotient is held
// opaque in a register: otherwise the compiler fuses the last fused
// multiply-add with a following conversion to fp16 (v_fma_mixlo_f16), which
// rounds once to fp16 where the scale is fp16 of the rounded fp32 quotient.
template <int Q>
__device__ __forceinline__ float div_by(float a) {
  constexpr float c = 1.0f / static_cast<float>(Q);
  const float q1 = __fmul_rn(a, c);
  const float r = fmaf(-q1, static_cast<float>(Q), a);
  float q = fmaf(r, c, q1);
  asm("" : "+v"(q));
  return q;
}

// 1.5 * 2^23 + 8: adding it to w*r leaves rint_even(w*r) + 8 in the low
// mantissa bits (valid while |w*r| < 2^22; larger values are clamped by the
// integer clamp below).
constexpr float kMagic = 12582920.0f;
constexpr int kMagicLo = 0x4B400000;   // bits of 1.5 * 2^23     (code -8)
constexpr int kMagicHi = 0x4B40000F;   // bits of 1.5 * 2^23 + 15 (code  7)

// Offset nibble of clamp(rint_even(w * r), -8, 7) in the low 4 bits; the
// upper bits hold the constant 0x4B40000 pattern.
__device__ __forceinline__ uint32_t quant_bits(float w, float r) {
  const int b = __builtin_bit_cast(int, fmaf(w, r, kMagic));
  return static_cast<uint32_t>(min(max(b, kMagicLo), kMagicHi));
}

// int8 codes: 1.5 * 2^23 + 128 leaves rint_even(w*r) + 128 in the low byte.
constexpr float kMagic8 = 12583040.0f;
constexpr int kMagic8Hi = 0x4B4000FF;   // bits of 1.5 * 2^23 + 255 (code 127)

// Offset byte of clamp(rint_even(w * r), -128, 127) in the low 8 bits.
__device__ __forceinline__ uint32_t quant_bits8(float w, float r) {
  const int b = __builtin_bit_cast(int, fmaf(w, r, kMagic8));
  return static_cast<uint32_t>(min(max(b, kMagicLo), kMagic8Hi));
}

// Byte of a channel pair: even channel in the low nibble.
__device__ __forceinline__ uint32_t pair_byte(uint32_t lo_bits, uint32_t hi_bits) {
  return lo_bits + (hi_bits << 4);   // low byte = n_even + 16 n_odd, no carry
}

// Four pair bytes (each in the low byte of its argument) -> one code word.
__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

}  // namespace kvq
