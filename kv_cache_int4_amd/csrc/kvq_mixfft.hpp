// Mixed-radix complex DFT of length M in registers, for head dimensions D =
// 2M that are not powers of two (D = 80: M = 40 = 4*2*5; D = 96: M = 48 =
// 4*4*3).  The pages prefer the Fourier transform to the Walsh-Hadamard one
// precisely because a DFT exists at every length, not only at powers of two
// (paper abstract); the rotation is the same unitary SRFT as at D = 128,
// factored over radices 2, 3, 4 and 5 instead of 4 alone.
//
// Decimation in frequency, first stage on the full length: a stage of radix
// r on sub-transforms of length L (Q = L / r) takes a_p = v[base + j + pQ],
// forms the r-point DFT y_k = sum_p a_p w_r^{pk}, multiplies y_k by the
// twiddle W_L^{jk} and stores it at base + j + kQ.  After all stages,
// frequency m sits at position mr_pos(m) (mixed-radix digit reversal).
// Every index is a compile-time constant once the loops unroll, so the
// twiddles become instruction literals.  The functions are host-callable so
// that the index logic can be checked against a library FFT on the CPU.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

// cos / sin (2 pi e / N) for e < N, from the Taylor series of kvq_device.hpp
// (double, rounded once to float); quarter turns are exact.
template <int N>
struct TwN {
  float c[N];
  float s[N];
};

template <int N>
constexpr TwN<N> make_twn() {
  TwN<N> t{};
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

template <int N>
struct TwHold {
  static constexpr TwN<N> t = make_twn<N>();
};

// Radices of a supported length, first stage first.
template <int M>
struct MixRadix;
template <>
struct MixRadix<48> {
  static constexpr int r0 = 4, r1 = 4, r2 = 3;
};
template <>
struct MixRadix<40> {
  static constexpr int r0 = 4, r1 = 2, r2 = 5;
};

template <int M>
__host__ __device__ constexpr int mr_radix(int s) {
  return s == 0 ? MixRadix<M>::r0 : s == 1 ? MixRadix<M>::r1 : s == 2 ? MixRadix<M>::r2 : 1;
}

// Position of frequency m after the stages s .. 2 on a block of length L.
template <int M>
__host__ __device__ constexpr int mr_pos_from(int m, int s, int L) {
  return s == 3 ? 0 : (m % mr_radix<M>(s)) * (L / mr_radix<M>(s)) +
                          mr_pos_from<M>(m / mr_radix<M>(s), s + 1, L / mr_radix<M>(s));
}

template <int M>
__host__ __device__ constexpr int mr_pos(int m) {
  return mr_pos_from<M>(m, 0, M);
}

// 1 / sqrt(n) in double by Newton's iteration (compile time).
constexpr double const_rsqrt(double n) {
  double y = 1.0 / n;
  for (int i = 0; i < 100; ++i) y = y * (1.5 - 0.5 * n * y * y);
  return y;
}

// Shear factors of the rotations by 2 pi k / (4 N), |k| <= N / 2 (at most
// an eighth of a turn), at index k + N / 2: tan of half the angle and its
// sine, in double, rounded once to float.
template <int N>
struct ShearN {
  float t[N + 1];
  float s[N + 1];
};

template <int N>
constexpr ShearN<N> make_shear_n() {
  ShearN<N> h{};
  for (int k = -N / 2; k <= N / 2; ++k) {
    const double x = 2.0 * kPi * k / (4.0 * N);
    const double sn = taylor_sin(x), cs = taylor_cos(x);
    h.t[k + N / 2] = static_cast<float>(sn / (1.0 + cs));
    h.s[k + N / 2] = static_cast<float>(sn);
  }
  return h;
}

template <int N>
struct ShearHold {
  static constexpr ShearN<N> h = make_shear_n<N>();
};

// (re + i im) * exp(-+ 2 pi i e / N): INV = false takes the forward kernel.
// As the power-of-two twiddles: the nearest quarter turn by renaming and
// sign flips (folded into the adds that use the result), the rest, at most
// an eighth of a turn, by three in-place shears.
template <int N, bool INV>
__host__ __device__ __forceinline__ void mr_rot(float& re, float& im, int e) {
  e %= N;
  const int A = INV ? e : (N - e) % N;        // angle 2 pi A / N
  const int Q = (8 * A + N) / (2 * N);        // nearest quarter turn
  const int k = 4 * A - Q * N;                // rest 2 pi k / (4 N)
  if (k != 0) {
    const float t = ShearHold<N>::h.t[k + N / 2], sn = ShearHold<N>::h.s[k + N / 2];
    re = fmaf(-t, im, re);
    im = fmaf(sn, re, im);
    re = fmaf(-t, im, re);
  }
  const float x = re, y = im;
  switch (Q & 3) {
    case 1: re = -y; im = x; break;     // times i
    case 2: re = -x; im = -y; break;    // times -1
    case 3: re = y; im = -x; break;     // times -i
    default: break;
  }
}

// R-point DFT of (ar, ai) in place, forward kernel w = exp(-2 pi i / R) or
// its conjugate.  Radix 3 and 5 use the symmetric sums a_p + a_{R-p} and
// differences a_p - a_{R-p}, so that each real constant multiplies once.
template <int R, bool INV>
__host__ __device__ __forceinline__ void mr_butterfly(float (&ar)[R], float (&ai)[R]) {
  // sg = +1 for the forward kernel: outputs y_k = m_k - i sg n_k, y_{R-k} =
  // m_k + i sg n_k
  constexpr float sg = INV ? -1.f : 1.f;
  if (R == 2) {
    const float r0 = ar[0] + ar[1 % R], i0 = ai[0] + ai[1 % R];
    const float r1 = ar[0] - ar[1 % R], i1 = ai[0] - ai[1 % R];
    ar[0] = r0; ai[0] = i0; ar[1 % R] = r1; ai[1 % R] = i1;
  } else if (R == 3) {
    constexpr float h = 0.866025403784438646763723170752936183f;   // sin(2 pi / 3)
    const float tr = ar[1 % R] + ar[2 % R], ti = ai[1 % R] + ai[2 % R];
    const float mr = fmaf(-0.5f, tr, ar[0]), mi = fmaf(-0.5f, ti, ai[0]);
    const float nr = sg * h * (ar[1 % R] - ar[2 % R]), ni = sg * h * (ai[1 % R] - ai[2 % R]);
    ar[0] += tr;
    ai[0] += ti;
    // m - i n = (mr + ni) + i (mi - nr)
    ar[1 % R] = mr + ni; ai[1 % R] = mi - nr;
    ar[2 % R] = mr - ni; ai[2 % R] = mi + nr;
  } else if (R == 4) {
    const float t0r = ar[0] + ar[2 % R], t0i = ai[0] + ai[2 % R];
    const float t1r = ar[0] - ar[2 % R], t1i = ai[0] - ai[2 % R];
    const float t2r = ar[1 % R] + ar[3 % R], t2i = ai[1 % R] + ai[3 % R];
    const float t3r = sg * (ar[1 % R] - ar[3 % R]), t3i = sg * (ai[1 % R] - ai[3 % R]);
    ar[0] = t0r + t2r; ai[0] = t0i + t2i;
    ar[2 % R] = t0r - t2r; ai[2 % R] = t0i - t2i;
    ar[1 % R] = t1r + t3i; ai[1 % R] = t1i - t3r;
    ar[3 % R] = t1r - t3i; ai[3 % R] = t1i + t3r;
  } else if (R == 5) {
    constexpr float c1 = TwHold<5>::t.c[1], c2 = TwHold<5>::t.c[2];
    constexpr float s1 = TwHold<5>::t.s[1], s2 = TwHold<5>::t.s[2];
    const float b1r = ar[1 % R] + ar[4 % R], b1i = ai[1 % R] + ai[4 % R];
    const float b2r = ar[2 % R] + ar[3 % R], b2i = ai[2 % R] + ai[3 % R];
    const float d1r = sg * (ar[1 % R] - ar[4 % R]), d1i = sg * (ai[1 % R] - ai[4 % R]);
    const float d2r = sg * (ar[2 % R] - ar[3 % R]), d2i = sg * (ai[2 % R] - ai[3 % R]);
    const float m1r = fmaf(c2, b2r, fmaf(c1, b1r, ar[0])), m1i = fmaf(c2, b2i, fmaf(c1, b1i, ai[0]));
    const float m2r = fmaf(c1, b2r, fmaf(c2, b1r, ar[0])), m2i = fmaf(c1, b2i, fmaf(c2, b1i, ai[0]));
    const float n1r = fmaf(s2, d2r, s1 * d1r), n1i = fmaf(s2, d2i, s1 * d1i);
    const float n2r = fmaf(-s1, d2r, s2 * d1r), n2i = fmaf(-s1, d2i, s2 * d1i);
    ar[0] += b1r + b2r;
    ai[0] += b1i + b2i;
    ar[1 % R] = m1r + n1i; ai[1 % R] = m1i - n1r;
    ar[4 % R] = m1r - n1i; ai[4 % R] = m1i + n1r;
    ar[2 % R] = m2r + n2i; ai[2 % R] = m2i - n2r;
    ar[3 % R] = m2r - n2i; ai[3 % R] = m2i + n2r;
  }
}

// One stage: radix R on blocks of length L of the M complex values
// v[2p] + i v[2p+1].
template <int M, int L, int R, bool INV>
__host__ __device__ __forceinline__ void mr_stage(float (&v)[2 * M]) {
  constexpr int Q = L / R;
#pragma unroll
  for (int base = 0; base < M; base += L) {
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      float ar[R], ai[R];
#pragma unroll
      for (int p = 0; p < R; ++p) {
        ar[p] = v[2 * (base + j + p * Q)];
        ai[p] = v[2 * (base + j + p * Q) + 1];
      }
      mr_butterfly<R, INV>(ar, ai);
#pragma unroll
      for (int k = 0; k < R; ++k) {
        mr_rot<L, INV>(ar[k], ai[k], j * k);
        v[2 * (base + j + k * Q)] = ar[k];
        v[2 * (base + j + k * Q) + 1] = ai[k];
      }
    }
  }
}

// Unnormalized M-point DFT of v (natural order in; frequency m at position
// mr_pos<M>(m) out).  INV selects the conjugate kernel.
template <int M, bool INV>
__host__ __device__ __forceinline__ void mr_fft(float (&v)[2 * M]) {
  using R = MixRadix<M>;
  mr_stage<M, M, R::r0, INV>(v);
  mr_stage<M, M / R::r0, R::r1, INV>(v);
  mr_stage<M, M / (R::r0 * R::r1), R::r2, INV>(v);
}

}  // namespace kvq
