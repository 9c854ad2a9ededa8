// device_common.h -- device helpers shared by the forward and backward kernels: element
// types, the step-size transform, rounding to bfloat16 and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace selscan {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|); e^-|x| lies in (0, 1], so nothing
// overflows.  log1p(e) is formed from the rounded sum t = 1 + e as log(t) * e / (t - 1), which
// gives back the bits of e that the sum drops (Goldberg, "What every computer scientist
// should know about floating-point arithmetic", Theorem 4); t == 1 leaves log1p(e) = e.
__device__ __forceinline__ float softplus_f32(float x) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float t = 1.f + e;
  const float lp = (t == 1.f) ? e : __builtin_amdgcn_logf(t) * kLn2 * (e * __builtin_amdgcn_rcpf(t - 1.f));
  return fmaxf(x, 0.f) + lp;
}

// The step size a token uses: delta + bias, through softplus when sp.
__device__ __forceinline__ float step_size(float raw, float bias, bool sp) {
  const float x = raw + bias;
  return sp ? softplus_f32(x) : x;
}

// The zero-order-hold input coefficient (e^x - 1)/a, x = delta * a, of one state with rate
// a != 0 ("state-space models" (aarnphm.xyz), section "From continuous time to tokens";
// Algenta "Sequence and state-space models", ssm_discretize_b), given ab = e^x already
// formed for the transition and ia = 1/a.  ab carries an error of about one ulp of 1
// whatever x is, so ab - 1 loses relative accuracy as |x| shrinks; from |x| = 1/8 down the
// coefficient is instead delta times the Taylor series of (e^x - 1)/x = 1 + x/2 + x^2/6 +
// x^3/24 + x^4/120 (truncation below 5e-8 relative at |x| = 1/8), and above it (ab - 1)/a
// is one fma, within about 1e-6 relative.  a == 0 (with ia == 0) gives x = 0: delta, the
// coefficient's limit.
__device__ __forceinline__ float zoh_coeff_exact(float dd, float a, float ia, float ab) {
  const float x = dd * a;
  const float ser = dd * fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.f / 120.f, 1.f / 24.f), 1.f / 6.f), 0.5f), 1.f);
  return fabsf(x) < 0.125f ? ser : fmaf(ab, ia, -ia);
}

// Rates below this magnitude (zero included) send a wavefront to the form above for every
// step.  The one-fma form (ab - 1)/a alone is kept where every rate a wavefront owns is at
// least this large: its relative error is about 2^-23 / |delta a|, 5e-4 at the smallest
// step of the canonical initialisation (delta = 1e-3) and this rate, less for larger ones.
constexpr float kSmallRate = 0.25f;

// element types: per-token tensors travel as raw bit patterns (see the buffer loads in the
// forward kernels) and are widened to fp32 when staged.

template <typename IO> struct io_traits;
template <> struct io_traits<float> {
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ float widen(float v) { return v; }
  static __device__ __forceinline__ float from_raw(uint32_t r) { return __uint_as_float(r); }
};
template <> struct io_traits<uint16_t> {   // bfloat16 bit patterns
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
  static __device__ __forceinline__ float from_raw(uint32_t r) { return __uint_as_float(r << 16); }
};

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t x = __float_as_uint(v);
  const uint32_t r = ((x & 0x7fffffffu) > 0x7f800000u) ? ((x >> 16) | 0x40u) : ((x + 0x7fffu + ((x >> 16) & 1u)) >> 16);
  return uint16_t(r);
}

// Blocks are dealt round-robin to the 8 XCDs; remap so that each XCD gets a contiguous
// range of work items (neighbouring channel groups of one batch row share B/C rows and
// the cache lines of u/delta/z/y, and those live in that XCD's L2).
__device__ __forceinline__ int xcd_contiguous_block(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int per = nblocks / kXcd, rem = nblocks % kXcd;
  const int xcd = bid % kXcd, pos = bid / kXcd;
  return (xcd < rem) ? xcd * (per + 1) + pos : rem * (per + 1) + (xcd - rem) * per + pos;
}

}  // namespace
}  // namespace selscan
