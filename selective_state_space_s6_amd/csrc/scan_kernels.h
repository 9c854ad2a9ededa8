// scan_kernels.h -- gfx950 kernels of the selective-scan forward (S6), as templates.
// Included by scan_kernels.hip (decode step, chunk prefix, launchers) and by the
// scan_inst_<io>_<pass>.hip units, each of which instantiates the scan kernels of one
// element type and one pass so that they compile in parallel.
//
// Recurrence per (batch b, channel d, state n), from a zero (or given) state:
//   Abar = exp(delta * A),  Bbar = (Abar - 1)/A * B  (delta * B when A == 0),
//   h = Abar * h + Bbar * u,  y = sum_n C h + Dskip * u,  y *= z * sigmoid(z).
// The input coefficient (Abar - 1)/A takes one of three forms, chosen once per wavefront:
// one fma from Abar and 1/A; the same with a Taylor series where |delta A| < 1/8
// (zoh_coeff_exact), for wavefronts that own a rate below kSmallRate (zero included); or
// the first-order coefficient Bbar = delta * B (Algenta "Sequence and state-space models",
// mamba_selective_scan_step), an option.  The step size delta + bias[d] through softplus
// (TorchLean "Selective Mamba", step) is another option, applied once per (token, channel)
// where delta is staged.
// Discretisation: "state-space models" (aarnphm.xyz), section "From continuous time to
// tokens" (ZOH); Algenta "Sequence and state-space models", section on state_space_models
// (ssm_discretize_zoh / ssm_discretize_b with the A == 0 fallback).  Selectivity and the
// shared per-token B/C: "state-space models", section "Mamba"; TorchLean "Selective Mamba",
// Parameters.  Readout of the updated state, feed-through, SiLU gate: "Selective Mamba",
// step.  Chunk composition by the associative combine (A1,b1).(A2,b2) = (A2 A1, A2 b1 + b2):
// chipfoundry glossary "State-Space Models & Long-Context Sequence Architectures (Mamba)",
// Appendix Lab 3.
//
// Work decomposition (one wavefront = 64 lanes):
//   lane = (c, s): c in [0, CW) is a channel of the wave's channel group, s in [0, S) a
//   state slot; CW * S = 64.  Lane (c, s) owns the K states n = s + S*k of channel c, held
//   in VGPRs.  The sequence is walked in tiles of 16 tokens.  For each tile the wave loads
//   its operands with plain per-lane global loads (issued one tile ahead) and stages them
//   in a wave-private LDS region: B and C transposed to [n][token] so every lane reads its
//   own state's four consecutive tokens with one 128-bit read, u and delta as [c][token]
//   so the S lanes of a channel read the same 128-bit row (broadcast).  Each step computes
//   a per-lane partial readout p[token] = sum_k C h_k.  After 16 steps the 16 x S partials
//   of a channel are transposed through LDS so that lane (c, s) sums the S partials of
//   tokens s, s+S, ...: every lane then finalises (feed-through, gate, store) 16/S tokens
//   with all 64 lanes busy, instead of one lane in S doing it for every token.
//   No block barrier is used: a wave only ever touches its own LDS region.
//
// Three modes share this code:
//   MODE_SINGLE: scan the whole sequence from h = 0, write y and last_state.
//   MODE_STATE : chunked pass 1 -- scan one chunk from h = 0 without readout; write the
//                chunk's end state and its sum of delta (the chunk's decay is
//                exp(A * sum delta), the product of its Abar).  The last chunk is skipped:
//                its map is never carried into another chunk.
//   MODE_APPLY : chunked pass 2 -- scan one chunk from the carried-in state, write y and,
//                for the final chunk, last_state.
// Between the two chunked passes, chunk_prefix_kernel composes the per-chunk affine maps
// (P, H) with a log-depth scan across the lanes of a wavefront (ds_bpermute shuffles) and
// leaves each chunk's carried-in state.
//
// Time-invariant coefficients (delta[d], B[d,n], C[d,n]) use the same skeleton with a
// scaled state g = h / Bbar (g = Abar g + u; y = sum_n (C Bbar) g), so a step costs two
// fused multiply-adds per state and no exp.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "scan_launch.h"

namespace selscan {
namespace {

constexpr int kTile = 16;        // tokens per tile
constexpr int kRowPad = 20;      // LDS row length (floats) of a 16-token row: 16 + 4 padding
constexpr int kPrefetchMax = 2;  // tiles of global loads kept in flight per wavefront (K <= 2)

enum { MODE_SINGLE = 0, MODE_STATE = 1, MODE_APPLY = 2 };
// Forms of the input coefficient in the cooperative scan, chosen once per wavefront:
// the one-fma ZOH form, the exact ZOH form (zoh_coeff_exact), first order (delta B).
enum { V_FAST = 0, V_EXACT = 1, V_EULER = 2 };

// Order this wave's LDS traffic: every LDS write before the barrier is visible to every
// lane's LDS read after it.  A wave's LDS instructions execute in issue order, so this
// only has to stop the compiler from moving accesses across it.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS floats one wave needs.
template <int S, int K, bool TI>
struct wave_lds {
  static constexpr int CW = 64 / S;
  static constexpr int NP = S * K;                    // padded states per channel
  static constexpr int kB = TI ? 0 : NP * kRowPad;    // sB[NP][20]
  static constexpr int kC = kB;                       // sC[NP][20]
  static constexpr int kU = CW * kRowPad;             // sU[CW][20]
  static constexpr int kD = TI ? 0 : CW * kRowPad;    // sD[CW][20]
  static constexpr int kChan = 21 * S;                // sP channel block: S rows of 20 + S pad
  static constexpr int kP = CW * kChan;               // sP[CW][S][20] (+pad per channel)
  static constexpr int total = kB + kC + kU + kD + kP;
};

// ---------------------------------------------------------------------------------------
// the scan kernel

// Register budget: at least kMinWaves wavefronts per SIMD (512 / kMinWaves VGPRs each).
template <int K> struct occupancy { static constexpr int kMinWaves = K == 1 ? 3 : 2; };

template <typename IO, int S, int K, bool TI, int MODE>
__global__ __launch_bounds__(kWavesPerBlock * 64)
__attribute__((amdgpu_waves_per_eu(occupancy<K>::kMinWaves, 8)))
void scan_kernel(ScanParams p) {
  using T = io_traits<IO>;
  using LDS = wave_lds<S, K, TI>;
  constexpr int CW = LDS::CW;
  constexpr int NP = LDS::NP;
  constexpr int M = kTile / S;          // tokens each lane stages / finalises per tile
  constexpr int NB = (NP * kTile) / 64; // B (and C) tile elements per lane
  constexpr bool READOUT = (MODE != MODE_STATE);
  constexpr int ES = T::kBytes;
  constexpr int kPrefetch = K <= 2 ? kPrefetchMax : 1;

  extern __shared__ __align__(16) float smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane / S, s = lane % S;

  const int item = xcd_contiguous_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wave;
  // The state pass skips the last chunk: its end state is never carried anywhere.
  const int nc_run = MODE == MODE_STATE ? p.n_chunks - 1 : p.n_chunks;
  if (item >= p.batch * nc_run * p.groups) return;       // whole wave exits together
  // item = ((b * nc_run) + chunk) * groups + g : neighbouring items share (b, chunk)
  const int g = item % p.groups;
  const int bc = item / p.groups;
  const int chunk = bc % nc_run;
  const int64_t b = bc / nc_run;

  float* const sB = smem + wave * LDS::total;
  float* const sC = sB + LDS::kB;
  float* const sU = sC + LDS::kC;
  float* const sD = sU + LDS::kU;
  float* const sP = sD + LDS::kD;

  const int64_t D = p.D, N = p.N;
  const int64_t d0 = int64_t(g) * CW;                     // first channel of the group (uniform)
  const int64_t d = d0 + c;
  const bool dvalid = d < D;
  const int64_t l_begin = int64_t(chunk) * p.chunk_len;
  const int64_t l_end = (l_begin + p.chunk_len < p.L) ? l_begin + p.chunk_len : p.L;

  // ---- per-lane constants of the K owned states
  float A2[K], iA[K], Af[K], h[K];
  float Ab[K], CB[K];                 // time-invariant: Abar and C*Bbar, hoisted
  bool any_exact = false;
  float dt_ti = 0.f;
  const IO* const Bti = static_cast<const IO*>(p.B);    // time-invariant: B[d][n], C[d][n]
  const IO* const Cti = static_cast<const IO*>(p.C);
  const float bias_d = (p.delta_bias != nullptr && dvalid) ? p.delta_bias[d] : 0.f;
  if (TI) dt_ti = dvalid ? T::widen(static_cast<const IO*>(p.delta)[d]) : 0.f;
  if (TI && p.dxf && dvalid) dt_ti = step_size(dt_ti, bias_d, p.softplus != 0);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t n = s + S * k;
    const bool ok = dvalid && n < N;
    const float a = ok ? p.A[d * N + n] : 0.f;
    const bool first_order = a == 0.f || p.euler;     // Bbar = delta * B
    A2[k] = a * kLog2e;
    iA[k] = first_order ? 0.f : 1.0f / a;
    Af[k] = p.euler ? 0.f : a;                        // first order: the exact form's x = 0, delta
    any_exact |= (ok && (p.euler || fabsf(a) < kSmallRate));
    h[k] = 0.f;
    if (TI) {
      // Abar = exp(delta a); Bbar = expm1(delta a)/a * B (delta * B when a == 0 or first order)
      const float bv = ok ? T::widen(Bti[d * p.B_sd + n]) : 0.f;
      const float cv = ok ? T::widen(Cti[d * p.C_sd + n]) : 0.f;
      Ab[k] = ok ? expf(dt_ti * a) : 1.f;
      const float coeff = first_order ? dt_ti : expm1f(dt_ti * a) / a;
      CB[k] = ok ? cv * coeff * bv : 0.f;
    } else {
      Ab[k] = 0.f;
      CB[k] = 0.f;
    }
  }
  // wave-uniform: does any owned state need the exact form of the input coefficient
  // (zoh_coeff_exact: a rate below kSmallRate, zero included, or first order)?
  const bool wave_zero = __builtin_amdgcn_readfirstlane(__ballot(any_exact) != 0ull ? 1 : 0) != 0;

  if (MODE == MODE_APPLY) {                // carried-in state (h, or g in time-invariant form)
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t n = s + S * k;
      if (dvalid && n < N) h[k] = p.ws_state[((b * D + d) * N + n) * p.n_chunks + chunk];
    }
  } else if (MODE == MODE_SINGLE && !TI && p.h0 != nullptr) {   // given initial state
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t n = s + S * k;
      if (dvalid && n < N) h[k] = p.h0[(b * D + d) * N + n];
    }
  }

  // ---- buffer resources.  Every per-token tensor is addressed through a buffer descriptor
  // whose base is this work item's first token (and, for u/delta/z/y, its first channel)
  // and whose size ends at the work item's last valid element.  Each lane keeps a fixed
  // 32-bit offset inside a tile; the tile's position goes into the scalar offset.  Reads
  // past the end (tokens at or after l_end, channels at or after D) return 0 and writes
  // there are dropped by the hardware range check, so no guard code is needed: a zero
  // token (delta = 0, u = 0) leaves the selective state unchanged (Abar = 1, Bbar = 0).
  constexpr uint32_t kOOB = 0x80000000u;    // an offset beyond every descriptor's size
  constexpr int kRsrcWord3 = 0x00020000;
  const int64_t nrows = l_end - l_begin;
  auto rsrc = [&](const void* base, int64_t sb, int64_t sl, int64_t col0, int64_t ncols) __attribute__((always_inline)) {
    const char* p0 = static_cast<const char*>(base) + (b * sb + l_begin * sl + col0) * ES;
    const int64_t bytes = nrows > 0 ? ((nrows - 1) * sl + ncols) * ES : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p0), (short)0, int(bytes), kRsrcWord3);
  };
  const int64_t z_sb = p.z != nullptr ? p.z_sb : p.u_sb, z_sl = p.z != nullptr ? p.z_sl : p.u_sl;
  const auto rU = rsrc(p.u, p.u_sb, p.u_sl, d0, D - d0);
  const auto rD = rsrc(p.delta, p.delta_sb, p.delta_sl, d0, D - d0);
  // without a gate the z loads re-read u (always valid memory) and are ignored
  const auto rZ = rsrc(p.z != nullptr ? p.z : p.u, z_sb, z_sl, d0, D - d0);
  const auto rY = rsrc(p.y, p.y_sb, p.y_sl, d0, D - d0);
  const auto rBd = rsrc(p.B, p.B_sb, p.B_sl, 0, N);
  const auto rCd = rsrc(p.C, p.C_sb, p.C_sl, 0, N);

  // per-lane offsets: token s + S m of the tile, channel c (out of range when d >= D)
  uint32_t offU[M], offD[M], offZ[M], offY[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int64_t tl = s + S * m;
    offU[m] = dvalid ? uint32_t((tl * p.u_sl + c) * ES) : kOOB;
    offD[m] = dvalid ? uint32_t((tl * p.delta_sl + c) * ES) : kOOB;
    offZ[m] = dvalid ? uint32_t((tl * z_sl + c) * ES) : kOOB;
    offY[m] = dvalid ? uint32_t((tl * p.y_sl + c) * ES) : kOOB;
  }
  // B/C tile element r of this lane: token tl0 + r * (64 / NP), state n0 (the same state for
  // every r, since NP divides 64).  The per-row part of the address is a scalar offset.
  static_assert(64 % NP == 0, "padded state count must divide the wavefront");
  constexpr int kRowsPerLoad = 64 / NP;
  const int tl0 = lane / NP, n0 = lane % NP;
  const uint32_t maskB = n0 < N ? 0xffffffffu : 0u;   // padded state slots read as zero
  const uint32_t offB0 = uint32_t((tl0 * p.B_sl + (n0 < N ? n0 : 0)) * ES);
  const uint32_t offC0 = uint32_t((tl0 * p.C_sl + (n0 < N ? n0 : 0)) * ES);

  // ---- staging registers: kPrefetch tiles of loads in flight, kept as raw bit patterns
  // (widened when staged into LDS, so no instruction waits on a load before then).
  uint32_t xB[kPrefetch][TI ? 1 : NB], xC[kPrefetch][TI ? 1 : NB];
  uint32_t xU[kPrefetch][M], xD[kPrefetch][M], xZ[kPrefetch][M];
  const bool gate = (p.z != nullptr) && READOUT;
  const bool has_d = (p.Dskip != nullptr) && READOUT;
  const float dskip = (has_d && dvalid) ? p.Dskip[d] : 0.f;

  auto load_raw = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t voff, int64_t soff) __attribute__((always_inline)) -> uint32_t {
    if (ES == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, voff, int(soff), 0);
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, int(soff), 0);
  };
  auto store_y = [&](float v, uint32_t voff, int64_t soff) __attribute__((always_inline)) {
    if (ES == 2) {
      // round to nearest even; NaN stays a quiet NaN
      const uint32_t x = __float_as_uint(v);
      const uint32_t rr = ((x & 0x7fffffffu) > 0x7f800000u) ? ((x >> 16) | 0x40u)
                                                            : ((x + 0x7fffu + ((x >> 16) & 1u)) >> 16);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)rr, rY, voff, int(soff), 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rY, voff, int(soff), 0);
    }
  };

  // Issue the loads of tile t (0-based within the work item) into register set SET.
  auto load_tile = [&](int64_t t, auto set_tag) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;
    const int64_t row0 = t * kTile;
    if (!TI) {
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        const int64_t row = row0 + int64_t(kRowsPerLoad) * r;
        xB[SET][r] = load_raw(rBd, offB0, row * p.B_sl * ES);
        if (READOUT) xC[SET][r] = load_raw(rCd, offC0, row * p.C_sl * ES);
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      xU[SET][m] = load_raw(rU, offU[m], row0 * p.u_sl * ES);
      if (!TI) xD[SET][m] = load_raw(rD, offD[m], row0 * p.delta_sl * ES);
      if (READOUT) xZ[SET][m] = load_raw(rZ, offZ[m], row0 * z_sl * ES);
    }
  };

  // Steps of the recurrence on the staged tile.  FULL: all 16 tokens; otherwise only the
  // first `nsteps` (a uniform count).  The tile is walked in four groups of four
  // tokens; the LDS operands of group q+1 are read while group q computes, and a scheduling
  // barrier between groups keeps the compiler from hoisting every read of the tile.  Each
  // group's four partial readouts go straight to this lane's row of sP.
  float* const prow = sP + c * LDS::kChan + s * kRowPad;
  auto compute_tile = [&](auto zero_tag, auto full_tag, int64_t nsteps) __attribute__((always_inline)) {
    constexpr bool ZERO = decltype(zero_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    float4 u4[2], d4[2], b4[2][K], c4[2][K];
    auto read_group = [&](int q, int buf) __attribute__((always_inline)) {
      u4[buf] = *reinterpret_cast<const float4*>(sU + c * kRowPad + 4 * q);
      if (!TI) {
        d4[buf] = *reinterpret_cast<const float4*>(sD + c * kRowPad + 4 * q);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          b4[buf][k] = *reinterpret_cast<const float4*>(sB + (s + S * k) * kRowPad + 4 * q);
          if (READOUT) c4[buf][k] = *reinterpret_cast<const float4*>(sC + (s + S * k) * kRowPad + 4 * q);
        }
      }
    };
    read_group(0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cur = q & 1;
      if (q + 1 < 4) read_group(q + 1, cur ^ 1);
      const float uu[4] = {u4[cur].x, u4[cur].y, u4[cur].z, u4[cur].w};
      float pacc[4] = {0.f, 0.f, 0.f, 0.f};
      if (TI) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!FULL && 4 * q + j >= nsteps) break;
          float acc = 0.f;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            h[k] = fmaf(Ab[k], h[k], uu[j]);                 // g = Abar g + u
            if (READOUT) acc = fmaf(CB[k], h[k], acc);       // y += C Bbar g
          }
          pacc[j] = acc;
        }
      } else {
        const float dd[4] = {d4[cur].x, d4[cur].y, d4[cur].z, d4[cur].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!FULL && 4 * q + j >= nsteps) break;
          float acc = 0.f;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            const float bj = j == 0 ? b4[cur][k].x : j == 1 ? b4[cur][k].y : j == 2 ? b4[cur][k].z : b4[cur][k].w;
            const float ab = __builtin_amdgcn_exp2f(dd[j] * A2[k]);   // Abar = exp(delta A)
            const float f = ZERO ? zoh_coeff_exact(dd[j], Af[k], iA[k], ab)   // exact form, or delta
                                 : fmaf(ab, iA[k], -iA[k]);                     // (Abar - 1)/A
            h[k] = fmaf(ab, h[k], f * (bj * uu[j]));                   // h = Abar h + Bbar u
            if (READOUT) {
              const float cj = j == 0 ? c4[cur][k].x : j == 1 ? c4[cur][k].y : j == 2 ? c4[cur][k].z : c4[cur][k].w;
              acc = fmaf(cj, h[k], acc);                               // C . h (updated state)
            }
          }
          pacc[j] = acc;
        }
      }
      if (READOUT) *reinterpret_cast<float4*>(prow + 4 * q) = make_float4(pacc[0], pacc[1], pacc[2], pacc[3]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  float dsum = 0.f;                         // MODE_STATE: sum of delta over the chunk
  const int64_t ntiles = (nrows + kTile - 1) / kTile;
  const int64_t last_steps = nrows - (ntiles - 1) * kTile;   // tokens in the final tile
  using true_t = std::integral_constant<bool, true>;
  using false_t = std::integral_constant<bool, false>;

  // One tile: stage set SET into LDS, refill SET with tile t + kPrefetch, run the steps,
  // reduce the partial readouts and finalise this lane's tokens.
  auto process = [&](int64_t t, auto set_tag, auto zero_tag) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;
    wave_lds_sync();                        // previous tile's LDS reads are done
    if (!TI) {
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        const int tl = tl0 + kRowsPerLoad * r;
        sB[n0 * kRowPad + tl] = T::from_raw(xB[SET][r] & maskB);
        if (READOUT) sC[n0 * kRowPad + tl] = T::from_raw(xC[SET][r] & maskB);
      }
    }
    float uo[M], zo[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float fu = T::from_raw(xU[SET][m]);
      sU[c * kRowPad + s + S * m] = fu;
      if (!TI) {
        float fd = T::from_raw(xD[SET][m]);
        if (p.dxf) fd = step_size(fd, bias_d, p.softplus != 0);   // once per (token, channel)
        sD[c * kRowPad + s + S * m] = fd;
        if (MODE == MODE_STATE) dsum += fd;      // lane sums its own tokens; reduced below
      }
      uo[m] = fu;
      zo[m] = gate ? T::from_raw(xZ[SET][m]) : 0.f;
    }
    if (t + kPrefetch < ntiles) load_tile(t + kPrefetch, set_tag);   // keep the ring full
    wave_lds_sync();

    // The ragged final tile runs only its real tokens: operands given with a zero token
    // stride (a per-channel delta, say) do not read as zero past the end.
    if (t == ntiles - 1 && last_steps < kTile) compute_tile(zero_tag, false_t{}, last_steps);
    else compute_tile(zero_tag, true_t{}, kTile);

    if (READOUT) {
      // ---- transpose the partial readouts of this channel: lane (c, s) -> tokens s + S m
      wave_lds_sync();
      const int64_t soff_y = t * kTile * p.y_sl * ES;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int tl = s + S * m;
        const float* col = sP + c * LDS::kChan + tl;
        float yv = col[0];
#pragma unroll
        for (int r = 1; r < S; ++r) yv += col[r * kRowPad];
        yv = fmaf(dskip, uo[m], yv);                                   // + D u
        if (gate) {
          const float zz = zo[m];
          const float sig = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zz * kLog2e));
          yv *= zz * sig;                                              // * SiLU(z)
        }
        store_y(yv, offY[m], soff_y);        // dropped past l_end or for d >= D
      }
    }
  };

  // The tile loop, for one of the two forms of the input coefficient (a wave-uniform
  // choice made once: waves with a small or zero rate, or first order, take the exact form).
  auto run = [&](auto zero_tag) __attribute__((always_inline)) {
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1 % kPrefetch>;
    using I2 = std::integral_constant<int, 2 % kPrefetch>;
    if (0 < ntiles) load_tile(0, I0{});
    if (kPrefetch > 1 && 1 < ntiles) load_tile(1, I1{});
    if (kPrefetch > 2 && 2 < ntiles) load_tile(2, I2{});
    for (int64_t t0 = 0; t0 < ntiles; t0 += kPrefetch) {
      process(t0, I0{}, zero_tag);
      if (kPrefetch > 1 && t0 + 1 < ntiles) process(t0 + 1, I1{}, zero_tag);
      if (kPrefetch > 2 && t0 + 2 < ntiles) process(t0 + 2, I2{}, zero_tag);
    }
  };
  static_assert(kPrefetch >= 1 && kPrefetch <= 3, "the ring prologue issues up to three tiles");
  if (wave_zero) run(true_t{});
  else run(false_t{});

  // ---- outputs that follow the last token of the work item
  if (MODE == MODE_STATE) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t n = s + S * k;
      if (dvalid && n < N) p.ws_state[((b * D + d) * N + n) * p.n_chunks + chunk] = h[k];
    }
    float sum;
    if (TI) {
      sum = dt_ti * float(l_end - l_begin);
    } else {   // every lane of channel c summed its own 16/S tokens of each tile: add them up
      sum = dsum;
#pragma unroll
      for (int off = 1; off < S; off <<= 1) sum += __shfl_xor(sum, off, S);
    }
    if (dvalid && s == 0) p.ws_dsum[(b * D + d) * p.n_chunks + chunk] = sum;
  } else if (p.last_state != nullptr && (MODE == MODE_SINGLE || chunk == p.n_chunks - 1)) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t n = s + S * k;
      if (dvalid && n < N) {
        float hv = h[k];
        if (TI) {   // h = Bbar * g
          const float a = p.A[d * N + n];
          const float bv = T::widen(Bti[d * p.B_sd + n]);
          const float coeff = (a != 0.f && !p.euler) ? expm1f(dt_ti * a) / a : dt_ti;
          hv = coeff * bv * hv;
        }
        p.last_state[(b * D + d) * N + n] = hv;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// The cooperative, software-pipelined scan.  Used when 16 lanes share a channel (N > 8),
// D % 4 == 0, u/delta/z/y rows sit on 4-element boundaries and per-token B/C rows can be
// read four states at a time (N % 4 == 0; always for time-invariant coefficients).
//
// A workgroup of 4 wavefronts (2 for time-invariant coefficients) owns 16 (8) neighbouring
// channels of one (batch row, chunk); wavefront w steps channels 4w .. 4w+3 exactly as scan_kernel does (lane (c, s)
// owns states s + 16 k of channel c, held in VGPRs).  What the four wavefronts share is the
// movement of data: each 16-token tile of u, delta, z, B and C is fetched ONCE per
// workgroup -- one 8-byte (bf16) or 16-byte (fp32) access per lane covers 4 channels of one
// token (or 4 states of B/C) -- and staged in LDS, and y leaves as one 32- or 64-byte row
// segment per token.  A wavefront owning only 4 channels would otherwise make one memory
// request per token row for 8 useful bytes; sharing cuts those requests by 4 and moves the
// per-tile staging work off three of the four wavefronts.  The roles (which tensor a
// wavefront fetches and stages, which one stores y) are fixed per wavefront and chosen
// through its descriptors and LDS destinations, so every wavefront runs the same code.
//
// Iteration t of the tile loop starts with one workgroup barrier and runs three
// independent streams:
//   finalise tile t-1   its partial readouts (private to the wavefront), D u, gate, y into
//                       the shared y tile; the y tile of t-2 is stored
//   stage tile t+1      LDS writes of the loads issued NS iterations earlier; loads of
//                       tile t+1+NS issued
//   steps of tile t     four groups of four tokens, each group's operands read one
//                       scheduling region ahead
// Staged tiles rotate over three LDS buffers (t mod 3): a tile is written in iteration t-1,
// stepped in iteration t and read by its finalise in iteration t+1.  The y tile alternates
// over two.  The partial-readout block is single: its finalise reads are issued before the
// steps overwrite it (a wavefront's LDS accesses run in issue order, and a compiler fence
// keeps that order).  Full tiles run in the loop; a ragged last tile runs after it with a
// step count (its padded tokens must not touch the state).
//
// Partial readouts (selective coefficients): before the LDS transpose, the readouts of
// states s and s ^ 1 are summed across the lane pair (a DPP add), so each channel's block
// holds 8 state-pair rows: half the LDS bytes of the transpose and 7 instead of 15 adds in
// the finalise, for 16 DPP adds per tile.  Time-invariant coefficients (a few VALU per state
// and token, their K states already summed in the lane) keep 16 rows.
//
// Issue priority: a compute unit holds two or three workgroups at once, and its arbiter
// prefers the oldest wavefront, so the first workgroup dealt to a compute unit ran ahead and
// the last one finished its sequence alone, with one wavefront per SIMD to hide latency.  The
// workgroups sharing a compute unit therefore take turns at the top priority: time is cut
// into slices of 2^11 ticks of the 100 MHz constant clock (20.48 us), and in each slice the
// workgroups of dispatch rounds r, r + 1 and r + 2 (mod 3) hold priorities 3, 2 and 1 (when the
// whole grid is resident at once; a longer grid keeps its compute units full by itself).  This
// changes only the order in which ready instructions issue.  The clock is read after a
// tile's barrier and acted on at the next tile's, so its latency is never waited for.

// LDS block of one channel's partial readouts: 8 (pair-summed, selective) or 16 rows of 16
// tokens, + 8 floats
template <bool TI> struct part_rows { static constexpr int R = TI ? 16 : 8; static constexpr int kChanP = 16 * R + 8; };
constexpr int kFairSliceShift = 11;       // priority rotation slice: 2^11 ticks of the 100 MHz clock

// Wavefronts per workgroup: 4 for selective coefficients (u, delta, z, B, C to share);
// 2 for time-invariant ones, where only u (and z) move per token and the per-tile work is
// small, so fewer barrier partners pay (measured).
template <bool TI> struct coop_width { static constexpr int W = TI ? 2 : 4; };

template <int K, bool TI, int MODE>
struct coop_lds {
  static constexpr bool READOUT = MODE != MODE_STATE;
  static constexpr int W = coop_width<TI>::W;
  static constexpr int kCh = 4 * W;                             // channels per workgroup
  static constexpr int kRowY = kCh + 4;                         // LDS row of the y tile
  static constexpr int NP = 16 * K;
  static constexpr int kT = kCh * kRowPad;                      // one token tile [channels][20]
  static constexpr int kB = TI ? 0 : NP * kRowPad;              // [NP][20]
  static constexpr int kC = (TI || !READOUT) ? 0 : kB;
  static constexpr int kU = kT;
  static constexpr int kD = TI ? 0 : kT;
  static constexpr int kZ = READOUT ? kT : 0;
  static constexpr int kBuf = kB + kC + kU + kD + kZ;           // one staged tile
  static constexpr int kNBuf = 3;
  static constexpr int kT4 = 16 * kRowPad;                      // a token tile of 4 vectors (16 channels)
  static constexpr int kSink = kT4 > kB ? kT4 : kB;             // writes of idle staging lanes and roles
  static constexpr int kP = READOUT ? 4 * part_rows<TI>::kChanP : 0;   // per wavefront
  static constexpr int kY = READOUT ? 2 * kTile * kRowY : 0;    // [2][16 tokens][kRowY]
  static constexpr int total = kNBuf * kBuf + kSink + W * kP + kY;
};

// Four consecutive elements (channels of a token, or states of B/C) as raw bits.
template <typename IO> struct quad_io;
template <> struct quad_io<float> {
  using raw_t = uint32_t __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ raw_t load(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __builtin_bit_cast(raw_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  }
  static __device__ __forceinline__ float get(raw_t v, int j) { return __uint_as_float(v[j]); }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, float4 y) {
    const raw_t v = {__float_as_uint(y.x), __float_as_uint(y.y), __float_as_uint(y.z), __float_as_uint(y.w)};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                           r, voff, soff, 0);
  }
};
template <> struct quad_io<uint16_t> {
  using raw_t = uint32_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ raw_t load(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __builtin_bit_cast(raw_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
  }
  static __device__ __forceinline__ float get(raw_t v, int j) {
    const uint32_t w = v[j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, float4 y) {
    // round to nearest even (v_cvt_pk_bf16_f32)
    const f32x2_t lo = {y.x, y.y}, hi = {y.z, y.w};
    const raw_t v = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t))};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v),
                                          r, voff, soff, 0);
  }
};

// Calls f(std::integral_constant<int, i>) for i = 0 .. n-1.
template <int I, int Nn, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < Nn) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, Nn>(f);
  }
}
template <int Nn, typename F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, Nn>(f); }

// Position of (row r, token j) in a channel's partial-readout block: rows of 16 tokens, the
// four 4-token groups of row r XOR-rotated by (r >> 1) & 3 so that the 128-bit row writes of
// a channel's lanes (its eight even lanes, or all 16) spread evenly over the 32 banks, and the
// column reads of the finalise (a channel block starts 8 banks after the previous one) hit
// every bank twice, the least a 64-lane read can.
__device__ __forceinline__ int part_pos(int r, int j) { return r * 16 + 4 * ((j >> 2) ^ ((r >> 1) & 3)) + (j & 3); }

// The value lane L of this lane's 16-lane row holds (DPP row_newbcast; folded into the VOP2
// instruction that consumes it).
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + L, 0xF, 0xF, false));
}

// Workgroup barrier for LDS traffic only: this wavefront's LDS accesses have completed and
// every wavefront has arrived.  Global loads stay in flight (no vmcnt wait).
__device__ __forceinline__ void block_lds_sync() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// DXF: the step size is transformed (delta + bias, softplus) by the wavefront that stages
// delta, once per (token, channel), before it reaches LDS; a separate instantiation so that
// the plain kernel carries none of it.
template <typename IO, int K, bool TI, int MODE, bool DXF>
__global__ __launch_bounds__(64 * coop_width<TI>::W)
__attribute__((amdgpu_waves_per_eu(occupancy<K>::kMinWaves)))
void scan_kernel_coop(ScanParams p) {
  using T = io_traits<IO>;
  using Qd = quad_io<IO>;
  using LDS = coop_lds<K, TI, MODE>;
  constexpr int W = LDS::W, kCh = LDS::kCh, kRowY = LDS::kRowY;
  constexpr int S = 16, NP = LDS::NP;
  constexpr int QG = NP / 4;                 // 4-state groups per token row
  constexpr int TPL = 64 / QG;               // tokens covered by one B/C load instruction
  constexpr int NL = kTile / TPL;            // B/C loads per lane per tile
  constexpr bool READOUT = LDS::READOUT;
  constexpr int ES = T::kBytes;
  constexpr uint32_t kOOB = 0x80000000u;
  constexpr int kRsrcWord3 = 0x00020000;
  // tiles of global loads in flight: measured best at 3 for both element types (fp32 at 130
  // VGPRs, within the three wavefronts per SIMD its grids take); 1 for 64 states per channel
  constexpr int NS = K >= 4 ? 1 : 3;
  // the loop is unrolled by six (below): a tile's load set, (t + 1) mod NS at its issue and at
  // its staging NS iterations later, is the same compile-time residue only if NS divides 6
  static_assert(6 % NS == 0, "load depth must divide the six-fold unroll");

  extern __shared__ __align__(16) float smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane / S, s = lane % S;      // step layout: channel 4w + c, state slot s
  const int it = lane >> 2, ic = lane & 3;   // finalise layout: token it, channel 4w + ic
  const int vr = lane & 15, vq = lane >> 4;  // tile I/O layout: token vr, channels 4vq .. 4vq+3

  const int64_t groups = (p.D + kCh - 1) / kCh;
  const int64_t wg = xcd_contiguous_block(blockIdx.x, gridDim.x);
  // The state pass skips the last chunk (its end state is never carried anywhere) unless
  // it checkpoints every chunk's tiles.
  const int nc_run = MODE == MODE_STATE && !p.state_all ? p.n_chunks - 1 : p.n_chunks;
  if (wg >= p.batch * nc_run * groups) return;               // whole workgroup exits together
  const int64_t g = wg % groups;
  const int64_t bc = wg / groups;
  const int chunk = int(bc % nc_run);
  const int64_t b = bc / nc_run;

  const int64_t D = p.D, N = p.N;
  const int64_t d0 = g * kCh;                // first channel of the workgroup
  const int64_t d = d0 + 4 * w + c;          // channel of the step layout
  const int64_t df = d0 + 4 * w + ic;        // channel of the finalise layout
  const bool dvalid = d < D, fvalid = df < D;
  const bool vvalid = vq < W && d0 + 4 * vq < D;   // D % 4 == 0: a 4-channel vector is all in or all out
  const int64_t l_begin = int64_t(chunk) * p.chunk_len;
  const int64_t l_end = (l_begin + p.chunk_len < p.L) ? l_begin + p.chunk_len : p.L;
  const int64_t nrows = l_end - l_begin;

  // ---- per-lane constants of the K owned states (see scan_kernel)
  float A2[K], iA[K], Af[K], h[K], Ab[K], CB[K];
  bool any_small = false;
  float dt_ti = 0.f;
  const IO* const Bti = static_cast<const IO*>(p.B);
  const IO* const Cti = static_cast<const IO*>(p.C);
  if (TI) dt_ti = dvalid ? T::widen(static_cast<const IO*>(p.delta)[d]) : 0.f;
  if (TI && p.dxf && dvalid)
    dt_ti = step_size(dt_ti, p.delta_bias != nullptr ? p.delta_bias[d] : 0.f, p.softplus != 0);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t n = s + S * k;
    const bool ok = dvalid && n < N;
    const float a = ok ? p.A[d * N + n] : 0.f;
    const bool first_order = a == 0.f || p.euler;     // Bbar = delta * B
    A2[k] = a * kLog2e;
    iA[k] = first_order ? 0.f : 1.0f / a;
    Af[k] = a;
    any_small |= (ok && !p.euler && fabsf(a) < kSmallRate);
    h[k] = 0.f;
    Ab[k] = 0.f;
    CB[k] = 0.f;
    if (TI) {
      const float bv = ok ? T::widen(Bti[d * p.B_sd + n]) : 0.f;
      const float cv = ok ? T::widen(Cti[d * p.C_sd + n]) : 0.f;
      Ab[k] = ok ? expf(dt_ti * a) : 1.f;
      const float coeff = first_order ? dt_ti : expm1f(dt_ti * a) / a;
      CB[k] = ok ? cv * coeff * bv : 0.f;
    }
  }
  // wave-uniform form of the input coefficient: first order; the exact ZOH form (some owned
  // rate below kSmallRate, zero included); or the one-fma ZOH form
  const bool wave_small = __builtin_amdgcn_readfirstlane(__ballot(any_small) != 0ull ? 1 : 0) != 0;
  if (MODE == MODE_APPLY) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t n = s + S * k;
      if (dvalid && n < N) h[k] = p.ws_state[((b * D + d) * N + n) * p.n_chunks + chunk];
    }
  } else if (MODE == MODE_SINGLE && !TI && p.h0 != nullptr) {   // given initial state
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t n = s + S * k;
      if (dvalid && n < N) h[k] = p.h0[(b * D + d) * N + n];
    }
  }

  // ---- buffer resources (see scan_kernel): based at the workgroup's first token and
  // channel, sized to its last element; reads past the end return 0, writes are dropped.
  auto rsrc = [&](const void* base, int64_t sb, int64_t sl, int64_t col0, int64_t ncols) __attribute__((always_inline)) {
    const char* p0 = static_cast<const char*>(base) + (b * sb + l_begin * sl + col0) * ES;
    const int64_t bytes = nrows > 0 ? ((nrows - 1) * sl + ncols) * ES : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p0), (short)0, int(bytes), kRsrcWord3);
  };
  const int64_t z_sb = p.z != nullptr ? p.z_sb : p.u_sb, z_sl = p.z != nullptr ? p.z_sl : p.u_sl;
  const auto rY = rsrc(p.y, p.y_sb, p.y_sl, d0, D - d0);

  // ---- staging roles.  Token-tile role (u, delta, z or none) and B/C-tile role (B, C or
  // none) of this wavefront; an idle role reads past the descriptor (no memory traffic)
  // and writes to an LDS sink.  Wavefront 0 also stores y.  Four wavefronts: u, delta, z
  // (gate only); C (readout only), B.  Two (time-invariant): u, z (gate only).
  static_assert(W == 4 || (W == 2 && TI), "two-wavefront workgroups move no delta, B or C");
  const int roleT = W == 4 ? w : (w == 0 ? 0 : 2);   // 0 u, 1 delta, 2 z, 3 none
  const bool onT = (roleT == 0) || (roleT == 1 && !TI) || (roleT == 2 && READOUT && p.z != nullptr);
  const bool onQ = !TI && ((w == 3) || (w == 2 && READOUT));
  const int64_t slT = roleT == 0 ? p.u_sl : roleT == 1 ? p.delta_sl : z_sl;
  const int64_t slQ = w == 3 ? p.B_sl : p.C_sl;
  const auto rT = roleT == 0 ? rsrc(p.u, p.u_sb, p.u_sl, d0, D - d0)
                : roleT == 1 ? rsrc(p.delta, p.delta_sb, p.delta_sl, d0, D - d0)
                             : rsrc(p.z != nullptr ? p.z : p.u, z_sb, z_sl, d0, D - d0);   // no gate: idle
  const auto rQ = w == 3 ? rsrc(p.B, p.B_sb, p.B_sl, 0, N) : rsrc(p.C, p.C_sb, p.C_sl, 0, N);
  const uint32_t voT = (onT && vvalid) ? uint32_t((vr * slT + 4 * vq) * ES) : kOOB;
  const int qg = lane / TPL, tq = lane % TPL;   // B/C: 4-state group qg of token tq (+TPL per load)
  const uint32_t voQ = (onQ && 4 * qg < N) ? uint32_t((tq * slQ + 4 * qg) * ES) : kOOB;
  const uint32_t voY = (w == 0 && vvalid) ? uint32_t((vr * p.y_sl + 4 * vq) * ES) : kOOB;

  const bool gate = (p.z != nullptr) && READOUT;
  const float dskip = (READOUT && p.Dskip != nullptr && fvalid) ? p.Dskip[df] : 0.f;

  // ---- LDS layout: three staged-tile buffers, the sink, per-wavefront partial readouts,
  // two y tiles
  float* const sStage = smem;
  float* const sSink = smem + LDS::kNBuf * LDS::kBuf;
  float* const sP = sSink + LDS::kSink + w * LDS::kP;
  float* const sY = sSink + LDS::kSink + W * LDS::kP;
  auto bufB = [&](int q) __attribute__((always_inline)) { return sStage + q * LDS::kBuf; };
  auto bufC = [&](int q) __attribute__((always_inline)) { return sStage + q * LDS::kBuf + LDS::kB; };
  auto bufU = [&](int q) __attribute__((always_inline)) { return sStage + q * LDS::kBuf + LDS::kB + LDS::kC; };
  auto bufD = [&](int q) __attribute__((always_inline)) { return bufU(q) + LDS::kU; };
  auto bufZ = [&](int q) __attribute__((always_inline)) { return bufU(q) + LDS::kU + LDS::kD; };
  // this wavefront's staging destinations inside buffer q
  const int offT = !onT ? -1 : roleT == 0 ? LDS::kB + LDS::kC : roleT == 1 ? LDS::kB + LDS::kC + LDS::kU
                                                                  : LDS::kB + LDS::kC + LDS::kU + LDS::kD;
  const int offQ = !onQ ? -1 : w == 3 ? 0 : LDS::kB;
  // lanes of channel vectors beyond the workgroup's W (two-wavefront groups) stage into the sink too
  const bool tlane = offT >= 0 && vq < W;
  // step-size transform: the bias of the four channels this lane stages (delta wavefront)
  static_assert(!(DXF && TI), "time-invariant step sizes are transformed once, at set-up");
  float dbias[4] = {0.f, 0.f, 0.f, 0.f};
  if (DXF && roleT == 1 && vvalid && p.delta_bias != nullptr) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dbias[j] = p.delta_bias[d0 + 4 * vq + j];
  }
  auto dstT = [&](int q) __attribute__((always_inline)) { return tlane ? sStage + q * LDS::kBuf + offT : sSink; };
  auto dstQ = [&](int q) __attribute__((always_inline)) { return offQ < 0 ? sSink : sStage + q * LDS::kBuf + offQ; };

  // ---- load sets: tile t's loads go to set t % NS, issued NS iterations before it is staged
  typename Qd::raw_t xT[NS], xQ[NS][TI ? 1 : NL];
  // tile counts and byte offsets inside a work item fit 32 bits (its span is below 2^30 bytes),
  // so the loop bookkeeping stays on the scalar unit
  const int ntiles = int((nrows + kTile - 1) / kTile);
  const int nfull = int(nrows / kTile);
  const int last_steps = int(nrows) - nfull * kTile;        // tokens of a ragged last tile
  const int tstrideT = kTile * int(slT) * ES, tstrideQ = kTile * int(slQ) * ES;
  // Idle roles load through an offset past their descriptor (no memory traffic) and stage
  // into the sink, so that every wavefront runs the same instruction stream.
  auto issue = [&](int t, auto set_tag) __attribute__((always_inline)) {
    constexpr int P = decltype(set_tag)::value;
    const int tt = t < ntiles ? t : ntiles - 1;               // past the end: reload the last tile
    xT[P] = Qd::load(rT, voT, tt * tstrideT);
    if (!TI) {
#pragma unroll
      for (int r = 0; r < NL; ++r) xQ[P][r] = Qd::load(rQ, voQ, tt * tstrideQ + r * (TPL * int(slQ) * ES));
    }
  };
  // Stage load set SET into LDS buffer q: token tiles channel-major ([c][token]), B/C
  // state-major ([n][token]).
  auto stage = [&](auto set_tag, int q) __attribute__((always_inline)) {
    constexpr int P = decltype(set_tag)::value;
    {
      float* const dt = dstT(q);
      float tv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) tv[j] = Qd::get(xT[P], j);
      if (DXF && roleT == 1) {               // wave-uniform: the delta wavefront
#pragma unroll
        for (int j = 0; j < 4; ++j) tv[j] = step_size(tv[j], dbias[j], p.softplus != 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) dt[(4 * vq + j) * kRowPad + vr] = tv[j];
    }
    if (!TI) {
      float* const dq = dstQ(q);
#pragma unroll
      for (int r = 0; r < NL; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dq[(4 * qg + j) * kRowPad + tq + TPL * r] = Qd::get(xQ[P][r], j);
      }
    }
  };

  // ---- steps: rd(q, grp) reads group grp's
  // operands of the tile in buffer q into register slot grp & 1; cmp(grp) runs its steps
  // and writes its four partial readouts.  Selective coefficients: the 16 lanes of a
  // channel form one DPP row, and lane s holds u and delta of the tile's token s (one
  // 4-byte LDS read each per tile, at group 0); step j of group grp takes them from lane
  // 4 grp + j of the row by a row broadcast folded into the multiply that consumes them.
  // First order (V_EULER) broadcasts delta * u instead of u, formed once per token by the
  // lane that holds it, so that the input term is one multiply.  The exact ZOH form
  // (V_EXACT) and time-invariant coefficients read u and delta four tokens at a time.
  float dsum = 0.f;
  constexpr int kChanP = part_rows<TI>::kChanP, PR = part_rows<TI>::R;
  float* const prow = sP + c * kChanP;
  const int cw = 4 * w + c;                  // step channel within the workgroup
  float4 rU4[2], rD4[2], rB4[2][K], rC4[2][K];
  float rU1 = 0.f, rD1 = 0.f;
  auto rd = [&](int q, auto grp_tag, auto var_tag) __attribute__((always_inline)) {
    constexpr int grp = decltype(grp_tag)::value;
    constexpr int V = decltype(var_tag)::value;
    constexpr bool BC = V != V_EXACT;          // u (or delta u) and delta by row broadcast
    const int sl = grp & 1;
    if (TI || !BC) rU4[sl] = *reinterpret_cast<const float4*>(bufU(q) + cw * kRowPad + 4 * grp);
    if (!TI) {
      if (grp == 0 && BC) {
        rU1 = bufU(q)[cw * kRowPad + s];
        rD1 = bufD(q)[cw * kRowPad + s];
        if (V == V_EULER) rU1 *= rD1;          // delta u of token s
      }
      if (!BC) rD4[sl] = *reinterpret_cast<const float4*>(bufD(q) + cw * kRowPad + 4 * grp);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        rB4[sl][k] = *reinterpret_cast<const float4*>(bufB(q) + (s + S * k) * kRowPad + 4 * grp);
        if (READOUT) rC4[sl][k] = *reinterpret_cast<const float4*>(bufC(q) + (s + S * k) * kRowPad + 4 * grp);
      }
    }
  };
  auto cmp = [&](auto grp_tag, auto var_tag, auto full_tag, int nsteps) __attribute__((always_inline)) {
    constexpr int grp = decltype(grp_tag)::value;
    constexpr int V = decltype(var_tag)::value;
    constexpr bool BC = V != V_EXACT;
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int sl = grp & 1;
    float pacc[4] = {0.f, 0.f, 0.f, 0.f};
    static_for<4>([&](auto j_tag) __attribute__((always_inline)) {
      constexpr int j = decltype(j_tag)::value;
      if (!FULL && 4 * grp + j >= nsteps) return;           // ragged tile: steps past its end
      float acc = 0.f;
      if (TI) {
        const float uu = j == 0 ? rU4[sl].x : j == 1 ? rU4[sl].y : j == 2 ? rU4[sl].z : rU4[sl].w;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          h[k] = fmaf(Ab[k], h[k], uu);                           // g = Abar g + u
          if (READOUT) acc = fmaf(CB[k], h[k], acc);              // y += C Bbar g
        }
      } else {
        // uu: u, or delta u for first order
        const float uu = BC ? row_bcast<4 * grp + j>(rU1)
                            : j == 0 ? rU4[sl].x : j == 1 ? rU4[sl].y : j == 2 ? rU4[sl].z : rU4[sl].w;
        const float dd = BC ? row_bcast<4 * grp + j>(rD1)
                            : j == 0 ? rD4[sl].x : j == 1 ? rD4[sl].y : j == 2 ? rD4[sl].z : rD4[sl].w;
        if (MODE == MODE_STATE) dsum += dd;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float4 b4 = rB4[sl][k];
          const float bj = j == 0 ? b4.x : j == 1 ? b4.y : j == 2 ? b4.z : b4.w;
          const float ab = __builtin_amdgcn_exp2f(dd * A2[k]);     // Abar = exp(delta A)
          if (V == V_EULER) {
            h[k] = fmaf(ab, h[k], bj * uu);                         // h = Abar h + B (delta u)
          } else {
            const float f = V == V_EXACT ? zoh_coeff_exact(dd, Af[k], iA[k], ab)
                                         : fmaf(ab, iA[k], -iA[k]); // (Abar - 1)/A
            h[k] = fmaf(ab, h[k], f * (bj * uu));                   // h = Abar h + Bbar u
          }
          if (READOUT) {
            const float4 c4 = rC4[sl][k];
            const float cj = j == 0 ? c4.x : j == 1 ? c4.y : j == 2 ? c4.z : c4.w;
            acc = fmaf(cj, h[k], acc);                              // C . h (updated state)
          }
        }
      }
      pacc[j] = acc;
    });
    if (READOUT && PR == 16) {
      *reinterpret_cast<float4*>(prow + s * 16 + 4 * (grp ^ ((s >> 1) & 3))) =
          make_float4(pacc[0], pacc[1], pacc[2], pacc[3]);
    } else if (READOUT) {
      // states s and s ^ 1 summed across the lane pair (DPP quad_perm [1,0,3,2]); the even
      // lane writes row s / 2
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pacc[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(pacc[j]), 0xB1, 0xF, 0xF, false));
      // the sums stay in the common block (the compiler would sink them into the even lanes'
      // branch, where the DPP move no longer folds into the add)
#pragma unroll
      for (int j = 0; j < 4; ++j) __asm__ volatile("" : "+v"(pacc[j]));
      if ((s & 1) == 0) {
        const int r = s >> 1;
        *reinterpret_cast<float4*>(prow + r * 16 + 4 * (grp ^ ((r >> 1) & 3))) =
            make_float4(pacc[0], pacc[1], pacc[2], pacc[3]);
      }
    }
  };

  // ---- finalise: the PR (pair-summed) partial readouts of (token it, channel 4w + ic),
  // feed-through and gate with u and z from the staged tile, result into the y tile.
  float part[PR], uF = 0.f, zF = 0.f;
  auto fin_read = [&](int q) __attribute__((always_inline)) {
    const float* const col = sP + ic * kChanP;
#pragma unroll
    for (int r = 0; r < PR; ++r) part[r] = col[part_pos(r, it)];
    uF = bufU(q)[(4 * w + ic) * kRowPad + it];
    zF = bufZ(q)[(4 * w + ic) * kRowPad + it];
  };
  auto fin_sum = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int wd = PR / 2; wd >= 1; wd >>= 1) {
#pragma unroll
      for (int r = 0; r < wd; ++r) part[r] += part[r + wd];
    }
  };
  auto fin_out = [&](int yq) __attribute__((always_inline)) {
    float yv = fmaf(dskip, uF, part[0]);                               // + D u
    // * SiLU(z) = z / (1 + exp(-z)); computed unconditionally and selected, so that the
    // iteration stays one basic block
    const float silu = zF * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zF * kLog2e));
    yv *= gate ? silu : 1.f;
    sY[yq * (kTile * kRowY) + it * kRowY + 4 * w + ic] = yv;
  };
  // store the y tile of tile t from y buffer yq (wavefront 0 only)
  const int tstrideY = kTile * int(p.y_sl) * ES;
  auto y_store = [&](int t, int yq) __attribute__((always_inline)) {
    if (w != 0) return;                                               // wave-uniform
    const float4 yv = *reinterpret_cast<const float4*>(sY + yq * (kTile * kRowY) + vr * kRowY + 4 * (vq < W ? vq : 0));
    Qd::store(rY, voY, t * tstrideY, yv);                             // dropped past l_end
  };
  auto order_lds = [] () __attribute__((always_inline)) { __asm__ __volatile__("" ::: "memory"); };
  auto region = [] () __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };

  using I0 = std::integral_constant<int, 0>;
  using G0 = std::integral_constant<int, 0>;
  using G1 = std::integral_constant<int, 1>;
  using G2 = std::integral_constant<int, 2>;
  using G3 = std::integral_constant<int, 3>;
  using true_t = std::integral_constant<bool, true>;
  using false_t = std::integral_constant<bool, false>;
  auto mod3 = [] (int t) __attribute__((always_inline)) { return t % 3; };

  // One loop iteration for full tile t; SET1 = (t + 1) % NS is compile-time.
  // state pass, optional: the state (from the chunk's zero start) and the running sum of
  // delta at the start of tile t
  auto checkpoint = [&](int t) __attribute__((always_inline)) {
    if constexpr (MODE == MODE_STATE && !TI) {
      if (p.ckpt != nullptr && dvalid) {
        const int64_t tile = l_begin / kTile + t;
        float* const ck = p.ckpt + ((b * p.ck_ntiles + tile) * D + d) * N;
#pragma unroll
        for (int k = 0; k < K; ++k)
          if (s + S * k < N) ck[s + S * k] = h[k];
        if (s == 0) p.ck_dsum[(b * p.ck_ntiles + tile) * D + d] = dsum;
      }
    }
  };
  // the issue-priority turn of this workgroup's dispatch round (see the kernel's header)
  // (only when the whole grid is resident at once, at most four workgroups per compute unit:
  // with more, finished workgroups are replaced and the compute units stay full anyway)
  const bool fair = p.sched_round > 0 && gridDim.x <= 4u * uint32_t(p.sched_round);
  const uint32_t fair_round = fair ? uint32_t(blockIdx.x) / uint32_t(p.sched_round) : 0u;
  uint64_t fair_clock = 0;                     // read after the previous tile's barrier
  auto fair_share = [&]() __attribute__((always_inline)) {
    if (!fair) return;
    const uint32_t ph = (uint32_t(fair_clock >> kFairSliceShift) + fair_round) % 3u;
    if (ph == 0) __builtin_amdgcn_s_setprio(3);
    else if (ph == 1) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(1);
  };
  // RES = t mod 6, known at compile time: the LDS buffers (t mod 3), the y tile (t mod 2) and
  // the load set ((t + 1) mod NS) are constants, folded into the instructions' offsets
  auto iteration = [&](int t, auto res_tag, auto var_tag, auto fin_tag, auto yst_tag) __attribute__((always_inline)) {
    constexpr int RES = decltype(res_tag)::value;
    constexpr bool FIN = decltype(fin_tag)::value && READOUT;
    constexpr bool YST = decltype(yst_tag)::value && READOUT;
    constexpr int q0 = RES % 3, q1 = (RES + 1) % 3, qm = (RES + 2) % 3;   // buffers of t, t+1, t-1
    using SET = std::integral_constant<int, (RES + 1) % NS>;
    checkpoint(t);
    fair_share();
    region();
    block_lds_sync();
    if (fair) fair_clock = __builtin_amdgcn_s_memrealtime();
    if (FIN) fin_read(qm);                             // tile t-1
    if (YST) y_store(t - 2, RES & 1);                  // tile t-2
    order_lds();
    rd(q0, G0{}, var_tag);
    stage(SET{}, q1);                                  // tile t+1
    issue(t + 1 + NS, SET{});
    region();
    rd(q0, G1{}, var_tag);
    cmp(G0{}, var_tag, true_t{}, kTile);
    if (FIN) fin_sum();
    region();
    rd(q0, G2{}, var_tag);
    cmp(G1{}, var_tag, true_t{}, kTile);
    if (FIN) fin_out((RES + 1) & 1);
    region();
    rd(q0, G3{}, var_tag);
    cmp(G2{}, var_tag, true_t{}, kTile);
    region();
    cmp(G3{}, var_tag, true_t{}, kTile);
  };
  // Six iterations from t (t mod 6 == 2), each only while t < nfull when GUARD.
  auto block = [&](int t, auto var_tag, auto guard_tag) __attribute__((always_inline)) {
    constexpr bool GUARD = decltype(guard_tag)::value;
    static_for<6>([&](auto k_tag) __attribute__((always_inline)) {
      constexpr int KK = decltype(k_tag)::value;
      using RES = std::integral_constant<int, (2 + KK) % 6>;
      if (!GUARD || t + KK < nfull) iteration(t + KK, RES{}, var_tag, true_t{}, true_t{});
    });
  };

  auto run = [&](auto var_tag) __attribute__((always_inline)) {
    static_for<NS>([&](auto k_tag) __attribute__((always_inline)) { issue(int(decltype(k_tag)::value), k_tag); });
    stage(I0{}, 0);                                     // tile 0 -> buffer 0
    issue(NS, I0{});
    int t = 0;
    if (nfull > 0) {
      iteration(0, std::integral_constant<int, 0>{}, var_tag, false_t{}, false_t{});
      t = 1;
    }
    if (nfull > 1) {
      iteration(1, std::integral_constant<int, 1>{}, var_tag, true_t{}, false_t{});
      t = 2;
    }
    for (; t + 6 <= nfull; t += 6) block(t, var_tag, false_t{});
    if (t < nfull) {
      block(t, var_tag, true_t{});
      t = nfull;
    }
    if (!READOUT) {                                     // state pass: only the ragged tile is left
      if (last_steps > 0) {
        checkpoint(nfull);
        block_lds_sync();
        const int qr = mod3(nfull);
        static_for<4>([&](auto g_tag) __attribute__((always_inline)) {
          rd(qr, g_tag, var_tag);
          cmp(g_tag, var_tag, false_t{}, last_steps);
        });
      }
      return;
    }
    // drain: finalise tile nfull-1 and store tile nfull-2; the ragged tile (staged in buffer
    // nfull % 3) runs its steps; then tile nfull-1's y, then the ragged tile's finalise
    block_lds_sync();
    if (nfull > 0) fin_read(mod3(nfull + 2));
    if (nfull > 1) y_store(nfull - 2, int(nfull & 1));
    order_lds();
    if (last_steps > 0) {
      const int qr = mod3(nfull);
      static_for<4>([&](auto g_tag) __attribute__((always_inline)) {
        rd(qr, g_tag, var_tag);
        cmp(g_tag, var_tag, false_t{}, last_steps);
      });
    }
    if (nfull > 0) {
      fin_sum();
      fin_out(int((nfull - 1) & 1));
    }
    block_lds_sync();
    if (nfull > 0) y_store(nfull - 1, int((nfull - 1) & 1));
    if (last_steps > 0) {
      fin_read(mod3(nfull));
      fin_sum();
      fin_out(int(nfull & 1));
      block_lds_sync();
      y_store(nfull, int(nfull & 1));
    }
  };
  if constexpr (TI) {
    run(std::integral_constant<int, V_FAST>{});
  } else {
    if (p.euler) run(std::integral_constant<int, V_EULER>{});
    else if (wave_small) run(std::integral_constant<int, V_EXACT>{});
    else run(std::integral_constant<int, V_FAST>{});
  }

  // ---- outputs after the last token (see scan_kernel)
  if (MODE == MODE_STATE) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t n = s + S * k;
      if (dvalid && n < N) p.ws_state[((b * D + d) * N + n) * p.n_chunks + chunk] = h[k];
    }
    const float sum = TI ? dt_ti * float(nrows) : dsum;     // every lane of c summed all tokens
    if (dvalid && s == 0) p.ws_dsum[(b * D + d) * p.n_chunks + chunk] = sum;
  } else if (p.last_state != nullptr && (MODE == MODE_SINGLE || chunk == p.n_chunks - 1)) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t n = s + S * k;
      if (dvalid && n < N) {
        float hv = h[k];
        if (TI) {
          const float a = p.A[d * N + n];
          const float bv = T::widen(Bti[d * p.B_sd + n]);
          const float coeff = (a != 0.f && !p.euler) ? expm1f(dt_ti * a) / a : dt_ti;
          hv = coeff * bv * hv;
        }
        p.last_state[(b * D + d) * N + n] = hv;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// One recurrent decode step: a single token per batch row, state [batch][D][N] updated in
// place (the recurrent form of the scan; aarnphm "state-space models", section "One
// recurrence, one convolution").  Moves the state in and out once: bound by HBM.
// Lane (c, s) owns states 4s .. 4s+3 of channel c of the wavefront's channel group (SL
// lanes per channel, 64/SL channels), so a channel's state row moves as 16-byte accesses;
// A and its derived constants stay in registers while the wavefront walks kStepRows batch
// rows, issuing every row's loads before computing any.  The readout is summed over the
// SL lanes of a channel with cross-lane adds; lane s == 0 adds the feed-through, applies
// the gate and stores y.
constexpr int kStepRows = 2;   // measured: 2 rows per wavefront beat 1, 4 and 8 (more loads in flight vs more waves)

// VEC: N % 4 == 0 and state / B / C rows aligned to 4 elements, so a lane's 4 states and
// its 4 B and C values move as one access each.
template <typename IO, bool TI, int SL, bool VEC>
__global__ __launch_bounds__(256)
void step_kernel(StepParams p) {
  using T = io_traits<IO>;
  using Qd = quad_io<IO>;
  constexpr int CW = 64 / SL;
  const int lane = threadIdx.x & 63;
  const int64_t wave = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t groups = (p.D + CW - 1) / CW;
  const int64_t rowblocks = (p.batch + kStepRows - 1) / kStepRows;
  if (wave >= groups * rowblocks) return;               // whole wavefront exits together
  const int64_t g = wave % groups, b0 = (wave / groups) * kStepRows;
  const int c = lane / SL, s = lane % SL;
  const int64_t d = g * CW + c;
  const bool dvalid = d < p.D;
  const IO* __restrict__ const u = static_cast<const IO*>(p.u);
  const IO* __restrict__ const dl = static_cast<const IO*>(p.delta);
  const IO* __restrict__ const Bv = static_cast<const IO*>(p.B);
  const IO* __restrict__ const Cv = static_cast<const IO*>(p.C);
  const IO* __restrict__ const zv = static_cast<const IO*>(p.z);
  float* __restrict__ const st = p.state;

  // per-lane constants of the 4 owned states
  float A2[4], iA[4], Af[4], Bt[4], Ct[4];
  bool nok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = 4 * s + j;
    nok[j] = dvalid && n < p.N;
    const float a = nok[j] ? p.A[d * p.N + n] : 0.f;
    A2[j] = a * kLog2e;
    const bool first_order = a == 0.f || p.euler;       // Bbar = delta * B
    iA[j] = first_order ? 0.f : 1.0f / a;
    Af[j] = p.euler ? 0.f : a;                           // first order: x = 0, the coefficient is delta
    Bt[j] = (TI && nok[j]) ? T::widen(Bv[d * p.B_sd + n]) : 0.f;
    Ct[j] = (TI && nok[j]) ? T::widen(Cv[d * p.C_sd + n]) : 0.f;
  }
  const float dskip = (dvalid && p.Dskip != nullptr) ? p.Dskip[d] : 0.f;
  const float bias_d = (p.delta_bias != nullptr && dvalid) ? p.delta_bias[d] : 0.f;
  float dt_ti = (TI && dvalid) ? T::widen(dl[d]) : 0.f;
  if (TI && p.dxf) dt_ti = step_size(dt_ti, bias_d, p.softplus != 0);

  // loads of all rows first
  float uu[kStepRows], dt[kStepRows], zz[kStepRows], h[kStepRows][4], bb[kStepRows][4], cc[kStepRows][4];
#pragma unroll
  for (int r = 0; r < kStepRows; ++r) {
    const int64_t b = b0 + r;
    const bool live = dvalid && b < p.batch;
    uu[r] = live ? T::widen(u[b * p.u_sb + d]) : 0.f;
    dt[r] = TI ? dt_ti : (live ? T::widen(dl[b * p.delta_sb + d]) : 0.f);
    if (!TI && p.dxf) dt[r] = step_size(dt[r], bias_d, p.softplus != 0);
    zz[r] = (live && zv != nullptr) ? T::widen(zv[b * p.z_sb + d]) : 0.f;
    if (VEC) {                                                   // all 4 states valid or none
      if (live && nok[0]) {
        const float4 hv = *reinterpret_cast<const float4*>(st + (b * p.D + d) * p.N + 4 * s);
        h[r][0] = hv.x; h[r][1] = hv.y; h[r][2] = hv.z; h[r][3] = hv.w;
        if (!TI) {
          const typename Qd::raw_t bq = *reinterpret_cast<const typename Qd::raw_t*>(Bv + b * p.B_sb + 4 * s);
          const typename Qd::raw_t cq = *reinterpret_cast<const typename Qd::raw_t*>(Cv + b * p.C_sb + 4 * s);
#pragma unroll
          for (int j = 0; j < 4; ++j) { bb[r][j] = Qd::get(bq, j); cc[r][j] = Qd::get(cq, j); }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) { h[r][j] = 0.f; bb[r][j] = 0.f; cc[r][j] = 0.f; }
      }
      if (TI) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { bb[r][j] = Bt[j]; cc[r][j] = Ct[j]; }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = 4 * s + j;
        const bool ok = live && nok[j];
        h[r][j] = ok ? st[(b * p.D + d) * p.N + n] : 0.f;
        bb[r][j] = TI ? Bt[j] : (ok ? T::widen(Bv[b * p.B_sb + n]) : 0.f);
        cc[r][j] = TI ? Ct[j] : (ok ? T::widen(Cv[b * p.C_sb + n]) : 0.f);
      }
    }
  }
  IO* __restrict__ const y = static_cast<IO*>(p.y);
#pragma unroll
  for (int r = 0; r < kStepRows; ++r) {
    const int64_t b = b0 + r;
    const bool live = dvalid && b < p.batch;
    float acc = 0.f, hn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ab = __builtin_amdgcn_exp2f(dt[r] * A2[j]);               // Abar = exp(delta A)
      const float f = zoh_coeff_exact(dt[r], Af[j], iA[j], ab);             // (Abar - 1)/A, or delta
      hn[j] = fmaf(ab, h[r][j], f * (bb[r][j] * uu[r]));                    // h = Abar h + Bbar u
      acc = fmaf(cc[r][j], hn[j], acc);                                     // C . h
      if (!VEC && live && nok[j]) st[(b * p.D + d) * p.N + 4 * s + j] = hn[j];
    }
    if (VEC && live && nok[0])
      *reinterpret_cast<float4*>(st + (b * p.D + d) * p.N + 4 * s) = make_float4(hn[0], hn[1], hn[2], hn[3]);
#pragma unroll
    for (int off = SL / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, SL);   // sum over the channel's lanes
    if (live && s == 0) {
      float yv = fmaf(dskip, uu[r], acc);                                   // + D u
      if (zv != nullptr) yv *= zz[r] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zz[r] * kLog2e));   // * SiLU(z)
      if (sizeof(IO) == 2) {
        // round to nearest even; NaN stays a quiet NaN
        const uint32_t x = __float_as_uint(yv);
        const uint32_t rr = ((x & 0x7fffffffu) > 0x7f800000u) ? ((x >> 16) | 0x40u)
                                                              : ((x + 0x7fffu + ((x >> 16) & 1u)) >> 16);
        reinterpret_cast<uint16_t*>(y)[b * p.y_sb + d] = uint16_t(rr);
      } else {
        reinterpret_cast<float*>(y)[b * p.y_sb + d] = yv;
      }
    }
  }
}

template <typename IO, bool TI, int SL>
hipError_t launch_step_sl(const StepParams& p, hipStream_t stream) {
  constexpr int CW = 64 / SL;
  const int64_t waves = ((p.D + CW - 1) / CW) * ((p.batch + kStepRows - 1) / kStepRows);
  const int64_t blocks = (waves + 3) / 4;
  if (blocks == 0) return hipSuccess;
  if (p.vec) hipLaunchKernelGGL((step_kernel<IO, TI, SL, true>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((step_kernel<IO, TI, SL, false>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename IO, bool TI>
hipError_t launch_step_t(const StepParams& p, hipStream_t stream) {
  const int64_t quads = (p.N + 3) / 4;                  // lanes per channel: 4 states each
  if (quads <= 1) return launch_step_sl<IO, TI, 1>(p, stream);
  if (quads <= 2) return launch_step_sl<IO, TI, 2>(p, stream);
  if (quads <= 4) return launch_step_sl<IO, TI, 4>(p, stream);
  if (quads <= 8) return launch_step_sl<IO, TI, 8>(p, stream);
  return launch_step_sl<IO, TI, 16>(p, stream);
}

template <typename IO, int S, int K, bool TI, int MODE>
hipError_t launch_scan(const ScanParams& p, hipStream_t stream) {
  constexpr size_t lds = size_t(wave_lds<S, K, TI>::total) * sizeof(float) * kWavesPerBlock;
  const int64_t items = p.batch * (MODE == MODE_STATE ? p.n_chunks - 1 : p.n_chunks) * p.groups;
  const int blocks = int((items + kWavesPerBlock - 1) / kWavesPerBlock);
  if (blocks == 0) return hipSuccess;
  if (lds > 65536) {   // above the default dynamic-LDS limit: opt in once per kernel
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&scan_kernel<IO, S, K, TI, MODE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL((scan_kernel<IO, S, K, TI, MODE>), dim3(blocks), dim3(kWavesPerBlock * 64), lds, stream, p);
  return hipGetLastError();
}

template <typename IO, int K, bool TI, int MODE, bool DXF>
hipError_t launch_scan_coop(const ScanParams& p, hipStream_t stream) {
  constexpr size_t lds = size_t(coop_lds<K, TI, MODE>::total) * sizeof(float);
  if (lds > 65536) {   // above the default dynamic-LDS limit: opt in once per kernel
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&scan_kernel_coop<IO, K, TI, MODE, DXF>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (attr != hipSuccess) return attr;
  }
  constexpr int kCh = coop_lds<K, TI, MODE>::kCh;
  const int64_t groups = (p.D + kCh - 1) / kCh;
  const int64_t blocks = p.batch * (MODE == MODE_STATE && !p.state_all ? p.n_chunks - 1 : p.n_chunks) * groups;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((scan_kernel_coop<IO, K, TI, MODE, DXF>), dim3(unsigned(blocks)), dim3(64 * coop_width<TI>::W),
                     lds, stream, p);
  return hipGetLastError();
}

template <typename IO, bool TI, int MODE>
hipError_t dispatch_sk(int S, int K, const ScanParams& p, hipStream_t stream) {
  if (p.pipelined && S == 16) {
    if (!TI && p.dxf) {
      if (K == 1) return launch_scan_coop<IO, 1, false, MODE, true>(p, stream);
      if (K == 2) return launch_scan_coop<IO, 2, false, MODE, true>(p, stream);
      if (K == 4) return launch_scan_coop<IO, 4, false, MODE, true>(p, stream);
    }
    if (K == 1) return launch_scan_coop<IO, 1, TI, MODE, false>(p, stream);
    if (K == 2) return launch_scan_coop<IO, 2, TI, MODE, false>(p, stream);
    if (K == 4) return launch_scan_coop<IO, 4, TI, MODE, false>(p, stream);
  }
  if (S == 4 && K == 1) return launch_scan<IO, 4, 1, TI, MODE>(p, stream);
  if (S == 8 && K == 1) return launch_scan<IO, 8, 1, TI, MODE>(p, stream);
  if (S == 16 && K == 1) return launch_scan<IO, 16, 1, TI, MODE>(p, stream);
  if (S == 16 && K == 2) return launch_scan<IO, 16, 2, TI, MODE>(p, stream);
  if (S == 16 && K == 4) return launch_scan<IO, 16, 4, TI, MODE>(p, stream);
  return hipErrorInvalidValue;
}


}  // namespace
}  // namespace selscan
