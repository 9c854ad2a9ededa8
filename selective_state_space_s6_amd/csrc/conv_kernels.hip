// conv_kernels.hip -- the convolution mode of fixed (time-invariant) coefficients on the fp32
// matrix cores of gfx950.
//
// With delta, B and C fixed per channel the scan is a causal convolution of u with the lag
// kernel K_k = sum_n C_n Abar_n^k Bbar_n ("state-space models" (aarnphm.xyz), section "One
// recurrence, one convolution"; Algenta "Sequence and state-space models", s4_kernel_element).
// The sequence is cut into blocks of 16 tokens, and each block's output is its own Toeplitz
// product plus the readout of the state carried in from the blocks before it:
//   y[tau, j]  = sum_{s <= tau} K_{tau-s} u[s, j]              (Toep, 16 x 16, per block j)
//              + sum_n C_n Abar_n^{tau+1} h_n[j-1]              (V, 16 x N)
//   h_n[j]     = Abar_n^16 h_n[j-1] + sum_s Abar_n^{15-s} Bbar_n u[s, j]   (W, N x 16)
// where u[s, j] is token s of block j and h_n[j] the state after block j.  Toep, W and V depend
// on the channel only, so for sixteen blocks at once (a 256-token super-tile) the three terms
// are matrix products with the blocks as the 16 columns: Toep.U and W.U (K = 16 tokens) and
// V.H (K = N states), 4 + 4N/16 + 4N/16 instructions of v_mfma_f32_16x16x4_f32 per
// wavefront.  The state carry between the sixteen blocks is a linear recurrence with the
// constant factor Abar^16 per state, done across the 16 lanes of a DPP row by a log-depth scan
// (row shifts by 1, 2, 4, 8 with factors q, q^2, q^4, q^8).  The readout of the carried state
// is formed for block j from the state after block j and added to block j + 1 (a row shift of
// the product), the last column feeding the next super-tile's first block.
//
// Work decomposition: one wavefront per (batch row, channel), 8 wavefronts (8 neighbouring
// channels) per workgroup, so that the workgroup stages u, and writes y, as rows of 8 channels
// through LDS; workgroups are dealt to the XCDs in contiguous runs of channel groups.  Per
// wavefront, the Toeplitz, W and V matrices live in VGPRs as MFMA fragments; the carry factors
// Abar^16 go to LDS and are read back per super-tile, and the readout over the state blocks
// accumulates into one register set, so that every state count fits 128 VGPRs: four
// wavefronts per SIMD, two workgroups per compute unit (the latency of the chain MFMA -> DPP
// scan -> MFMA is what a second workgroup hides).  Fragment layouts of v_mfma_f32_16x16x4_f32 (wave64): lane l = 16 g + j holds
// A[i = j][k = g] and B[k = g][col = j]; the four result registers r hold D[4 g + r][j].
// The state index of the carried product's k-steps is chosen as n = 16 a + 4 g + r, which is
// the row of the W.U result in register (a, r): the scanned states feed V.H without a
// transpose.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "scan_launch.h"

namespace selscan {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 16;                  // tokens per block (rows of the Toeplitz product)
constexpr int kNBlk = 16;                 // blocks per super-tile (columns of every product)
constexpr int kSup = kBlk * kNBlk;        // tokens per super-tile
constexpr int kCW = 8;                    // wavefronts, and channels, per workgroup
constexpr int kThreads = 64 * kCW;
// LDS row of one channel's 256 tokens: one pad word per 16-token block (so that the lanes of a
// fragment read, 16 blocks apart, fall in different banks) and one more
constexpr int kRow = kSup + kNBlk + 1;
__device__ __forceinline__ int tpos(int t) { return t + (t >> 4); }

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {   // DPP lane move within rows of 16, zero where no source
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;   // row_shr:1 .. 8
constexpr int kBcast15 = 0x15F;                                               // row_newbcast:15

template <typename IO> struct conv_io;
template <> struct conv_io<float> {
  using raw_t = float4;
  static __device__ __forceinline__ raw_t load(const void* p, int64_t off) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
  }
  static __device__ __forceinline__ float get(const raw_t& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
  static __device__ __forceinline__ raw_t zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ void store(void* p, int64_t off, float4 y) {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + off) = y;
  }
};
template <> struct conv_io<uint16_t> {       // bfloat16 bit patterns
  using raw_t = uint2;
  static __device__ __forceinline__ raw_t load(const void* p, int64_t off) {
    return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + off);
  }
  static __device__ __forceinline__ float get(const raw_t& v, int i) {
    const uint32_t w = (i < 2) ? v.x : v.y;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  static __device__ __forceinline__ raw_t zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ void store(void* p, int64_t off, float4 y) {
    const uint2 v = make_uint2(uint32_t(bf16_rne(y.x)) | (uint32_t(bf16_rne(y.y)) << 16),
                               uint32_t(bf16_rne(y.z)) | (uint32_t(bf16_rne(y.w)) << 16));
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + off) = v;
  }
};

// NB: blocks of 16 states (N <= 16 NB; states past N are padded with Bbar = C = 0).
template <typename IO, int NB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void conv_ti_kernel(ConvParams p) {
  using T = io_traits<IO>;
  using Io = conv_io<IO>;
  __shared__ __align__(16) float sU[2][kCW * kRow];      // u of a super-tile, [channel][token], two buffers
  __shared__ __align__(16) float sY[kCW * kRow];         // y of a super-tile (and set-up scratch)
  __shared__ __align__(16) float4 sQ[kCW][NB][64];       // each lane's Abar^16 of its four result rows, per state block

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;                // fragment lane: column (block) j, row group g
  // neighbouring channel groups share the 128-byte lines of u and y: the XCD-contiguous order
  // puts them on one XCD, whose L2 then fetches each line once
  const int64_t groups = (p.D + kCW - 1) / kCW;
  const int64_t item = xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int64_t b = item / groups;
  const int64_t d0 = (item % groups) * kCW;
  const int64_t d = d0 + w;                              // this wavefront's channel
  const bool dvalid = d < p.D;
  const int64_t L = p.L, N = p.N;

  // ---- per-channel constants.  Lane n computes state n's log-transition delta*a, Bbar and C
  // into LDS scratch; the fragments are then formed from them.
  float* const scr = sY + w * 4 * 64;                    // da[64], bbar[64], c[64], 4 x 16 partial sums of K
  static_assert(kCW * kRow >= kCW * 4 * 64, "set-up scratch fits the y tile");
  {
    float dt = dvalid ? T::widen(static_cast<const IO*>(p.delta)[d]) : 0.f;
    if (p.dxf && dvalid) dt = step_size(dt, p.delta_bias != nullptr ? p.delta_bias[d] : 0.f, p.softplus != 0);
    const int n = lane;
    const bool ok = dvalid && n < N;
    const float a = ok ? p.A[d * N + n] : 0.f;
    const float bv = ok ? T::widen(static_cast<const IO*>(p.B)[d * p.B_sd + n]) : 0.f;
    const float cv = ok ? T::widen(static_cast<const IO*>(p.C)[d * p.C_sd + n]) : 0.f;
    const float coeff = (a == 0.f || p.euler) ? dt : expm1f(dt * a) / a;   // Bbar / B (ZOH or first order)
    scr[n] = dt * a;
    scr[64 + n] = coeff * bv;
    scr[128 + n] = cv;
  }
  __syncthreads();
  // K_k, k = 0..15: lane (j, g) sums the states n = g + 4 i
  {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 16 * NB / 4; ++i) {
      const int n = g + 4 * i;
      acc = fmaf(scr[128 + n] * scr[64 + n], expf(float(j) * scr[n]), acc);
    }
    scr[192 + g * 16 + j] = acc;
  }
  __syncthreads();
  float tf[4];                                            // Toep: A[tau = j][sigma = 4 s + g]
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int sig = 4 * s + g, k = j - sig;
    float kv = 0.f;
    if (k >= 0) kv = scr[192 + k] + scr[192 + 16 + k] + scr[192 + 32 + k] + scr[192 + 48 + k];
    tf[s] = kv;
  }
  float wf[NB][4], vf[NB][4], q[NB][4];                  // q goes to LDS (sQ)
#pragma unroll
  for (int a = 0; a < NB; ++a) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {                         // W: A[state 16 a + j][sigma = 4 s + g]
      const int n = 16 * a + j, sig = 4 * s + g;
      wf[a][s] = expf(float(15 - sig) * scr[n]) * scr[64 + n];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {                         // V: A[tau = j][state 16 a + 4 g + r]; q per result row
      const int n = 16 * a + 4 * g + r;
      vf[a][r] = scr[128 + n] * expf(float(j + 1) * scr[n]);
      q[a][r] = expf(16.f * scr[n]);
    }
  }
  // computed once: opaque to the compiler, which would otherwise rematerialise the
  // exponentials inside the loop to save registers
#pragma unroll
  for (int s = 0; s < 4; ++s) __asm__ __volatile__("" : "+v"(tf[s]));
#pragma unroll
  for (int a = 0; a < NB; ++a) {
#pragma unroll
    for (int k = 0; k < 4; ++k) __asm__ __volatile__("" : "+v"(wf[a][k]), "+v"(vf[a][k]));
    sQ[w][a][lane] = make_float4(q[a][0], q[a][1], q[a][2], q[a][3]);
  }
  __syncthreads();                                        // the scratch (in sY) is free again

  // ---- the super-tiles
  const IO* const ub = static_cast<const IO*>(p.u) + b * p.u_sb;
  const IO* const zb = p.z != nullptr ? static_cast<const IO*>(p.z) + b * p.z_sb : nullptr;
  IO* const yb = static_cast<IO*>(p.y) + b * p.y_sb;
  // cooperative I/O layout: thread -> token tt (of 256), channels d0 + 4 c4 .. + 3
  constexpr int kQuads = kCW / 4;
  static_assert(kQuads * kSup == kThreads, "one 4-channel vector per thread and super-tile");
  const int tt = tid / kQuads, c4 = tid % kQuads;
  const int64_t dq = d0 + 4 * c4;
  const bool qvalid = dq < p.D;                           // D % 4 == 0: a quad is all in or all out
  float dsk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dsk[i] = (p.Dskip != nullptr && qvalid) ? p.Dskip[dq + i] : 0.f;
  const int64_t ntile = (L + kSup - 1) / kSup;
  auto load_u = [&](int64_t t0) __attribute__((always_inline)) {
    const int64_t l = t0 + tt;
    return (qvalid && l < L) ? Io::load(ub, l * p.u_sl + dq) : Io::zero();
  };
  auto stage_u = [&](float* dst, const typename Io::raw_t& v) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(4 * c4 + i) * kRow + tpos(tt)] = Io::get(v, i);
  };

  f32x4 X[NB];                                            // state after each block: X[a][r] = h[16a+4g+r][j]
  f32x4 Zp = {0.f, 0.f, 0.f, 0.f};                        // carried readout of the previous super-tile
#pragma unroll
  for (int a = 0; a < NB; ++a) X[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  typename Io::raw_t nxt = load_u(0);
  stage_u(sU[0], nxt);
  if (ntile > 1) nxt = load_u(kSup);
  // The two workgroups sharing a compute unit take turns at the top issue priority, in slices of
  // 2^11 ticks of the 100 MHz clock (the arbiter otherwise prefers the older one, and the
  // younger finishes alone); only when the whole grid is resident at once (two per compute
  // unit).  The clock is read after a super-tile's barrier and used at the next one's.
  const bool fair = p.sched_round > 0 && gridDim.x <= 2u * uint32_t(p.sched_round);
  const uint32_t fair_round = fair ? uint32_t(blockIdx.x) / uint32_t(p.sched_round) : 0u;
  uint64_t fair_clock = 0;
  for (int64_t it = 0; it < ntile; ++it) {
    const int cur = int(it & 1);
    if (fair) {
      const uint32_t ph = (uint32_t(fair_clock >> 11) + fair_round) % 3u;
      if (ph == 0) __builtin_amdgcn_s_setprio(3);
      else if (ph == 1) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(1);
    }
    __syncthreads();                                      // tile it staged; the other buffer and sY are free
    if (fair) fair_clock = __builtin_amdgcn_s_memrealtime();
    typename Io::raw_t zr = Io::zero();
    if (zb != nullptr && qvalid && it * kSup + tt < L) zr = Io::load(zb, (it * kSup + tt) * p.z_sl + dq);
    const float* const uc = sU[cur] + w * kRow;
    float uf[4];                                          // U: B[sigma = 4 s + g][block j]
#pragma unroll
    for (int s = 0; s < 4; ++s) uf[s] = uc[17 * j + 4 * s + g];
    f32x4 Y = zero4;
#pragma unroll
    for (int s = 0; s < 4; ++s) Y = mfma4(tf[s], uf[s], Y);              // Toep . U
    // final state (last super-tile): the state entering the block of the last token is kept
    // in the free u buffer; the tokens of that block up to the last are then stepped serially
    const bool fin = (it == ntile - 1) && p.last_state != nullptr;
    const int e = int(L - 1 - it * kSup);                 // last valid token of the tile (when fin)
    const int jl = e >> 4, m = (e & 15) + 1;
    float* const hs = sU[cur ^ 1] + w * kRow;             // nothing is staged after the last tile
    // per block of 16 states: W . U, the scan over the 16 blocks, and its readout V . X
    f32x4 Z = {0.f, 0.f, 0.f, 0.f};                       // V . X summed over the state blocks
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      f32x4 S = zero4;
#pragma unroll
      for (int s = 0; s < 4; ++s) S = mfma4(wf[a][s], uf[s], S);           // W . U
      const float4 qa = sQ[w][a][lane];
      const float qv[4] = {qa.x, qa.y, qa.z, qa.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // the state entering the super-tile (last column of the previous one) enters block 0
        const float hin = dpp<kBcast15>(X[a][r]);
        if (fin && jl == 0 && j == 0) hs[16 * a + 4 * g + r] = hin;
        float x = S[r];
        if (j == 0) x = fmaf(qv[r], hin, x);
        // inclusive scan over the 16 blocks: x_j += q^m x_{j-m}, m = 1, 2, 4, 8
        float qm = qv[r];
        x = fmaf(dpp<kShr1>(x), qm, x);
        qm *= qm;
        x = fmaf(dpp<kShr2>(x), qm, x);
        qm *= qm;
        x = fmaf(dpp<kShr4>(x), qm, x);
        qm *= qm;
        x = fmaf(dpp<kShr8>(x), qm, x);
        X[a][r] = x;
        if (fin && jl > 0 && j == jl - 1) hs[16 * a + 4 * g + r] = x;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Z = mfma4(vf[a][r], X[a][r], Z);   // readout of the state after block j
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {                         // block j takes the readout of block j - 1
      const float prev = dpp<kShr1>(Z[r]);
      const float last = dpp<kBcast15>(Zp[r]);
      Y[r] += (j == 0) ? last : prev;
    }
    Zp = Z;
    float* const yc = sY + w * kRow;
#pragma unroll
    for (int r = 0; r < 4; ++r) yc[17 * j + 4 * g + r] = Y[r];            // token 16 j + 4 g + r
    if (fin) {                                            // uniform over the workgroup
      __syncthreads();
      if (lane < N && dvalid) {
        const int n = lane;
        float dt = T::widen(static_cast<const IO*>(p.delta)[d]);
        if (p.dxf) dt = step_size(dt, p.delta_bias != nullptr ? p.delta_bias[d] : 0.f, p.softplus != 0);
        const float a = p.A[d * N + n];
        const float bv = T::widen(static_cast<const IO*>(p.B)[d * p.B_sd + n]);
        const float coeff = (a == 0.f || p.euler) ? dt : expm1f(dt * a) / a;
        const float ab = expf(dt * a), bb = coeff * bv;
        float h = hs[n];
        for (int s = 0; s < m; ++s) h = fmaf(ab, h, bb * uc[17 * jl + s]);
        p.last_state[(b * p.D + d) * N + n] = h;
      }
    }
    __syncthreads();                                      // y tile complete; u tile it still readable
    // coalesced output: token tt, channels dq .. dq+3: + D u, gate, store
    const int64_t l = it * kSup + tt;
    if (qvalid && l < L) {
      float4 yv;
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sY[(4 * c4 + i) * kRow + tpos(tt)];
        v = fmaf(dsk[i], sU[cur][(4 * c4 + i) * kRow + tpos(tt)], v);
        if (zb != nullptr) {
          const float zz = Io::get(zr, i);
          v *= zz * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zz * kLog2e));
        }
        o[i] = v;
      }
      yv = make_float4(o[0], o[1], o[2], o[3]);
      Io::store(yb, l * p.y_sl + dq, yv);
    }
    if (it + 1 < ntile) {                                 // stage the next tile into the other buffer
      stage_u(sU[cur ^ 1], nxt);
      if (it + 2 < ntile) nxt = load_u((it + 2) * kSup);
    }
  }
}

template <typename IO>
hipError_t launch_conv_io(int nb, const ConvParams& p, hipStream_t stream) {
  const int64_t blocks = p.batch * ((p.D + kCW - 1) / kCW);
  if (blocks == 0) return hipSuccess;
  const dim3 grid{unsigned(blocks)}, block{unsigned(kThreads)};
  switch (nb) {
    case 1: hipLaunchKernelGGL((conv_ti_kernel<IO, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((conv_ti_kernel<IO, 2>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((conv_ti_kernel<IO, 3>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((conv_ti_kernel<IO, 4>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_ti(bool bf16, const ConvParams& p, hipStream_t stream) {
  const int nb = int((p.N + 15) / 16);
  return bf16 ? launch_conv_io<uint16_t>(nb, p, stream) : launch_conv_io<float>(nb, p, stream);
}

}  // namespace selscan
