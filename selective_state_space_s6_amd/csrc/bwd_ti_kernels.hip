// bwd_ti_kernels.hip -- the backward pass of the selective scan with fixed (time-invariant)
// coefficients: delta[d], B[d][n] and C[d][n] shared by every batch row and token.
//
// The same reverse-time recurrence as the selective backward (the rustytorch commit log's
// hand-written VJP of the selective scan: lambda_t = dy'_t C + Abar lambda_{t+1}, every
// gradient by the chain rule through one step), with Abar = exp(delta a) and the input
// coefficient c = Bbar / B constant per (channel, state).  So no exponential is evaluated per
// element, and the gradients of the shared coefficients are sums over batch rows and tokens
// that each lane accumulates for its own (channel, state) pairs:
//   dB[d][n]     = c  sum_{b,t} lambda_t u_t
//   dC[d][n]     = sum_{b,t} dy'_t h_t
//   dA[d][n]     = sum_{b,t} lambda_t (delta Abar h_{t-1} + dc/da B u_t)
//   ddelta[d]    = sum_{b,t,n} lambda_t (a Abar h_{t-1} + dc/ddelta B u_t)   (times softplus')
// with dc/ddelta = Abar and dc/da = (delta Abar - c)/a, by its series near zero (ZOH), or
// 1 and 0 (first order).  Since delta, B and dc/da are fixed, dA and ddelta are formed once per
// chunk from R = sum_t lambda_t h_{t-1} and G = sum_t lambda_t u_t (dB's own sum).  Per token,
// only du and dz leave.
//
// Work decomposition as the selective backward: SL = N/4 lanes per channel, 4 states per
// lane, a workgroup of four wavefronts per (batch row, chunk, 4 * 64 / SL channels); u, dy'
// and the gate's derivative factor are staged per 16-token tile in LDS by coalesced loads
// issued one tile ahead.  A split sequence takes three kernels of this file and two of the
// selective backward's: the chunk end states from a zero start (TI_STATE), composed into
// carried-in states by chunk_prefix_kernel; the chunk adjoints from a zero start (TI_ADJOINT),
// combined by bwd_adjoint_combine_kernel; then the main pass (TI_MAIN), which checkpoints each
// chunk's tiles from its carried-in state, walks the tiles backwards and writes per-(batch row,
// chunk) partial sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "scan_launch.h"

namespace selscan {
namespace {

constexpr int kTTile = 16;      // tokens per tile (one checkpoint each)
constexpr int kTRow = 20;       // LDS row of one channel's 16 tokens: 16 + 4 padding

enum { TI_STATE = 0, TI_ADJOINT = 1, TI_MAIN = 2 };

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the SL consecutive lanes of a channel, result in every one of them.
template <int SL>
__device__ __forceinline__ float chan_sum(float v) {
  v += dpp_mov<0xB1>(v);                     // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);                     // quad_perm [2,3,0,1]
  if (SL >= 8) v += dpp_mov<0x141>(v);       // row_half_mirror
  if (SL >= 16) v += dpp_mov<0x140>(v);      // row_mirror
  return v;
}

template <typename IO, int SL, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_ti_kernel(BwdParams p) {
  using T = io_traits<IO>;
  constexpr int CW = 64 / SL, CWG = 4 * CW;
  constexpr int ET = CWG * kTTile / 256;     // token-tensor elements each thread stages
  constexpr int kTStep = 256 / CWG;
  __shared__ __align__(16) float sTok[3][CWG][kTRow];   // u, dy through the gate, dz factor

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane / SL, s = lane % SL;
  const int cw = w * CW + c;
  const int64_t item = xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int nc = p.n_chunks;
  // TI_STATE: chunks 0 .. nc-2 (the last chunk's end state is never used); TI_ADJOINT:
  // chunks 1 .. nc-1 (the first chunk's adjoint map is never used); TI_MAIN: all
  const int nc_run = MODE == TI_MAIN ? nc : nc - 1;
  const int64_t g = item % p.groups, bc = item / p.groups;
  const int chunk = int(bc % nc_run) + (MODE == TI_ADJOINT ? 1 : 0);
  const int64_t b = bc / nc_run;
  const int64_t D = p.D, N = p.N, L = p.L;
  const int64_t d0 = g * CWG, d = d0 + cw;
  const bool dvalid = d < D;
  const int64_t dq = dvalid ? d : D - 1;
  const bool sp = p.softplus != 0, gated = p.z != nullptr, first = p.euler != 0;
  const int64_t l_begin = int64_t(chunk) * p.chunk_len;
  const int64_t l_end = (l_begin + p.chunk_len < L) ? l_begin + p.chunk_len : L;
  const int64_t ntiles = (l_end - l_begin + kTTile - 1) / kTTile;
  const int64_t tile0 = l_begin / kTTile;
  const int last_nt = int(l_end - l_begin - (ntiles - 1) * kTTile);

  // ---- the channel's constants
  const float raw = T::widen(static_cast<const IO*>(p.delta)[dq]);
  const float bias = p.delta_bias != nullptr ? p.delta_bias[dq] : 0.f;
  const float dt = p.dxf ? step_size(raw, bias, sp) : raw;
  // d dt / d raw: the logistic function of the softplus argument, or 1
  const float dsig = sp ? __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-(raw + bias) * kLog2e)) : 1.f;
  float a[4], ab[4], cfv[4], cb[4], Bv[4], Cv[4], dcdd[4], dcda[4];
  bool nok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = 4 * s + i;
    nok[i] = dvalid && n < N;
    a[i] = nok[i] ? p.A[d * N + n] : 0.f;
    ab[i] = __builtin_amdgcn_exp2f(dt * a[i] * kLog2e);
    const float ia = a[i] != 0.f ? 1.f / a[i] : 0.f;
    const float cf = first ? dt : zoh_coeff_exact(dt, a[i], ia, ab[i]);
    Bv[i] = nok[i] ? T::widen(static_cast<const IO*>(p.B)[d * p.B_sd + n]) : 0.f;
    Cv[i] = nok[i] ? T::widen(static_cast<const IO*>(p.C)[d * p.C_sd + n]) : 0.f;
    cfv[i] = cf;
    cb[i] = cf * Bv[i];
    dcdd[i] = first ? 1.f : ab[i];
    // dc/da = (delta Abar - c) / a, or delta^2 phi(x), x = delta a, by the series of
    // phi(x) = (x e^x - (e^x - 1)) / x^2 near 0 (where the first form cancels, and at a == 0)
    const float x = dt * a[i];
    const float series = fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.f / 144.f, 1.f / 30.f), 1.f / 8.f), 1.f / 3.f), 0.5f);
    dcda[i] = first ? 0.f : (fabsf(x) < 0.1f ? dt * dt * series : fmaf(dt, ab[i], -cf) * ia);
  }
  const float dskip = (dvalid && p.Dskip != nullptr) ? p.Dskip[d] : 0.f;

  // ---- staging: element e = tid + 256 r is token e / CWG of channel d0 + e % CWG
  const IO* const u_b = static_cast<const IO*>(p.u) + b * p.u_sb;
  const IO* const dy_b = static_cast<const IO*>(p.dy) + b * p.dy_sb;
  const IO* const z_b = gated ? static_cast<const IO*>(p.z) + b * p.z_sb : u_b;
  const int64_t z_sl = gated ? p.z_sl : p.u_sl;
  const int tj0 = tid / CWG, tc = tid % CWG;
  const bool tcok = d0 + tc < D;
  const int64_t tdq = tcok ? d0 + tc : D - 1;
  IO xu[ET], xy[ET], xz[ET];
  int pend_nt = kTTile;
  constexpr bool kU = MODE != TI_ADJOINT, kY = MODE != TI_STATE;
  auto issue = [&](int64_t t) __attribute__((always_inline)) {
    const int nt = t == ntiles - 1 ? last_nt : kTTile;
    pend_nt = nt;
    const int64_t l0 = l_begin + t * kTTile;
#pragma unroll
    for (int r = 0; r < ET; ++r) {
      const int j = tj0 + kTStep * r;
      const int jq = j < nt ? j : nt - 1;                  // clamped: read in bounds, zeroed when staged
      if (kU) xu[r] = u_b[(l0 + jq) * p.u_sl + tdq];
      if (kY) {
        xy[r] = dy_b[(l0 + jq) * p.dy_sl + tdq];
        xz[r] = z_b[(l0 + jq) * z_sl + tdq];
      }
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
    const int nt = pend_nt;
#pragma unroll
    for (int r = 0; r < ET; ++r) {
      const int j = tj0 + kTStep * r;
      const bool ok = tcok && j < nt;
      if (kU) sTok[0][tc][j] = ok ? T::widen(xu[r]) : 0.f;
      if (kY) {
        const float vy = ok ? T::widen(xy[r]) : 0.f;
        float dyp = vy, gzf = 0.f;
        if (gated) {           // y = yp * z sigmoid(z): dyp = dy z sigmoid(z); dz = yp * gzf
          const float zz = ok ? T::widen(xz[r]) : 0.f;
          const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zz * kLog2e));
          dyp = vy * zz * sg;
          gzf = vy * sg * fmaf(zz, 1.f - sg, 1.f);
        }
        sTok[1][tc][j] = dyp;
        if (MODE == TI_MAIN) sTok[2][tc][j] = gzf;
      }
    }
  };
  // (b, d, n) of a per-chunk workspace array [batch][D][N][n_chunks]
  auto chunk_slot = [&](int i, int cc) { return ((b * D + d) * N + 4 * s + i) * nc + cc; };
  const float dsum = dt * float(l_end - l_begin);       // the chunk's sum of delta

  if constexpr (MODE == TI_STATE) {
    // the chunk's end state from a zero start
    float h[4] = {0.f, 0.f, 0.f, 0.f};
    issue(0);
    for (int64_t t = 0; t < ntiles; ++t) {
      __syncthreads();                                      // the previous tile's LDS reads are done
      stage();
      __syncthreads();
      if (t + 1 < ntiles) issue(t + 1);
      const int nt = t == ntiles - 1 ? last_nt : kTTile;
      for (int j = 0; j < nt; ++j) {
        const float uu = sTok[0][cw][j];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = fmaf(ab[i], h[i], cb[i] * uu);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nok[i]) p.carry[chunk_slot(i, chunk)] = h[i];
    if (dvalid && s == 0) p.sdsum[(b * D + d) * nc + chunk] = dsum;   // the chunk's sum of delta, for the prefix
    return;
  }

  if constexpr (MODE == TI_ADJOINT) {
    // mu_{t-1} = Abar (dyp_t C + mu_t), from mu = 0 after the chunk's last token
    float mu[4] = {0.f, 0.f, 0.f, 0.f};
    issue(ntiles - 1);
    for (int64_t t = ntiles - 1; t >= 0; --t) {
      __syncthreads();
      stage();
      __syncthreads();
      if (t > 0) issue(t - 1);
      const int nt = t == ntiles - 1 ? last_nt : kTTile;
      for (int j = nt - 1; j >= 0; --j) {
        const float dyp = sTok[1][cw][j];
#pragma unroll
        for (int i = 0; i < 4; ++i) mu[i] = ab[i] * fmaf(dyp, Cv[i], mu[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nok[i]) p.adjG[chunk_slot(i, chunk)] = mu[i];
    if (dvalid && s == 0) p.adjS[(b * D + d) * nc + chunk] = dsum;   // its decay is exp(A sum delta)
    return;
  }

  // ---- TI_MAIN.  Pass 1: forward from the chunk's carried-in state, checkpoint at every tile
  // start (the last tile's state is the one pass 1 ends with).
  float* const ck_b = p.ckpt + (b * p.ntiles + tile0) * D * N;
  const int64_t ck_d = dq * N;
  float h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float h_in = 0.f;
    if (nok[i]) {
      if (nc > 1) h_in = p.carry[chunk_slot(i, chunk)];
      else if (p.h0 != nullptr) h_in = p.h0[(b * D + d) * N + 4 * s + i];
    }
    h[i] = h_in;
  }
  if (ntiles > 1) issue(0);
  for (int64_t t = 0; t < ntiles - 1; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nok[i]) ck_b[t * D * N + ck_d + 4 * s + i] = h[i];
    __syncthreads();
    stage();
    __syncthreads();
    if (t + 1 < ntiles - 1) issue(t + 1);
#pragma unroll
    for (int j = 0; j < kTTile; ++j) {                      // every tile before the last is full
      const float uu = sTok[0][cw][j];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = fmaf(ab[i], h[i], cb[i] * uu);
    }
  }
  __syncthreads();                                          // pass 1's LDS reads are done

  // Pass 2: tiles backwards, from the adjoint reaching the chunk's end.  With delta, B and C
  // fixed per channel, the A and delta gradients factor through two per-state sums:
  //   sum_t lambda_t (delta Abar h_{t-1} + dc/da B u_t) = delta Abar R + dc/da B G,
  //   sum_t lambda_t (a Abar h_{t-1} + dc/ddelta B u_t) = a Abar R + dc/ddelta B G,
  // R = sum_t lambda_t h_{t-1}, G = sum_t lambda_t u_t (which dB needs as well), so a token
  // accumulates R and G and the rest is formed once per chunk.
  float mu[4], gR[4], gB[4], gC[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = 0.f;
    if (nok[i]) {
      if (nc > 1) m = p.adj_in[chunk_slot(i, chunk)];
      else if (p.dlast != nullptr) m = p.dlast[(b * D + d) * N + 4 * s + i];
    }
    mu[i] = m;
    gR[i] = gB[i] = gC[i] = 0.f;
  }
  float gD = 0.f;
  auto put = [&](IO* ptr, float v) __attribute__((always_inline)) {
    if constexpr (sizeof(IO) == 2) *ptr = bf16_rne(v);
    else *ptr = v;
  };
  issue(ntiles - 1);
  for (int64_t t = ntiles - 1; t >= 0; --t) {
    stage();                                                // the previous tile's LDS reads ended at its barrier
    __syncthreads();
    const int nt = t == ntiles - 1 ? last_nt : kTTile;
    if (t < ntiles - 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = nok[i] ? ck_b[t * D * N + ck_d + 4 * s + i] : 0.f;
    }
    if (t > 0) issue(t - 1);
    // the tile's states: hp[j] before token j (padded tokens: the state after the last one)
    float hp[kTTile][4];
#pragma unroll
    for (int j = 0; j < kTTile; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) hp[j][i] = h[i];
      if (j < nt) {
        const float uu = sTok[0][cw][j];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = fmaf(ab[i], h[i], cb[i] * uu);
      }
    }
#pragma unroll
    for (int j = kTTile - 1; j >= 0; --j) {
      if (j < nt) {
        const float uu = sTok[0][cw][j], dyp = sTok[1][cw][j], gzf = sTok[2][cw][j];
        float gu = 0.f, spart = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ha = j + 1 < kTTile ? hp[j + 1][i] : h[i];   // the state after token j
          const float lam = fmaf(dyp, Cv[i], mu[i]);
          spart = fmaf(Cv[i], ha, spart);
          gu = fmaf(lam, cb[i], gu);
          gR[i] = fmaf(lam, hp[j][i], gR[i]);
          gB[i] = fmaf(lam, uu, gB[i]);
          gC[i] = fmaf(dyp, ha, gC[i]);
          mu[i] = ab[i] * lam;
        }
        gu = chan_sum<SL>(gu);
        const float gz = gated ? fmaf(dskip, uu, chan_sum<SL>(spart)) * gzf : 0.f;
        gD = fmaf(dyp, uu, gD);
        if (s == 0) {                                       // this wavefront owns the channel's rows
          sTok[0][cw][j] = fmaf(dskip, dyp, gu);
          sTok[2][cw][j] = gz;
        }
      }
    }
    __syncthreads();
    // the tile's du (and dz), coalesced over the workgroup's channels
    {
      const int64_t o = (b * L + l_begin + t * kTTile) * D + d0 + tc;
      IO* const du_t = static_cast<IO*>(p.du) + o;
      IO* const dz_t = p.dz != nullptr ? static_cast<IO*>(p.dz) + o : nullptr;
#pragma unroll
      for (int r = 0; r < ET; ++r) {
        const int j = tj0 + kTStep * r;
        if (tcok && j < nt) {
          put(du_t + j * D, sTok[0][tc][j]);
          if (dz_t != nullptr) put(dz_t + j * D, sTok[2][tc][j]);
        }
      }
    }
    if (t > 0) __syncthreads();                             // the next tile's staging reuses the rows
  }

  // ---- per-(batch row, chunk) partial sums, and (first chunk) the initial state's gradient
  const int64_t bq = b * nc + chunk;
  float gdt = 0.f, gA[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float bg = Bv[i] * gB[i];
    gA[i] = fmaf(dt * ab[i], gR[i], dcda[i] * bg);
    gdt = fmaf(a[i] * ab[i], gR[i], fmaf(dcdd[i], bg, gdt));
  }
  gdt = chan_sum<SL>(gdt);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!nok[i]) continue;
    const int64_t o = (bq * D + d) * N + 4 * s + i;
    p.pA[o] = gA[i];
    p.pB[o] = cfv[i] * gB[i];
    p.pC[o] = gC[i];
    if (p.dh0 != nullptr && chunk == 0) p.dh0[(b * D + d) * N + 4 * s + i] = mu[i];
  }
  if (dvalid && s == 0) {
    p.pD[bq * D + d] = gD;
    p.pbias[bq * D + d] = gdt * dsig;
  }
}

template <typename IO, int SL, int MODE>
hipError_t launch_ti_k(const BwdParams& p, hipStream_t stream) {
  const int64_t blocks = p.batch * int64_t(MODE == TI_MAIN ? p.n_chunks : p.n_chunks - 1) * p.groups;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_ti_kernel<IO, SL, MODE>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename IO, int MODE>
hipError_t launch_ti_m(const BwdParams& p, hipStream_t stream) {
  const int SL = bwd_lanes_per_channel(p.N);
  if (SL == 4) return launch_ti_k<IO, 4, MODE>(p, stream);
  if (SL == 8) return launch_ti_k<IO, 8, MODE>(p, stream);
  return launch_ti_k<IO, 16, MODE>(p, stream);
}

template <typename IO>
hipError_t launch_ti_io(int pass, const BwdParams& p, hipStream_t stream) {
  if (pass == kTiPassState) return launch_ti_m<IO, TI_STATE>(p, stream);
  if (pass == kTiPassAdjoint) return launch_ti_m<IO, TI_ADJOINT>(p, stream);
  return launch_ti_m<IO, TI_MAIN>(p, stream);
}

}  // namespace

hipError_t launch_bwd_ti(bool bf16, int pass, const BwdParams& p, hipStream_t stream) {
  return bf16 ? launch_ti_io<uint16_t>(pass, p, stream) : launch_ti_io<float>(pass, p, stream);
}

}  // namespace selscan
