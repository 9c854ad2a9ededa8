// microbench.hip -- issue-rate and bandwidth probes of the GPU the scan runs on, built with the
// same compiler flags as the scan kernels (packed fp32 disabled).  They set the practical roofs
// the scan's measurements are read against:
//   fma     : independent fp32 fused multiply-add chains, one VALU instruction per lane each
//   exp     : independent v_exp_f32 (exp2) chains, the transcendental the scan issues per element
//   mix     : one exp2 per `ratio` FMAs in independent chains (does the transcendental overlap?)
//   dpp     : independent fp32 multiplies whose first operand is a DPP row broadcast of another
//             lane (v_mul_f32 with row_newbcast), the form the scan uses for u and delta
//   copy    : streaming 16-byte-per-lane copy of one buffer into another (HBM read + write)
//   fill    : streaming 16-byte-per-lane writes (HBM write only)
//   arbiter : workgroups of four wavefronts that repeat 64 FMAs and a workgroup barrier (the
//             per-tile shape of the scan), launched 2.5 per compute unit; every wavefront
//             records its compute unit, SIMD, start and end, with and without the scan's
//             issue-priority rotation (how the dispatcher places workgroups, and how the
//             arbiter shares a SIMD between the wavefronts of workgroups dealt to it in turn)
// Every probe records, in wavefront 0 of workgroup 0, the shader-clock counter (clock64) and the
// constant-rate wall counter (wall_clock64) around its loop, so that the clock the GPU ran at is
// measured too.  Host entry points return the kernel time from HIP events on their own stream.
// Not part of the scan library: bench.py loads it for its --microbench report only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 8;
constexpr int kRounds = 8;   // unrolled rounds per loop iteration

__device__ __forceinline__ void stamp(uint64_t* clk, int slot) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[2 * slot] = clock64();
    clk[2 * slot + 1] = wall_clock64();
  }
}

__global__ __launch_bounds__(kThreads) void fma_kernel(float* out, int iters, float a, float b, uint64_t* clk) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = float(threadIdx.x) * 1e-3f + float(c);
  stamp(clk, 0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) x[c] = fmaf(x[c], a, b);
    }
  }
  stamp(clk, 1);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void exp_kernel(float* out, int iters, float a, uint64_t* clk) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = a - float(c) - float(threadIdx.x) * 1e-3f;
  stamp(clk, 0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(x[c]);
    }
  }
  stamp(clk, 1);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// kChains chains x[c] = bcast15(x[c]) * a: the row-broadcast operand folds into the multiply
// (one v_mul_f32_dpp) only when the other operand is a VGPR, as in the scan, where it is a
// per-lane constant; a is therefore held in a VGPR (a multiply by an SGPR would issue a
// separate v_mov_b32_dpp first)
__global__ __launch_bounds__(kThreads) void dpp_kernel(float* out, int iters, float a_arg, uint64_t* clk) {
  float a = a_arg;
  __asm__ volatile("" : "+v"(a));
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = float(threadIdx.x) * 1e-3f + float(c);
  stamp(clk, 0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        x[c] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[c]), 0x15F, 0xF, 0xF, true)) * a;
    }
  }
  stamp(clk, 1);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// Arbitration probe.  Each wavefront runs `iters` iterations of 64 FMAs (8 chains) and a
// workgroup barrier; `lds` bytes of dynamic LDS per workgroup bound how many share a compute
// unit.  Lane 0 of every wavefront records [start, end] (s_memrealtime, 100 MHz), HW_ID and
// XCC_ID into rec[(block * 4 + wave) * 4 ...].  ROTATE: the workgroups of dispatch rounds
// (block / cus) take turns at the top issue priority in slices of 2^11 ticks, as the scan does.
template <bool ROTATE>
__global__ __launch_bounds__(kThreads) void arbiter_kernel(float* out, uint64_t* rec, int iters, float a, float b,
                                                           int cus) {
  extern __shared__ float lds_pad[];
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);
  const uint32_t round = uint32_t(blockIdx.x) / uint32_t(cus);
  uint64_t clk = 0;
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = float(threadIdx.x) * 1e-3f + float(c);
  for (int i = 0; i < iters; ++i) {
    if (ROTATE) {
      const uint32_t ph = (uint32_t(clk >> 11) + round) % 3u;
      if (ph == 0) __builtin_amdgcn_s_setprio(3);
      else if (ph == 1) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(1);
    }
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) x[c] = fmaf(x[c], a, b);
    }
    __syncthreads();
    if (ROTATE) clk = __builtin_amdgcn_s_memrealtime();
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) sum += x[c];
  if (iters < 0) lds_pad[threadIdx.x] = sum;   // never taken; keeps the LDS request
  out[blockIdx.x * kThreads + threadIdx.x] = sum;
  if ((threadIdx.x & 63) == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    uint64_t* q = rec + (size_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 4;
    q[0] = t0; q[1] = t1; q[2] = hw; q[3] = xcc;
  }
}

// RATIO fma per exp2: kChains exp2 chains and kChains fma chains, each fma chain stepped RATIO
// times per exp2 step
template <int RATIO>
__global__ __launch_bounds__(kThreads) void mix_kernel(float* out, int iters, float a, float b, uint64_t* clk) {
  float x[kChains], y[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    x[c] = a - float(c) - float(threadIdx.x) * 1e-3f;
    y[c] = float(threadIdx.x) * 1e-3f + float(c);
  }
  stamp(clk, 0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        x[c] = __builtin_amdgcn_exp2f(x[c]);
#pragma unroll
        for (int k = 0; k < RATIO; ++k) y[c] = fmaf(y[c], a, b);
      }
    }
  }
  stamp(clk, 1);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c] + y[c];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                        int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void fill_kernel(float4* __restrict__ dst, int64_t n, float v) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) dst[i] = make_float4(v, v, v, v);
}

thread_local int g_err = 0;

// Time `launch` (called with the stream) between two events; 0 on success.
template <typename F>
int timed(F&& launch, hipStream_t s, float* ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1;
  if (hipEventCreate(&e1) != hipSuccess) { (void)hipEventDestroy(e0); return -1; }
  hipError_t e = hipEventRecord(e0, s);
  if (e == hipSuccess) { launch(); e = hipGetLastError(); }
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  g_err = int(e);
  return e == hipSuccess ? 0 : -1;
}

}  // namespace

extern "C" {

// The last hipError_t a probe met (0: none).
int selscan_mb_last_error(void) { return g_err; }

// Compute-rate probes.  kind: 0 fma, 1 exp2, 2 mix with 1 fma per exp2, 3 ratio 2, 4 ratio 4,
// 5 ratio 8, 6 multiply with a DPP row-broadcast operand.  blocks workgroups of 256 lanes run `iters` loop iterations of 8 rounds over 8
// independent chains.  Outputs: kernel milliseconds, the shader-clock cycles and the wall-clock
// ticks wavefront 0 of workgroup 0 measured around its loop.  Returns 0 on success.
int selscan_mb_compute(int kind, int blocks, int iters, float* ms, uint64_t* cycles, uint64_t* ticks) {
  if (blocks < 1 || iters < 1 || kind < 0 || kind > 6) return -2;
  float* out = nullptr;
  uint64_t* clk = nullptr;
  hipStream_t s = nullptr;
  if (hipMalloc(&out, size_t(blocks) * kThreads * sizeof(float)) != hipSuccess) return -1;
  if (hipMalloc(&clk, 4 * sizeof(uint64_t)) != hipSuccess) { (void)hipFree(out); return -1; }
  if (hipStreamCreate(&s) != hipSuccess) { (void)hipFree(out); (void)hipFree(clk); return -1; }
  const float a = 0.999f, b = 1e-3f;
  auto launch = [&]() {
    const dim3 g{unsigned(blocks)}, t{unsigned(kThreads)};
    switch (kind) {
      case 0: hipLaunchKernelGGL(fma_kernel, g, t, 0, s, out, iters, a, b, clk); break;
      case 1: hipLaunchKernelGGL(exp_kernel, g, t, 0, s, out, iters, -4.f, clk); break;
      case 2: hipLaunchKernelGGL(mix_kernel<1>, g, t, 0, s, out, iters, a, b, clk); break;
      case 3: hipLaunchKernelGGL(mix_kernel<2>, g, t, 0, s, out, iters, a, b, clk); break;
      case 4: hipLaunchKernelGGL(mix_kernel<4>, g, t, 0, s, out, iters, a, b, clk); break;
      case 5: hipLaunchKernelGGL(mix_kernel<8>, g, t, 0, s, out, iters, a, b, clk); break;
      default: hipLaunchKernelGGL(dpp_kernel, g, t, 0, s, out, iters, a, clk); break;
    }
  };
  launch();                                                   // warm-up
  int rc = hipStreamSynchronize(s) == hipSuccess ? timed(launch, s, ms) : -1;
  uint64_t h[4] = {0, 0, 0, 0};
  if (rc == 0 && hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) rc = -1;
  *cycles = h[2] - h[0];
  *ticks = h[3] - h[1];
  (void)hipStreamDestroy(s);
  (void)hipFree(out);
  (void)hipFree(clk);
  return rc;
}

// Bandwidth probes over `bytes` bytes (a multiple of 16): kind 0 copies one buffer into
// another (bytes read and bytes written), kind 1 fills one buffer.  The best of `reps` timed
// runs, in milliseconds.
int selscan_mb_bandwidth(int kind, int64_t bytes, int blocks, int reps, float* ms) {
  if (bytes < 16 || bytes % 16 != 0 || blocks < 1 || reps < 1 || kind < 0 || kind > 1) return -2;
  float4* a = nullptr;
  float4* b = nullptr;
  hipStream_t s = nullptr;
  if (hipMalloc(&a, size_t(bytes)) != hipSuccess) return -1;
  if (hipMalloc(&b, size_t(bytes)) != hipSuccess) { (void)hipFree(a); return -1; }
  if (hipStreamCreate(&s) != hipSuccess) { (void)hipFree(a); (void)hipFree(b); return -1; }
  const int64_t n = bytes / 16;
  hipLaunchKernelGGL(fill_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, a, n, 1.f);
  auto launch = [&]() {
    if (kind == 0) hipLaunchKernelGGL(copy_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, a, b, n);
    else hipLaunchKernelGGL(fill_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, b, n, 2.f);
  };
  launch();
  int rc = hipStreamSynchronize(s) == hipSuccess ? 0 : -1;
  float best = 0.f;
  for (int r = 0; rc == 0 && r < reps; ++r) {
    float t = 0.f;
    rc = timed(launch, s, &t);
    if (rc == 0 && (r == 0 || t < best)) best = t;
  }
  *ms = best;
  (void)hipStreamDestroy(s);
  (void)hipFree(a);
  (void)hipFree(b);
  return rc;
}

// Arbitration probe (see arbiter_kernel): `blocks` workgroups, `iters` iterations, `lds_bytes`
// of LDS per workgroup (at most 65536), rotate 0/1.  rec (host, blocks * 16 values) receives
// each wavefront's [start, end, HW_ID, XCC_ID]; ms the kernel time (HIP events, second run).
int selscan_mb_arbiter(int rotate, int blocks, int iters, int lds_bytes, uint64_t* rec, float* ms) {
  if (blocks < 1 || iters < 1 || lds_bytes < 0 || lds_bytes > 65536 || rec == nullptr) return -2;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -1;
  float* out = nullptr;
  uint64_t* drec = nullptr;
  hipStream_t s = nullptr;
  const size_t rec_bytes = size_t(blocks) * 16 * sizeof(uint64_t);
  if (hipMalloc(&out, size_t(blocks) * kThreads * sizeof(float)) != hipSuccess) return -1;
  if (hipMalloc(&drec, rec_bytes) != hipSuccess) { (void)hipFree(out); return -1; }
  if (hipStreamCreate(&s) != hipSuccess) { (void)hipFree(out); (void)hipFree(drec); return -1; }
  auto launch = [&]() {
    const dim3 g{unsigned(blocks)}, t{unsigned(kThreads)};
    if (rotate) hipLaunchKernelGGL(arbiter_kernel<true>, g, t, size_t(lds_bytes), s, out, drec, iters, 0.999f, 1e-3f, cus);
    else hipLaunchKernelGGL(arbiter_kernel<false>, g, t, size_t(lds_bytes), s, out, drec, iters, 0.999f, 1e-3f, cus);
  };
  launch();                                                   // warm-up
  int rc = hipStreamSynchronize(s) == hipSuccess ? timed(launch, s, ms) : -1;
  if (rc == 0 && hipMemcpy(rec, drec, rec_bytes, hipMemcpyDeviceToHost) != hipSuccess) rc = -1;
  (void)hipStreamDestroy(s);
  (void)hipFree(out);
  (void)hipFree(drec);
  return rc;
}

// The wall-clock counter's rate (kHz), for converting ticks to seconds.
int selscan_mb_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

}  // extern "C"
