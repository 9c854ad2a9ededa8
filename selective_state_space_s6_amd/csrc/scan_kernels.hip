// scan_kernels.hip -- launchers of the selective-scan forward (S6): the decode step, the
// chunk prefix, the fills, and the dispatch of a scan pass to the unit that instantiates
// it (scan_inst_<io>_<pass>.hip).  The kernels themselves are in scan_kernels.h.
#include "scan_kernels.h"

namespace selscan {
namespace {

// ---------------------------------------------------------------------------------------
// chunk prefix: per (b, d, n), turn chunk end states into carried-in states.
// Lanes of a segment are the chunks 0 .. n_chunks-1 (segment width W = pow2 >= n_chunks).
// Chunk c's map is h -> P_c h + H_c with P_c = exp(A sum_{t in c} delta_t); an inclusive
// log-depth scan composes (P1,H1).(P2,H2) = (P2 P1, P2 H1 + H2); the carried-in state of
// chunk c is the composed H up to chunk c-1 (the initial state for chunk 0, which also
// enters chunk 0's map as P_0 h0 + H_0).

__global__ __launch_bounds__(256)
void chunk_prefix_kernel(PrefixParams p) {
  const int lane = threadIdx.x & 63;
  const int W = p.seg_width;                         // power of two, <= 64
  const int seg_in_wave = lane / W, i = lane % W;
  const int64_t seg = (int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6)) * (64 / W) + seg_in_wave;
  const int64_t nseg = p.batch * p.D * p.N;
  const bool live = seg < nseg && i < p.n_chunks;
  float P = 1.f, H = 0.f, h0 = 0.f;
  int64_t b = 0, d = 0, n = 0;
  if (live) {
    n = seg % p.N;
    d = (seg / p.N) % p.D;
    b = seg / (p.N * p.D);
    const float a2 = p.A[d * p.N + n] * kLog2e;
    if (i < p.n_chunks - 1) {          // the last chunk's map is never used (nor computed)
      P = __builtin_amdgcn_exp2f(a2 * p.dsum[(b * p.D + d) * p.n_chunks + i]);
      H = p.state[seg * p.n_chunks + i];
    }
    if (p.h0 != nullptr) {             // a given initial state enters through chunk 0's map
      h0 = p.h0[seg];
      if (i == 0) H = fmaf(P, h0, H);
    }
  }
  for (int off = 1; off < W; off <<= 1) {
    const float Pp = __shfl_up(P, off, W);
    const float Hp = __shfl_up(H, off, W);
    if (i >= off) {
      H = fmaf(P, Hp, H);
      P = P * Pp;
    }
  }
  const float carry = __shfl_up(H, 1, W);
  if (live) p.state[seg * p.n_chunks + i] = (i == 0) ? h0 : carry;
}

// zero-fill (empty sequence: last_state = 0); a kernel, not a memset, so callers may
// capture it in a graph.
__global__ __launch_bounds__(256)
void fill_zero_kernel(float* x, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    x[i] = 0.f;
}

// copy (empty sequence with an initial state: last_state = initial_state)
__global__ __launch_bounds__(256)
void copy_kernel(float* dst, const float* src, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

}  // namespace

void lanes_for_states(int64_t N, int* S, int* K) {
  if (N <= 4) { *S = 4; *K = 1; }
  else if (N <= 8) { *S = 8; *K = 1; }
  else if (N <= 16) { *S = 16; *K = 1; }
  else if (N <= 32) { *S = 16; *K = 2; }
  else { *S = 16; *K = 4; }
}

hipError_t launch_scan_pass(int pass, bool bf16, bool ti, int S, int K, const ScanParams& p, hipStream_t stream) {
  switch (pass) {
    case kPassSingle: return bf16 ? launch_scan_bf16_single(ti, S, K, p, stream) : launch_scan_f32_single(ti, S, K, p, stream);
    case kPassState: return bf16 ? launch_scan_bf16_state(ti, S, K, p, stream) : launch_scan_f32_state(ti, S, K, p, stream);
    case kPassApply: return bf16 ? launch_scan_bf16_apply(ti, S, K, p, stream) : launch_scan_f32_apply(ti, S, K, p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_prefix(const PrefixParams& p, hipStream_t stream) {
  const int64_t segs = p.batch * p.D * p.N;
  const int per_wave = 64 / p.seg_width;
  const int64_t waves = (segs + per_wave - 1) / per_wave;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(chunk_prefix_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_copy(float* dst, const float* src, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, dst, src, n);
  return hipGetLastError();
}

hipError_t launch_step(bool bf16, bool ti, const StepParams& p, hipStream_t stream) {
  if (bf16) return ti ? launch_step_t<uint16_t, true>(p, stream) : launch_step_t<uint16_t, false>(p, stream);
  return ti ? launch_step_t<float, true>(p, stream) : launch_step_t<float, false>(p, stream);
}

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, x, n);
  return hipGetLastError();
}

}  // namespace selscan
