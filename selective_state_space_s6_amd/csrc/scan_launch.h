// scan_launch.h -- internal interface between the C ABI (selscan_api.cpp) and the
// kernels (scan_kernels.h and the units that instantiate it).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace selscan {

constexpr int kWavesPerBlock = 4;
enum { kPassSingle = 0, kPassState = 1, kPassApply = 2 };

// Everything one scan-kernel launch needs.  Strides are in elements.
struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;   // may be null
  const void* z;        // may be null
  void* y;
  float* last_state;    // may be null
  const float* h0;      // initial state [batch][D][N], may be null (zero); selective only
  const float* delta_bias;   // [D], may be null (zero)
  int32_t euler;        // 1: Bbar = delta * B (first-order input coefficient)
  int32_t dxf;          // 1: the step size is transformed: delta + delta_bias, then softplus if
  int32_t softplus;     //    softplus is 1
  int64_t batch, L, D, N;
  int64_t u_sb, u_sl, delta_sb, delta_sl, z_sb, z_sl, y_sb, y_sl;
  int64_t B_sb, B_sl, B_sd, C_sb, C_sl, C_sd;
  int64_t chunk_len;    // tokens per chunk (L for the single pass)
  int32_t n_chunks;     // 1 for the single pass
  int32_t groups;       // channel groups per batch row: ceil(D / channels-per-wave)
  int32_t total_items;  // batch * n_chunks * groups (one wavefront each)
  float* ws_state;      // chunked: [batch][D][N][n_chunks] end states, then carries
  float* ws_dsum;       // chunked: [batch][D][n_chunks] sum of delta per chunk
  int32_t pipelined;    // 1: scan_kernel_coop (16 lanes per channel, D % 4 == 0, u/delta/z/y
                        //    rows and B/C rows readable four elements at a time); 0: scan_kernel
  // state pass of scan_kernel_coop, selective coefficients, optional: the state from a zero
  // start and the running sum of delta at the start of every 16-token tile of the chunk
  float* ckpt;          // [batch][ck_ntiles][D][N], tile index l / 16, or null
  float* ck_dsum;       // [batch][ck_ntiles][D]
  int64_t ck_ntiles;
  int32_t state_all;    // scan_kernel_coop: the state pass runs the last chunk too (its end
                        //    state is never carried; wanted for its checkpoints)
  int32_t sched_round;  // workgroups the GPU deals out per round (its compute units; 0 if
                        //    unknown: no rotation): workgroup b arrives on its compute unit in
                        //    round b / sched_round, which sets its turn in scan_kernel_coop's
                        //    issue-priority rotation
};

struct PrefixParams {
  const float* A;
  const float* dsum;
  const float* h0;      // initial state [batch][D][N], may be null (zero)
  float* state;
  int64_t batch, D, N;
  int32_t n_chunks;
  int32_t seg_width;    // power of two >= n_chunks, <= 64
};

// Lanes per channel (S) and states per lane (K) for N states.
void lanes_for_states(int64_t N, int* S, int* K);

hipError_t launch_scan_pass(int pass, bool bf16, bool ti, int S, int K, const ScanParams& p, hipStream_t stream);
// one scan pass of one element type (scan_inst_<io>_<pass>.hip); launch_scan_pass picks one
hipError_t launch_scan_f32_single(bool ti, int S, int K, const ScanParams& p, hipStream_t stream);
hipError_t launch_scan_f32_state(bool ti, int S, int K, const ScanParams& p, hipStream_t stream);
hipError_t launch_scan_f32_apply(bool ti, int S, int K, const ScanParams& p, hipStream_t stream);
hipError_t launch_scan_bf16_single(bool ti, int S, int K, const ScanParams& p, hipStream_t stream);
hipError_t launch_scan_bf16_state(bool ti, int S, int K, const ScanParams& p, hipStream_t stream);
hipError_t launch_scan_bf16_apply(bool ti, int S, int K, const ScanParams& p, hipStream_t stream);
hipError_t launch_chunk_prefix(const PrefixParams& p, hipStream_t stream);
hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t stream);
hipError_t launch_copy(float* dst, const float* src, int64_t n, hipStream_t stream);

// One decode step (seqlen 1), state updated in place.
struct StepParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;   // may be null
  const void* z;        // may be null
  void* y;
  float* state;         // [batch][D][N]
  const float* delta_bias;   // [D], may be null (zero)
  int32_t euler;        // 1: Bbar = delta * B
  int32_t dxf;          // 1: step size delta + delta_bias, then softplus if softplus is 1
  int32_t softplus;
  int64_t batch, D, N;
  int64_t u_sb, delta_sb, z_sb, y_sb, B_sb, B_sd, C_sb, C_sd;
  int32_t vec;          // 1: N % 4 == 0, state and per-token B/C rows aligned to 4 elements
};
hipError_t launch_step(bool bf16, bool ti, const StepParams& p, hipStream_t stream);

// The convolution mode of fixed coefficients (conv_kernels.hip): delta [D], B/C [D][*] with
// channel strides B_sd / C_sd; u, z, y rows of D channels, D % 4 == 0, rows 16-byte (fp32) or
// 8-byte (bf16) aligned.
struct ConvParams {
  const void* u;
  const void* delta;
  const float* delta_bias;   // may be null
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;        // may be null
  const void* z;             // may be null
  void* y;
  float* last_state;         // may be null
  int32_t euler, dxf, softplus;
  int64_t batch, L, D, N;
  int64_t u_sb, u_sl, z_sb, z_sl, y_sb, y_sl, B_sd, C_sd;
  int32_t sched_round;       // compute units of the GPU (0 if unknown): the workgroup's dispatch
                             //    round, blockIdx / sched_round, sets its issue-priority turn
};
hipError_t launch_conv_ti(bool bf16, const ConvParams& p, hipStream_t stream);

}  // namespace selscan

namespace selscan {

// The backward pass (selective coefficients).  Strides in elements; the gradients du,
// ddelta, dz are contiguous [batch][L][D] in the I/O type.
struct BwdParams {
  const void* u;
  const void* delta;
  const float* delta_bias;   // may be null
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;   // may be null
  const void* z;        // may be null
  const float* h0;      // may be null
  const void* dy;
  const float* dlast;   // may be null
  void* du;
  void* ddelta;
  void* dz;             // may be null (then not written)
  float* dh0;           // may be null
  float* ckpt;          // [batch][ntiles][D][N] state at the start of every tile
  float* pB;            // [groups][batch][L][N] per-channel-group partial sums of dB
  float* pC;            // [groups][batch][L][N] per-group partial sums of dC
  float* pA;            // [batch][n_chunks][D][N] partial sums of dA
  float* pD;            // [batch][n_chunks][D] partial sums of dDskip
  float* pbias;         // [batch][n_chunks][D] partial sums of the bias gradient
  float* carry;         // [batch][D][N][n_chunks] state entering each chunk (n_chunks > 1)
  float* adjG;          // [batch][D][N][n_chunks] adjoint a chunk hands back from a zero start
  float* adjS;          // [batch][D][n_chunks] sum of delta over each chunk
  float* adj_in;        // [batch][D][N][n_chunks] adjoint reaching each chunk's end
  int64_t batch, L, D, N;
  int64_t u_sb, u_sl, delta_sb, delta_sl, z_sb, z_sl, dy_sb, dy_sl, B_sb, B_sl, C_sb, C_sl;
  int64_t ntiles;       // ceil(L / 16)
  int64_t chunk_len;    // tokens per chunk, a multiple of 16
  int32_t n_chunks;
  int32_t groups;       // ceil(D / channels per workgroup)
  int32_t euler;
  int32_t dxf;
  int32_t softplus;
  // 1: the forward state pass wrote each tile's zero-start state into ckpt and its running
  // sum of delta into ck_dsum, for every chunk
  int32_t ck_fwd;
  const float* ck_dsum; // [batch][ntiles][D]
  // fixed coefficients: [batch][D][n_chunks] each chunk's sum of delta (the chunk state pass
  // writes it for chunk_prefix_kernel)
  float* sdsum;
  // fixed coefficients: B_sd, C_sd (element stride between channels of B[d][n], C[d][n])
  int64_t B_sd, C_sd;
  // 1: u, delta, dy, z and du, ddelta, dz move as 4-channel vectors (D % 4 == 0; their row
  // and batch strides multiples of 4 elements, rows at least D long; bases aligned to 4
  // elements; a chunk's span under 2^31 bytes)
  int32_t vec;
};
// lanes per channel of the backward kernel (4 states per lane): 4, 8 or 16
int bwd_lanes_per_channel(int64_t N);
hipError_t launch_bwd(bool bf16, const BwdParams& p, hipStream_t stream);
// backward of fixed coefficients (bwd_ti_kernels.hip): the chunk end states from zero (for
// chunk_prefix_kernel), the chunk adjoints from zero (for bwd_adjoint_combine_kernel), or the
// main pass
enum { kTiPassState = 0, kTiPassAdjoint = 1, kTiPassMain = 2 };
hipError_t launch_bwd_ti(bool bf16, int pass, const BwdParams& p, hipStream_t stream);
// the adjoint combine of the selective backward, on its own (fixed coefficients)
hipError_t launch_bwd_adjoint_combine(const BwdParams& p, hipStream_t stream);
// out[i] = sum_{j < nparts} part[j * stride + i], i < m; out in the I/O type when bf16
hipError_t launch_sum_partials(const float* part, int64_t nparts, int64_t stride, void* out, int64_t m, bool bf16,
                               hipStream_t stream);

}  // namespace selscan

namespace selscan {

// The scalar-decay (Mamba-2) layer: bf16 x, delta, B, C, z, y; fp32 A [H], Dskip [H*P],
// states.  Contiguous: x, z, y [batch][L][H][64]; delta [batch][L][H]; B, C [batch][L][N].
struct SsdParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;   // may be null
  const void* z;        // may be null
  void* y;
  const float* h0;      // [batch][H][64][N], may be null
  float* last_state;    // [batch][H][64][N], may be null
  float* state;         // workspace [batch][H][n_chunks][64][N]: chunk states (transposed)
  uint16_t* carry;      // workspace [batch][H][n_chunks][64][N]: bf16 state entering each chunk
  float* decay;         // workspace [batch][H][n_chunks]: exp(A sum delta) of each chunk
  float* seg_state;     // workspace [batch][H][n_seg][64][N]: segment end states, then carried-in states
  float* seg_decay;     // workspace [batch][H][n_seg]: exp(A sum delta) of each segment
  int64_t batch, L, H, N;
  int64_t n_chunks;     // ceil(L / 64)
  int64_t n_seg;        // on-chip path: sequence segments (1: the whole sequence per workgroup)
  int64_t seg_chunks;   // chunks per segment (the last may have fewer)
  int32_t euler;
  int32_t fused;        // 1: on chip, one workgroup per (batch, segment, head), the state in registers
};
hipError_t launch_ssd(const SsdParams& p, hipStream_t stream);

}  // namespace selscan
