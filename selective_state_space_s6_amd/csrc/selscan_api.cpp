// selscan_api.cpp -- the C ABI of libselscan.so: argument checks, path choice, workspace,
// and the launch sequence.  The operation itself is documented in include/selscan.h.
#include "selscan.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "scan_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = int(e);
  return SELSCAN_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Plan {
  bool ti = false;
  bool bf16 = false;
  int S = 16, K = 1;
  int64_t groups = 0;         // channel groups per batch row
  bool chunked = false;
  bool conv = false;          // the convolution mode of fixed coefficients
  int64_t chunk_len = 0;
  int32_t n_chunks = 1;
  size_t ws_bytes = 0;        // workspace the chunked path needs
  size_t ws_state_bytes = 0;
};

constexpr int64_t kMaxChunks = 64;
constexpr int64_t kTargetWaves = 4096;   // about four wavefronts per SIMD on 256 CUs

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Validate dims and choose the schedule.  Does not look at pointers.
// The automatic path takes the convolution mode for fixed coefficients when it has one
// wavefront per (batch row, channel) for at least this many and the sequence fills a 256-token
// super-tile: measured faster than the recurrence on the time-invariant workload (batch 4,
// L 8192, D 1024, N 64).  Fewer (batch, channel) pairs leave the recurrence's sequence chunks
// as the better source of parallelism.
constexpr int64_t kConvMinWaves = 1024;
constexpr int64_t kConvMinLen = 256;

int make_plan(const selscan_dims* dims, Plan* plan, bool allow_auto_conv = true) {
  if (!dims) return SELSCAN_ERR_NULL;
  if (dims->abi_version != SELSCAN_ABI_VERSION) return SELSCAN_ERR_ABI;
  const selscan_dims& d = *dims;
  if (d.batch < 0 || d.seqlen < 0 || d.dim < 1 || d.dstate < 1) return SELSCAN_ERR_DIMS;
  const int64_t strides[] = {d.u_sb, d.u_sl, d.delta_sb, d.delta_sl, d.z_sb, d.z_sl, d.y_sb, d.y_sl,
                             d.B_sb, d.B_sl, d.B_sd, d.C_sb, d.C_sl, d.C_sd};
  for (int64_t s : strides)
    if (s < 0) return SELSCAN_ERR_DIMS;
  if (d.dstate > 64) return SELSCAN_ERR_UNSUPPORTED;
  if (d.io_dtype != SELSCAN_F32 && d.io_dtype != SELSCAN_BF16) return SELSCAN_ERR_UNSUPPORTED;
  const int32_t path = d.path & ~int32_t(SELSCAN_PATH_FLAG_SCALAR_IO);
  if (path != SELSCAN_PATH_AUTO && path != SELSCAN_PATH_SINGLE && path != SELSCAN_PATH_CHUNKED &&
      path != SELSCAN_PATH_CONV)
    return SELSCAN_ERR_UNSUPPORTED;
  if (d.chunk_len < 0 || d.chunk_len % 16 != 0) return SELSCAN_ERR_UNSUPPORTED;
  if (d.discretization != SELSCAN_DISC_ZOH && d.discretization != SELSCAN_DISC_EULER) return SELSCAN_ERR_UNSUPPORTED;
  // y rows must not overlap (every (b, l, d) is written exactly once)
  if ((d.seqlen > 1 && d.y_sl < d.dim) || (d.batch > 1 && d.y_sb < d.seqlen * d.y_sl && d.seqlen > 0))
    return SELSCAN_ERR_UNSUPPORTED;
  // the kernels address a 16-token tile with 32-bit byte offsets from a per-tile base
  const int64_t kMaxRowStride = int64_t(1) << 26;
  if (d.u_sl > kMaxRowStride || d.delta_sl > kMaxRowStride || d.z_sl > kMaxRowStride || d.y_sl > kMaxRowStride ||
      d.B_sl > kMaxRowStride || d.C_sl > kMaxRowStride || d.dim > kMaxRowStride)
    return SELSCAN_ERR_UNSUPPORTED;
  // grid-size limits of this implementation (item indices are 32-bit)
  if (d.dim > (int64_t(1) << 30) || d.batch > (int64_t(1) << 30)) return SELSCAN_ERR_UNSUPPORTED;

  const bool bc_per_token = d.B_sd == 0 && d.C_sd == 0;
  const bool bc_per_channel = d.B_sb == 0 && d.B_sl == 0 && d.C_sb == 0 && d.C_sl == 0 && d.B_sd >= d.dstate &&
                              d.C_sd >= d.dstate;
  const bool delta_per_channel = d.delta_sb == 0 && d.delta_sl == 0;
  Plan p;
  if (bc_per_token) p.ti = false;
  else if (bc_per_channel && delta_per_channel) p.ti = true;
  else return SELSCAN_ERR_UNSUPPORTED;
  p.bf16 = d.io_dtype == SELSCAN_BF16;
  // whole 4-channel vectors of u, z and y per token (their pointers are checked per call)
  const bool conv_ok = p.ti && d.dim % 4 == 0 && d.u_sb % 4 == 0 && d.u_sl % 4 == 0 && d.z_sb % 4 == 0 &&
                       d.z_sl % 4 == 0 && d.y_sb % 4 == 0 && d.y_sl % 4 == 0 && d.chunk_len == 0;
  const bool auto_conv = path == SELSCAN_PATH_AUTO && allow_auto_conv && conv_ok &&
                         d.batch * d.dim >= kConvMinWaves && d.seqlen >= kConvMinLen;
  if (path == SELSCAN_PATH_CONV || auto_conv) {
    if (!conv_ok) return SELSCAN_ERR_UNSUPPORTED;
    p.conv = true;
    p.chunk_len = d.seqlen;
    p.n_chunks = 1;
    p.groups = (d.dim + 15) / 16;
    *plan = p;
    return SELSCAN_OK;
  }
  selscan::lanes_for_states(d.dstate, &p.S, &p.K);
  const int cw = 64 / p.S;
  p.groups = (d.dim + cw - 1) / cw;
  const int64_t waves_single = d.batch * p.groups;
  if (waves_single > (int64_t(1) << 31) - 1) return SELSCAN_ERR_UNSUPPORTED;

  // Each work item addresses its tokens through 32-bit buffer offsets; inactive lanes use
  // offset 2^31, so a work item may span at most 2^30 bytes of any tensor (no wrap-around).
  const int64_t es = d.io_dtype == SELSCAN_BF16 ? 2 : 4;
  int64_t max_sl = d.u_sl;
  for (int64_t v : {d.delta_sl, d.z_sl, d.y_sl, d.B_sl, d.C_sl}) max_sl = v > max_sl ? v : max_sl;
  const int64_t max_cols = d.dim > d.dstate ? d.dim : d.dstate;
  const int64_t kSpan = int64_t(1) << 30;
  auto span_ok = [&](int64_t rows) { return (rows * max_sl + max_cols + 16 * max_sl) * es <= kSpan; };
  int64_t max_rows = max_sl > 0 ? (kSpan / es - max_cols) / max_sl - 16 : d.seqlen;
  max_rows = max_rows / 16 * 16;
  if (max_cols * es > kSpan / 2 || max_rows < 16) return SELSCAN_ERR_UNSUPPORTED;

  // chunking: when the single pass leaves the GPU under-filled and the sequence is long,
  // or when one pass over the whole sequence would exceed the addressing span
  bool chunk = false;
  int64_t nc = 1;
  if (path != SELSCAN_PATH_CHUNKED && !span_ok(d.seqlen)) {
    if (path == SELSCAN_PATH_SINGLE) return SELSCAN_ERR_UNSUPPORTED;
    chunk = true;
    nc = (d.seqlen + max_rows - 1) / max_rows;
  } else if (path == SELSCAN_PATH_CHUNKED) {
    chunk = d.seqlen > 0;
    if (d.chunk_len > 0) nc = (d.seqlen + d.chunk_len - 1) / d.chunk_len;
    else nc = (d.seqlen + 63) / 64 < kMaxChunks ? (d.seqlen + 63) / 64 : kMaxChunks;
  } else if (path == SELSCAN_PATH_AUTO && d.seqlen >= 256 && waves_single > 0 && waves_single < kTargetWaves / 2) {
    nc = (kTargetWaves + waves_single - 1) / waves_single;
    const int64_t by_len = d.seqlen / 128;               // chunks of at least 128 tokens
    if (nc > by_len) nc = by_len;
    if (nc > kMaxChunks) nc = kMaxChunks;
    chunk = nc >= 2;
  }
  if (chunk) {
    if (nc < 1) nc = 1;
    if (nc > kMaxChunks) return SELSCAN_ERR_UNSUPPORTED;   // forced chunk_len too small
    p.chunk_len = d.chunk_len > 0 ? d.chunk_len : round_up((d.seqlen + nc - 1) / nc, 16);
    if (!span_ok(p.chunk_len)) return SELSCAN_ERR_UNSUPPORTED;
    p.n_chunks = int32_t((d.seqlen + p.chunk_len - 1) / p.chunk_len);
    p.chunked = true;
    p.ws_state_bytes = size_t(round_up(int64_t(sizeof(float)) * d.batch * d.dim * d.dstate * p.n_chunks, 256));
    p.ws_bytes = p.ws_state_bytes + size_t(round_up(int64_t(sizeof(float)) * d.batch * d.dim * p.n_chunks, 256));
  } else {
    p.chunk_len = d.seqlen;
    p.n_chunks = 1;
  }
  if (d.batch * p.n_chunks * p.groups > (int64_t(1) << 31) - 1) return SELSCAN_ERR_UNSUPPORTED;
  *plan = p;
  return SELSCAN_OK;
}

int check_pointers(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* Dskip, const void* z, const void* y, const float* last_state, int io_dtype,
                   bool no_tokens) {
  // With no tokens (batch * seqlen == 0) nothing is read from the per-token tensors, and an
  // empty tensor may legitimately have a NULL address.
  if (!A || (!no_tokens && (!u || !delta || !B || !C || !y))) return SELSCAN_ERR_NULL;
  const size_t es = io_dtype == SELSCAN_BF16 ? 2 : 4;
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(y, es) ||
      (z && !aligned(z, es)))
    return SELSCAN_ERR_ALIGN;
  if (!aligned(A, 4) || (Dskip && !aligned(Dskip, 4)) || (last_state && !aligned(last_state, 4)))
    return SELSCAN_ERR_ALIGN;
  return SELSCAN_OK;
}

// Compute units of the GPU that `stream` belongs to, looked up once per GPU; 0 if the lookup
// fails (the issue-priority rotation of scan_kernel_coop then takes every workgroup as round 0).
constexpr int kMaxCuDevices = 64;
std::atomic<int> g_cu_count[kMaxCuDevices];
int compute_units(hipStream_t stream) {
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
    (void)hipGetLastError();              // not an error of this call's launches
    return 0;
  }
  if (dev < 0 || dev >= kMaxCuDevices) return 0;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      return 0;
    }
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Kernel parameters of one forward call (chunk plan, options, path choice); the chunked
// path's workspace pointers are set by the caller.
selscan::ScanParams scan_params(const void* u, const void* delta, const float* delta_bias, const float* A,
                                const void* B, const void* C, const float* Dskip, const void* z, void* y,
                                const float* h0, float* last_state, const selscan_dims& d, const Plan& plan) {
  selscan::ScanParams p{};
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = Dskip; p.z = z; p.y = y;
  p.last_state = last_state;
  p.h0 = h0;
  p.delta_bias = delta_bias;
  p.euler = d.discretization == SELSCAN_DISC_EULER ? 1 : 0;
  p.softplus = d.delta_softplus != 0 ? 1 : 0;
  p.dxf = (p.softplus || delta_bias != nullptr) ? 1 : 0;
  p.batch = d.batch; p.L = d.seqlen; p.D = d.dim; p.N = d.dstate;
  p.u_sb = d.u_sb; p.u_sl = d.u_sl; p.delta_sb = d.delta_sb; p.delta_sl = d.delta_sl;
  p.z_sb = d.z_sb; p.z_sl = d.z_sl; p.y_sb = d.y_sb; p.y_sl = d.y_sl;
  p.B_sb = d.B_sb; p.B_sl = d.B_sl; p.B_sd = d.B_sd; p.C_sb = d.C_sb; p.C_sl = d.C_sl; p.C_sd = d.C_sd;
  p.chunk_len = plan.chunk_len;
  p.n_chunks = plan.n_chunks;
  p.groups = int32_t(plan.groups);
  p.total_items = int32_t(d.batch * plan.n_chunks * plan.groups);
  // cooperative pipelined kernel: 16 lanes per channel, whole 4-channel vectors (D % 4 == 0,
  // u/delta/z/y rows on 4-element boundaries) and per-token B/C rows readable four states
  // at a time (N % 4 == 0, rows on 4-element boundaries)
  {
    const uintptr_t qbytes = uintptr_t(4) * (plan.bf16 ? 2 : 4);
    auto quad_ok = [&](const void* ptr, int64_t sb, int64_t sl) {
      return ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) % qbytes == 0 && sb % 4 == 0 && sl % 4 == 0);
    };
    const bool io_ok = d.dim % 4 == 0 && quad_ok(u, d.u_sb, d.u_sl) && quad_ok(z, d.z_sb, d.z_sl) &&
                       quad_ok(y, d.y_sb, d.y_sl) && (plan.ti || quad_ok(delta, d.delta_sb, d.delta_sl));
    const bool bc_ok = plan.ti || (d.dstate % 4 == 0 && quad_ok(B, d.B_sb, d.B_sl) && quad_ok(C, d.C_sb, d.C_sl));
    p.pipelined = (plan.S == 16 && io_ok && bc_ok && !(d.path & SELSCAN_PATH_FLAG_SCALAR_IO)) ? 1 : 0;
  }
  return p;
}

int run(const void* u, const void* delta, const float* delta_bias, const float* A, const void* B, const void* C,
        const float* Dskip, const void* z, void* y, const float* h0, float* last_state, const selscan_dims* dims,
        const Plan& plan, void* workspace, hipStream_t stream) {
  const selscan_dims& d = *dims;
  if (d.batch == 0) return SELSCAN_OK;
  if (d.seqlen == 0) {                     // no tokens: the initial state is handed back
    if (last_state && last_state != h0) {
      const int64_t n = d.batch * d.dim * d.dstate;
      hipError_t e = h0 ? selscan::launch_copy(last_state, h0, n, stream) : selscan::launch_fill_zero(last_state, n, stream);
      if (e != hipSuccess) return hip_fail(e);
    }
    return SELSCAN_OK;
  }
  hipError_t e;
  if (plan.conv) {
    selscan::ConvParams c{};
    c.u = u; c.delta = delta; c.delta_bias = delta_bias; c.A = A; c.B = B; c.C = C; c.Dskip = Dskip; c.z = z;
    c.y = y; c.last_state = last_state;
    c.euler = d.discretization == SELSCAN_DISC_EULER ? 1 : 0;
    c.softplus = d.delta_softplus != 0 ? 1 : 0;
    c.dxf = (c.softplus || delta_bias != nullptr) ? 1 : 0;
    c.batch = d.batch; c.L = d.seqlen; c.D = d.dim; c.N = d.dstate;
    c.u_sb = d.u_sb; c.u_sl = d.u_sl; c.z_sb = d.z_sb; c.z_sl = d.z_sl; c.y_sb = d.y_sb; c.y_sl = d.y_sl;
    c.B_sd = d.B_sd; c.C_sd = d.C_sd;
    c.sched_round = compute_units(stream);
    e = selscan::launch_conv_ti(plan.bf16, c, stream);
    return e == hipSuccess ? SELSCAN_OK : hip_fail(e);
  }
  selscan::ScanParams p = scan_params(u, delta, delta_bias, A, B, C, Dskip, z, y, h0, last_state, d, plan);
  p.sched_round = compute_units(stream);
  if (!plan.chunked) {
    e = selscan::launch_scan_pass(selscan::kPassSingle, plan.bf16, plan.ti, plan.S, plan.K, p, stream);
    return e == hipSuccess ? SELSCAN_OK : hip_fail(e);
  }
  char* ws = static_cast<char*>(workspace);
  p.ws_state = reinterpret_cast<float*>(ws);
  p.ws_dsum = reinterpret_cast<float*>(ws + plan.ws_state_bytes);
  e = selscan::launch_scan_pass(selscan::kPassState, plan.bf16, plan.ti, plan.S, plan.K, p, stream);
  if (e != hipSuccess) return hip_fail(e);
  selscan::PrefixParams q{};
  q.A = A; q.dsum = p.ws_dsum; q.state = p.ws_state; q.h0 = h0;
  q.batch = d.batch; q.D = d.dim; q.N = d.dstate; q.n_chunks = plan.n_chunks;
  int w = 1;
  while (w < plan.n_chunks) w <<= 1;
  q.seg_width = w;
  e = selscan::launch_chunk_prefix(q, stream);
  if (e != hipSuccess) return hip_fail(e);
  e = selscan::launch_scan_pass(selscan::kPassApply, plan.bf16, plan.ti, plan.S, plan.K, p, stream);
  return e == hipSuccess ? SELSCAN_OK : hip_fail(e);
}

// The forward pass with an optional initial state.  A missing workspace is allocated
// stream-ordered when allow_alloc, else reported.
int fwd_impl(const void* u, const void* delta, const float* delta_bias, const float* A, const void* B,
             const void* C, const float* Dskip, const void* z, void* y, const float* h0, float* last_state,
             const selscan_dims* dims, void* workspace, size_t workspace_bytes, bool allow_alloc,
             hipStream_t stream) {
  Plan plan;
  int st = make_plan(dims, &plan);
  if (st != SELSCAN_OK) return st;
  st = check_pointers(u, delta, A, B, C, Dskip, z, y, last_state, dims->io_dtype, dims->batch * dims->seqlen == 0);
  if (st != SELSCAN_OK) return st;
  if (h0 != nullptr) {
    if (plan.ti) return SELSCAN_ERR_UNSUPPORTED;      // the time-invariant kernels keep a scaled state
    if (!aligned(h0, 4)) return SELSCAN_ERR_ALIGN;
  }
  if (delta_bias != nullptr && !aligned(delta_bias, 4)) return SELSCAN_ERR_ALIGN;
  if (plan.conv) {                                    // vectors of 4 channels per access
    const size_t vb = dims->io_dtype == SELSCAN_BF16 ? 8 : 16;
    if (!aligned(u, vb) || !aligned(y, vb) || (z != nullptr && !aligned(z, vb))) {
      const int32_t path = dims->path & ~int32_t(SELSCAN_PATH_FLAG_SCALAR_IO);
      if (path != SELSCAN_PATH_AUTO) return SELSCAN_ERR_UNSUPPORTED;
      st = make_plan(dims, &plan, false);               // the automatic path falls back to the recurrence
      if (st != SELSCAN_OK) return st;
    }
  }
  const bool need_ws = plan.chunked && dims->batch > 0 && dims->seqlen > 0;
  if (!need_ws || workspace != nullptr) {
    if (need_ws && (workspace_bytes < plan.ws_bytes || !aligned(workspace, 256))) return SELSCAN_ERR_WORKSPACE;
    return run(u, delta, delta_bias, A, B, C, Dskip, z, y, h0, last_state, dims, plan, workspace, stream);
  }
  if (!allow_alloc) return SELSCAN_ERR_WORKSPACE;
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, plan.ws_bytes, stream);
  if (e != hipSuccess) return hip_fail(e);
  st = run(u, delta, delta_bias, A, B, C, Dskip, z, y, h0, last_state, dims, plan, ws, stream);
  e = hipFreeAsync(ws, stream);
  if (st == SELSCAN_OK && e != hipSuccess) return hip_fail(e);
  return st;
}

// ---- the no-allocation forward (selective_scan_fwd_noalloc)
// The chunked path's workspace lives in this file-scope device array, one copy per GPU that
// loads the library, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is a stand-in, not a device address): the device address of
// each GPU's copy is looked up once, with that GPU current, and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = SELSCAN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of the scratch array on the GPU that `stream` belongs to.
int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return SELSCAN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e);
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e);
    if (back != hipSuccess) return hip_fail(back);
    if (ptr == nullptr) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SELSCAN_OK;
}

int fwd_noalloc(const void* u, const void* delta, const float* delta_bias, const float* A, const void* B,
                const void* C, const float* Dskip, const void* z, void* y, const float* h0, float* last_state,
                const selscan_dims* dims, hipStream_t stream) {
  Plan plan;
  int st = make_plan(dims, &plan);
  if (st != SELSCAN_OK) return st;
  const bool need_ws = plan.chunked && dims->batch > 0 && dims->seqlen > 0;
  if (!need_ws)
    return fwd_impl(u, delta, delta_bias, A, B, C, Dskip, z, y, h0, last_state, dims, nullptr, 0, false, stream);
  if (plan.ws_bytes > kScratchBytes) return SELSCAN_ERR_SCRATCH_LIMIT;
  // argument errors are reported before the device is touched (fwd_impl repeats them)
  st = check_pointers(u, delta, A, B, C, Dskip, z, y, last_state, dims->io_dtype, false);
  if (st != SELSCAN_OK) return st;
  if (h0 != nullptr && plan.ti) return SELSCAN_ERR_UNSUPPORTED;
  if ((h0 != nullptr && !aligned(h0, 4)) || (delta_bias != nullptr && !aligned(delta_bias, 4)))
    return SELSCAN_ERR_ALIGN;
  void* ws = nullptr;
  st = scratch_for_stream(stream, &ws);
  if (st != SELSCAN_OK) return st;
  return fwd_impl(u, delta, delta_bias, A, B, C, Dskip, z, y, h0, last_state, dims, ws, kScratchBytes, false,
                  stream);
}

// ---- backward pass
struct BwdPlan {
  Plan fwd;                   // the forward plan whose chunked state pass supplies the carries
  bool ti = false;            // fixed coefficients (bwd_ti_kernels.hip)
  int64_t groups = 0, ntiles = 0, chunk_len = 0;
  int32_t n_chunks = 1;
  size_t off_pB = 0, off_pC = 0, off_pA = 0, off_pD = 0, off_pbias = 0;
  size_t off_state = 0, off_dsum = 0, off_adjG = 0, off_adjS = 0, off_adjin = 0, off_ckdsum = 0, bytes = 0;
};

// Main-pass workgroups resident on MI355X at once: 256 compute units x 2 (the selective
// main-pass instantiations take 214-256 VGPRs per lane and at most 80.9 KB of LDS; those of
// fixed coefficients 173-203 up to 32 states), or x 3 for fixed coefficients with 16 lanes
// per channel (33..64 states: 153-154 VGPRs, three wavefronts per SIMD).
constexpr int64_t kBwdSlots = 512;
constexpr int64_t kBwdSlotsTi16 = 768;

// Validate dims for the backward pass and lay out its workspace (groups: channel groups of
// one workgroup, 64, 32 or 16 channels):
//   ckpt [batch][ntiles][D][N], pB and pC [groups][batch][L][N], pA [batch][D][N],
//   pD and pbias [batch][D]  (fp32, each 256-byte aligned).
int make_bwd_plan(const selscan_dims* dims, BwdPlan* out) {
  Plan plan;
  int st = make_plan(dims, &plan);
  if (st != SELSCAN_OK) return st;
  const selscan_dims& d = *dims;
  BwdPlan b;
  b.ti = plan.ti;
  const int64_t cwg = 4 * 64 / selscan::bwd_lanes_per_channel(d.dstate);   // channels per workgroup
  b.groups = (d.dim + cwg - 1) / cwg;
  b.ntiles = (d.seqlen + 15) / 16;
  // Chunks of the sequence: each workgroup's tokens are a serial chain, so the time is about
  // (rounds of resident workgroups) x (tokens per workgroup).  The smallest such cost wins;
  // fewer chunks win unless more are at least 3 % cheaper (each chunk adds a carry and an
  // adjoint pass over its tokens).
  int64_t nc = 1;
  const int64_t items = d.batch * b.groups;
  if (items > 0 && d.seqlen >= 128) {
    int64_t max_nc = d.seqlen / 64;                              // chunks of at least 64 tokens
    if (max_nc > kMaxChunks) max_nc = kMaxChunks;
    const int64_t slots = (plan.ti && selscan::bwd_lanes_per_channel(d.dstate) == 16) ? kBwdSlotsTi16 : kBwdSlots;
    auto cost = [&](int64_t n) {
      const int64_t rounds = (items * n + slots - 1) / slots;
      return rounds * round_up((d.seqlen + n - 1) / n, 16);
    };
    int64_t best = cost(1);
    for (int64_t n = 2; n <= max_nc; ++n) {
      const int64_t c = cost(n);
      if (c * 100 < best * 97) {
        best = c;
        nc = n;
      }
    }
  }
  b.chunk_len = nc > 1 ? round_up((d.seqlen + nc - 1) / nc, 16) : round_up(d.seqlen > 0 ? d.seqlen : 1, 16);
  // a forward plan chunked for its 32-bit tile addressing bounds the chunk length (the
  // selective backward takes its carries from that plan's state pass)
  if (!plan.ti && plan.chunked && plan.chunk_len < b.chunk_len) b.chunk_len = plan.chunk_len;
  b.n_chunks = d.seqlen > 0 ? int32_t((d.seqlen + b.chunk_len - 1) / b.chunk_len) : 1;
  if (d.batch * b.n_chunks * b.groups > (int64_t(1) << 31) - 1) return SELSCAN_ERR_UNSUPPORTED;
  b.fwd = plan;
  if (b.n_chunks > 1) {
    // the forward plan of the carries: its state pass over the same chunks
    b.fwd.chunked = true;
    b.fwd.chunk_len = b.chunk_len;
    b.fwd.n_chunks = b.n_chunks;
  }
  auto al = [](int64_t x) { return size_t(round_up(x, 256)); };
  const int64_t f = int64_t(sizeof(float));
  const int64_t bdn = d.batch * d.dim * d.dstate, ncq = b.n_chunks;
  size_t off = al(f * d.batch * b.ntiles * d.dim * d.dstate);
  // dB, dC partials: per channel group and token (selective), per batch row and chunk (fixed)
  const int64_t pbc = b.ti ? ncq * bdn : b.groups * d.batch * d.seqlen * d.dstate;
  b.off_pB = off;
  off += al(f * pbc);
  b.off_pC = off;
  off += al(f * pbc);
  b.off_pA = off;
  off += al(f * ncq * bdn);
  b.off_pD = off;
  off += al(f * ncq * d.batch * d.dim);
  b.off_pbias = off;
  off += al(f * ncq * d.batch * d.dim);
  if (b.n_chunks > 1) {
    b.off_state = off;
    off += al(f * ncq * bdn);
    b.off_dsum = off;
    off += al(f * ncq * d.batch * d.dim);
    b.off_adjG = off;
    off += al(f * ncq * bdn);
    b.off_adjS = off;
    off += al(f * ncq * d.batch * d.dim);
    b.off_adjin = off;
    off += al(f * ncq * bdn);
    if (!b.ti) {
      b.off_ckdsum = off;                                 // running sum of delta at every tile start
      off += al(f * d.batch * b.ntiles * d.dim);
    }
  }
  b.bytes = (d.batch * d.seqlen > 0) ? off : 0;
  *out = b;
  return SELSCAN_OK;
}

// Fixed coefficients: chunk end states and prefix, chunk adjoints and combine (a split
// sequence), the main pass, then the sums of the per-(batch row, chunk) partials: dB, dC and
// ddelta in the I/O type ([D][N], [D][N], [D]), dA, dDskip and ddelta_bias in fp32.
int bwd_run_ti(selscan::BwdParams& p, const float* A, const float* h0, void* ddelta, float* ddelta_bias, float* dA,
               void* dB, void* dC, float* dDskip, const selscan_dims& d, const BwdPlan& plan, char* ws,
               hipStream_t stream) {
  const bool bf16 = d.io_dtype == SELSCAN_BF16;
  p.B_sd = d.B_sd;
  p.C_sd = d.C_sd;
  hipError_t e = hipSuccess;
  if (plan.n_chunks > 1) {
    p.carry = reinterpret_cast<float*>(ws + plan.off_state);
    p.sdsum = reinterpret_cast<float*>(ws + plan.off_dsum);
    p.adjG = reinterpret_cast<float*>(ws + plan.off_adjG);
    p.adjS = reinterpret_cast<float*>(ws + plan.off_adjS);
    p.adj_in = reinterpret_cast<float*>(ws + plan.off_adjin);
    e = selscan::launch_bwd_ti(bf16, selscan::kTiPassState, p, stream);
    selscan::PrefixParams q{};
    q.A = A; q.dsum = p.sdsum; q.state = p.carry; q.h0 = h0;
    q.batch = d.batch; q.D = d.dim; q.N = d.dstate; q.n_chunks = plan.n_chunks;
    int sw = 1;
    while (sw < plan.n_chunks) sw <<= 1;
    q.seg_width = sw;
    if (e == hipSuccess) e = selscan::launch_chunk_prefix(q, stream);
    if (e == hipSuccess) e = selscan::launch_bwd_ti(bf16, selscan::kTiPassAdjoint, p, stream);
    if (e == hipSuccess) e = selscan::launch_bwd_adjoint_combine(p, stream);
  }
  if (e == hipSuccess) e = selscan::launch_bwd_ti(bf16, selscan::kTiPassMain, p, stream);
  const int64_t nbc = d.batch * plan.n_chunks, dn = d.dim * d.dstate;
  if (e == hipSuccess) e = selscan::launch_sum_partials(p.pB, nbc, dn, dB, dn, bf16, stream);
  if (e == hipSuccess) e = selscan::launch_sum_partials(p.pC, nbc, dn, dC, dn, bf16, stream);
  if (e == hipSuccess) e = selscan::launch_sum_partials(p.pA, nbc, dn, dA, dn, false, stream);
  if (e == hipSuccess && dDskip) e = selscan::launch_sum_partials(p.pD, nbc, d.dim, dDskip, d.dim, false, stream);
  if (e == hipSuccess) e = selscan::launch_sum_partials(p.pbias, nbc, d.dim, ddelta, d.dim, bf16, stream);
  if (e == hipSuccess && ddelta_bias)
    e = selscan::launch_sum_partials(p.pbias, nbc, d.dim, ddelta_bias, d.dim, false, stream);
  return e == hipSuccess ? SELSCAN_OK : hip_fail(e);
}

int bwd_run(const void* u, const void* delta, const float* delta_bias, const float* A, const void* B, const void* C,
            const float* Dskip, const void* z, const float* h0, const void* dy, const float* dlast, void* du,
            void* ddelta, float* ddelta_bias, float* dA, void* dB, void* dC, float* dDskip, void* dz, float* dh0,
            const selscan_dims& d, const BwdPlan& plan, char* ws, hipStream_t stream) {
  const bool bf16 = d.io_dtype == SELSCAN_BF16;
  hipError_t e;
  if (d.batch * d.seqlen == 0) {
    // no tokens: every sum is empty; the initial state's gradient is dlast itself
    e = selscan::launch_fill_zero(dA, d.dim * d.dstate, stream);
    if (e == hipSuccess && dDskip) e = selscan::launch_fill_zero(dDskip, d.dim, stream);
    if (e == hipSuccess && ddelta_bias) e = selscan::launch_fill_zero(ddelta_bias, d.dim, stream);
    if (e == hipSuccess && dh0 && d.batch > 0)
      e = dlast ? selscan::launch_copy(dh0, dlast, d.batch * d.dim * d.dstate, stream)
                : selscan::launch_fill_zero(dh0, d.batch * d.dim * d.dstate, stream);
    if (plan.ti) {          // the shared coefficients' gradients are empty sums too (zero parts)
      const int64_t dn = d.dim * d.dstate;
      if (e == hipSuccess && dB) e = selscan::launch_sum_partials(nullptr, 0, 0, dB, dn, bf16, stream);
      if (e == hipSuccess && dC) e = selscan::launch_sum_partials(nullptr, 0, 0, dC, dn, bf16, stream);
      if (e == hipSuccess && ddelta) e = selscan::launch_sum_partials(nullptr, 0, 0, ddelta, d.dim, bf16, stream);
    }
    return e == hipSuccess ? SELSCAN_OK : hip_fail(e);
  }
  selscan::BwdParams p{};
  p.u = u; p.delta = delta; p.delta_bias = delta_bias; p.A = A; p.B = B; p.C = C; p.Dskip = Dskip; p.z = z;
  p.h0 = h0; p.dy = dy; p.dlast = dlast; p.du = du; p.ddelta = ddelta; p.dz = z ? dz : nullptr; p.dh0 = dh0;
  p.ckpt = reinterpret_cast<float*>(ws);
  p.pB = reinterpret_cast<float*>(ws + plan.off_pB);
  p.pC = reinterpret_cast<float*>(ws + plan.off_pC);
  p.pA = reinterpret_cast<float*>(ws + plan.off_pA);
  p.pD = reinterpret_cast<float*>(ws + plan.off_pD);
  p.pbias = reinterpret_cast<float*>(ws + plan.off_pbias);
  p.batch = d.batch; p.L = d.seqlen; p.D = d.dim; p.N = d.dstate;
  p.u_sb = d.u_sb; p.u_sl = d.u_sl; p.delta_sb = d.delta_sb; p.delta_sl = d.delta_sl;
  p.z_sb = d.z_sb; p.z_sl = d.z_sl; p.dy_sb = d.y_sb; p.dy_sl = d.y_sl;
  p.B_sb = d.B_sb; p.B_sl = d.B_sl; p.C_sb = d.C_sb; p.C_sl = d.C_sl;
  p.ntiles = plan.ntiles;
  p.chunk_len = plan.chunk_len;
  p.n_chunks = plan.n_chunks;
  p.groups = int32_t(plan.groups);
  p.euler = d.discretization == SELSCAN_DISC_EULER ? 1 : 0;
  p.softplus = d.delta_softplus != 0 ? 1 : 0;
  p.dxf = (p.softplus || delta_bias != nullptr) ? 1 : 0;
  {
    const int64_t es = bf16 ? 2 : 4, span_max = (int64_t(1) << 31) / es - d.dim;
    auto vec_ok = [&](const void* q, int64_t sb, int64_t sl) {
      return q == nullptr || (aligned(q, size_t(4 * es)) && sb % 4 == 0 && sl % 4 == 0 && sl >= d.dim &&
                              plan.chunk_len * sl < span_max);
    };
    p.vec = (d.dim % 4 == 0 && vec_ok(u, d.u_sb, d.u_sl) && vec_ok(delta, d.delta_sb, d.delta_sl) &&
             vec_ok(dy, d.y_sb, d.y_sl) && vec_ok(z, d.z_sb, d.z_sl) && vec_ok(du, d.seqlen * d.dim, d.dim) &&
             vec_ok(ddelta, d.seqlen * d.dim, d.dim) && vec_ok(z ? dz : nullptr, d.seqlen * d.dim, d.dim))
                ? 1 : 0;
  }
  if (plan.ti) return bwd_run_ti(p, A, h0, ddelta, ddelta_bias, dA, dB, dC, dDskip, d, plan, ws, stream);
  if (plan.n_chunks > 1) {
    // the state entering every chunk: the forward's chunked state pass and prefix
    selscan::ScanParams f = scan_params(u, delta, delta_bias, A, B, C, Dskip, z, nullptr, h0, nullptr, d, plan.fwd);
    f.sched_round = compute_units(stream);
    f.ws_state = reinterpret_cast<float*>(ws + plan.off_state);
    f.ws_dsum = reinterpret_cast<float*>(ws + plan.off_dsum);
    if (f.pipelined) {                                    // the state pass also checkpoints its tiles
      f.ckpt = p.ckpt;
      f.ck_dsum = reinterpret_cast<float*>(ws + plan.off_ckdsum);
      f.ck_ntiles = plan.ntiles;
      f.state_all = 1;                                    // the last chunk's tiles too
      p.ck_fwd = 1;
      p.ck_dsum = f.ck_dsum;
    }
    e = selscan::launch_scan_pass(selscan::kPassState, bf16, false, plan.fwd.S, plan.fwd.K, f, stream);
    if (e != hipSuccess) return hip_fail(e);
    selscan::PrefixParams q{};
    q.A = A; q.dsum = f.ws_dsum; q.state = f.ws_state; q.h0 = h0;
    q.batch = d.batch; q.D = d.dim; q.N = d.dstate; q.n_chunks = plan.n_chunks;
    int sw = 1;
    while (sw < plan.n_chunks) sw <<= 1;
    q.seg_width = sw;
    e = selscan::launch_chunk_prefix(q, stream);
    if (e != hipSuccess) return hip_fail(e);
    p.carry = f.ws_state;
    p.adjG = reinterpret_cast<float*>(ws + plan.off_adjG);
    p.adjS = reinterpret_cast<float*>(ws + plan.off_adjS);
    p.adj_in = reinterpret_cast<float*>(ws + plan.off_adjin);
  }
  e = selscan::launch_bwd(bf16, p, stream);
  const int64_t m_bc = d.batch * d.seqlen * d.dstate;
  if (e == hipSuccess) e = selscan::launch_sum_partials(p.pB, plan.groups, m_bc, dB, m_bc, bf16, stream);
  if (e == hipSuccess) e = selscan::launch_sum_partials(p.pC, plan.groups, m_bc, dC, m_bc, bf16, stream);
  const int64_t nbc = d.batch * plan.n_chunks;              // partials: one per (batch row, chunk)
  if (e == hipSuccess)
    e = selscan::launch_sum_partials(p.pA, nbc, d.dim * d.dstate, dA, d.dim * d.dstate, false, stream);
  if (e == hipSuccess && dDskip) e = selscan::launch_sum_partials(p.pD, nbc, d.dim, dDskip, d.dim, false, stream);
  if (e == hipSuccess && ddelta_bias)
    e = selscan::launch_sum_partials(p.pbias, nbc, d.dim, ddelta_bias, d.dim, false, stream);
  return e == hipSuccess ? SELSCAN_OK : hip_fail(e);
}

}  // namespace

extern "C" {

void selscan_dims_init(selscan_dims* dims, int io_dtype, int64_t batch, int64_t seqlen, int64_t dim,
                       int64_t dstate, int time_invariant) {
  if (!dims) return;
  selscan_dims d{};
  d.abi_version = SELSCAN_ABI_VERSION;
  d.io_dtype = io_dtype;
  d.batch = batch; d.seqlen = seqlen; d.dim = dim; d.dstate = dstate;
  d.u_sb = d.z_sb = d.y_sb = seqlen * dim;
  d.u_sl = d.z_sl = d.y_sl = dim;
  if (time_invariant) {
    d.delta_sb = d.delta_sl = 0;
    d.B_sb = d.B_sl = d.C_sb = d.C_sl = 0;
    d.B_sd = d.C_sd = dstate;
  } else {
    d.delta_sb = seqlen * dim;
    d.delta_sl = dim;
    d.B_sb = d.C_sb = seqlen * dstate;
    d.B_sl = d.C_sl = dstate;
    d.B_sd = d.C_sd = 0;
  }
  d.path = SELSCAN_PATH_AUTO;
  d.chunk_len = 0;
  d.discretization = SELSCAN_DISC_ZOH;
  d.delta_softplus = 0;
  *dims = d;
}

int selective_scan_plan_path(const selscan_dims* dims) {
  Plan plan;
  const int st = make_plan(dims, &plan);
  if (st != SELSCAN_OK) return st;
  return plan.conv ? SELSCAN_PATH_CONV : plan.chunked ? SELSCAN_PATH_CHUNKED : SELSCAN_PATH_SINGLE;
}

size_t selective_scan_workspace_size(const selscan_dims* dims) {
  Plan plan;
  if (make_plan(dims, &plan) != SELSCAN_OK) return 0;
  return plan.ws_bytes;
}

int selective_scan_fwd_ws(const void* u, const void* delta, const float* A, const void* B, const void* C,
                          const float* Dskip, const void* z, void* y, float* last_state, const selscan_dims* dims,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(u, delta, nullptr, A, B, C, Dskip, z, y, nullptr, last_state, dims, workspace, workspace_bytes,
                  false, static_cast<hipStream_t>(stream));
}

int selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, void* y, float* last_state, const selscan_dims* dims,
                       void* stream) {
  return fwd_impl(u, delta, nullptr, A, B, C, Dskip, z, y, nullptr, last_state, dims, nullptr, 0, true,
                  static_cast<hipStream_t>(stream));
}

int selective_scan_fwd_ex(const void* u, const void* delta, const float* delta_bias, const float* A, const void* B,
                          const void* C, const float* Dskip, const void* z, void* y, const float* initial_state,
                          float* last_state, const selscan_dims* dims, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return fwd_impl(u, delta, delta_bias, A, B, C, Dskip, z, y, initial_state, last_state, dims, workspace,
                  workspace_bytes, workspace == nullptr, static_cast<hipStream_t>(stream));
}

int selective_scan_fwd_noalloc(const void* u, const void* delta, const float* delta_bias, const float* A,
                               const void* B, const void* C, const float* Dskip, const void* z, void* y,
                               const float* initial_state, float* last_state, const selscan_dims* dims,
                               void* stream) {
  return fwd_noalloc(u, delta, delta_bias, A, B, C, Dskip, z, y, initial_state, last_state, dims,
                     static_cast<hipStream_t>(stream));
}

int selective_scan_step(const void* u, const void* delta, const float* delta_bias, const float* A, const void* B,
                        const void* C, const float* Dskip, const void* z, void* y, float* state,
                        const selscan_dims* dims, void* stream) {
  Plan plan;
  int st = make_plan(dims, &plan);
  if (st != SELSCAN_OK) return st;
  if (dims->seqlen != 1) return SELSCAN_ERR_DIMS;
  if (!state) return SELSCAN_ERR_NULL;
  st = check_pointers(u, delta, A, B, C, Dskip, z, y, state, dims->io_dtype, dims->batch == 0);
  if (st != SELSCAN_OK) return st;
  if (delta_bias != nullptr && !aligned(delta_bias, 4)) return SELSCAN_ERR_ALIGN;
  if (dims->batch * dims->dim > (int64_t(1) << 36)) return SELSCAN_ERR_UNSUPPORTED;   // grid size
  if (dims->batch == 0) return SELSCAN_OK;
  selscan::StepParams q{};
  q.u = u; q.delta = delta; q.A = A; q.B = B; q.C = C; q.Dskip = Dskip; q.z = z; q.y = y; q.state = state;
  q.delta_bias = delta_bias;
  q.euler = dims->discretization == SELSCAN_DISC_EULER ? 1 : 0;
  q.softplus = dims->delta_softplus != 0 ? 1 : 0;
  q.dxf = (q.softplus || delta_bias != nullptr) ? 1 : 0;
  q.batch = dims->batch; q.D = dims->dim; q.N = dims->dstate;
  q.u_sb = dims->u_sb; q.delta_sb = dims->delta_sb; q.z_sb = dims->z_sb; q.y_sb = dims->y_sb;
  q.B_sb = dims->B_sb; q.B_sd = dims->B_sd; q.C_sb = dims->C_sb; q.C_sd = dims->C_sd;
  {
    const uintptr_t qb = uintptr_t(4) * (plan.bf16 ? 2 : 4);
    const bool bc_vec = plan.ti || (aligned(B, qb) && aligned(C, qb) && dims->B_sb % 4 == 0 && dims->C_sb % 4 == 0);
    q.vec = (dims->dstate % 4 == 0 && aligned(state, 16) && bc_vec) ? 1 : 0;
  }
  const hipError_t e = selscan::launch_step(plan.bf16, plan.ti, q, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SELSCAN_OK : hip_fail(e);
}

size_t selective_scan_bwd_workspace_size(const selscan_dims* dims) {
  BwdPlan plan;
  if (make_bwd_plan(dims, &plan) != SELSCAN_OK) return 0;
  return plan.bytes;
}

int selective_scan_bwd(const void* u, const void* delta, const float* delta_bias, const float* A, const void* B,
                       const void* C, const float* Dskip, const void* z, const float* initial_state, const void* dy,
                       const float* dlast_state, void* du, void* ddelta, float* ddelta_bias, float* dA, void* dB,
                       void* dC, float* dDskip, void* dz, float* dinitial_state, const selscan_dims* dims,
                       void* workspace, size_t workspace_bytes, void* stream) {
  BwdPlan plan;
  int st = make_bwd_plan(dims, &plan);
  if (st != SELSCAN_OK) return st;
  const selscan_dims& d = *dims;
  const bool no_tokens = d.batch * d.seqlen == 0;
  st = check_pointers(u, delta, A, B, C, Dskip, z, dy, nullptr, d.io_dtype, no_tokens);
  if (st != SELSCAN_OK) return st;
  if (!dA || (!no_tokens && (!du || !ddelta || !dB || !dC))) return SELSCAN_ERR_NULL;
  const size_t es = d.io_dtype == SELSCAN_BF16 ? 2 : 4;
  if (!aligned(du, es) || !aligned(ddelta, es) || !aligned(dB, es) || !aligned(dC, es) || (dz && !aligned(dz, es)))
    return SELSCAN_ERR_ALIGN;
  for (const float* f : {delta_bias, initial_state, dlast_state, static_cast<const float*>(ddelta_bias),
                         static_cast<const float*>(dA), static_cast<const float*>(dDskip),
                         static_cast<const float*>(dinitial_state)})
    if (f && !aligned(f, 4)) return SELSCAN_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.bytes == 0 || workspace != nullptr) {
    if (plan.bytes > 0 && (workspace_bytes < plan.bytes || !aligned(workspace, 256))) return SELSCAN_ERR_WORKSPACE;
    return bwd_run(u, delta, delta_bias, A, B, C, Dskip, z, initial_state, dy, dlast_state, du, ddelta, ddelta_bias,
                   dA, dB, dC, dDskip, dz, dinitial_state, d, plan, static_cast<char*>(workspace), s);
  }
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, plan.bytes, s);
  if (e != hipSuccess) return hip_fail(e);
  st = bwd_run(u, delta, delta_bias, A, B, C, Dskip, z, initial_state, dy, dlast_state, du, ddelta, ddelta_bias, dA,
               dB, dC, dDskip, dz, dinitial_state, d, plan, static_cast<char*>(ws), s);
  e = hipFreeAsync(ws, s);
  if (st == SELSCAN_OK && e != hipSuccess) return hip_fail(e);
  return st;
}

// Automatic path: chunk-parallel up to this many (batch, head, 64-token chunk) units (short,
// narrow calls, where launches dominate), else on chip over the modelled best segment count
// (measured crossover on MI355X).
constexpr int64_t kSsdChunkParallelMaxUnits = 512;

struct SsdPlan {
  int64_t n_chunks = 0;
  bool fused = false;
  int64_t n_seg = 1, seg_chunks = 0;
  size_t ws_bytes = 0;
  size_t seg_state_bytes = 0;                 // offset of the segment decays in the workspace
};

// Segments of n_chunks chunks for a requested count: equal runs of ceil(n_chunks / count)
// chunks, none empty.
static void ssd_set_segments(SsdPlan& pl, int64_t count) {
  const int64_t nc = pl.n_chunks > 0 ? pl.n_chunks : 1;
  const int64_t want = count < 1 ? 1 : count > nc ? nc : count;
  pl.seg_chunks = (nc + want - 1) / want;
  pl.n_seg = (nc + pl.seg_chunks - 1) / pl.seg_chunks;
}

// Modelled time (us, N = 128) of the on-chip path over `count` segments, from times measured
// on MI355X (256 CUs): the output walk costs t_pair per 64-token chunk for each of two
// workgroups sharing a CU (four wavefronts each), t_alone for a workgroup alone on its CU,
// t_alone8 when every workgroup has a CU of its own and so runs eight wavefronts (measured on
// the whole-sequence walk at 130M widths: 0.142 ms for 32 chunks), and its workgroups are
// dealt out in rounds of two per CU; the segment state pass costs
// t_state1 per chunk alone on a CU plus t_state_more per further workgroup sharing it (up to
// four at once); the segment carries move every segment state twice at about 5 TB/s; and
// splitting at all costs two more launches and the carried-in states' loads (t_split).
static double ssd_onchip_cost(int64_t items, int64_t nc, int64_t dstate, int64_t count) {
  constexpr double t_pair = 6.25, t_alone = 4.1, t_alone8 = 4.45, t_state1 = 1.6, t_state_more = 0.6, t_split = 12.0;
  constexpr int64_t kCUs = 256;
  SsdPlan pl;
  pl.n_chunks = nc;
  ssd_set_segments(pl, count);
  const double len = double(pl.seg_chunks);
  const int64_t w = items * pl.n_seg;
  double t;
  if (w <= kCUs) {
    t = len * t_alone8;                                  // one eight-wavefront workgroup per CU
  } else {
    const int64_t full = w / (2 * kCUs), rem = w % (2 * kCUs);
    t = double(full) * len * t_pair + (rem == 0 ? 0.0 : rem <= kCUs ? len * t_alone : len * t_pair);
  }
  if (pl.n_seg > 1) {
    const int64_t per_cu = (items * (pl.n_seg - 1) + kCUs - 1) / kCUs;
    const int64_t rounds = (per_cu + 3) / 4, conc = per_cu < 4 ? per_cu : 4;
    t += double(rounds) * len * (t_state1 + double(conc - 1) * t_state_more);
    t += double(w) * double(dstate) * 64.0 * 8.0 / 5.0e6 + t_split;
  }
  return t;
}

// Segment count of the automatic on-chip path: the modelled fastest split, fewer segments on
// a near tie; no split unless it saves at least 8 % (a split re-reads x for the segment state
// pass and moves the segment states, about 1.4x the layer's bytes at 2.7B widths).
static int64_t ssd_auto_segments(int64_t items, int64_t nc, int64_t dstate) {
  static const int64_t kCounts[] = {2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32, 48, 64, 96, 128};
  int64_t best = 0;
  double best_t = 0.0;
  for (int64_t c : kCounts) {
    if (c > nc) break;
    const double t = ssd_onchip_cost(items, nc, dstate, c);
    if (best == 0 || t < best_t * 0.98) {
      best = c;
      best_t = t;
    }
  }
  return best != 0 && best_t < 0.92 * ssd_onchip_cost(items, nc, dstate, 1) ? best : 1;
}

static int ssd_check(const selscan_ssd_dims* d, SsdPlan* pl) {
  if (!d) return SELSCAN_ERR_NULL;
  if (d->abi_version != SELSCAN_ABI_VERSION) return SELSCAN_ERR_ABI;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1) return SELSCAN_ERR_DIMS;
  if (d->headdim != 64 || (d->dstate != 64 && d->dstate != 128)) return SELSCAN_ERR_UNSUPPORTED;
  if (d->discretization != SELSCAN_DISC_ZOH && d->discretization != SELSCAN_DISC_EULER) return SELSCAN_ERR_UNSUPPORTED;
  const int64_t nc = (d->seqlen + 63) / 64;
  // (the on-chip kernels address a chunk of one head's x, z and y with 32-bit offsets)
  if (d->batch * d->nheads * nc > (int64_t(1) << 31) - 1 || d->batch * d->nheads * d->dstate * 64 > (int64_t(1) << 36) ||
      d->nheads * 64 * 64 * 2 >= (int64_t(1) << 31))
    return SELSCAN_ERR_UNSUPPORTED;
  if (d->path < 0 || d->path > 3 || d->segments < 0 || (d->segments != 0 && d->path != 3)) return SELSCAN_ERR_UNSUPPORTED;
  const int64_t items = d->batch * d->nheads, bhc = items * nc;
  SsdPlan p;
  p.n_chunks = nc;
  p.fused = d->path == 1 || d->path == 3 || (d->path == 0 && items * nc > kSsdChunkParallelMaxUnits);
  // the segment state pass addresses one batch row of x through a buffer resource (32-bit offsets)
  const bool seg_ok = (d->seqlen + 64) * d->nheads * 64 * 2 < (int64_t(1) << 31);
  if (d->path == 3 && !seg_ok) return SELSCAN_ERR_UNSUPPORTED;
  if (d->path == 3) ssd_set_segments(p, d->segments > 0 ? d->segments : ssd_auto_segments(items, nc, d->dstate));
  else if (d->path == 0 && p.fused && seg_ok) ssd_set_segments(p, ssd_auto_segments(items, nc, d->dstate));
  else ssd_set_segments(p, 1);
  if (d->batch * d->seqlen == 0) {
    p.ws_bytes = 0;
  } else if (!p.fused) {
    p.ws_bytes = size_t(round_up(bhc * d->dstate * 64 * int64_t(sizeof(float)), 256) +
                        round_up(bhc * int64_t(sizeof(float)), 256) + round_up(bhc * d->dstate * 64 * 2, 256));
  } else if (p.n_seg > 1) {
    p.seg_state_bytes = size_t(round_up(items * p.n_seg * d->dstate * 64 * int64_t(sizeof(float)), 256));
    p.ws_bytes = p.seg_state_bytes + size_t(round_up(items * p.n_seg * int64_t(sizeof(float)), 256));
  }
  *pl = p;
  return SELSCAN_OK;
}

size_t selective_scan_ssd_workspace_size(const selscan_ssd_dims* dims) {
  SsdPlan pl;
  return ssd_check(dims, &pl) == SELSCAN_OK ? pl.ws_bytes : 0;
}

int selective_scan_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, void* y, const float* initial_state, float* last_state,
                           const selscan_ssd_dims* dims, void* workspace, size_t workspace_bytes, void* stream) {
  SsdPlan pl;
  int st = ssd_check(dims, &pl);
  if (st != SELSCAN_OK) return st;
  const size_t need = pl.ws_bytes;
  const int64_t nc = pl.n_chunks;
  const bool fused = pl.fused;
  const selscan_ssd_dims& d = *dims;
  const bool no_tokens = d.batch * d.seqlen == 0;
  if (!A || (!no_tokens && (!x || !delta || !B || !C || !y))) return SELSCAN_ERR_NULL;
  if (delta && !aligned(delta, 2)) return SELSCAN_ERR_ALIGN;
  for (const void* q : {x, B, C, z, static_cast<const void*>(y)})     // moved 16 bytes at a time
    if (q && !aligned(q, 16)) return SELSCAN_ERR_ALIGN;
  for (const float* f : {A, Dskip, initial_state, static_cast<const float*>(last_state)})
    if (f && !aligned(f, 4)) return SELSCAN_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (d.batch == 0) return SELSCAN_OK;
  if (d.seqlen == 0) {                         // no tokens: the initial state is handed back
    if (last_state && last_state != initial_state) {
      const int64_t n = d.batch * d.nheads * 64 * d.dstate;
      e = initial_state ? selscan::launch_copy(last_state, initial_state, n, s) : selscan::launch_fill_zero(last_state, n, s);
    }
    return e == hipSuccess ? SELSCAN_OK : hip_fail(e);
  }
  void* ws = workspace;
  if (need > 0 && ws != nullptr) {
    if (workspace_bytes < need || !aligned(ws, 256)) return SELSCAN_ERR_WORKSPACE;
  } else if (need > 0) {
    e = hipMallocAsync(&ws, need, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  selscan::SsdParams p{};
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = Dskip; p.z = z; p.y = y;
  p.h0 = initial_state; p.last_state = last_state;
  p.batch = d.batch; p.L = d.seqlen; p.H = d.nheads; p.N = d.dstate; p.n_chunks = nc;
  p.euler = d.discretization == SELSCAN_DISC_EULER ? 1 : 0;
  p.fused = fused ? 1 : 0;
  p.n_seg = pl.n_seg;
  p.seg_chunks = pl.seg_chunks;
  if (fused && pl.n_seg > 1) {
    p.seg_state = static_cast<float*>(ws);
    p.seg_decay = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.seg_state_bytes);
  }
  if (!fused) {
    p.state = static_cast<float*>(ws);
    const int64_t bhc = d.batch * d.nheads * nc;
    char* const wsc = static_cast<char*>(ws);
    p.decay = reinterpret_cast<float*>(wsc + round_up(bhc * d.dstate * 64 * int64_t(sizeof(float)), 256));
    p.carry = reinterpret_cast<uint16_t*>(wsc + round_up(bhc * d.dstate * 64 * int64_t(sizeof(float)), 256) +
                                          round_up(bhc * int64_t(sizeof(float)), 256));
  }
  e = selscan::launch_ssd(p, s);
  st = e == hipSuccess ? SELSCAN_OK : hip_fail(e);
  if (workspace == nullptr && need > 0) {
    const hipError_t f = hipFreeAsync(ws, s);
    if (st == SELSCAN_OK && f != hipSuccess) st = hip_fail(f);
  }
  return st;
}

const char* selective_scan_strerror(int status) {
  switch (status) {
    case SELSCAN_OK: return "success";
    case SELSCAN_ERR_NULL: return "a required pointer is NULL";
    case SELSCAN_ERR_DIMS: return "a size or stride is out of range";
    case SELSCAN_ERR_UNSUPPORTED: return "unsupported dtype, state count, path, discretization or stride pattern";
    case SELSCAN_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case SELSCAN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case SELSCAN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SELSCAN_ERR_ABI: return "selscan_dims.abi_version does not match the library";
    case SELSCAN_ERR_SCRATCH_LIMIT:
      return "the chunked path needs more scratch than the no-allocation entry point holds "
             "(SELSCAN_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int selective_scan_last_hip_error(void) { return g_last_hip_error; }

int selective_scan_abi_version(void) { return SELSCAN_ABI_VERSION; }

}  // extern "C"
