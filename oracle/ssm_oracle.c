/*
 * ssm_oracle.c -- plain, slow, double-precision CPU oracle for the S6 selective-scan
 * forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header, table or
 * helper with the GPU library: it is a second, independent statement of the method.
 *
 * What it computes, with the passage each step follows:
 *
 *   - Zero-order-hold discretisation of a diagonal continuous-time system, one scalar
 *     per (position, channel, state):
 *        Abar = exp(delta * a)                     ("state-space models", aarnphm.xyz,
 *                                                   section "From continuous time to
 *                                                   tokens", ZOH equation; Algenta
 *                                                   "Sequence and state-space models",
 *                                                   section on state_space_models,
 *                                                   ssm_discretize_zoh)
 *        Bbar = (Abar - 1) / a * b,  and delta * b when a == 0
 *                                                  (Algenta page, ssm_discretize_b and its
 *                                                   a == 0 fallback; the ZOH integral on
 *                                                   the aarnphm page stays finite when A is
 *                                                   singular and its limit is delta * b)
 *     (Abar - 1)/a is evaluated as expm1(delta*a)/a so that the small-|delta*a| regime
 *     keeps full double precision.
 *   - Optional first-order input coefficient ("Euler"): Abar = exp(delta * a) as above but
 *     Bbar = delta * b for every state (Algenta page, mamba_selective_scan_step and the
 *     worked example after it: h_1 = delta * b * x = 1.0 at a = -1, delta = 0.5, b = 2,
 *     x = 1; TorchLean "Selective Mamba", step: the input term is delta[d] * B[n] * u[d];
 *     chipfoundry glossary, Lab 2: B_bar = delta * B).
 *   - Optional step-size transform: delta_eff = delta + delta_bias[d], then, when asked,
 *     softplus(delta_eff) = log(1 + exp(delta_eff))  (TorchLean "Selective Mamba", step:
 *     the time step is softplus of the projection plus dtBias, one bias per channel;
 *     Algenta page, mamba_delta_softplus), evaluated in the overflow-free form
 *     log1p(exp(-|x|)) + max(x, 0)  (chipfoundry glossary, Lab 2, softplus).
 *   - Selectivity: delta, B and C are given per token (B, C shared by every channel of
 *     a token); A is fixed and diagonal per (channel, state)  ("state-space models",
 *     section "Mamba"; TorchLean "Selective Mamba", Parameters: bProj/cProj describe one
 *     B and one C vector per token shared by the expanded channels).
 *   - Recurrence h_t = Abar_t * h_{t-1} + Bbar_t * u_t from h_{-1} = 0, and readout of the
 *     UPDATED state y_t = C_t . h_t   (aarnphm page, ZOH equation block and section "One
 *     recurrence, one convolution" for the zero initial state; Algenta page,
 *     ssm_recurrence_step / ssm_output_step; TorchLean "Selective Mamba", step: the
 *     readout contracts the new hidden state).
 *   - Direct feed-through y += D * u before gating, then the gate y *= z * sigmoid(z)
 *     (chipfoundry glossary "State-Space Models & Long-Context Sequence Architectures
 *     (Mamba)", section "Mathematical Formulation", continuous system with D; TorchLean
 *     "Selective Mamba", step: adds dSkip * u, then gates by SiLU of the z projection).
 *   - The final hidden state after the last token, one N-vector per channel
 *     (TorchLean "Selective Mamba", State.hidden and runArray: the state a following
 *     chunk continues from).
 *   - An optional initial state h_{-1} (default zero): a call continues from the state a
 *     previous call ended in, so running two chunks one after the other equals running
 *     their concatenation, and a call with no tokens hands its initial state back unchanged
 *     (TorchLean "Selective Mamba", step / runArray with an explicit state; the zero state
 *     is zeroState).  A one-token call is the recurrent decode step (aarnphm, "One
 *     recurrence, one convolution": the recurrent form generates one token at a time).
 *
 * Backward pass (ssm_oracle_bwd): the vector-Jacobian product of the same forward, taken
 * by the reverse-time recurrence over the cached state trajectory that the rustytorch commit
 * log describes for its hand-written VJP of the selective scan ("Hand-written VJP of the
 * selective-scan forward": the scan differentiated analytically, backwards in time, over the
 * cached h).  With lambda_t = dL/dh_t (the total derivative through every later token):
 *     lambda_t = dyp_t * C_t + Abar_{t+1} * lambda_{t+1}        (lambda_L-1 picks up dlast)
 * where dyp_t = dy_t * SiLU(z_t) is the derivative at the pre-gate output; every input's
 * gradient is then the chain rule through one step of the forward:
 *     h_t = Abar_t h_{t-1} + c_t B_t u_t,   Abar_t = exp(delta_t a),  c_t = Bbar_t / B_t,
 * with dc/ddelta = Abar_t (ZOH, also at a == 0) or 1 (first order), and dc/da =
 * (delta Abar_t - c_t)/a (ZOH, limit delta^2/2 at a == 0) or 0 (first order).
 *
 * Layouts (row-major, all contiguous):
 *   u, delta, z, y : [batch][L][D]           (time-invariant mode: delta is [D])
 *   B, C           : [batch][L][N]           (time-invariant mode: [D][N])
 *   A              : [D][N]
 *   Dskip          : [D]      (may be NULL: no feed-through)
 *   z              : may be NULL (no gate)
 *   h0             : [batch][D][N]  float, the initial state (may be NULL: zero)
 *   delta_bias     : [D]      (may be NULL: zero)
 *   last_state     : [batch][D][N]  (may be NULL)
 * Inputs are fp32 (bf16 data arrives already widened to fp32, which is exact); every
 * intermediate and every output is double.  The summation over states runs n = 0..N-1
 * in that fixed order.  Threads split the (batch, channel) pairs; each pair is computed
 * by exactly one thread with the same code, so results do not depend on the thread
 * count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const float *u, *delta, *A, *B, *C, *Dskip, *z, *h0, *delta_bias;
  double *y, *last_state;
  int64_t batch, L, D, N;
  int time_invariant;
  int euler;               /* Bbar = delta * b instead of the ZOH coefficient */
  int delta_softplus;      /* delta_eff = softplus(delta + bias) instead of delta + bias */
  int64_t next_pair;       /* work counter, guarded by mu */
  pthread_mutex_t mu;
} oracle_job;

/* ZOH input coefficient (Abar - 1) / a, with the a == 0 limit delta. */
static double zoh_input_coeff(double dt, double a) {
  if (a == 0.0) return dt;
  return expm1(dt * a) / a;
}

/* softplus(x) = log(1 + e^x), written so that e^x never overflows. */
static double softplus(double x) { return log1p(exp(-fabs(x))) + fmax(x, 0.0); }

/* The step size a token uses: the given delta, plus the channel's bias, through softplus
 * when asked. */
static double step_size(const oracle_job* j, double raw, int64_t d) {
  double x = raw;
  if (j->delta_bias) x += (double)j->delta_bias[d];
  return j->delta_softplus ? softplus(x) : x;
}

static void scan_one_channel(oracle_job* j, int64_t b, int64_t d, double* h) {
  const int64_t L = j->L, D = j->D, N = j->N;
  for (int64_t n = 0; n < N; ++n)                                /* h_{-1}: given, else 0 */
    h[n] = j->h0 ? (double)j->h0[(b * D + d) * N + n] : 0.0;
  for (int64_t l = 0; l < L; ++l) {
    const int64_t tok = (b * L + l) * D + d;
    const double uu = (double)j->u[tok];
    const double dt = step_size(j, j->time_invariant ? (double)j->delta[d] : (double)j->delta[tok], d);
    const float* Brow = j->time_invariant ? j->B + d * N : j->B + (b * L + l) * N;
    const float* Crow = j->time_invariant ? j->C + d * N : j->C + (b * L + l) * N;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = (double)j->A[d * N + n];
      const double abar = exp(dt * a);
      const double bbar = (j->euler ? dt : zoh_input_coeff(dt, a)) * (double)Brow[n];
      h[n] = abar * h[n] + bbar * uu;
      acc += (double)Crow[n] * h[n];
    }
    double yv = acc;
    if (j->Dskip) yv += (double)j->Dskip[d] * uu;
    if (j->z) {
      const double zz = (double)j->z[tok];
      yv *= zz / (1.0 + exp(-zz));
    }
    j->y[tok] = yv;
  }
  if (j->last_state)
    for (int64_t n = 0; n < N; ++n) j->last_state[(b * D + d) * N + n] = h[n];
}

static void* worker(void* arg) {
  oracle_job* j = (oracle_job*)arg;
  double* h = (double*)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
  if (!h) return (void*)1;
  const int64_t total = j->batch * j->D;
  for (;;) {
    pthread_mutex_lock(&j->mu);
    const int64_t p = j->next_pair++;
    pthread_mutex_unlock(&j->mu);
    if (p >= total) break;
    scan_one_channel(j, p / j->D, p % j->D, h);
  }
  free(h);
  return NULL;
}

/* Returns 0 on success, -1 on invalid arguments, -2 on allocation/thread failure. */
int ssm_oracle_fwd(const float* u, const float* delta, const float* A, const float* B,
                   const float* C, const float* Dskip, const float* z, const float* h0,
                   const float* delta_bias, double* y, double* last_state, int64_t batch, int64_t L,
                   int64_t D, int64_t N, int time_invariant, int euler, int delta_softplus,
                   int nthreads) {
  if (batch < 0 || L < 0 || D <= 0 || N <= 0) return -1;
  if (batch == 0) return 0;
  if (L > 0 && (!u || !delta || !A || !B || !C || !y)) return -1;
  if (L == 0) {                                 /* no tokens: the state is handed back */
    if (last_state)
      for (int64_t i = 0; i < batch * D * N; ++i) last_state[i] = h0 ? (double)h0[i] : 0.0;
    return 0;
  }
  oracle_job j;
  j.u = u; j.delta = delta; j.A = A; j.B = B; j.C = C; j.Dskip = Dskip; j.z = z; j.h0 = h0;
  j.delta_bias = delta_bias; j.euler = euler; j.delta_softplus = delta_softplus;
  j.y = y; j.last_state = last_state;
  j.batch = batch; j.L = L; j.D = D; j.N = N; j.time_invariant = time_invariant;
  j.next_pair = 0;
  pthread_mutex_init(&j.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0, rc = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, worker, &j) != 0) { rc = -2; break; }
    ++started;
  }
  if (worker(&j) != NULL) rc = -2;
  for (int t = 1; t <= started; ++t) {
    void* r = NULL;
    pthread_join(th[t], &r);
    if (r != NULL) rc = -2;
  }
  pthread_mutex_destroy(&j.mu);
  return rc;
}

/* The two ZOH coefficients for one scalar, exposed so the worked numbers printed for
 * the scalar example (a = -1, delta = 0.5, b = 2) can be checked on their own. */
void ssm_oracle_discretize(double a, double b, double dt, double* abar, double* bbar) {
  *abar = exp(dt * a);
  *bbar = zoh_input_coeff(dt, a) * b;
}

/* The first-order ("Euler") pair for one scalar: the same Abar, Bbar = delta * b. */
void ssm_oracle_discretize_euler(double a, double b, double dt, double* abar, double* bbar) {
  *abar = exp(dt * a);
  *bbar = dt * b;
}

/* softplus of one value, exposed so the printed values can be checked on their own. */
double ssm_oracle_softplus(double x) { return softplus(x); }


/* ------------------------------------------------------------------------------------- */
/* Backward pass.  Gradients (all double, all contiguous):
 *   du, ddelta, dz : [batch][L][D]   (ddelta is the gradient of the GIVEN delta, i.e. of the
 *                                     softplus argument's raw part when delta_softplus)
 *   dB, dC         : [batch][L][N]   (time-invariant mode: [D][N])
 *   dA             : [D][N]
 *   dDskip, ddelta_bias : [D]       (may be NULL)
 *   dh0            : [batch][D][N]   (may be NULL)
 *   ddelta in time-invariant mode: [D]
 * dy: [batch][L][D] float; dlast: [batch][D][N] float or NULL (the gradient reaching the
 * final state).  Single-threaded over (b, d) in a fixed order, so the sums over channels
 * (dB, dC) and over batch and tokens (dA, dDskip, ddelta_bias) have a fixed order. */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* d c / d a for the ZOH coefficient c = expm1(dt a)/a: (dt e^{dt a} - c)/a, written through
 * x = dt a as dt^2 * (x e^x - expm1(x)) / x^2, with its series 1/2 + x/3 + x^2/8 + x^3/30
 * + x^4/144 where |x| is small enough for the closed form to cancel. */
static double zoh_coeff_da(double dt, double a) {
  const double x = dt * a;
  if (fabs(x) < 1e-3) return dt * dt * (0.5 + x * (1.0 / 3.0 + x * (1.0 / 8.0 + x * (1.0 / 30.0 + x / 144.0))));
  return dt * dt * (x * exp(x) - expm1(x)) / (x * x);
}

int ssm_oracle_bwd(const float* u, const float* delta, const float* A, const float* B, const float* C,
                   const float* Dskip, const float* z, const float* h0, const float* delta_bias,
                   const float* dy, const float* dlast,
                   double* du, double* ddelta, double* dA, double* dB, double* dC, double* dDskip,
                   double* dz, double* ddelta_bias, double* dh0,
                   int64_t batch, int64_t L, int64_t D, int64_t N, int time_invariant, int euler,
                   int delta_softplus) {
  if (batch < 0 || L < 0 || D <= 0 || N <= 0) return -1;
  if (!A || !du || !ddelta || !dA || !dB || !dC || !dz) return -1;
  if (batch * L > 0 && (!u || !delta || !B || !C || !dy)) return -1;
  const int ti = time_invariant;
  memset(du, 0, sizeof(double) * (size_t)(batch * L * D));
  memset(dz, 0, sizeof(double) * (size_t)(batch * L * D));
  memset(ddelta, 0, sizeof(double) * (size_t)(ti ? D : batch * L * D));
  memset(dB, 0, sizeof(double) * (size_t)(ti ? D * N : batch * L * N));
  memset(dC, 0, sizeof(double) * (size_t)(ti ? D * N : batch * L * N));
  memset(dA, 0, sizeof(double) * (size_t)(D * N));
  if (dDskip) memset(dDskip, 0, sizeof(double) * (size_t)D);
  if (ddelta_bias) memset(ddelta_bias, 0, sizeof(double) * (size_t)D);
  if (dh0) memset(dh0, 0, sizeof(double) * (size_t)(batch * D * N));
  if (batch == 0) return 0;
  double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));   /* h_{-1} .. h_{L-1} */
  double* lam = (double*)malloc(sizeof(double) * (size_t)N);
  if (!hs || !lam) { free(hs); free(lam); return -2; }
  oracle_job j;                       /* only the fields step_size reads */
  memset(&j, 0, sizeof(j));
  j.delta_bias = delta_bias; j.delta_softplus = delta_softplus;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      /* forward, caching the trajectory */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? (double)h0[(b * D + d) * N + n] : 0.0;
      for (int64_t l = 0; l < L; ++l) {
        const int64_t tok = (b * L + l) * D + d;
        const double uu = (double)u[tok];
        const double dt = step_size(&j, ti ? (double)delta[d] : (double)delta[tok], d);
        const float* Brow = ti ? B + d * N : B + (b * L + l) * N;
        for (int64_t n = 0; n < N; ++n) {
          const double a = (double)A[d * N + n];
          const double c = euler ? dt : zoh_input_coeff(dt, a);
          hs[(l + 1) * N + n] = exp(dt * a) * hs[l * N + n] + c * (double)Brow[n] * uu;
        }
      }
      /* reverse */
      for (int64_t n = 0; n < N; ++n) lam[n] = dlast ? (double)dlast[(b * D + d) * N + n] : 0.0;
      for (int64_t l = L - 1; l >= 0; --l) {
        const int64_t tok = (b * L + l) * D + d;
        const double uu = (double)u[tok];
        const double raw = ti ? (double)delta[d] : (double)delta[tok];
        const double dt = step_size(&j, raw, d);
        const float* Brow = ti ? B + d * N : B + (b * L + l) * N;
        const float* Crow = ti ? C + d * N : C + (b * L + l) * N;
        double* dBrow = ti ? dB + d * N : dB + (b * L + l) * N;
        double* dCrow = ti ? dC + d * N : dC + (b * L + l) * N;
        /* pre-gate output and the gate */
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) s += (double)Crow[n] * hs[(l + 1) * N + n];
        const double yp = s + (Dskip ? (double)Dskip[d] * uu : 0.0);
        double dyp = (double)dy[tok];
        if (z) {
          const double zz = (double)z[tok], sg = sigmoid(zz);
          dz[tok] = dyp * yp * sg * (1.0 + zz * (1.0 - sg));
          dyp *= zz * sg;
        }
        if (Dskip) dDskip[d] += dyp * uu;
        double g_u = Dskip ? (double)Dskip[d] * dyp : 0.0, g_dt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double a = (double)A[d * N + n];
          const double abar = exp(dt * a);
          const double c = euler ? dt : zoh_input_coeff(dt, a);
          const double dc_ddt = euler ? 1.0 : abar;
          const double dc_da = euler ? 0.0 : (a == 0.0 ? 0.5 * dt * dt : zoh_coeff_da(dt, a));
          const double hp = hs[l * N + n], bn = (double)Brow[n];
          const double ln = dyp * (double)Crow[n] + lam[n];        /* lambda_t */
          dCrow[n] += dyp * hs[(l + 1) * N + n];
          dBrow[n] += ln * c * uu;
          g_u += ln * c * bn;
          g_dt += ln * (a * abar * hp + dc_ddt * bn * uu);
          dA[d * N + n] += ln * (dt * abar * hp + dc_da * bn * uu);
          lam[n] = abar * ln;                                       /* carried to token l-1 */
        }
        du[tok] = g_u;
        const double g_raw = g_dt * (delta_softplus ? sigmoid(raw + (delta_bias ? (double)delta_bias[d] : 0.0)) : 1.0);
        if (ti) ddelta[d] += g_raw;
        else ddelta[tok] = g_raw;
        if (ddelta_bias) ddelta_bias[d] += g_raw;
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = lam[n];
    }
  }
  free(hs);
  free(lam);
  return 0;
}
