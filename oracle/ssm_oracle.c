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
