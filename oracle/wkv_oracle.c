/*
 * wkv_oracle.c -- plain, slow, fp64 CPU oracle for the RWKV-4 WKV time-mixing path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header, table
 * or helper with the GPU library; the two meet only through the seeded inputs.
 *
 * What is computed (the WKV operator of the RWKV paper, arXiv 2305.13048, which
 * the "RWKV-4 14B" architecture page cites; the TR-2026-0009 port report,
 * sections Abstract, Methods and Reproducibility, describes the same operator as
 * a per-channel numerator/denominator/max recurrence with fp32 state, a
 * receptance gate and a token shift):
 *
 *   For one channel with decay w (natural-log units, w <= 0) and bonus u, keys
 *   k_0..k_{T-1}, values v_0..v_{T-1}, and an optional prior state whose
 *   numerator and denominator are N0 = aa0 * e^pp0 and D0 = bb0 * e^pp0:
 *
 *     num_t = e^{t w} N0 + sum_{i<t} e^{(t-1-i) w + k_i} v_i + e^{u + k_t} v_t
 *     den_t = e^{t w} D0 + sum_{i<t} e^{(t-1-i) w + k_i}     + e^{u + k_t}
 *     wkv_t = num_t / den_t
 *
 *   The newest past token (i = t-1) carries no decay; every older one loses one
 *   factor e^w per step.  The current token gets the bonus u instead of a decay.
 *   The prior-state term follows from feeding the state through t updates.
 *   Gated output: y_t = wkv_t / (1 + e^{-r_t}).
 *
 *   The state after T tokens is the triple (aa, bb, pp) with
 *     pp = max( pp0 + T w  [only with a prior state],  max_i k_i + (T-1-i) w ),
 *     aa = e^{-pp} * (e^{T w} N0 + sum_i e^{(T-1-i) w + k_i} v_i),  bb likewise,
 *   i.e. the numerator/denominator scaled by their largest term, which is what a
 *   running-max ("max-trick") recurrence carries.
 *
 * Error yardstick: scale_t applies the same weights to |v_i| and |aa0|,
 * so |wkv_t| <= scale_t.  The tests measure GPU error relative to it.
 *
 * Precision: everything in fp64 and in linear space (no max-trick).  Callers keep
 * |k|, |pp| well below 700 so that no exponential overflows; each routine reports
 * a non-finite result through its return code.
 *
 * Layout: activations [B, T, C] row-major (C fastest); per-channel w, u, mix [C];
 * states planar [3, B, C] = (aa, bb, pp).  All arrays are fp64.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX(b, t, c) (((int64_t)(b) * T + (t)) * C + (c))

/* e^{n w}, with the convention e^{0 * w} = 1 even when w = -inf. */
static double decay_pow(int64_t n, double w)
{
    if (n == 0) return 1.0;
    return exp((double)n * w);
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Threads of the routines that take no thread count (LayerNorm, the gate); 0 leaves it. */
void oracle_set_num_threads(int nthreads) { set_threads(nthreads); }

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One output of one lane by the direct sums of the definition above.
 * kl, vl point at the lane's first token and advance by `stride` per token.
 */
static void direct_point(int64_t t, int64_t stride, double w, double u,
                         const double *kl, const double *vl, int has_prior,
                         double aa0, double bb0, double pp0,
                         double *y, double *s)
{
    double num = 0.0, den = 0.0, absn = 0.0;
    if (has_prior) {
        double f = decay_pow(t, w) * exp(pp0);
        num += f * aa0;
        den += f * bb0;
        absn += f * fabs(aa0);
    }
    for (int64_t i = 0; i < t; ++i) {
        const int64_t age = t - 1 - i;
        const double e = exp((age == 0) ? kl[i * stride] : (double)age * w + kl[i * stride]);
        num += e * vl[i * stride];
        den += e;
        absn += e * fabs(vl[i * stride]);
    }
    double eb = exp(u + kl[t * stride]);
    num += eb * vl[t * stride];
    den += eb;
    absn += eb * fabs(vl[t * stride]);
    *y = num / den;
    *s = absn / den;
}

static double logistic(double r) { return 1.0 / (1.0 + exp(-r)); }

/*
 * Every output of every lane by the direct sums: O(T^2) per lane.
 * r (nullable) gates the output; state_in (nullable) is the prior state.
 * y, scale: [B, T, C].  Returns 0, or 1 if any output is not finite.
 */
int oracle_wkv_direct(int64_t B, int64_t T, int64_t C,
                      const double *w, const double *u,
                      const double *k, const double *v, const double *r,
                      const double *state_in, double *y, double *scale, int nthreads)
{
    set_threads(nthreads);
    int bad = 0;
    const int64_t lanes = B * C;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t lane = 0; lane < lanes; ++lane) {
        const int64_t b = lane / C, c = lane % C;
        const double *kl = k + IDX(b, 0, c), *vl = v + IDX(b, 0, c);
        double aa0 = 0, bb0 = 0, pp0 = 0;
        if (state_in) {
            aa0 = state_in[0 * lanes + lane];
            bb0 = state_in[1 * lanes + lane];
            pp0 = state_in[2 * lanes + lane];
        }
        for (int64_t t = 0; t < T; ++t) {
            double yt, st;
            direct_point(t, C, w[c], u[c], kl, vl, state_in != NULL, aa0, bb0, pp0, &yt, &st);
            if (r) {
                double g = logistic(r[IDX(b, t, c)]);
                yt *= g;
                st *= g;
            }
            if (!isfinite(yt) || !isfinite(st)) bad |= 1;
            y[IDX(b, t, c)] = yt;
            scale[IDX(b, t, c)] = st;
        }
    }
    return bad;
}

/*
 * Selected outputs only, by the same direct sums: npts points (b, t, c) given as
 * three index arrays.  O(t) per point, so usable at any sequence length.
 */
int oracle_wkv_points(int64_t B, int64_t T, int64_t C,
                      const double *w, const double *u,
                      const double *k, const double *v, const double *r,
                      const double *state_in, int64_t npts,
                      const int64_t *pb, const int64_t *pt, const int64_t *pc,
                      double *y, double *scale, int nthreads)
{
    set_threads(nthreads);
    int bad = 0;
    const int64_t lanes = B * C;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t n = 0; n < npts; ++n) {
        const int64_t b = pb[n], t = pt[n], c = pc[n];
        const int64_t lane = b * C + c;
        double aa0 = 0, bb0 = 0, pp0 = 0;
        if (state_in) {
            aa0 = state_in[0 * lanes + lane];
            bb0 = state_in[1 * lanes + lane];
            pp0 = state_in[2 * lanes + lane];
        }
        double yt, st;
        direct_point(t, C, w[c], u[c], k + IDX(b, 0, c), v + IDX(b, 0, c),
                     state_in != NULL, aa0, bb0, pp0, &yt, &st);
        if (r) {
            double g = logistic(r[IDX(b, t, c)]);
            yt *= g;
            st *= g;
        }
        if (!isfinite(yt) || !isfinite(st)) bad |= 1;
        y[n] = yt;
        scale[n] = st;
    }
    return bad;
}

/*
 * The state after all T tokens, by its definition (see the file header):
 * pp is the largest log-weight, aa and bb are the sums scaled by e^{-pp}.
 * state_out [3, B, C].  Also returns |aa| scale in abs_out[B*C] (nullable):
 * the same weights applied to |v| and |aa0|.
 */
int oracle_wkv_state(int64_t B, int64_t T, int64_t C,
                     const double *w, const double *k, const double *v,
                     const double *state_in, double *state_out, double *abs_out, int nthreads)
{
    set_threads(nthreads);
    int bad = 0;
    const int64_t lanes = B * C;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t lane = 0; lane < lanes; ++lane) {
        const int64_t b = lane / C, c = lane % C;
        const double wc = w[c];
        double aa0 = 0, bb0 = 0, pp0 = 0;
        if (state_in) {
            aa0 = state_in[0 * lanes + lane];
            bb0 = state_in[1 * lanes + lane];
            pp0 = state_in[2 * lanes + lane];
        }
        /* largest log-weight among all terms of the numerator/denominator */
        double pmax = -INFINITY;
        if (state_in) pmax = (T == 0) ? pp0 : (double)T * wc + pp0;
        for (int64_t i = 0; i < T; ++i) {
            int64_t age = T - 1 - i;
            double lw = (age == 0) ? k[IDX(b, i, c)] : (double)age * wc + k[IDX(b, i, c)];
            if (lw > pmax) pmax = lw;
        }
        double aa = 0.0, bb = 0.0, ab = 0.0;
        if (state_in) {
            double f = exp(((T == 0) ? pp0 : (double)T * wc + pp0) - pmax);
            aa += f * aa0;
            bb += f * bb0;
            ab += f * fabs(aa0);
        }
        for (int64_t i = 0; i < T; ++i) {
            int64_t age = T - 1 - i;
            double lw = (age == 0) ? k[IDX(b, i, c)] : (double)age * wc + k[IDX(b, i, c)];
            double e = exp(lw - pmax);
            aa += e * v[IDX(b, i, c)];
            bb += e;
            ab += e * fabs(v[IDX(b, i, c)]);
        }
        /* pp = -inf is the empty state (T = 0, no prior) and is not an error */
        if (!isfinite(aa) || !isfinite(bb) || isnan(pmax) || pmax == INFINITY) bad |= 1;
        state_out[0 * lanes + lane] = aa;
        state_out[1 * lanes + lane] = bb;
        state_out[2 * lanes + lane] = pmax;
        if (abs_out) abs_out[lane] = ab;
    }
    return bad;
}

/*
 * The recurrence the port report describes (a numerator and a denominator
 * carried per channel from token to token), in fp64 linear space:
 *   output at t :  wkv_t = (N + e^{u+k_t} v_t) / (D + e^{u+k_t})
 *   then update :  N <- e^w N + e^{k_t} v_t,   D <- e^w D + e^{k_t}
 * starting from N = aa0 e^pp0, D = bb0 e^pp0 (zero without a prior state).
 * Summing the geometric decays of this recurrence gives exactly the direct
 * sums above, in O(T) per lane instead of O(T^2).  No max-trick: fp64 has the
 * range for every input the tests draw.  y, scale [B, T, C]; the final state is
 * left to oracle_wkv_state.
 */
int oracle_wkv_recurrence(int64_t B, int64_t T, int64_t C,
                          const double *w, const double *u,
                          const double *k, const double *v, const double *r,
                          const double *state_in, double *y, double *scale, int nthreads)
{
    set_threads(nthreads);
    int bad = 0;
    const int64_t lanes = B * C;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t lane = 0; lane < lanes; ++lane) {
        const int64_t b = lane / C, c = lane % C;
        const double ew = exp(w[c]), eu = exp(u[c]);
        double N = 0.0, D = 0.0, A = 0.0;
        if (state_in) {
            double e = exp(state_in[2 * lanes + lane]);
            N = state_in[0 * lanes + lane] * e;
            D = state_in[1 * lanes + lane] * e;
            A = fabs(state_in[0 * lanes + lane]) * e;
        }
        for (int64_t t = 0; t < T; ++t) {
            const double kt = k[IDX(b, t, c)], vt = v[IDX(b, t, c)];
            const double ek = exp(kt);
            const double den = D + eu * ek;
            double yt = (N + eu * ek * vt) / den;
            double st = (A + eu * ek * fabs(vt)) / den;
            if (r) {
                double g = logistic(r[IDX(b, t, c)]);
                yt *= g;
                st *= g;
            }
            if (!isfinite(yt) || !isfinite(st)) bad |= 1;
            y[IDX(b, t, c)] = yt;
            scale[IDX(b, t, c)] = st;
            N = ew * N + ek * vt;
            D = ew * D + ek;
            A = ew * A + ek * fabs(vt);
        }
    }
    return bad;
}

/*
 * Token shift (the port report's "mix current and previous token"):
 * the shifted sequence is xs_0 = x_prev (zeros when x_prev is NULL), xs_t = x_{t-1};
 * out_t = mix * x_t + (1 - mix) * xs_t per channel.  out [B, T, C].
 */
void oracle_token_shift(int64_t B, int64_t T, int64_t C,
                        const double *x, const double *x_prev, const double *mix, double *out)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t c = 0; c < C; ++c) {
                double xs = (t > 0) ? x[IDX(b, t - 1, c)] : (x_prev ? x_prev[b * C + c] : 0.0);
                out[IDX(b, t, c)] = mix[c] * x[IDX(b, t, c)] + (1.0 - mix[c]) * xs;
            }
}

/*
 * LayerNorm over the channels of every row (the "RWKV-4 14B" page, Facts table: the norm is
 * LayerNorm and sits before each mixer, ln1 before time mixing and ln2 before channel mixing;
 * the port report's Abstract lists pre-LN).  The textbook definition: per row, the mean and the
 * biased variance (divided by C) of its C values, z = (x - mean) / sqrt(var + eps), and the
 * per-channel affine out = z * weight + bias.  x and out [rows, C]; weight, bias [C].
 */
void oracle_layer_norm(int64_t rows, int64_t C, const double *x, const double *weight,
                       const double *bias, double eps, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * C;
        double mean = 0.0;
        for (int64_t c = 0; c < C; ++c) mean += xr[c];
        mean /= (double)C;
        double var = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            const double d = xr[c] - mean;
            var += d * d;
        }
        var /= (double)C;
        const double inv = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < C; ++c) out[r * C + c] = (xr[c] - mean) * inv * weight[c] + bias[c];
    }
}

/*
 * Receptance gate of channel mixing (the port report's "time-mix / channel-mix gating"; the
 * "RWKV-4 14B" page, field table: channel mixing has its own d x d receptance matrix):
 * y = residual + kv / (1 + e^{-r}) elementwise over n values; residual NULL = 0.
 */
void oracle_receptance_gate(int64_t n, const double *r, const double *kv, const double *residual,
                            double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const double g = kv[i] / (1.0 + exp(-r[i]));
        y[i] = residual ? residual[i] + g : g;
    }
}
