/*
 * ssq_oracle.c -- the CPU oracle for the quantized recurrent-state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline do.  It shares no code, header, table or constant with the GPU
 * library; it is plain, single-threaded C built with -ffp-contract=off, so
 * that every fp32 operation below is exactly one IEEE rounding and fmaf()
 * appears only where the evaluation order says "fused".
 *
 * What it computes (sources are the pages on recurrent-state quantization):
 *
 *  Mamba-2 layer, per row (sequence b, head h, head-dim p) of N state
 *  entries -- "ssm-state-quantization" README, Setup:
 *    lambda = exp(dt*A)                          decay of the head
 *    h'_n   = lambda*h_n + dt*x*B_n              write of the token
 *    y      = sum_n C_n*r_n + D*x                readout, r = the state after
 *                                                quantization (the README reads
 *                                                the output from the quantized
 *                                                state) or, as an option, before
 *  The row is then refit and rounded to nearest (Setup, quantizer bullets):
 *    symmetric  grid [-amax, amax], step amax/(2^(b-1)-1), codes in
 *               [-(2^(b-1)-1), 2^(b-1)-1]
 *    asymmetric grid [min, max], step (max-min)/(2^b-1), integer zero point,
 *               codes in [0, 2^b-1]
 *  refit every step from the new fp32 row.
 *
 *  Rounding is to nearest, or stochastic (README, Findings 9): the code is
 *  floor(v + U) for the exact v = h*inv + z and U uniform in [0, 1) drawn from
 *  SplitMix64 by (seed, token, state row, entry); the grid is the same.
 *
 *  Delta rule (GDN/KDA-style), one dk x dv matrix S per (sequence, head) --
 *  "Mamba state quantization for inference", sections "Mamba state
 *  quantization changes persistent state" and "Quantization error returns on
 *  the next token": decay plus a delta-rule correction write the next state,
 *    S' = alpha*(I - beta*k*k^T)*S + beta*k*v^T,   o = S'^T q,
 *  each key channel i (a row of S over the value dimension) quantized like a
 *  Mamba-2 row.
 *
 * Fixed fp32 evaluation order (the pages give the formulas, not the rounding
 * order; fl() is one fp32 rounding):
 *    lambda = fl32(exp_double(fl(dt*A)))          exp taken in double
 *    w      = fl(dt*x)
 *    quantized row (scale s, zero z, codes c): reconstruct, then recur
 *      hh_n = fl(s*fl(c_n - z))                   the stored row in fp32
 *      h'_n = fma(lambda, hh_n, fl(w*B_n))         the fp32 update below
 *    fp32 row:  h'_n = fma(lambda, h_n, fl(w*B_n))
 *    refit, asymmetric: mn, mx = min/max h'; s' = fl(fl(mx-mn)/(2^b-1));
 *      inv = fl(1/s'); z' = -rne(mn*inv);
 *      c'_n = clamp(rne(h'_n*inv + z'), 0, 2^b-1)
 *    refit, symmetric: s' = fl(amax/(2^(b-1)-1)); inv = fl(1/s');
 *      c'_n = clamp(rne(h'_n*inv), -(2^(b-1)-1), 2^(b-1)-1)
 *    where rne() rounds the exact real value (the product h'*inv is not
 *      rounded first) to the nearest integer, a tie going to the even code.
 *    degenerate rows: if s' is zero or subnormal the row carries no usable
 *      step.  Asymmetric rows are then stored as the constant mn (s' = |mn|,
 *      z' = -sign(mn), all codes 0, which dequantizes to mn exactly);
 *      symmetric rows are stored as zero (s' = 0, codes 0).
 *    a zero point of zero is stored as +0.
 *    dequantized value: fl(s*fl(c - z)).
 *    Readouts (y, o) are output only: they are accumulated here in double and
 *    rounded once, so they are the most accurate value any order can give.
 *    Delta rule: a quantized S is first reconstructed row by row,
 *      S_ij = fl(s_i*fl(c_ij - z_i)); then u_j = RN32(sum_i k_i*S_ij) with the
 *      products and the sum taken in double; w_j = fl(beta*fl(v_j - fl(alpha*u_j)));
 *      S'_ij = fma(alpha, S_ij, fl(k_i*w_j)).
 *    The quantized paths thus run the fp32 recurrence on the reconstructed
 *    state ("Mamba state quantization for inference", "Mixed precision spends
 *    bits on persistent channels": the fused kernel reconstructs the low tier,
 *    computes the recurrence in FP32, refits and writes back; README, Setup:
 *    the decay and the write act on the state).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must be built without -ffast-math"
#endif

/* ------------------------------------------------------------------------ */
/* decay                                                                    */
/* ------------------------------------------------------------------------ */

float orc_decay(float dt, float A)
{
    float e = dt * A; /* fl(dt*A) */
    return (float)exp((double)e);
}

/* ------------------------------------------------------------------------ */
/* one row: refit and round to nearest                                       */
/* ------------------------------------------------------------------------ */

/* The integer nearest to the real number p + z (p a double, z an integer
 * valued double), a tie going to the even result.  p - floor(p) is exact, so
 * the decision is exact even where p + z itself is not representable. */
static double rne_sum(double p, double z)
{
    double f = floor(p);
    double r = p - f;
    double k;
    if (r > 0.5)
        k = f + 1.0;
    else if (r < 0.5)
        k = f;
    else
        k = (fmod(f + z, 2.0) == 0.0) ? f : f + 1.0;
    return k + z;
}

/* Stochastic rounding ("ssm-state-quantization" README, Findings 9: the state
 * rounded stochastically instead of to nearest).  The code is floor(v + U)
 * for the exact real v = p + z (p = h*inv, z an integer) and a uniform U in
 * [0, 1) that is a multiple of 2^-16, U = K/2^16: it rounds up with the
 * probability that the fraction of v, taken down to a multiple of 2^-16, reaches
 * 1 - U.  floor(p + U) = floor(p) + [t + K >= 2^16] with t = floor(2^16 frac(p))
 * = floor(2^16 p) - 2^16 floor(p): both terms are exact integers in double and
 * so is their difference (it lies in [0, 2^16)), for every p. */
static double sr_sum(double p, double z, float u)
{
    double K = (double)u * 65536.0;
    double f = floor(p);
    double t = floor(p * 65536.0) - f * 65536.0;
    return f + z + (t + K >= 65536.0 ? 1.0 : 0.0);
}

/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): output number i >= 1 of the generator whose state
 * starts at `seed`, i.e. the state advanced i times by the golden gamma and
 * passed through the finalizer. */
uint64_t orc_splitmix64(uint64_t seed, uint64_t i)
{
    uint64_t x = seed + i * 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

/* The uniform that entry n of state row r draws at token `step`, for the flat
 * counter ctr = (step*rows + r)*N + n: every output of the generator gives four
 * 16-bit uniforms, counter ctr taking bits 16k .. 16k+15 (k = ctr mod 4) of
 * output number floor(ctr/4) + 1, scaled by 2^-16. */
float orc_sr_uniform(uint64_t seed, uint64_t step, int64_t rows, int64_t r, int N, int n)
{
    uint64_t ctr = (step * (uint64_t)rows + (uint64_t)r) * (uint64_t)N + (uint64_t)n;
    uint64_t out = orc_splitmix64(seed, ctr / 4 + 1);
    uint32_t K = (uint32_t)(out >> (16 * (ctr % 4))) & 0xFFFFu;
    return (float)K * (1.0f / 65536.0f);
}

/* the N uniforms of state row r at token `step` */
void orc_sr_row_uniforms(uint64_t seed, uint64_t step, int64_t rows, int64_t r, int N, float *U)
{
    int n;
    for (n = 0; n < N; ++n)
        U[n] = orc_sr_uniform(seed, step, rows, r, N, n);
}

static float sign_of(float c)
{
    if (c > 0.0f)
        return 1.0f;
    if (c < 0.0f)
        return -1.0f;
    return 0.0f;
}

/* Quantize the n entries of h with a b-bit grid (bits in 2..8).  Writes the
 * integer codes, the scale and the zero point (0 for the symmetric grid).
 * v_out, if not NULL, receives fl(h_n*inv), the value that is rounded (to
 * within half an ulp: the rounding itself uses the exact product).  U NULL:
 * round to nearest; else U[i] in [0, 1) rounds entry i stochastically.  The
 * grid (scale, zero point) does not depend on the rounding. */
void orc_quantize_row_sr(const float *h, int n, int bits, int asym, int32_t *code, float *s_out,
                         float *z_out, float *v_out, const float *U)
{
    int i;
    if (asym) {
        const float cmax = (float)((1 << bits) - 1);
        float mn = h[0], mx = h[0];
        for (i = 1; i < n; ++i) {
            if (h[i] < mn)
                mn = h[i];
            if (h[i] > mx)
                mx = h[i];
        }
        float range = mx - mn;
        float s = range / cmax;
        if (!(s >= FLT_MIN)) {
            *s_out = fabsf(mn);
            *z_out = -sign_of(mn) + 0.0f; /* a zero zero point is stored as +0 */
            for (i = 0; i < n; ++i) {
                code[i] = 0;
                if (v_out)
                    v_out[i] = 0.0f;
            }
            return;
        }
        float inv = 1.0f / s;
        /* products of two floats are exact in double */
        float z = (float)(-rne_sum((double)mn * (double)inv, 0.0)) + 0.0f; /* +0, never -0 */
        for (i = 0; i < n; ++i) {
            float v = h[i] * inv;
            double p = (double)h[i] * (double)inv;
            double t = U ? sr_sum(p, (double)z, U[i]) : rne_sum(p, (double)z);
            if (t < 0.0)
                t = 0.0;
            if (t > (double)cmax)
                t = (double)cmax;
            code[i] = (int32_t)t;
            if (v_out)
                v_out[i] = v;
        }
        *s_out = s;
        *z_out = z;
    } else {
        const float cmax = (float)((1 << (bits - 1)) - 1);
        float amax = 0.0f;
        for (i = 0; i < n; ++i) {
            float a = fabsf(h[i]);
            if (a > amax)
                amax = a;
        }
        float s = amax / cmax;
        if (!(s >= FLT_MIN)) {
            *s_out = 0.0f;
            *z_out = 0.0f;
            for (i = 0; i < n; ++i) {
                code[i] = 0;
                if (v_out)
                    v_out[i] = 0.0f;
            }
            return;
        }
        float inv = 1.0f / s;
        for (i = 0; i < n; ++i) {
            float v = h[i] * inv;
            double p = (double)h[i] * (double)inv;
            double t = U ? sr_sum(p, 0.0, U[i]) : rne_sum(p, 0.0);
            if (t < -(double)cmax)
                t = -(double)cmax;
            if (t > (double)cmax)
                t = (double)cmax;
            code[i] = (int32_t)t;
            if (v_out)
                v_out[i] = v;
        }
        *s_out = s;
        *z_out = 0.0f;
    }
}

void orc_quantize_row(const float *h, int n, int bits, int asym, int32_t *code, float *s_out,
                      float *z_out, float *v_out)
{
    orc_quantize_row_sr(h, n, bits, asym, code, s_out, z_out, v_out, NULL);
}

void orc_dequantize_row(const int32_t *code, int n, float s, float z, float *out)
{
    int i;
    for (i = 0; i < n; ++i) {
        float d = (float)code[i] - z;
        out[i] = s * d;
    }
}

void orc_quantize_rows(int64_t rows, int n, int bits, int asym, const float *h, int32_t *code,
                       float *s, float *z, float *v_out)
{
    int64_t r;
    for (r = 0; r < rows; ++r)
        orc_quantize_row(h + r * n, n, bits, asym, code + r * n, s + r, z + r,
                         v_out ? v_out + r * n : NULL);
}

void orc_dequantize_rows(int64_t rows, int n, const int32_t *code, const float *s, const float *z,
                         float *out)
{
    int64_t r;
    for (r = 0; r < rows; ++r)
        orc_dequantize_row(code + r * n, n, s[r], z[r], out + r * n);
}

/* ------------------------------------------------------------------------ */
/* Mamba-2: one token for one row                                            */
/* ------------------------------------------------------------------------ */

/* bits == 0: fp32 state in h (code/s/z unused).  Otherwise the row's codes,
 * scale and zero point are read and replaced.  hpre (optional) receives the
 * new row before rounding, vq (optional) the fp32 values that were rounded.
 * Returns y. */
static float mamba2_row_step(int N, int bits, int asym, int32_t *code, float *s, float *z,
                             float *h, float x, float dt, float A, const float *Bn,
                             const float *Cn, float D, int readout_pre, float *hpre, float *vq,
                             float *work, const float *U)
{
    int n;
    float lam = orc_decay(dt, A);
    float w = dt * x;
    float dx = D * x;
    double acc = 0.0;

    if (bits == 0) {
        for (n = 0; n < N; ++n) {
            float wb = w * Bn[n];
            h[n] = fmaf(lam, h[n], wb);
            if (hpre)
                hpre[n] = h[n];
            acc += (double)Cn[n] * (double)h[n];
        }
        return (float)(acc + (double)dx);
    }

    /* reconstruct the stored row, then the fp32 update of the row above */
    orc_dequantize_row(code, N, *s, *z, work);
    for (n = 0; n < N; ++n) {
        float wb = w * Bn[n];
        work[n] = fmaf(lam, work[n], wb);
        if (hpre)
            hpre[n] = work[n];
    }
    if (readout_pre) {
        for (n = 0; n < N; ++n)
            acc += (double)Cn[n] * (double)work[n];
    }
    orc_quantize_row_sr(work, N, bits, asym, code, s, z, vq, U);
    if (!readout_pre) {
        orc_dequantize_row(code, N, *s, *z, work);
        for (n = 0; n < N; ++n)
            acc += (double)Cn[n] * (double)work[n];
    }
    return (float)(acc + (double)dx);
}

/* One decode step of one layer.
 *   code [Bsz][H][P][N] int32, s, z [Bsz][H][P]   (quantized formats)
 *   h    [Bsz][H][P][N] fp32                       (bits == 0)
 *   x [Bsz][H][P], dt [Bsz][H], A [H], Bm/Cm [Bsz][G][N], D [H], y [Bsz][H][P]
 *   hpre, vq: optional [Bsz][H][P][N] diagnostics.
 * Returns 0, or -1 on bad sizes. */
/* As orc_mamba2_step_sr for the sequences of a larger state: the arrays hold sequences
 * b0 .. b0+Bsz-1 of a state of rows_total rows, and stochastic rounding draws the uniforms of
 * those rows' places in it (row r of the slice is state row b0*H*P + r). */
int orc_mamba2_step_sr_part(int Bsz, int H, int G, int P, int N, int bits, int asym, int32_t *code,
                            float *s, float *z, float *h, const float *x, const float *dt,
                            const float *A, const float *Bm, const float *Cm, const float *D,
                            float *y, int readout_pre, float *hpre, float *vq, int sr,
                            uint64_t seed, uint64_t step, int64_t b0, int64_t rows_total)
{
    int b, hh, p;
    float *work, *U;
    int64_t rows = rows_total, row0 = b0 * H * P;
    if (Bsz <= 0 || H <= 0 || G <= 0 || P <= 0 || N <= 0 || H % G != 0 || b0 < 0 ||
        row0 + (int64_t)Bsz * H * P > rows_total)
        return -1;
    work = (float *)malloc(sizeof(float) * (size_t)N);
    U = (float *)malloc(sizeof(float) * (size_t)N);
    if (!work || !U) {
        free(work);
        free(U);
        return -1;
    }
    for (b = 0; b < Bsz; ++b)
        for (hh = 0; hh < H; ++hh) {
            int g = hh / (H / G);
            const float *Bn = Bm + ((int64_t)b * G + g) * N;
            const float *Cn = Cm + ((int64_t)b * G + g) * N;
            float dtv = dt[(int64_t)b * H + hh];
            for (p = 0; p < P; ++p) {
                int64_t r = ((int64_t)b * H + hh) * P + p;
                if (sr)
                    orc_sr_row_uniforms(seed, step, rows, row0 + r, N, U);
                y[r] = mamba2_row_step(N, bits, asym, code ? code + r * N : NULL, s ? s + r : NULL,
                                       z ? z + r : NULL, h ? h + r * N : NULL, x[r], dtv, A[hh],
                                       Bn, Cn, D[hh], readout_pre, hpre ? hpre + r * N : NULL,
                                       vq ? vq + r * N : NULL, work, sr ? U : NULL);
            }
        }
    free(work);
    free(U);
    return 0;
}

int orc_mamba2_step_sr(int Bsz, int H, int G, int P, int N, int bits, int asym, int32_t *code,
                       float *s, float *z, float *h, const float *x, const float *dt, const float *A,
                       const float *Bm, const float *Cm, const float *D, float *y, int readout_pre,
                       float *hpre, float *vq, int sr, uint64_t seed, uint64_t step)
{
    return orc_mamba2_step_sr_part(Bsz, H, G, P, N, bits, asym, code, s, z, h, x, dt, A, Bm, Cm, D,
                                   y, readout_pre, hpre, vq, sr, seed, step, 0,
                                   (int64_t)Bsz * H * P);
}

int orc_mamba2_step(int Bsz, int H, int G, int P, int N, int bits, int asym, int32_t *code,
                    float *s, float *z, float *h, const float *x, const float *dt, const float *A,
                    const float *Bm, const float *Cm, const float *D, float *y, int readout_pre,
                    float *hpre, float *vq)
{
    return orc_mamba2_step_sr(Bsz, H, G, P, N, bits, asym, code, s, z, h, x, dt, A, Bm, Cm, D, y,
                              readout_pre, hpre, vq, 0, 0, 0);
}

/* T tokens of one layer, the state rounded after every token: plain repetition
 * of orc_mamba2_step on token-t slices.
 *   x [Bsz][T][H][P], dt [Bsz][T][H], Bm/Cm [Bsz][T][G][N], y [Bsz][T][H][P] */
int orc_mamba2_scan_sr(int Bsz, int T, int H, int G, int P, int N, int bits, int asym,
                       int32_t *code, float *s, float *z, float *h, const float *x, const float *dt,
                       const float *A, const float *Bm, const float *Cm, const float *D, float *y,
                       int readout_pre, int sr, uint64_t seed, uint64_t step)
{
    int t, b;
    int rc = 0;
    size_t nx = (size_t)Bsz * H * P, ndt = (size_t)Bsz * H, nbc = (size_t)Bsz * G * N;
    float *xs, *dts, *Bs, *Cs, *ys;
    if (T <= 0)
        return -1;
    xs = (float *)malloc(sizeof(float) * nx);
    ys = (float *)malloc(sizeof(float) * nx);
    dts = (float *)malloc(sizeof(float) * ndt);
    Bs = (float *)malloc(sizeof(float) * nbc);
    Cs = (float *)malloc(sizeof(float) * nbc);
    if (!xs || !ys || !dts || !Bs || !Cs) {
        rc = -1;
        goto done;
    }
    for (t = 0; t < T; ++t) {
        for (b = 0; b < Bsz; ++b) {
            memcpy(xs + (size_t)b * H * P, x + ((size_t)b * T + t) * H * P, sizeof(float) * H * P);
            memcpy(dts + (size_t)b * H, dt + ((size_t)b * T + t) * H, sizeof(float) * H);
            memcpy(Bs + (size_t)b * G * N, Bm + ((size_t)b * T + t) * G * N, sizeof(float) * G * N);
            memcpy(Cs + (size_t)b * G * N, Cm + ((size_t)b * T + t) * G * N, sizeof(float) * G * N);
        }
        /* token t draws the uniforms of step + t */
        rc = orc_mamba2_step_sr(Bsz, H, G, P, N, bits, asym, code, s, z, h, xs, dts, A, Bs, Cs, D,
                                ys, readout_pre, NULL, NULL, sr, seed, step + (uint64_t)t);
        if (rc)
            goto done;
        for (b = 0; b < Bsz; ++b)
            memcpy(y + ((size_t)b * T + t) * H * P, ys + (size_t)b * H * P, sizeof(float) * H * P);
    }
done:
    free(xs);
    free(ys);
    free(dts);
    free(Bs);
    free(Cs);
    return rc;
}

int orc_mamba2_scan(int Bsz, int T, int H, int G, int P, int N, int bits, int asym, int32_t *code,
                    float *s, float *z, float *h, const float *x, const float *dt, const float *A,
                    const float *Bm, const float *Cm, const float *D, float *y, int readout_pre)
{
    return orc_mamba2_scan_sr(Bsz, T, H, G, P, N, bits, asym, code, s, z, h, x, dt, A, Bm, Cm, D, y,
                              readout_pre, 0, 0, 0);
}

/* T tokens for R independent rows, each with its own inputs (for checking
 * sampled rows of a large state):
 *   code/h [R][N], s/z [R], x/dt/y [R][T], A/D [R], Bm/Cm [R][T][N] */
int orc_mamba2_rows_scan_sr(int64_t R, int T, int N, int bits, int asym, int32_t *code, float *s,
                            float *z, float *h, const float *x, const float *dt, const float *A,
                            const float *Bm, const float *Cm, const float *D, float *y,
                            int readout_pre, int sr, uint64_t seed, uint64_t step, int64_t rows,
                            const int64_t *row_id)
{
    int64_t r;
    int t;
    float *work = (float *)malloc(sizeof(float) * (size_t)N);
    float *U = (float *)malloc(sizeof(float) * (size_t)N);
    if (!work || !U) {
        free(work);
        free(U);
        return -1;
    }
    for (r = 0; r < R; ++r)
        for (t = 0; t < T; ++t) {
            int64_t rt = r * T + t;
            if (sr)
                orc_sr_row_uniforms(seed, step + (uint64_t)t, rows, row_id[r], N, U);
            y[rt] = mamba2_row_step(N, bits, asym, code ? code + r * N : NULL, s ? s + r : NULL,
                                    z ? z + r : NULL, h ? h + r * N : NULL, x[rt], dt[rt], A[r],
                                    Bm + rt * N, Cm + rt * N, D[r], readout_pre, NULL, NULL, work,
                                    sr ? U : NULL);
        }
    free(work);
    free(U);
    return 0;
}

int orc_mamba2_rows_scan(int64_t R, int T, int N, int bits, int asym, int32_t *code, float *s,
                         float *z, float *h, const float *x, const float *dt, const float *A,
                         const float *Bm, const float *Cm, const float *D, float *y,
                         int readout_pre)
{
    return orc_mamba2_rows_scan_sr(R, T, N, bits, asym, code, s, z, h, x, dt, A, Bm, Cm, D, y,
                                   readout_pre, 0, 0, 0, 0, NULL);
}

/* ------------------------------------------------------------------------ */
/* delta rule: one step of one (sequence, head) matrix                       */
/* ------------------------------------------------------------------------ */

/* code [dk][dv], s/z [dk] (quantized) or S [dk][dv] fp32 (bits == 0); q, k [dk];
 * v [dv]; o [dv].  Spre, vq: optional [dk][dv] diagnostics.
 * avec NULL: one decay alpha for the matrix (Gated DeltaNet):
 *   u = k^T S, w = beta*(v - alpha*u), S' = alpha*S + k w^T.
 * avec [dk]: a decay per key channel (Kimi Delta Attention's channel-wise gate):
 *   S' = (I - beta k k^T) Diag(avec) S + beta k v^T, i.e.
 *   u = k^T Diag(avec) S, w = beta*(v - u), S'_ij = avec_i*S_ij + k_i*w_j. */
static int delta_matrix_step(int dk, int dv, int bits, int asym, int32_t *code, float *s, float *z,
                             float *S, const float *q, const float *k, const float *v, float alpha,
                             float beta, float *o, int readout_pre, float *Spre, float *vq,
                             const float *U, const float *avec)
{
    int i, j;
    float *u = (float *)malloc(sizeof(float) * (size_t)dv);
    float *w = (float *)malloc(sizeof(float) * (size_t)dv);
    float *Sn = (float *)malloc(sizeof(float) * (size_t)dk * dv);
    float *Sh = (float *)malloc(sizeof(float) * (size_t)dk * dv);
    double *acc = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!u || !w || !Sn || !Sh || !acc) {
        free(u);
        free(w);
        free(Sn);
        free(Sh);
        free(acc);
        return -1;
    }

    /* the state the step starts from, in fp32: a quantized state is reconstructed
     * row by row, fl(s_i*fl(c_ij - z_i)) */
    if (bits == 0)
        memcpy(Sh, S, sizeof(float) * (size_t)dk * dv);
    else
        for (i = 0; i < dk; ++i)
            orc_dequantize_row(code + (int64_t)i * dv, dv, s[i], z[i], Sh + (int64_t)i * dv);

    /* u = k^T S, or k^T Diag(avec) S */
    for (j = 0; j < dv; ++j) {
        double a = 0.0;
        for (i = 0; i < dk; ++i) {
            double kd = avec ? (double)k[i] * (double)avec[i] : (double)k[i];
            a += kd * (double)Sh[(int64_t)i * dv + j];
        }
        u[j] = (float)a;
    }
    /* w = beta*(v - alpha*u), or beta*(v - u) when the decay is already in u */
    for (j = 0; j < dv; ++j) {
        float vm;
        if (avec) {
            vm = v[j] - u[j];
        } else {
            float au = alpha * u[j];
            vm = v[j] - au;
        }
        w[j] = beta * vm;
    }
    /* S' = alpha*S + k w^T, alpha the key channel's own decay with avec */
    for (i = 0; i < dk; ++i) {
        float al = avec ? avec[i] : alpha;
        for (j = 0; j < dv; ++j) {
            float kw = k[i] * w[j];
            Sn[(int64_t)i * dv + j] = fmaf(al, Sh[(int64_t)i * dv + j], kw);
        }
    }
    if (Spre)
        memcpy(Spre, Sn, sizeof(float) * (size_t)dk * dv);

    for (j = 0; j < dv; ++j)
        acc[j] = 0.0;
    if (bits == 0 || readout_pre) {
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                acc[j] += (double)q[i] * (double)Sn[(int64_t)i * dv + j];
    }
    if (bits == 0) {
        memcpy(S, Sn, sizeof(float) * (size_t)dk * dv);
    } else {
        for (i = 0; i < dk; ++i)
            orc_quantize_row_sr(Sn + (int64_t)i * dv, dv, bits, asym, code + (int64_t)i * dv, s + i,
                                z + i, vq ? vq + (int64_t)i * dv : NULL,
                                U ? U + (int64_t)i * dv : NULL);
        if (!readout_pre) {
            for (i = 0; i < dk; ++i) {
                orc_dequantize_row(code + (int64_t)i * dv, dv, s[i], z[i], Sn + (int64_t)i * dv);
                for (j = 0; j < dv; ++j)
                    acc[j] += (double)q[i] * (double)Sn[(int64_t)i * dv + j];
            }
        }
    }
    for (j = 0; j < dv; ++j)
        o[j] = (float)acc[j];

    free(u);
    free(w);
    free(Sn);
    free(Sh);
    free(acc);
    return 0;
}

/* One delta-rule step of one layer.
 *   code [Bsz][H][dk][dv], s/z [Bsz][H][dk] or S [Bsz][H][dk][dv]
 *   q, k [Bsz][H][dk], v [Bsz][H][dv], alpha/beta [Bsz][H], o [Bsz][H][dv]
 *   Spre, vq: optional [Bsz][H][dk][dv] */
int orc_delta_step_sr(int Bsz, int H, int dk, int dv, int bits, int asym, int32_t *code, float *s,
                      float *z, float *S, const float *q, const float *k, const float *v,
                      const float *alpha, const float *beta, float *o, int readout_pre, float *Spre,
                      float *vq, int sr, uint64_t seed, uint64_t step)
{
    int64_t m, nm = (int64_t)Bsz * H, i;
    float *U = NULL;
    if (Bsz <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (sr) {
        U = (float *)malloc(sizeof(float) * (size_t)dk * dv);
        if (!U)
            return -1;
    }
    for (m = 0; m < nm; ++m) {
        int64_t mat = m * dk * dv;
        int rc;
        if (sr) /* key row i of matrix m is state row m*dk + i */
            for (i = 0; i < dk; ++i)
                orc_sr_row_uniforms(seed, step, nm * dk, m * dk + i, dv, U + i * dv);
        rc = delta_matrix_step(dk, dv, bits, asym, code ? code + mat : NULL,
                               s ? s + m * dk : NULL, z ? z + m * dk : NULL,
                               S ? S + mat : NULL, q + m * dk, k + m * dk, v + m * dv,
                               alpha[m], beta[m], o + m * dv, readout_pre,
                               Spre ? Spre + mat : NULL, vq ? vq + mat : NULL, U, NULL);
        if (rc) {
            free(U);
            return rc;
        }
    }
    free(U);
    return 0;
}

int orc_delta_step(int Bsz, int H, int dk, int dv, int bits, int asym, int32_t *code, float *s,
                   float *z, float *S, const float *q, const float *k, const float *v,
                   const float *alpha, const float *beta, float *o, int readout_pre, float *Spre,
                   float *vq)
{
    return orc_delta_step_sr(Bsz, H, dk, dv, bits, asym, code, s, z, S, q, k, v, alpha, beta, o,
                             readout_pre, Spre, vq, 0, 0, 0);
}

/* One Kimi-Delta-Attention-style step of one layer: the delta rule with a decay
 * per key channel ("Mamba state quantization for inference": KDA keeps one
 * dk x dv matrix per head, and DAMP finds persistence differing per key
 * channel), S' = (I - beta k k^T) Diag(alpha) S + beta k v^T, o = S'^T q.
 *   alpha [Bsz][H][dk]; everything else as orc_delta_step_sr. */
int orc_kda_step_sr(int Bsz, int H, int dk, int dv, int bits, int asym, int32_t *code, float *s,
                    float *z, float *S, const float *q, const float *k, const float *v,
                    const float *alpha, const float *beta, float *o, int readout_pre, float *Spre,
                    float *vq, int sr, uint64_t seed, uint64_t step)
{
    int64_t m, nm = (int64_t)Bsz * H, i;
    float *U = NULL;
    if (Bsz <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (sr) {
        U = (float *)malloc(sizeof(float) * (size_t)dk * dv);
        if (!U)
            return -1;
    }
    for (m = 0; m < nm; ++m) {
        int64_t mat = m * dk * dv;
        int rc;
        if (sr)
            for (i = 0; i < dk; ++i)
                orc_sr_row_uniforms(seed, step, nm * dk, m * dk + i, dv, U + i * dv);
        rc = delta_matrix_step(dk, dv, bits, asym, code ? code + mat : NULL,
                               s ? s + m * dk : NULL, z ? z + m * dk : NULL,
                               S ? S + mat : NULL, q + m * dk, k + m * dk, v + m * dv,
                               0.0f, beta[m], o + m * dv, readout_pre,
                               Spre ? Spre + mat : NULL, vq ? vq + mat : NULL, U, alpha + m * dk);
        if (rc) {
            free(U);
            return rc;
        }
    }
    free(U);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Mamba-2 prefill with chunk-final quantization                              */
/* ------------------------------------------------------------------------ */

/* T prompt tokens of one layer, the state quantized only at the end of each
 * chunk of `chunk` tokens and after the last token ("Mamba state quantization
 * for inference", "Mamba state quantization needs phase-aware benchmarks":
 * DAMP runs the recurrence in FP32 inside each chunk and writes the
 * chunk-final state into the packed cache).  Per row: the stored state is
 * dequantized once, then every token applies the fp32 update
 * h'_n = fma(lambda, h_n, fl(w*B_n)); inside a chunk y is read from that fp32
 * state; at a chunk end the row is refit and rounded (to nearest, or
 * stochastically with the uniforms of token step + t), y is read from the
 * state the readout flag names, and the next chunk starts from the
 * dequantized new codes.  bits == 0 (fp32 state): the plain fp32 scan.
 * Shapes as orc_mamba2_scan. */
int orc_mamba2_prefill_sr(int Bsz, int T, int chunk, int H, int G, int P, int N, int bits, int asym,
                          int32_t *code, float *s, float *z, float *h, const float *x,
                          const float *dt, const float *A, const float *Bm, const float *Cm,
                          const float *D, float *y, int readout_pre, int sr, uint64_t seed,
                          uint64_t step)
{
    int b, hh, p, t, n;
    int64_t rows = (int64_t)Bsz * H * P;
    float *r, *U;
    if (Bsz <= 0 || T <= 0 || chunk <= 0 || H <= 0 || G <= 0 || P <= 0 || N <= 0 || H % G != 0)
        return -1;
    if (bits == 0)
        return orc_mamba2_scan(Bsz, T, H, G, P, N, 0, 0, NULL, NULL, NULL, h, x, dt, A, Bm, Cm, D, y,
                               readout_pre);
    r = (float *)malloc(sizeof(float) * (size_t)N);
    U = (float *)malloc(sizeof(float) * (size_t)N);
    if (!r || !U) {
        free(r);
        free(U);
        return -1;
    }
    for (b = 0; b < Bsz; ++b)
        for (hh = 0; hh < H; ++hh) {
            int g = hh / (H / G);
            for (p = 0; p < P; ++p) {
                int64_t row = ((int64_t)b * H + hh) * P + p;
                int32_t *c = code + row * N;
                orc_dequantize_row(c, N, s[row], z[row], r);
                for (t = 0; t < T; ++t) {
                    int64_t bt = (int64_t)b * T + t;
                    const float *Bn = Bm + (bt * G + g) * N;
                    const float *Cn = Cm + (bt * G + g) * N;
                    float xv = x[(bt * H + hh) * P + p];
                    float dtv = dt[bt * H + hh];
                    float lam = orc_decay(dtv, A[hh]);
                    float w = dtv * xv;
                    float dx = D[hh] * xv;
                    int end = ((t + 1) % chunk == 0) || t == T - 1;
                    double acc = 0.0;
                    for (n = 0; n < N; ++n) {
                        float wb = w * Bn[n];
                        r[n] = fmaf(lam, r[n], wb);
                    }
                    if (!end || readout_pre)
                        for (n = 0; n < N; ++n)
                            acc += (double)Cn[n] * (double)r[n];
                    if (end) {
                        if (sr)
                            orc_sr_row_uniforms(seed, step + (uint64_t)t, rows, row, N, U);
                        orc_quantize_row_sr(r, N, bits, asym, c, s + row, z + row, NULL,
                                            sr ? U : NULL);
                        orc_dequantize_row(c, N, s[row], z[row], r);
                        if (!readout_pre)
                            for (n = 0; n < N; ++n)
                                acc += (double)Cn[n] * (double)r[n];
                    }
                    y[(bt * H + hh) * P + p] = (float)(acc + (double)dx);
                }
            }
        }
    free(r);
    free(U);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* DAMP-style two-tier delta state                                          */
/* ------------------------------------------------------------------------ */

/* The nearest IEEE half-precision value to x (ties to even), as a float:
 * 10 fraction bits, quantum 2^(e-10) for 2^e <= |x| < 2^(e+1) and e >= -14,
 * 2^-24 below (subnormals); a result above 65504 is infinite.  x/q is exact
 * (a power-of-two scaling), and rint() rounds it half to even. */
float orc_round_half(float x)
{
    double a = fabs((double)x), q, r;
    int e;
    if (a == 0.0 || x != x)
        return x;
    e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a) /* log2 rounding near powers of two */
        e -= 1;
    else if (ldexp(1.0, e + 1) <= a)
        e += 1;
    if (e < -14)
        e = -14;
    q = ldexp(1.0, e - 10);
    r = rint((double)x / q) * q;
    if (fabs(r) > 65504.0)
        return x > 0 ? INFINITY : -INFINITY;
    return (float)r;
}

/* Entry (j, i) of the scaled Sylvester-Hadamard matrix Hs = H_128 / 16: (-1)^popcount(i & j) / 16.
 * Hs is symmetric and Hs*Hs = I/2. */
static double hs(int j, int i)
{
    int v = i & j, c = 0;
    while (v) {
        c += v & 1;
        v >>= 1;
    }
    return (c & 1) ? -1.0 / 16.0 : 1.0 / 16.0;
}

/* One step of the two-tier delta-rule state of one layer ("Mamba state
 * quantization for inference", "Mixed precision spends bits on persistent
 * channels": a Hadamard transform along each key channel's value dimension,
 * the protected key channels in FP16 and the rest in INT8 with scale and
 * zero point, selected channels permuted to be contiguous; the fused kernel
 * reconstructs the low tier, runs the recurrence in FP32, refits and writes
 * the packed state back).  The protected channels are key channels 0 .. nhi-1
 * (the model's key projection is permuted offline so that they come first).
 * The stored matrix is the rotated St = S Hs, row by row; in those
 * coordinates the step is the scalar-decay delta rule with v rotated and o
 * rotated back (Hs is symmetric and Hs Hs = I/2):
 *   vt = Hs v  (exact in double, rounded once)
 *   St = the stored rows in fp32: FP16 rows as they are, INT8 rows
 *        reconstructed as fl(s_i*fl(c_ij - z_i))
 *   ut = k^T St  (double, rounded once), wt = fl(beta*fl(vt - fl(alpha*ut)))
 *   St'_ij = fma(alpha, St_ij, fl(k_i*wt_j))            (every row)
 *   FP16 rows stored rounded to half, INT8 rows refit and rounded (asymmetric)
 *   ot = St'^T q over the stored (post) or pre-rounding rows, o = 2 Hs ot
 *   (ot and o in double, o rounded once).
 *   hi [Bsz][H][nhi][dv] (half values held in floats), code [Bsz][H][dk-nhi][dv],
 *   s/z [Bsz][H][dk-nhi]; q, k [Bsz][H][dk], v [Bsz][H][dv], alpha/beta [Bsz][H],
 *   o [Bsz][H][dv].  dv must be 128. */
int orc_damp_step_sr(int Bsz, int H, int dk, int dv, int nhi, float *hi, int32_t *code, float *s,
                     float *z, const float *q, const float *k, const float *v, const float *alpha,
                     const float *beta, float *o, int readout_pre, float *Spre, int sr, uint64_t seed,
                     uint64_t step)
{
    int64_t m, nm = (int64_t)Bsz * H;
    int nlo = dk - nhi, i, j;
    int64_t rows = nm * nlo;
    float *St, *Sh, *vt, *ut, *wt, *U;
    double *ot;
    if (Bsz <= 0 || H <= 0 || dk <= 0 || dv != 128 || nhi < 0 || nhi > dk)
        return -1;
    St = (float *)malloc(sizeof(float) * (size_t)dk * dv);
    Sh = (float *)malloc(sizeof(float) * (size_t)dk * dv);
    vt = (float *)malloc(sizeof(float) * (size_t)dv);
    ut = (float *)malloc(sizeof(float) * (size_t)dv);
    wt = (float *)malloc(sizeof(float) * (size_t)dv);
    U = (float *)malloc(sizeof(float) * (size_t)dv);
    ot = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!St || !Sh || !vt || !ut || !wt || !U || !ot) {
        free(St); free(Sh); free(vt); free(ut); free(wt); free(U); free(ot);
        return -1;
    }
    for (m = 0; m < nm; ++m) {
        float al = alpha[m], be = beta[m];
        const float *km = k + m * dk, *qm = q + m * dk, *vm = v + m * dv;
        float *him = hi + m * (int64_t)nhi * dv;
        int32_t *cm = code + m * (int64_t)nlo * dv;
        float *sm = s + m * nlo, *zm = z + m * nlo;
        /* vt = Hs v: 128 multiples of 1/16 of floats, exact in double */
        for (j = 0; j < dv; ++j) {
            double a = 0.0;
            for (i = 0; i < dv; ++i)
                a += hs(j, i) * (double)vm[i];
            vt[j] = (float)a;
        }
        /* the stored matrix in fp32: half rows as they are, uint8 rows reconstructed,
         * fl(s*fl(c - z)) */
        for (i = 0; i < dk; ++i) {
            if (i < nhi)
                memcpy(Sh + (int64_t)i * dv, him + (int64_t)i * dv, sizeof(float) * (size_t)dv);
            else
                orc_dequantize_row(cm + (int64_t)(i - nhi) * dv, dv, sm[i - nhi], zm[i - nhi],
                                   Sh + (int64_t)i * dv);
        }
        /* ut = k^T St */
        for (j = 0; j < dv; ++j) {
            double a = 0.0;
            for (i = 0; i < dk; ++i)
                a += (double)km[i] * (double)Sh[(int64_t)i * dv + j];
            ut[j] = (float)a;
        }
        for (j = 0; j < dv; ++j) {
            float au = al * ut[j];
            float vmj = vt[j] - au;
            wt[j] = be * vmj;
        }
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j) {
                float kw = km[i] * wt[j];
                St[(int64_t)i * dv + j] = fmaf(al, Sh[(int64_t)i * dv + j], kw);
            }
        if (Spre)
            memcpy(Spre + m * (int64_t)dk * dv, St, sizeof(float) * (size_t)dk * dv);
        for (j = 0; j < dv; ++j)
            ot[j] = 0.0;
        if (readout_pre)
            for (i = 0; i < dk; ++i)
                for (j = 0; j < dv; ++j)
                    ot[j] += (double)qm[i] * (double)St[(int64_t)i * dv + j];
        for (i = 0; i < dk; ++i) {
            float *row = St + (int64_t)i * dv;
            if (i < nhi) {
                for (j = 0; j < dv; ++j) {
                    him[(int64_t)i * dv + j] = orc_round_half(row[j]);
                    row[j] = him[(int64_t)i * dv + j];
                }
            } else {
                int li = i - nhi;
                if (sr)
                    orc_sr_row_uniforms(seed, step, rows, m * nlo + li, dv, U);
                orc_quantize_row_sr(row, dv, 8, 1, cm + (int64_t)li * dv, sm + li, zm + li, NULL,
                                    sr ? U : NULL);
                orc_dequantize_row(cm + (int64_t)li * dv, dv, sm[li], zm[li], row);
            }
        }
        if (!readout_pre)
            for (i = 0; i < dk; ++i)
                for (j = 0; j < dv; ++j)
                    ot[j] += (double)qm[i] * (double)St[(int64_t)i * dv + j];
        /* o = 2 Hs ot */
        for (j = 0; j < dv; ++j) {
            double a = 0.0;
            for (i = 0; i < dv; ++i)
                a += hs(j, i) * ot[i];
            o[m * dv + j] = (float)(2.0 * a);
        }
    }
    free(St); free(Sh); free(vt); free(ut); free(wt); free(U); free(ot);
    return 0;
}

/* The two-tier state from an fp32 state S [Bsz][H][dk][dv] (original coordinates):
 * every row rotated, St = S Hs (double, rounded once), the first nhi rows of each
 * matrix rounded to half, the rest quantized (asymmetric int8, to nearest). */
int orc_damp_from_fp32(int Bsz, int H, int dk, int dv, int nhi, const float *S, float *hi,
                       int32_t *code, float *s, float *z)
{
    int64_t m, nm = (int64_t)Bsz * H;
    int nlo = dk - nhi, i, j, c;
    float *row = (float *)malloc(sizeof(float) * (size_t)dv);
    if (!row || dv != 128)
        return -1;
    for (m = 0; m < nm; ++m)
        for (i = 0; i < dk; ++i) {
            const float *src = S + (m * dk + i) * (int64_t)dv;
            for (j = 0; j < dv; ++j) {
                double a = 0.0;
                for (c = 0; c < dv; ++c)
                    a += (double)src[c] * hs(c, j);
                row[j] = (float)a;
            }
            if (i < nhi) {
                for (j = 0; j < dv; ++j)
                    hi[(m * nhi + i) * (int64_t)dv + j] = orc_round_half(row[j]);
            } else {
                int64_t li = m * nlo + (i - nhi);
                orc_quantize_row(row, dv, 8, 1, code + li * dv, s + li, z + li, NULL);
            }
        }
    free(row);
    return 0;
}
