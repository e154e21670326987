/*
 * conv2d_oracle.c -- plain fp64 CPU oracle for NHWC conv2d (fprop / dgrad / wgrad).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct definition
 * that the HIP library is checked against.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it.  It shares no source,
 * header, table or helper with the library under convolution_nhwc_implicit_amd/.
 *
 * What it computes (deep-learning convolution = cross-correlation, no filter flip):
 *   "Declaring and running a Conv2d Fprop" in the CUTLASS Python Conv2d notebook
 *   checks fprop against aten.conv2d; "Declaring and running Conv2d Dgrad and
 *   Wgrad" checks the two gradients against torch.nn.grad.conv2d_input /
 *   conv2d_weight.  Those three operations are written out here by their
 *   definitions, one output element at a time, in double precision.
 *
 * Layouts (the notebook's "General setup" declares channel-last tensors):
 *   x, dx  [N][H][W][C]          w, dw  [K][R][S][C/G]
 *   y, dy  [N][P][Q][K]          bias   [K]
 * Groups: output channel k belongs to group g = k / (K/G) and reads input
 * channels [g*C/G, (g+1)*C/G)  (contiguous channel blocks).
 *
 * Problem vector `d` (14 ints):
 *   d[0]=N d[1]=C d[2]=H d[3]=W d[4]=K d[5]=R d[6]=S
 *   d[7]=pad_h d[8]=pad_w d[9]=stride_h d[10]=stride_w d[11]=dil_h d[12]=dil_w d[13]=G
 *
 * Every function is deterministic; the OpenMP loops only split independent
 * output elements across threads, and each element is summed in a fixed order.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Output size.                                                              */
/* The tensorcore Conv2D page ("Surface") gives out = floor((H + 2p - kH)/s) + 1 */
/* for dilation 1.  With dilation d the filter spans d*(kH-1)+1 input rows,   */
/* which is what CUTLASS's Conv2d.output_size takes in ("General setup").     */
/* Returns -1 when the padded input is shorter than the dilated filter.      */
/* ------------------------------------------------------------------------ */
int oracle_out_size(int in, int pad, int k, int stride, int dil)
{
    long span = (long)dil * (k - 1) + 1;
    long padded = (long)in + 2L * pad;
    if (in <= 0 || k <= 0 || stride <= 0 || dil <= 0 || pad < 0) return -1;
    if (padded < span) return -1;
    /* both operands are non-negative here, so C division is floor division */
    return (int)((padded - span) / stride + 1);
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

typedef struct {
    long N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, G, P, Q, Cg, Kg;
} prob_t;

static int load_prob(const int *d, prob_t *p)
{
    p->N = d[0]; p->C = d[1]; p->H = d[2]; p->W = d[3]; p->K = d[4];
    p->R = d[5]; p->S = d[6]; p->ph = d[7]; p->pw = d[8];
    p->sh = d[9]; p->sw = d[10]; p->dh = d[11]; p->dw = d[12]; p->G = d[13];
    if (p->G <= 0 || p->C % p->G || p->K % p->G) return -1;
    p->P = oracle_out_size(d[2], d[7], d[5], d[9], d[11]);
    p->Q = oracle_out_size(d[3], d[8], d[6], d[10], d[12]);
    if (p->P < 1 || p->Q < 1 || p->N < 1 || p->C < 1 || p->K < 1) return -1;
    p->Cg = p->C / p->G;
    p->Kg = p->K / p->G;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* fprop, one element:                                                       */
/*   y[n,p,q,k] = sum_{r,s,c'} x[n, p*sh - ph + r*dh, q*sw - pw + s*dw,      */
/*                              g*Cg + c'] * w[k,r,s,c']                     */
/* with taps outside the input counted as zero (zero padding).               */
/* ------------------------------------------------------------------------ */
static double fprop_at(const prob_t *p, const double *x, const double *w,
                       long n, long oh, long ow, long k)
{
    long g = k / p->Kg;
    double acc = 0.0;
    for (long r = 0; r < p->R; ++r) {
        long h = oh * p->sh - p->ph + r * p->dh;
        if (h < 0 || h >= p->H) continue;
        for (long s = 0; s < p->S; ++s) {
            long wc = ow * p->sw - p->pw + s * p->dw;
            if (wc < 0 || wc >= p->W) continue;
            const double *xp = x + ((n * p->H + h) * p->W + wc) * p->C + g * p->Cg;
            const double *wp = w + ((k * p->R + r) * p->S + s) * p->Cg;
            for (long c = 0; c < p->Cg; ++c) acc += xp[c] * wp[c];
        }
    }
    return acc;
}

/* ------------------------------------------------------------------------ */
/* dgrad, one element: the adjoint of x -> fprop(x, w) applied to dy.        */
/* Input row h is read by output row p through tap r exactly when            */
/* p*sh - ph + r*dh == h, i.e. when (h + ph - r*dh) is a non-negative        */
/* multiple of sh whose quotient is a valid output row (same for columns).   */
/* ------------------------------------------------------------------------ */
static double dgrad_at(const prob_t *p, const double *dy, const double *w,
                       long n, long h, long wc, long c)
{
    long g = c / p->Cg, cl = c - g * p->Cg;
    double acc = 0.0;
    for (long r = 0; r < p->R; ++r) {
        long th = h + p->ph - r * p->dh;
        if (th < 0 || th % p->sh) continue;
        long oh = th / p->sh;
        if (oh >= p->P) continue;
        for (long s = 0; s < p->S; ++s) {
            long tw = wc + p->pw - s * p->dw;
            if (tw < 0 || tw % p->sw) continue;
            long ow = tw / p->sw;
            if (ow >= p->Q) continue;
            const double *dyp = dy + ((n * p->P + oh) * p->Q + ow) * p->K;
            for (long kl = 0; kl < p->Kg; ++kl) {
                long k = g * p->Kg + kl;
                acc += dyp[k] * w[((k * p->R + r) * p->S + s) * p->Cg + cl];
            }
        }
    }
    return acc;
}

/* ------------------------------------------------------------------------ */
/* wgrad, one element: the adjoint with respect to w,                        */
/*   dw[k,r,s,c'] = sum_{n,p,q} dy[n,p,q,k] * x[n, p*sh-ph+r*dh,             */
/*                                             q*sw-pw+s*dw, g*Cg+c']        */
/* The sum runs over every output pixel (the GEMM-K of N*P*Q that the TVM     */
/* wgrad pull request calls very large).                                     */
/* ------------------------------------------------------------------------ */
static double wgrad_at(const prob_t *p, const double *x, const double *dy,
                       long k, long r, long s, long cl)
{
    long g = k / p->Kg;
    long c = g * p->Cg + cl;
    double acc = 0.0;
    for (long n = 0; n < p->N; ++n)
        for (long oh = 0; oh < p->P; ++oh) {
            long h = oh * p->sh - p->ph + r * p->dh;
            if (h < 0 || h >= p->H) continue;
            for (long ow = 0; ow < p->Q; ++ow) {
                long wc = ow * p->sw - p->pw + s * p->dw;
                if (wc < 0 || wc >= p->W) continue;
                acc += dy[((n * p->P + oh) * p->Q + ow) * p->K + k] *
                       x[((n * p->H + h) * p->W + wc) * p->C + c];
            }
        }
    return acc;
}

/* ------------------------------------------------------------------------ */
/* Linear-combination epilogue of the CUTLASS Python notebook: every pass it  */
/* runs (fprop "Run the Conv2d", dgrad and wgrad) produces                   */
/* D = alpha * conv + beta * C for a source tensor C of the output's shape.  */
/* With a bias and ReLU (fprop) the bias is added to that sum and ReLU comes */
/* last, as in the plain epilogue below (conv, bias, ReLU).  r holds the     */
/* pass's exact result, out[i] = relu(alpha*r[i] + beta*c[i] + bias[i % K]). */
/* ------------------------------------------------------------------------ */
void oracle_linear_combination(const double *r, const double *c, long count, long K, double alpha,
                               double beta, const double *bias, int relu, double *out)
{
    for (long i = 0; i < count; ++i) {
        double v = alpha * r[i];
        if (c) v += beta * c[i];
        if (bias) v += bias[i % K];
        if (relu && !(v > 0.0)) v = 0.0;
        out[i] = v;
    }
}

/* ------------------------------------------------------------------------ */
/* Epilogue of the float paths: + bias, then ReLU.  The order (conv, bias,    */
/* ReLU) is the one the quantized cuDNN conv builds in its op graph          */
/* (apply_impl_helper, "kReluFused" page).  ReLU maps every v <= 0 to +0.    */
/* ------------------------------------------------------------------------ */
static double bias_relu(double v, const double *bias, long k, int relu)
{
    if (bias) v += bias[k];
    if (relu && !(v > 0.0)) v = 0.0;
    return v;
}

/* Full tensors.  All return 0 on success, -1 on an invalid problem. */
int oracle_fprop(const int *d, const double *x, const double *w, const double *bias,
                 int relu, double *y)
{
    prob_t p;
    if (load_prob(d, &p)) return -1;
    long total = p.N * p.P * p.Q;
#pragma omp parallel for schedule(dynamic, 16)
    for (long pix = 0; pix < total; ++pix) {
        long n = pix / (p.P * p.Q), rem = pix % (p.P * p.Q);
        long oh = rem / p.Q, ow = rem % p.Q;
        for (long k = 0; k < p.K; ++k)
            y[pix * p.K + k] = bias_relu(fprop_at(&p, x, w, n, oh, ow, k), bias, k, relu);
    }
    return 0;
}

int oracle_dgrad(const int *d, const double *dy, const double *w, double *dx)
{
    prob_t p;
    if (load_prob(d, &p)) return -1;
    long total = p.N * p.H * p.W;
#pragma omp parallel for schedule(dynamic, 16)
    for (long pix = 0; pix < total; ++pix) {
        long n = pix / (p.H * p.W), rem = pix % (p.H * p.W);
        long h = rem / p.W, wc = rem % p.W;
        for (long c = 0; c < p.C; ++c)
            dx[pix * p.C + c] = dgrad_at(&p, dy, w, n, h, wc, c);
    }
    return 0;
}

int oracle_wgrad(const int *d, const double *x, const double *dy, double *dw)
{
    prob_t p;
    if (load_prob(d, &p)) return -1;
    long total = p.K * p.R * p.S * p.Cg;
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < total; ++i) {
        long cl = i % p.Cg, t = i / p.Cg;
        long s = t % p.S; t /= p.S;
        long r = t % p.R, k = t / p.R;
        dw[i] = wgrad_at(&p, x, dy, k, r, s, cl);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Bias gradient.  fprop adds bias[k] to every output pixel of channel k     */
/* (the tensorcore Conv2D page, forward algorithm, step 3), so the gradient  */
/* with respect to the bias is the adjoint of that broadcast:                */
/* db[k] = sum over all n, p, q of dy[n,p,q,k].  One fp64 sum per channel,   */
/* pixels in ascending order.                                                */
/* ------------------------------------------------------------------------ */
int oracle_bias_grad(const int *d, const double *dy, double *db)
{
    prob_t p;
    if (load_prob(d, &p)) return -1;
    long total = p.N * p.P * p.Q;
#pragma omp parallel for schedule(static)
    for (long k = 0; k < p.K; ++k) {
        double acc = 0.0;
        for (long pix = 0; pix < total; ++pix) acc += dy[pix * p.K + k];
        db[k] = acc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sampled outputs: idx holds `count` flat output indices (row-major in the  */
/* output layout); out[i] receives the value at idx[i].  Used to check       */
/* full-size problems at a sample of points.                                 */
/* ------------------------------------------------------------------------ */
int oracle_fprop_sampled(const int *d, const double *x, const double *w, const double *bias,
                         int relu, const int64_t *idx, long count, double *out)
{
    prob_t p;
    if (load_prob(d, &p)) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (long i = 0; i < count; ++i) {
        long e = (long)idx[i];
        long k = e % p.K, pix = e / p.K;
        long ow = pix % p.Q, t = pix / p.Q;
        long oh = t % p.P, n = t / p.P;
        out[i] = bias_relu(fprop_at(&p, x, w, n, oh, ow, k), bias, k, relu);
    }
    return 0;
}

int oracle_dgrad_sampled(const int *d, const double *dy, const double *w,
                         const int64_t *idx, long count, double *out)
{
    prob_t p;
    if (load_prob(d, &p)) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (long i = 0; i < count; ++i) {
        long e = (long)idx[i];
        long c = e % p.C, pix = e / p.C;
        long wc = pix % p.W, t = pix / p.W;
        long h = t % p.H, n = t / p.H;
        out[i] = dgrad_at(&p, dy, w, n, h, wc, c);
    }
    return 0;
}

int oracle_wgrad_sampled(const int *d, const double *x, const double *dy,
                         const int64_t *idx, long count, double *out)
{
    prob_t p;
    if (load_prob(d, &p)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < count; ++i) {
        long e = (long)idx[i];
        long cl = e % p.Cg, t = e / p.Cg;
        long s = t % p.S; t /= p.S;
        long r = t % p.R, k = t / p.R;
        out[i] = wgrad_at(&p, x, dy, k, r, s, cl);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* int8 requantisation, after the quantized cuDNN conv's op graph            */
/* (apply_impl_helper on the "kReluFused" page): the integer conv result     */
/* plus the int32 bias (already in accumulator units), then ReLU when fused, */
/* then multiplication by the requantize multiplier act*w/out, which that    */
/* code forms in double precision.  The product is rounded half-to-even and  */
/* saturated to int8 ([0,127] after ReLU follows from the clamp).            */
/* acc holds exact integers (fp64 represents them exactly below 2^53).       */
/* ------------------------------------------------------------------------ */
double oracle_requant_multiplier(double act_scale, double w_scale, double out_scale)
{
    return act_scale * w_scale / out_scale;
}

static int8_t requant_one(double v, double m)
{
    double t = v * m;
    double q = nearbyint(t); /* default rounding mode: to nearest, ties to even */
    if (q > 127.0) q = 127.0;
    if (q < -128.0) q = -128.0;
    return (int8_t)q;
}

/* acc[count] are conv sums for flat output indices idx (NULL = 0..count-1). */
void oracle_requant(const double *acc, const int64_t *idx, long count, long K,
                    const int32_t *bias, int relu, double multiplier, int8_t *out)
{
    for (long i = 0; i < count; ++i) {
        long e = idx ? (long)idx[i] : i;
        double v = acc[i];
        if (bias) v += (double)bias[e % K];
        if (relu && v < 0.0) v = 0.0;
        out[i] = requant_one(v, multiplier);
    }
}

/* ------------------------------------------------------------------------ */
/* One rounding of an fp64 result to the output type: IEEE binary16 or       */
/* bfloat16, round to nearest with ties to even, overflow to +-Inf.  Written  */
/* from the format definitions: scale |v| by an exact power of two so the    */
/* representable neighbours are consecutive integers, round with             */
/* nearbyint, then pack sign / exponent / mantissa.                          */
/* ------------------------------------------------------------------------ */
static uint16_t round_to_small_float(double v, int mant_bits, int exp_bias, int exp_max_field)
{
    uint16_t sign = signbit(v) ? (uint16_t)(1u << 15) : 0;
    double a = fabs(v);
    uint16_t inf = (uint16_t)(exp_max_field << mant_bits);
    if (isnan(v)) return (uint16_t)(sign | inf | (1u << (mant_bits - 1)));
    if (isinf(v)) return (uint16_t)(sign | inf);
    int emin = 1 - exp_bias; /* exponent of the smallest normal */
    if (a < ldexp(1.0, emin)) {
        /* subnormal range: quantum 2^(emin - mant_bits) */
        double m = nearbyint(ldexp(a, mant_bits - emin));
        /* m == 2^mant_bits lands exactly on the smallest normal, whose field
           value is the same integer */
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;         /* a in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(a, mant_bits - e)); /* in [2^mb, 2^(mb+1)] */
    if (m >= ldexp(1.0, mant_bits + 1)) { m = ldexp(m, -1); e += 1; }
    int field = e + exp_bias;
    if (field >= exp_max_field) return (uint16_t)(sign | inf);
    return (uint16_t)(sign | (uint16_t)(field << mant_bits) |
                      (uint16_t)((long)m - (1L << mant_bits)));
}

void oracle_round_f16(const double *v, long count, uint16_t *out)
{
    for (long i = 0; i < count; ++i) out[i] = round_to_small_float(v[i], 10, 15, 31);
}

void oracle_round_bf16(const double *v, long count, uint16_t *out)
{
    for (long i = 0; i < count; ++i) out[i] = round_to_small_float(v[i], 7, 127, 255);
}
