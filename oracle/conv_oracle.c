/*
 * Convolution oracle: plain direct nested-loop cross-correlation in double
 * precision, and its two backward passes (input and weight gradients,
 * below the forward code).  TEST INFRASTRUCTURE ONLY -- the library never links,
 * loads or calls this file; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg do.
 *
 * What it computes (the plain definition the im2col + GEMM lowering must
 * reproduce up to summation order):
 *
 *   pre[n,od,oh,ow,g,k] = b[g,k] (if bias)
 *       + sum_{z<Z, y<Y, x<X, c<C}  x[n, id, ih, iw, g, c] * w[g, k, z, y, x, c]
 *   with id = od*sd - pd + z*dd, ih = oh*sh - ph + y*dh, iw = ow*sw - pw + x*dw,
 *   a term being left out when any of id, ih, iw lies outside [0, Di/Hi/Wi).
 *   out = GELU(pre) = 0.5 * pre * erfc(-pre / sqrt(2))  if gelu, else pre.
 *   Output extent per spatial dim: O = floor((I + 2p - d*(F-1) - 1) / s) + 1.
 *
 * Sources: the ExecuTorch issue "[ET-VK] conv1d runs at ~3% of the GPU's
 * matmul throughput" (sections "Describe the bug", "Suggested fix": conv1d
 * is nn.Conv2d with a singleton height, the aten.convolution semantics), and
 * the Composable Kernel note "Learnings -- Grouped-Conv Heuristic (Forward,
 * 2D + 3D)" (intro: layouts NHWGC x GKYXC -> NHWGK; section 2: 3-D problems
 * with per-dimension dilation).  The pages never print the formula; the one
 * above is the standard deep-learning (no kernel flip, symmetric zero
 * padding) definition those pages name.
 *
 * Layouts (channels innermost; 1-D and 2-D use D = 1 and H = 1):
 *   x : N x Di x Hi x Wi x G x C
 *   w : G x K x Z x Y x X x C
 *   b : G x K
 *   y : N x Do x Ho x Wo x G x K
 *
 * Nothing is rounded: inputs arrive as doubles (exact copies of the fp32 or
 * bf16 values the device sees), every product and sum is in double.
 * Built with -O2 -ffp-contract=off so no fused multiply-add changes a value.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

typedef struct {
    int64_t N, G, C, K;
    int64_t in[3];       /* Di, Hi, Wi */
    int64_t filt[3];     /* Z, Y, X */
    int64_t stride[3];
    int64_t pad[3];
    int64_t dil[3];
} oracle_desc;

static int64_t out_extent(int64_t I, int64_t F, int64_t s, int64_t p, int64_t d)
{
    int64_t span = I + 2 * p - d * (F - 1) - 1;
    if (span < 0) return 0;
    return span / s + 1;
}

/* Returns 0 and fills out[3] = (Do, Ho, Wo); returns -1 on a degenerate
 * descriptor (non-positive sizes or an empty output). */
int oracle_out_dims(const oracle_desc *d, int64_t out[3])
{
    if (d->N < 0 || d->G < 1 || d->C < 1 || d->K < 1) return -1;
    for (int i = 0; i < 3; ++i) {
        if (d->in[i] < 1 || d->filt[i] < 1 || d->stride[i] < 1 ||
            d->dil[i] < 1 || d->pad[i] < 0)
            return -1;
        out[i] = out_extent(d->in[i], d->filt[i], d->stride[i], d->pad[i], d->dil[i]);
        if (out[i] < 1) return -1;
    }
    return 0;
}

static double gelu_exact(double v)
{
    return 0.5 * v * erfc(-v / sqrt(2.0));
}

/* One output element (n, od, oh, ow, g, k).  Writes the pre- or
 * post-activation value to *yv and sum |b| + sum |x*w| to *ad. */
static void one_output(const oracle_desc *d, const int64_t o[3],
                       const double *x, const double *w, const double *b,
                       int gelu, int64_t n, int64_t od, int64_t oh, int64_t ow,
                       int64_t g, int64_t k, double *yv, double *ad)
{
    const int64_t Di = d->in[0], Hi = d->in[1], Wi = d->in[2];
    const int64_t Z = d->filt[0], Y = d->filt[1], X = d->filt[2];
    const int64_t G = d->G, C = d->C, K = d->K;
    double acc = 0.0, absacc = 0.0;
    (void)o;
    if (b) {
        acc = b[g * K + k];
        absacc = fabs(acc);
    }
    for (int64_t z = 0; z < Z; ++z) {
        int64_t id = od * d->stride[0] - d->pad[0] + z * d->dil[0];
        if (id < 0 || id >= Di) continue;
        for (int64_t y = 0; y < Y; ++y) {
            int64_t ih = oh * d->stride[1] - d->pad[1] + y * d->dil[1];
            if (ih < 0 || ih >= Hi) continue;
            for (int64_t xx = 0; xx < X; ++xx) {
                int64_t iw = ow * d->stride[2] - d->pad[2] + xx * d->dil[2];
                if (iw < 0 || iw >= Wi) continue;
                const double *xp = x + ((((n * Di + id) * Hi + ih) * Wi + iw) * G + g) * C;
                const double *wp = w + ((((g * K + k) * Z + z) * Y + y) * X + xx) * C;
                for (int64_t c = 0; c < C; ++c) {
                    double p = xp[c] * wp[c];
                    acc += p;
                    absacc += fabs(p);
                }
            }
        }
    }
    *yv = gelu ? gelu_exact(acc) : acc;
    *ad = absacc;
}

/* Full output.  y (and absdot, when not NULL) hold N*Do*Ho*Wo*G*K doubles.
 * b may be NULL (no bias).  Returns 0, or -1 on a degenerate descriptor. */
int oracle_conv_fwd(const oracle_desc *d, const double *x, const double *w,
                    const double *b, int gelu, double *y, double *absdot)
{
    int64_t o[3];
    if (oracle_out_dims(d, o) != 0) return -1;
    const int64_t G = d->G, K = d->K;
    const int64_t rows = d->N * o[0] * o[1];
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = r / (o[0] * o[1]);
        int64_t od = (r / o[1]) % o[0];
        int64_t oh = r % o[1];
        for (int64_t ow = 0; ow < o[2]; ++ow)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t k = 0; k < K; ++k) {
                    int64_t idx = ((((n * o[0] + od) * o[1] + oh) * o[2] + ow) * G + g) * K + k;
                    double yv, ad;
                    one_output(d, o, x, w, b, gelu, n, od, oh, ow, g, k, &yv, &ad);
                    y[idx] = yv;
                    if (absdot) absdot[idx] = ad;
                }
    }
    return 0;
}

/* Selected outputs: idx[i] is a flat index into the y layout above.
 * Returns 0, -1 on a degenerate descriptor, -2 on an index out of range. */
int oracle_conv_fwd_points(const oracle_desc *d, const double *x, const double *w,
                           const double *b, int gelu, int64_t npts,
                           const int64_t *idx, double *y, double *absdot)
{
    int64_t o[3];
    if (oracle_out_dims(d, o) != 0) return -1;
    const int64_t G = d->G, K = d->K;
    const int64_t total = d->N * o[0] * o[1] * o[2] * G * K;
    for (int64_t i = 0; i < npts; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -2;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t t = idx[i];
        int64_t k = t % K;  t /= K;
        int64_t g = t % G;  t /= G;
        int64_t ow = t % o[2]; t /= o[2];
        int64_t oh = t % o[1]; t /= o[1];
        int64_t od = t % o[0]; t /= o[0];
        int64_t n = t;
        double yv, ad;
        one_output(d, o, x, w, b, gelu, n, od, oh, ow, g, k, &yv, &ad);
        y[i] = yv;
        if (absdot) absdot[i] = ad;
    }
    return 0;
}

/* ---- Backward passes -----------------------------------------------------
 * The Composable Kernel note (section 6, "Backward Variants Not Yet
 * Upgraded") names the bf16 grouped backward-data and backward-weight
 * convolutions on gfx950 beside the forward one, in the same layouts.  Their
 * plain definitions are the two partial derivatives of the forward sum
 * above (no bias, no activation: the backward of the linear convolution):
 *
 *   dx[n,id,ih,iw,g,c] = sum over (z,y,x,k) and the output (od,oh,ow) with
 *        od*sd - pd + z*dd = id, oh*sh - ph + y*dh = ih, ow*sw - pw + x*dw = iw
 *        of  dy[n,od,oh,ow,g,k] * w[g,k,z,y,x,c]
 *   dw[g,k,z,y,x,c] = sum over (n,od,oh,ow) whose tap (z,y,x) lies inside
 *        the input of  dy[n,od,oh,ow,g,k] * x[n,id,ih,iw,g,c]
 *
 * dx has x's layout, dw has w's; absdot holds the matching sums of |terms|.
 */

/* Output coordinate that tap t of an output reads input coordinate i with,
 * or -1 when no output does (o*s - p + t*d = i has no solution in range). */
static int64_t out_of(int64_t i, int64_t t, int64_t s, int64_t p, int64_t d, int64_t O)
{
    int64_t num = i + p - t * d;
    if (num < 0 || num % s != 0) return -1;
    num /= s;
    return num < O ? num : -1;
}

static void one_dx(const oracle_desc *d, const int64_t o[3], const double *dy, const double *w,
                   int64_t n, int64_t id, int64_t ih, int64_t iw, int64_t g, int64_t c,
                   double *v, double *ad)
{
    const int64_t Z = d->filt[0], Y = d->filt[1], X = d->filt[2];
    const int64_t G = d->G, C = d->C, K = d->K;
    double acc = 0.0, absacc = 0.0;
    for (int64_t z = 0; z < Z; ++z) {
        int64_t od = out_of(id, z, d->stride[0], d->pad[0], d->dil[0], o[0]);
        if (od < 0) continue;
        for (int64_t y = 0; y < Y; ++y) {
            int64_t oh = out_of(ih, y, d->stride[1], d->pad[1], d->dil[1], o[1]);
            if (oh < 0) continue;
            for (int64_t xx = 0; xx < X; ++xx) {
                int64_t ow = out_of(iw, xx, d->stride[2], d->pad[2], d->dil[2], o[2]);
                if (ow < 0) continue;
                const double *dyp = dy + ((((n * o[0] + od) * o[1] + oh) * o[2] + ow) * G + g) * K;
                for (int64_t k = 0; k < K; ++k) {
                    double p = dyp[k] * w[((((g * K + k) * Z + z) * Y + y) * X + xx) * C + c];
                    acc += p;
                    absacc += fabs(p);
                }
            }
        }
    }
    *v = acc;
    *ad = absacc;
}

/* Full input gradient: dx (and absdot, when not NULL) hold N*Di*Hi*Wi*G*C
 * doubles.  Returns 0, or -1 on a degenerate descriptor. */
int oracle_conv_bwd_data(const oracle_desc *d, const double *dy, const double *w, double *dx, double *absdot)
{
    int64_t o[3];
    if (oracle_out_dims(d, o) != 0) return -1;
    const int64_t Di = d->in[0], Hi = d->in[1], Wi = d->in[2], G = d->G, C = d->C;
    const int64_t rows = d->N * Di * Hi;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = r / (Di * Hi), id = (r / Hi) % Di, ih = r % Hi;
        for (int64_t iw = 0; iw < Wi; ++iw)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t c = 0; c < C; ++c) {
                    int64_t idx = ((((n * Di + id) * Hi + ih) * Wi + iw) * G + g) * C + c;
                    double v, ad;
                    one_dx(d, o, dy, w, n, id, ih, iw, g, c, &v, &ad);
                    dx[idx] = v;
                    if (absdot) absdot[idx] = ad;
                }
    }
    return 0;
}

/* Selected input-gradient elements (flat indices into the x layout).
 * Returns 0, -1 on a degenerate descriptor, -2 on an index out of range. */
int oracle_conv_bwd_data_points(const oracle_desc *d, const double *dy, const double *w, int64_t npts,
                                const int64_t *idx, double *dx, double *absdot)
{
    int64_t o[3];
    if (oracle_out_dims(d, o) != 0) return -1;
    const int64_t Di = d->in[0], Hi = d->in[1], Wi = d->in[2], G = d->G, C = d->C;
    const int64_t total = d->N * Di * Hi * Wi * G * C;
    for (int64_t i = 0; i < npts; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -2;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t t = idx[i];
        int64_t c = t % C;  t /= C;
        int64_t g = t % G;  t /= G;
        int64_t iw = t % Wi; t /= Wi;
        int64_t ih = t % Hi; t /= Hi;
        int64_t id = t % Di; t /= Di;
        double v, ad;
        one_dx(d, o, dy, w, t, id, ih, iw, g, c, &v, &ad);
        dx[i] = v;
        if (absdot) absdot[i] = ad;
    }
    return 0;
}

static void one_dw(const oracle_desc *d, const int64_t o[3], const double *x, const double *dy,
                   int64_t g, int64_t k, int64_t z, int64_t y, int64_t xx, int64_t c, double *v, double *ad)
{
    const int64_t Di = d->in[0], Hi = d->in[1], Wi = d->in[2];
    const int64_t G = d->G, C = d->C, K = d->K;
    double acc = 0.0, absacc = 0.0;
    for (int64_t n = 0; n < d->N; ++n)
        for (int64_t od = 0; od < o[0]; ++od) {
            int64_t id = od * d->stride[0] - d->pad[0] + z * d->dil[0];
            if (id < 0 || id >= Di) continue;
            for (int64_t oh = 0; oh < o[1]; ++oh) {
                int64_t ih = oh * d->stride[1] - d->pad[1] + y * d->dil[1];
                if (ih < 0 || ih >= Hi) continue;
                for (int64_t ow = 0; ow < o[2]; ++ow) {
                    int64_t iw = ow * d->stride[2] - d->pad[2] + xx * d->dil[2];
                    if (iw < 0 || iw >= Wi) continue;
                    double p = dy[((((n * o[0] + od) * o[1] + oh) * o[2] + ow) * G + g) * K + k] *
                               x[((((n * Di + id) * Hi + ih) * Wi + iw) * G + g) * C + c];
                    acc += p;
                    absacc += fabs(p);
                }
            }
        }
    *v = acc;
    *ad = absacc;
}

/* Full weight gradient: dw (and absdot, when not NULL) hold G*K*Z*Y*X*C
 * doubles.  Returns 0, or -1 on a degenerate descriptor. */
int oracle_conv_bwd_weight(const oracle_desc *d, const double *x, const double *dy, double *dw, double *absdot)
{
    int64_t o[3];
    if (oracle_out_dims(d, o) != 0) return -1;
    const int64_t Z = d->filt[0], Y = d->filt[1], X = d->filt[2], C = d->C;
    const int64_t rows = d->G * d->K;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t g = r / d->K, k = r % d->K;
        for (int64_t z = 0; z < Z; ++z)
            for (int64_t y = 0; y < Y; ++y)
                for (int64_t xx = 0; xx < X; ++xx)
                    for (int64_t c = 0; c < C; ++c) {
                        int64_t idx = (((r * Z + z) * Y + y) * X + xx) * C + c;
                        double v, ad;
                        one_dw(d, o, x, dy, g, k, z, y, xx, c, &v, &ad);
                        dw[idx] = v;
                        if (absdot) absdot[idx] = ad;
                    }
    }
    return 0;
}

/* Selected weight-gradient elements (flat indices into the w layout).
 * Returns 0, -1 on a degenerate descriptor, -2 on an index out of range. */
int oracle_conv_bwd_weight_points(const oracle_desc *d, const double *x, const double *dy, int64_t npts,
                                  const int64_t *idx, double *dw, double *absdot)
{
    int64_t o[3];
    if (oracle_out_dims(d, o) != 0) return -1;
    const int64_t Z = d->filt[0], Y = d->filt[1], X = d->filt[2], C = d->C, K = d->K;
    const int64_t total = d->G * K * Z * Y * X * C;
    for (int64_t i = 0; i < npts; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -2;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t t = idx[i];
        int64_t c = t % C;  t /= C;
        int64_t xx = t % X; t /= X;
        int64_t y = t % Y;  t /= Y;
        int64_t z = t % Z;  t /= Z;
        int64_t k = t % K;  t /= K;
        double v, ad;
        one_dw(d, o, x, dy, t, k, z, y, xx, c, &v, &ad);
        dw[i] = v;
        if (absdot) absdot[i] = ad;
    }
    return 0;
}

/* Threads the OpenMP runtime will use (reported beside the CPU timing). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
