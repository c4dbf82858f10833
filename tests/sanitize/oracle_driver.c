/*
 * Runs every entry point of the fp64 convolution oracle (oracle/conv_oracle.c)
 * on a grid of small problems -- 1-D, 2-D and 3-D, strides, padding wider
 * than the filter, dilation, groups -- with every buffer allocated at its
 * exact size, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer reports any read or write outside a tensor and
 * any undefined integer or pointer arithmetic.  Prints one checksum line per
 * problem and "oracle sanitize ok" at the end.  Test infrastructure only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    int64_t N, G, C, K;
    int64_t in[3], filt[3], stride[3], pad[3], dil[3];
} oracle_desc;

int oracle_out_dims(const oracle_desc *d, int64_t out[3]);
int oracle_conv_fwd(const oracle_desc *d, const double *x, const double *w, const double *b, int gelu, double *y,
                    double *absdot);
int oracle_conv_fwd_points(const oracle_desc *d, const double *x, const double *w, const double *b, int gelu,
                           int64_t npts, const int64_t *idx, double *y, double *absdot);
int oracle_conv_bwd_data(const oracle_desc *d, const double *dy, const double *w, double *dx, double *absdot);
int oracle_conv_bwd_data_points(const oracle_desc *d, const double *dy, const double *w, int64_t npts,
                                const int64_t *idx, double *v, double *absdot);
int oracle_conv_bwd_weight(const oracle_desc *d, const double *x, const double *dy, double *dw, double *absdot);
int oracle_conv_bwd_weight_points(const oracle_desc *d, const double *x, const double *dy, int64_t npts,
                                  const int64_t *idx, double *v, double *absdot);

static uint64_t state = 12345;
static double rnd(void)
{
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(int64_t)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *fill(int64_t n)
{
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}

static double sum(const double *p, int64_t n)
{
    double s = 0;
    for (int64_t i = 0; i < n; ++i) s += p[i];
    return s;
}

static int run(const oracle_desc *d)
{
    int64_t o[3];
    if (oracle_out_dims(d, o) != 0) return 0;   /* degenerate: nothing to run */
    const int64_t taps = d->filt[0] * d->filt[1] * d->filt[2];
    const int64_t nx = d->N * d->in[0] * d->in[1] * d->in[2] * d->G * d->C;
    const int64_t nw = d->G * d->K * taps * d->C;
    const int64_t ny = d->N * o[0] * o[1] * o[2] * d->G * d->K;
    double *x = fill(nx), *w = fill(nw), *b = fill(d->G * d->K), *dy = fill(ny);
    double *y = fill(ny), *ad = fill(ny), *dx = fill(nx), *adx = fill(nx), *dw = fill(nw), *adw = fill(nw);
    int rc = 0;
    rc |= oracle_conv_fwd(d, x, w, b, 1, y, ad);
    rc |= oracle_conv_fwd(d, x, w, NULL, 0, y, NULL);
    rc |= oracle_conv_bwd_data(d, dy, w, dx, adx);
    rc |= oracle_conv_bwd_weight(d, x, dy, dw, adw);
    /* every element through the point entry points, last first */
    int64_t nmax = ny > nx ? ny : nx;
    nmax = nmax > nw ? nmax : nw;
    int64_t *idx = (int64_t *)malloc((size_t)nmax * sizeof(int64_t));
    double *pv = fill(nmax), *pa = fill(nmax);
    for (int64_t i = 0; i < ny; ++i) idx[i] = ny - 1 - i;
    rc |= oracle_conv_fwd_points(d, x, w, b, 1, ny, idx, pv, pa);
    for (int64_t i = 0; i < nx; ++i) idx[i] = nx - 1 - i;
    rc |= oracle_conv_bwd_data_points(d, dy, w, nx, idx, pv, pa);
    for (int64_t i = 0; i < nw; ++i) idx[i] = nw - 1 - i;
    rc |= oracle_conv_bwd_weight_points(d, x, dy, nw, idx, pv, pa);
    /* an index past the end is refused, not read */
    idx[0] = ny;
    if (oracle_conv_fwd_points(d, x, w, b, 0, 1, idx, pv, pa) != -2) rc |= 1;
    printf("out %lld %lld %lld  sums %.6g %.6g %.6g\n", (long long)o[0], (long long)o[1], (long long)o[2],
           sum(y, ny), sum(dx, nx), sum(dw, nw));
    free(x); free(w); free(b); free(dy); free(y); free(ad); free(dx); free(adx); free(dw); free(adw);
    free(idx); free(pv); free(pa);
    return rc;
}

int main(void)
{
    int rc = 0, count = 0;
    static const int64_t I[] = {1, 4, 7};
    static const int64_t F[] = {1, 2, 3};
    for (int dim = 0; dim < 3; ++dim)
        for (int a = 0; a < 3; ++a)
            for (int f = 0; f < 3; ++f)
                for (int64_t s = 1; s <= 3; s += 2)
                    for (int64_t p = 0; p <= 3; p += 3)
                        for (int64_t dl = 1; dl <= 2; ++dl) {
                            oracle_desc d = {2, 2, 3, 2, {1, 1, 1}, {1, 1, 1}, {1, 1, 1}, {0, 0, 0}, {1, 1, 1}};
                            for (int k = 2 - dim; k < 3; ++k) {   /* the used spatial dims */
                                d.in[k] = I[(a + k) % 3];
                                d.filt[k] = F[(f + k) % 3];
                                d.stride[k] = s;
                                d.pad[k] = p;
                                d.dil[k] = dl;
                            }
                            rc |= run(&d);
                            ++count;
                        }
    /* a degenerate descriptor is refused */
    oracle_desc bad = {1, 1, 1, 1, {1, 1, 2}, {1, 1, 5}, {1, 1, 1}, {0, 0, 0}, {1, 1, 1}};
    int64_t o[3];
    if (oracle_out_dims(&bad, o) != -1) rc |= 1;
    double one = 1.0;
    if (oracle_conv_fwd(&bad, &one, &one, NULL, 0, &one, NULL) != -1) rc |= 1;
    printf("%d problems; oracle sanitize %s\n", count, rc ? "FAILED" : "ok");
    return rc ? 1 : 0;
}
