/*
 * cc3d_oracle.c -- plain, slow, fp64 reference for the causal 3-D convolution
 * of a chunked video-decoder stack.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the GPU library; the GPU path never calls it.
 *
 * What it computes (the definition, written out with no blocking or fusion):
 *
 *   Y[o,t,h,w] = B[o] + sum_c sum_a sum_b sum_d
 *                  Wt[o,c,a,b,d] * Xp[c, t+a, h+b-ph, w+d-pw]
 *
 *   Xp is the already temporally padded input sequence (the caller prepends the
 *   k_t-1 history frames; see oracle.py), ph=(k_h-1)/2, pw=(k_w-1)/2, and a
 *   spatial index outside the image reads 0.  The tap a = k_t-1 is the current
 *   frame, so output frame t sees padded frames t..t+k_t-1 only: causal.
 *   This is the cross-correlation convention of PyTorch's conv3d that the
 *   SwiftVR page's decoder runs on ("Experimental Setup and Validation": PyTorch
 *   and cuDNN); the MemoryBlock of that page ("ReAE: Causal Halo Exchange") is
 *   the k_t = 2 case: (current, previous) input pairs.
 *
 * With strides (a strided conv, as an encoder that reduces the frame rate and
 * the frame size takes it; the SwiftVR page, "ReAE: Causal Halo Exchange", puts
 * the ReAE encoder under the same causal-state rule as the decoder), output
 * (t, h, w) reads padded frame t0 + st*t + a and pixel (ss*h + b - ph,
 * ss*w + d - pw): the same sum taken at every st-th frame from t0 and every
 * ss-th pixel, the PyTorch conv3d convention for stride and padding.
 *
 * Three entry points:
 *   cc3d_oracle_conv_valid   -- every output of the definition above, fp64
 *   cc3d_oracle_conv_strided -- the same with strides and a first frame t0
 *   cc3d_oracle_conv_points  -- the same sum at a list of output positions, with
 *                               an optional nearest spatial upsample of the input
 *                               ("TemporalGrow: Compute Before Spatial
 *                               Upsampling": nearest upsampling copies each
 *                               position to four outputs), reading a float32
 *                               input of any strides, or a spatial stride.  Used
 *                               for sampled checks of full-size layers.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double* xp;
    const double* wt;
    const double* bias;
    double* y;
    int cin, tp, h, w, cout, kt, kh, kw;
    int t0, st, ss;             /* first padded frame, temporal and spatial stride */
    int t_out, h_out, w_out;
    int64_t row_begin, row_end; /* rows = (o, t, h) triples of the output */
} valid_job;

static void* valid_worker(void* arg)
{
    valid_job* j = (valid_job*)arg;
    const int ph = (j->kh - 1) / 2, pw = (j->kw - 1) / 2;
    const int64_t plane = (int64_t)j->h * j->w;
    for (int64_t r = j->row_begin; r < j->row_end; ++r) {
        const int hh = (int)(r % j->h_out);
        const int t = (int)((r / j->h_out) % j->t_out);
        const int o = (int)(r / ((int64_t)j->h_out * j->t_out));
        const int tz = j->t0 + j->st * t; /* first padded frame of the window */
        for (int ww = 0; ww < j->w_out; ++ww) {
            double s = j->bias ? j->bias[o] : 0.0;
            for (int c = 0; c < j->cin; ++c)
                for (int a = 0; a < j->kt; ++a)
                    for (int b = 0; b < j->kh; ++b) {
                        const int ih = j->ss * hh + b - ph;
                        if (ih < 0 || ih >= j->h) continue;
                        for (int d = 0; d < j->kw; ++d) {
                            const int iw = j->ss * ww + d - pw;
                            if (iw < 0 || iw >= j->w) continue;
                            const double wv =
                                j->wt[((((int64_t)o * j->cin + c) * j->kt + a) * j->kh + b) * j->kw + d];
                            const double xv =
                                j->xp[((int64_t)c * j->tp + (tz + a)) * plane + (int64_t)ih * j->w + iw];
                            s += wv * xv;
                        }
                    }
            j->y[(((int64_t)o * j->t_out + t) * j->h_out + hh) * j->w_out + ww] = s;
        }
    }
    return NULL;
}

/*
 * xp   : [cin][tp][h][w] fp64, the padded sequence (tp >= t0 + kt)
 * wt   : [cout][cin][kt][kh][kw] fp64 (PyTorch weight order)
 * bias : [cout] fp64 or NULL (reads as 0)
 * t0, st, ss : first padded frame of output 0 (>= 0), temporal stride and
 *        spatial stride (>= 1)
 * y    : [cout][t_out][h_out][w_out] fp64, written, with
 *        t_out = (tp - kt - t0) / st + 1, h_out = (h - 1) / ss + 1,
 *        w_out = (w - 1) / ss + 1 (integer division)
 * Returns 0, or -1 on a bad argument (nothing written).
 */
int cc3d_oracle_conv_strided(const double* xp, int cin, int tp, int h, int w,
                             const double* wt, int cout, int kt, int kh, int kw,
                             const double* bias, int t0, int st, int ss, double* y, int nthreads)
{
    if (!xp || !wt || !y || cin <= 0 || cout <= 0 || h <= 0 || w <= 0 || kt <= 0 ||
        kh <= 0 || kw <= 0 || (kh % 2) == 0 || (kw % 2) == 0 || t0 < 0 || st < 1 || ss < 1 ||
        tp < t0 + kt)
        return -1;
    const int t_out = (tp - kt - t0) / st + 1;
    const int h_out = (h - 1) / ss + 1, w_out = (w - 1) / ss + 1;
    const int64_t rows = (int64_t)cout * t_out * h_out;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > rows) nthreads = (int)rows;
    pthread_t th[256];
    valid_job jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        valid_job* j = &jobs[i];
        j->xp = xp; j->wt = wt; j->bias = bias; j->y = y;
        j->cin = cin; j->tp = tp; j->h = h; j->w = w; j->cout = cout;
        j->kt = kt; j->kh = kh; j->kw = kw;
        j->t0 = t0; j->st = st; j->ss = ss;
        j->t_out = t_out; j->h_out = h_out; j->w_out = w_out;
        j->row_begin = rows * i / nthreads;
        j->row_end = rows * (i + 1) / nthreads;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, valid_worker, &jobs[i]) != 0) break;
        started = i;
    }
    valid_worker(&jobs[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    /* rows the failed threads would have done */
    for (int i = started + 1; i < nthreads; ++i) valid_worker(&jobs[i]);
    return 0;
}

/* The definition without strides: y is [cout][tp-kt+1][h][w]. */
int cc3d_oracle_conv_valid(const double* xp, int cin, int tp, int h, int w,
                           const double* wt, int cout, int kt, int kh, int kw,
                           const double* bias, double* y, int nthreads)
{
    return cc3d_oracle_conv_strided(xp, cin, tp, h, w, wt, cout, kt, kh, kw, bias, 0, 1, 1, y, nthreads);
}

typedef struct {
    const float* z;
    int64_t sc, st, sh, sw;
    int cin, tz, hin, win, up, down;
    const double* wt;
    const double* bias;
    int cout, kt, kh, kw;
    const int32_t* pts;
    double* out;
    int64_t begin, end;
} points_job;

static void* points_worker(void* arg)
{
    points_job* j = (points_job*)arg;
    const int ph = (j->kh - 1) / 2, pw = (j->kw - 1) / 2;
    const int hu = j->hin * j->up, wu = j->win * j->up; /* upsampled size */
    const int ds = j->down;
    for (int64_t p = j->begin; p < j->end; ++p) {
        const int t = j->pts[3 * p + 0], yy = j->pts[3 * p + 1], xx = j->pts[3 * p + 2];
        for (int o = 0; o < j->cout; ++o) {
            double s = j->bias ? j->bias[o] : 0.0;
            for (int c = 0; c < j->cin; ++c)
                for (int a = 0; a < j->kt; ++a)
                    for (int b = 0; b < j->kh; ++b) {
                        const int uh = ds * yy + b - ph;     /* row of the upsampled image */
                        if (uh < 0 || uh >= hu) continue;
                        const int ih = uh / j->up;           /* nearest: floor(h / s) */
                        for (int d = 0; d < j->kw; ++d) {
                            const int uw = ds * xx + d - pw;
                            if (uw < 0 || uw >= wu) continue;
                            const int iw = uw / j->up;
                            const double wv =
                                j->wt[((((int64_t)o * j->cin + c) * j->kt + a) * j->kh + b) * j->kw + d];
                            const double xv = (double)j->z[c * j->sc + (int64_t)(t + a) * j->st +
                                                           ih * j->sh + iw * j->sw];
                            s += wv * xv;
                        }
                    }
            j->out[p * j->cout + o] = s;
        }
    }
    return NULL;
}

/*
 * z      : float32 padded input sequence Z[c][tau][h][w] addressed with element
 *          strides (sc, st, sh, sw); tau in [0, tz), h < hin, w < win
 * up     : nearest spatial upsample factor applied to Z before the conv (1 or 2)
 * down   : spatial stride of the conv (1 or 2; not with up = 2): output (y, x)
 *          is centred on pixel (down*y, down*x)
 * pts    : npts x (t, y, x) output positions, t the window's first frame of Z;
 *          down*y < hin*up, down*x < win*up, t + kt - 1 < tz
 * out    : npts x cout fp64, written
 * Returns 0, or -1 on a bad argument (nothing written).
 */
int cc3d_oracle_conv_points(const float* z, int64_t sc, int64_t st, int64_t sh, int64_t sw,
                            int cin, int tz, int hin, int win, int up, int down,
                            const double* wt, int cout, int kt, int kh, int kw,
                            const double* bias, const int32_t* pts, int64_t npts,
                            double* out, int nthreads)
{
    if (!z || !wt || !pts || !out || cin <= 0 || cout <= 0 || up < 1 || down < 1 || kt <= 0 ||
        (kh % 2) == 0 || (kw % 2) == 0 || npts < 0)
        return -1;
    for (int64_t p = 0; p < npts; ++p) {
        const int t = pts[3 * p], yy = pts[3 * p + 1], xx = pts[3 * p + 2];
        if (t < 0 || t + kt > tz || yy < 0 || down * yy >= hin * up || xx < 0 || down * xx >= win * up)
            return -1;
    }
    if (npts == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > npts) nthreads = (int)npts;
    pthread_t th[256];
    points_job jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        points_job* j = &jobs[i];
        j->z = z; j->sc = sc; j->st = st; j->sh = sh; j->sw = sw;
        j->cin = cin; j->tz = tz; j->hin = hin; j->win = win; j->up = up; j->down = down;
        j->wt = wt; j->bias = bias; j->cout = cout; j->kt = kt; j->kh = kh; j->kw = kw;
        j->pts = pts; j->out = out;
        j->begin = npts * i / nthreads;
        j->end = npts * (i + 1) / nthreads;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, points_worker, &jobs[i]) != 0) break;
        started = i;
    }
    points_worker(&jobs[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    for (int i = started + 1; i < nthreads; ++i) points_worker(&jobs[i]);
    return 0;
}
