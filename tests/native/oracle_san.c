/* Host program for the sanitizer tier: runs every oracle entry point on
 * small shapes (1-D and 2-D, stride, padding, output_padding, dilation,
 * groups, empty batches, the iSTFT pieces, the per-point evaluators) and
 * checks a few identities, so that AddressSanitizer and
 * UndefinedBehaviorSanitizer watch every loop and index of the oracle.
 * Prints "ok <cases>" and exits 0 when every call returned as expected. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ctconv_oracle_output_shape(int, const int64_t*, const int64_t*, const int64_t*,
                               const int64_t*, const int64_t*, const int64_t*, int64_t*);
int ctconv_oracle_conv_transpose(int, int64_t, int64_t, int64_t, const int64_t*,
                                 const int64_t*, const int64_t*, const int64_t*,
                                 const int64_t*, const int64_t*, const double*, const double*,
                                 const double*, double*);
int ctconv_oracle_points(int, int64_t, int64_t, int64_t, const int64_t*, const int64_t*,
                         const int64_t*, const int64_t*, const int64_t*, const int64_t*,
                         const double*, const double*, const double*, const int64_t*, int64_t,
                         double*);
int ctconv_oracle_conv_transpose_grouped(int, int64_t, int64_t, int64_t, int64_t,
                                         const int64_t*, const int64_t*, const int64_t*,
                                         const int64_t*, const int64_t*, const int64_t*,
                                         const double*, const double*, const double*, double*);
int ctconv_oracle_points_grouped(int, int64_t, int64_t, int64_t, int64_t, const int64_t*,
                                 const int64_t*, const int64_t*, const int64_t*,
                                 const int64_t*, const int64_t*, const double*, const double*,
                                 const double*, const int64_t*, int64_t, double*);
int ctconv_oracle_istft_ola(int64_t, int64_t, int64_t, int64_t, const double*, double*);
int ctconv_oracle_rfft(int64_t, const double*, double*, double*);
void ctconv_oracle_elu(int64_t, const double*, double*);

static uint64_t st = 88172645463325252ull;
static double rnd(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (double)(st >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static int64_t rint_(int64_t lo, int64_t hi) { return lo + (int64_t)((rnd() + 1.0) * 0.5 * (hi - lo + 1)) % (hi - lo + 1); }
static double* arr(int64_t n) {
    double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) a[i] = rnd();
    return a;
}

int main(void) {
    int cases = 0;
    for (int it = 0; it < 300; ++it) {
        const int nd = 1 + it % 2;
        int64_t in[2], k[2], s[2], p[2], op[2], d[2], o[2];
        for (int a = 0; a < nd; ++a) {
            in[a] = rint_(1, nd == 1 ? 9 : 5);
            k[a] = rint_(1, 5);
            s[a] = rint_(1, 4);
            d[a] = rint_(1, 3);
            p[a] = rint_(0, (d[a] * (k[a] - 1)) / 2);
            op[a] = rint_(0, (s[a] > d[a] ? s[a] : d[a]) - 1);
        }
        if (ctconv_oracle_output_shape(nd, in, k, s, p, op, d, o) != 0) continue;
        const int64_t groups = (it % 3 == 0) ? rint_(1, 3) : 1;
        const int64_t N = rint_(0, 2), Ci = groups * rint_(1, 3), Co = groups * rint_(1, 3);
        int64_t xin = N * Ci, xo = N * Co, K = 1;
        for (int a = 0; a < nd; ++a) {
            xin *= in[a];
            xo *= o[a];
            K *= k[a];
        }
        double* x = arr(xin);
        double* w = arr(Ci * (Co / groups) * K);
        double* b = arr(Co);
        double* y = arr(xo);
        double* y2 = arr(xo);
        int r;
        if (groups == 1)
            r = ctconv_oracle_conv_transpose(nd, N, Ci, Co, in, k, s, p, op, d, x, w,
                                             (it & 4) ? b : NULL, y);
        else
            r = ctconv_oracle_conv_transpose_grouped(nd, N, Ci, Co, groups, in, k, s, p, op, d, x,
                                                     w, (it & 4) ? b : NULL, y);
        if (r != 0) {
            printf("conv failed at case %d\n", it);
            return 1;
        }
        /* every output again through the per-point evaluator */
        int64_t np = xo;
        int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * 4 * (size_t)(np > 0 ? np : 1));
        int64_t e = 0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t c = 0; c < Co; ++c)
                for (int64_t oy = 0; oy < (nd == 2 ? o[0] : 1); ++oy)
                    for (int64_t ox = 0; ox < o[nd - 1]; ++ox) {
                        idx[4 * e + 0] = n;
                        idx[4 * e + 1] = c;
                        idx[4 * e + 2] = oy;
                        idx[4 * e + 3] = ox;
                        ++e;
                    }
        if (groups == 1)
            r = ctconv_oracle_points(nd, N, Ci, Co, in, k, s, p, op, d, x, w, (it & 4) ? b : NULL,
                                     idx, np, y2);
        else
            r = ctconv_oracle_points_grouped(nd, N, Ci, Co, groups, in, k, s, p, op, d, x, w,
                                             (it & 4) ? b : NULL, idx, np, y2);
        if (r != 0) {
            printf("points failed at case %d\n", it);
            return 1;
        }
        for (int64_t i = 0; i < np; ++i)
            if (fabs(y[i] - y2[i]) > 1e-9 * (1.0 + fabs(y[i]))) {
                printf("points disagree at case %d\n", it);
                return 1;
            }
        free(idx);
        free(x);
        free(w);
        free(b);
        free(y);
        free(y2);
        ++cases;
    }
    /* iSTFT pieces */
    {
        const int64_t n_fft = 16, hop = 4, T = 5, N = 2, F = n_fft / 2 + 1;
        double* spec = arr(N * 2 * F * T);
        double* y = arr(N * ((T - 1) * hop + n_fft));
        if (ctconv_oracle_istft_ola(N, n_fft, hop, T, spec, y) != 0) return 1;
        double* fr = arr(n_fft);
        double* re = arr(F);
        double* im = arr(F);
        if (ctconv_oracle_rfft(n_fft, fr, re, im) != 0) return 1;
        double* e1 = arr(64);
        double* e2 = arr(64);
        ctconv_oracle_elu(64, e1, e2);
        free(spec);
        free(y);
        free(fr);
        free(re);
        free(im);
        free(e1);
        free(e2);
        cases += 3;
    }
    printf("ok %d\n", cases);
    return 0;
}
