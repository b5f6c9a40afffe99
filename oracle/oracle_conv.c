/*
 * CPU oracle for the int8 2-D convolution.  TEST INFRASTRUCTURE ONLY: nothing
 * in the product library calls, links or includes this file; only the tests,
 * the smoke check and the CPU-baseline leg of the bench use it.  It shares no
 * code, header or table with the GPU path.
 *
 * What it computes (the plain definition, no lowering to a matrix product):
 *
 *   y[n][p][q][k] = wrap32( sum_{r<R, s<S, c<C} x[n][ih][iw][c] * w[k][r][s][c] )
 *   ih = p*stride_h + r*dil_h - pad_h,  iw = q*stride_w + s*dil_w - pad_w,
 *
 * terms with ih or iw outside the image being zero (zero padding), x and w
 * read as signed int8, the sum taken exactly in int64, wrap32 the two's-
 * complement reduction mod 2^32.  The input position of a tap is the one the
 * contest write-up's im2col kernel computes ("先导杯比赛回顾", 多批次展开的
 * Im2col 方法: input row = kernel row - pad + output row * stride, input
 * column = output column * stride - pad + kernel column), with a dilation
 * factor on the tap offset; the convolution is the one the write-up lowers
 * to a matrix product (卷积转化).
 *
 * Layouts (all dense): x is N x H x W x C (NHWC), w is K x R x S x C (KRSC),
 * y is N x P x Q x K with P = (H + 2 pad_h - dil_h (R-1) - 1) / stride_h + 1
 * and Q likewise (0 when the numerator is negative).
 *
 * Output rows (n, p) are spread over OpenMP threads.  The return value counts
 * outputs whose exact sum fell outside the int32 range.
 */
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int32_t cwrap32(int64_t s) { return (int32_t)(uint32_t)(uint64_t)s; }

static int64_t out_extent(int64_t H, int64_t R, int64_t pad, int64_t stride, int64_t dil)
{
    const int64_t span = H + 2 * pad - dil * (R - 1) - 1;
    return span < 0 ? 0 : span / stride + 1;
}

int64_t oracle_conv_out_extent(int64_t H, int64_t R, int64_t pad, int64_t stride, int64_t dil)
{
    return out_extent(H, R, pad, stride, dil);
}

static int64_t conv_point(int64_t n, int64_t p, int64_t q, int64_t k,
                          int64_t H, int64_t W, int64_t C, int64_t R, int64_t S,
                          int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w,
                          int64_t dil_h, int64_t dil_w, const int8_t *x, const int8_t *w)
{
    int64_t sum = 0;
    for (int64_t r = 0; r < R; ++r) {
        const int64_t ih = p * stride_h + r * dil_h - pad_h;
        if (ih < 0 || ih >= H) continue;
        for (int64_t s = 0; s < S; ++s) {
            const int64_t iw = q * stride_w + s * dil_w - pad_w;
            if (iw < 0 || iw >= W) continue;
            const int8_t *xp = x + ((n * H + ih) * W + iw) * C;
            const int8_t *wp = w + ((k * R + r) * S + s) * C;
            for (int64_t c = 0; c < C; ++c) sum += (int64_t)xp[c] * (int64_t)wp[c];
        }
    }
    return sum;
}

int64_t oracle_conv2d_s8s8s32(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                              int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w,
                              int64_t dil_h, int64_t dil_w, const int8_t *x, const int8_t *w, int32_t *y)
{
    const int64_t P = out_extent(H, R, pad_h, stride_h, dil_h);
    const int64_t Q = out_extent(W, S, pad_w, stride_w, dil_w);
    int64_t overflow = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : overflow)
    for (int64_t np = 0; np < N * P; ++np) {
        const int64_t n = np / P, p = np % P;
        for (int64_t q = 0; q < Q; ++q)
            for (int64_t k = 0; k < K; ++k) {
                const int64_t s = conv_point(n, p, q, k, H, W, C, R, S, pad_h, pad_w, stride_h, stride_w,
                                             dil_h, dil_w, x, w);
                overflow += (s < INT32_MIN || s > INT32_MAX);
                y[((n * P + p) * Q + q) * K + k] = cwrap32(s);
            }
    }
    return overflow;
}

/* out[t] = y[n[t]][p[t]][q[t]][k[t]] for sampled outputs. */
void oracle_conv2d_points(int64_t count, const int64_t *nn, const int64_t *pp, const int64_t *qq, const int64_t *kk,
                          int64_t H, int64_t W, int64_t C, int64_t R, int64_t S,
                          int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w,
                          int64_t dil_h, int64_t dil_w, const int8_t *x, const int8_t *w, int32_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t)
        out[t] = cwrap32(conv_point(nn[t], pp[t], qq[t], kk[t], H, W, C, R, S, pad_h, pad_w, stride_h, stride_w,
                                    dil_h, dil_w, x, w));
}
