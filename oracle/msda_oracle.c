/*
 * Reference oracle for the multi-scale deformable attention (MSDeformAttn) core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The HIP library
 * shares no source with it and never calls it.
 *
 * What it computes (definition followed):
 *   "Deformable DETR walkthrough" (zhangshiyu.com/post/59697), section 2.2.4
 *   (source analysis), function ms_deform_attn_core_pytorch: the flattened
 *   value is split per level into maps of shape (H_l, W_l); each level is
 *   sampled with grid_sample(mode=bilinear, padding_mode=zeros,
 *   align_corners=False) at grid = 2*loc - 1; every sample is multiplied by
 *   its attention weight and the L*P weighted samples of one (batch, query,
 *   head) are summed into output channels head*D .. head*D+D-1.
 *   Tensor layouts follow the Ascend DrivingSDK API page for
 *   multi_scale_deformable_attn (parameter list and return value):
 *     value               [bs, num_keys, M, D]
 *     spatial_shapes      [L, 2] = (H, W)
 *     level_start_index   [L]
 *     sampling_locations  [bs, Q, M, L, P, 2], last dim = (x, y)
 *     attention_weights   [bs, Q, M, L, P]
 *     output              [bs, Q, M*D]
 *   The backward returns gradients for value, sampling_locations and
 *   attention_weights only ("DQ-DETR ops directory" CSDN page, section 2(3),
 *   MSDeformAttnFunction.backward).
 *
 * Arithmetic:
 *   - float inputs arrive already widened (exactly) to float32, except the
 *     attention weights, which arrive as float64 (a float32 weight widened
 *     exactly, or a float64 softmax weight of the fused prologue);
 *   - the pixel coordinate is formed in float32 with two separate roundings,
 *     x = (loc_x * W) - 0.5, y = (loc_y * H) - 0.5 (align_corners=False maps
 *     normalised 0 and 1 to the outer pixel edges, so pixel centres land on
 *     integers); build with -ffp-contract=off so no fused multiply-add is
 *     formed here;
 *   - a sample takes part only when -1 < x < W and -1 < y < H (strict; NaN
 *     fails); a sample outside contributes nothing and receives zero
 *     gradient;
 *   - corners are floor(x), floor(x)+1 (likewise y); a corner outside the
 *     map reads as zero (padding_mode=zeros), per corner;
 *   - everything after the floor decision is float64.
 *
 * Every function here is pinned by tests/test_oracle_pins.py (closed forms,
 * brute force, a float64 grid_sample transcription, finite differences).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One bilinear sample: pixel coordinates, corner indices and weights. */
typedef struct {
    int valid;          /* passes -1 < x < W and -1 < y < H */
    int64_t x0, y0;     /* floor of the pixel coordinates */
    double lx, ly;      /* fractional parts */
    double hx, hy;      /* 1 - fractional parts */
} bilinear_t;

static bilinear_t make_sample(float loc_x, float loc_y, int64_t H, int64_t W)
{
    bilinear_t s;
    memset(&s, 0, sizeof(s));
    float x = loc_x * (float)W;   /* rounding 1 */
    x = x - 0.5f;                 /* rounding 2 */
    float y = loc_y * (float)H;
    y = y - 0.5f;
    if (!(x > -1.0f && x < (float)W && y > -1.0f && y < (float)H))
        return s;
    s.valid = 1;
    double fx = floor((double)x), fy = floor((double)y);
    s.x0 = (int64_t)fx;
    s.y0 = (int64_t)fy;
    s.lx = (double)x - fx;
    s.ly = (double)y - fy;
    s.hx = 1.0 - s.lx;
    s.hy = 1.0 - s.ly;
    return s;
}

/* Pointer to value[b, start + yc*W + xc, m, 0:D], or NULL when the corner is
 * off the map (it then reads as zero). */
static const float *corner_row(const float *value, int64_t K, int64_t M, int64_t D,
                               int64_t b, int64_t m, int64_t start, int64_t H, int64_t W,
                               int64_t yc, int64_t xc)
{
    if (yc < 0 || yc >= H || xc < 0 || xc >= W)
        return NULL;
    int64_t key = start + yc * W + xc;
    return value + ((b * K + key) * M + m) * D;
}

static double row_at(const float *row, int64_t d) { return row ? (double)row[d] : 0.0; }

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Number of threads an OpenMP region will use after set_threads(n). */
int oracle_threads(int nthreads)
{
#ifdef _OPENMP
    set_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Forward at one (b, q, m): out_d[d] = sum_{l,p} w[b,q,m,l,p] * sample_{l,p}[d],
 * sample = sum over the 4 corners of (bilinear weight) * value row.
 */
void oracle_forward_one(int64_t K, int64_t M, int64_t D, int64_t L, int64_t P, int64_t Q,
                        const int64_t *shapes, const int64_t *starts, const float *value,
                        const float *loc, const double *attw, int64_t b, int64_t q, int64_t m,
                        double *out_d)
{
    int64_t bq = b * Q + q;
    for (int64_t d = 0; d < D; ++d)
        out_d[d] = 0.0;
    for (int64_t l = 0; l < L; ++l) {
        int64_t H = shapes[2 * l], W = shapes[2 * l + 1], s0 = starts[l];
        for (int64_t p = 0; p < P; ++p) {
            int64_t idx = ((bq * M + m) * L + l) * P + p;
            bilinear_t s = make_sample(loc[2 * idx], loc[2 * idx + 1], H, W);
            if (!s.valid)
                continue;
            const float *v00 = corner_row(value, K, M, D, b, m, s0, H, W, s.y0, s.x0);
            const float *v01 = corner_row(value, K, M, D, b, m, s0, H, W, s.y0, s.x0 + 1);
            const float *v10 = corner_row(value, K, M, D, b, m, s0, H, W, s.y0 + 1, s.x0);
            const float *v11 = corner_row(value, K, M, D, b, m, s0, H, W, s.y0 + 1, s.x0 + 1);
            double w = attw[idx];
            for (int64_t d = 0; d < D; ++d) {
                double smp = s.hy * s.hx * row_at(v00, d) + s.hy * s.lx * row_at(v01, d) +
                             s.ly * s.hx * row_at(v10, d) + s.ly * s.lx * row_at(v11, d);
                out_d[d] += w * smp;
            }
        }
    }
}

/* Forward over the whole problem: out[bs, Q, M*D]. */
void oracle_forward(int64_t bs, int64_t K, int64_t M, int64_t D, int64_t L, int64_t P,
                    int64_t Q, const int64_t *shapes, const int64_t *starts,
                    const float *value, const float *loc, const double *attw,
                    double *out, int nthreads)
{
    set_threads(nthreads);
    int64_t nbq = bs * Q;
#pragma omp parallel for schedule(static)
    for (int64_t bq = 0; bq < nbq; ++bq)
        for (int64_t m = 0; m < M; ++m)
            oracle_forward_one(K, M, D, L, P, Q, shapes, starts, value, loc, attw,
                               bq / Q, bq % Q, m, out + (bq * M + m) * D);
}

/*
 * Backward.  g = grad_out[b, q, m*D : (m+1)*D].
 *   grad_w[b,q,m,l,p]     = sum_d g[d] * sample[d]
 *   grad_loc[..., 0]      = W * w * sum_d g[d] * d(sample[d])/dx
 *   grad_loc[..., 1]      = H * w * sum_d g[d] * d(sample[d])/dy
 *   grad_value[corner]   += w * (bilinear weight of that corner) * g
 * The chain factors W and H come from x = loc_x * W - 0.5.  At integer
 * coordinates the derivative is the one of the cell selected by floor (right
 * derivative).  grad_value is written in full (rows never sampled are 0).
 */
void oracle_backward(int64_t bs, int64_t K, int64_t M, int64_t D, int64_t L, int64_t P,
                     int64_t Q, const int64_t *shapes, const int64_t *starts,
                     const float *value, const float *loc, const double *attw,
                     const float *grad_out, double *grad_value, double *grad_loc,
                     double *grad_w, int nthreads)
{
    set_threads(nthreads);
    int64_t nbq = bs * Q;

    /* grad_loc and grad_w: independent per (b, q). */
#pragma omp parallel for schedule(static)
    for (int64_t bq = 0; bq < nbq; ++bq) {
        int64_t b = bq / Q;
        for (int64_t m = 0; m < M; ++m) {
            const float *g = grad_out + (bq * M + m) * D;
            for (int64_t l = 0; l < L; ++l) {
                int64_t H = shapes[2 * l], W = shapes[2 * l + 1], s0 = starts[l];
                for (int64_t p = 0; p < P; ++p) {
                    int64_t idx = ((bq * M + m) * L + l) * P + p;
                    bilinear_t s = make_sample(loc[2 * idx], loc[2 * idx + 1], H, W);
                    grad_w[idx] = 0.0;
                    grad_loc[2 * idx] = 0.0;
                    grad_loc[2 * idx + 1] = 0.0;
                    if (!s.valid)
                        continue;
                    const float *v00 = corner_row(value, K, M, D, b, m, s0, H, W, s.y0, s.x0);
                    const float *v01 = corner_row(value, K, M, D, b, m, s0, H, W, s.y0, s.x0 + 1);
                    const float *v10 = corner_row(value, K, M, D, b, m, s0, H, W, s.y0 + 1, s.x0);
                    const float *v11 = corner_row(value, K, M, D, b, m, s0, H, W, s.y0 + 1, s.x0 + 1);
                    double w = attw[idx];
                    double gw = 0.0, gx = 0.0, gy = 0.0;
                    for (int64_t d = 0; d < D; ++d) {
                        double a = row_at(v00, d), bb = row_at(v01, d);
                        double c = row_at(v10, d), e = row_at(v11, d);
                        double smp = s.hy * s.hx * a + s.hy * s.lx * bb + s.ly * s.hx * c + s.ly * s.lx * e;
                        double dsdx = s.hy * (bb - a) + s.ly * (e - c);
                        double dsdy = s.hx * (c - a) + s.lx * (e - bb);
                        double gd = (double)g[d];
                        gw += gd * smp;
                        gx += gd * dsdx;
                        gy += gd * dsdy;
                    }
                    grad_w[idx] = gw;
                    grad_loc[2 * idx] = (double)W * w * gx;
                    grad_loc[2 * idx + 1] = (double)H * w * gy;
                }
            }
        }
    }

    /* grad_value: each (b, m) owns a disjoint slice, so no two threads add
     * into the same element. */
    int64_t nbm = bs * M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bm = 0; bm < nbm; ++bm) {
        int64_t b = bm / M, m = bm % M;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t d = 0; d < D; ++d)
                grad_value[((b * K + k) * M + m) * D + d] = 0.0;
        for (int64_t q = 0; q < Q; ++q) {
            int64_t bq = b * Q + q;
            const float *g = grad_out + (bq * M + m) * D;
            for (int64_t l = 0; l < L; ++l) {
                int64_t H = shapes[2 * l], W = shapes[2 * l + 1], s0 = starts[l];
                for (int64_t p = 0; p < P; ++p) {
                    int64_t idx = ((bq * M + m) * L + l) * P + p;
                    bilinear_t s = make_sample(loc[2 * idx], loc[2 * idx + 1], H, W);
                    if (!s.valid)
                        continue;
                    double w = attw[idx];
                    const int64_t dy[4] = {0, 0, 1, 1}, dx[4] = {0, 1, 0, 1};
                    const double cw[4] = {s.hy * s.hx, s.hy * s.lx, s.ly * s.hx, s.ly * s.lx};
                    for (int c = 0; c < 4; ++c) {
                        int64_t yc = s.y0 + dy[c], xc = s.x0 + dx[c];
                        if (yc < 0 || yc >= H || xc < 0 || xc >= W)
                            continue;
                        int64_t key = s0 + yc * W + xc;
                        double *gv = grad_value + ((b * K + key) * M + m) * D;
                        for (int64_t d = 0; d < D; ++d)
                            gv[d] += w * cw[c] * (double)g[d];
                    }
                }
            }
        }
    }
}
