/*
 * oracle_asan_driver.c -- the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (test infrastructure, CPU only).
 *
 * Built with gcc together with oracle/mq_oracle.c. Every exported oracle function runs on small
 * ragged tensors and convolutions (odd channel and batch counts, partial squares, 1x1 / 3x3 /
 * 1x3 kernels, strides 1-3, paddings that differ between height and width, NaN input), into
 * buffers of exactly the documented sizes, so that any read or write past them, or any undefined
 * arithmetic, stops the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct { int32_t N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw; } conv_t;

double mqo_e2m1_value(int code);
double mqo_e2m3_value(int code);
double mqo_e4m3_value(int code);
double mqo_elem_value(int fmt, int code);
int mqo_e4m3_cast(float s);
int mqo_elem_rne(int fmt, float a);
int mqo_elem_sr(int fmt, float a, uint32_t u16);
void mqo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t mqo_sr_u16(uint64_t seed, int64_t t, int e);
int64_t mqo_num_squares(int O0, int O1, int R, int S);
int mqo_quantize(const float *src, int O0, int O1, int R, int S, int fmt, int rnd, uint64_t seed,
                 uint8_t *codes, uint8_t *scales, float *tscale);
int64_t mqo_packed_bytes(int64_t nsq, int fmt);
void mqo_pack(const uint8_t *codes, int64_t nsq, int fmt, uint8_t *out);
void mqo_unpack(const uint8_t *packed, int64_t nsq, int fmt, uint8_t *codes);
void mqo_dequant(const uint8_t *codes, const uint8_t *scales, float T, int O0, int O1, int R,
                 int S, int fmt, double *out);
void mqo_nchw_to_cbf(const float *src, float *dst, int N, int C, int H, int W);
void mqo_cbf_to_nchw(const float *src, float *dst, int N, int C, int H, int W);
void mqo_oihw_to_tap_major(const float *src, float *dst, int Cout, int Cin, int Kh, int Kw);
void mqo_tap_major_to_oihw(const float *src, float *dst, int Cout, int Cin, int Kh, int Kw);
int mqo_conv_fwd(const conv_t *p, const double *x, const double *w, double *y, double *yabs);
int mqo_conv_wgrad(const conv_t *p, const double *g, const double *x, double *gw, double *gwabs);
int mqo_conv_dgrad(const conv_t *p, const double *w, const double *g, double *gx, double *gxabs);
int mqo_conv_fwd_at(const conv_t *p, const double *x, const double *w, const int32_t *idx,
                    int64_t n, double *out, double *outabs);
int mqo_conv_wgrad_at(const conv_t *p, const double *g, const double *x, const int32_t *idx,
                      int64_t n, double *out, double *outabs);
int mqo_conv_dgrad_at(const conv_t *p, const double *w, const double *g, const int32_t *idx,
                      int64_t n, double *out, double *outabs);
void mqo_e4m3_cast_array(const float *s, int64_t n, uint8_t *out);
void mqo_elem_rne_array(int fmt, const float *a, int64_t n, uint8_t *out);
void mqo_elem_sr_array(int fmt, const float *a, const uint32_t *u16, int64_t n, uint8_t *out);
void mqo_sr_u16_array(uint64_t seed, const int64_t *t, const int32_t *e, int64_t n, uint32_t *out);

static uint64_t g_s = 12345;
static float rnd(void)
{
    g_s = g_s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((int64_t)(g_s >> 11) % 2000001 - 1000000) * 1e-6f;
}

static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) abort(); return p; }

/* quantize / pack / unpack / dequantize a [O0][O1][R][S] tensor in exactly sized buffers */
static void quant_roundtrip(int O0, int O1, int R, int S, int fmt, int rnd_mode, int with_nan)
{
    const int64_t n = (int64_t)O0 * O1 * R * S, nsq = mqo_num_squares(O0, O1, R, S);
    float *x = xmalloc(n * sizeof(float));
    for (int64_t i = 0; i < n; i++) x[i] = rnd() * (i % 5 == 0 ? 100.0f : 1.0f);
    if (with_nan) x[n / 2] = NAN;
    uint8_t *codes = xmalloc(nsq * 16), *scales = xmalloc(nsq);
    uint8_t *packed = xmalloc(mqo_packed_bytes(nsq, fmt)), *back = xmalloc(nsq * 16);
    float T;
    if (mqo_quantize(x, O0, O1, R, S, fmt, rnd_mode, 77, codes, scales, &T) != 0) abort();
    mqo_pack(codes, nsq, fmt, packed);
    mqo_unpack(packed, nsq, fmt, back);
    for (int64_t i = 0; i < nsq * 16; i++)
        if (back[i] != codes[i]) abort();
    double *deq = xmalloc(n * sizeof(double));
    mqo_dequant(codes, scales, T, O0, O1, R, S, fmt, deq);
    free(x); free(codes); free(scales); free(packed); free(back); free(deq);
}

static double *rand_d(int64_t n)
{
    double *a = xmalloc(n * sizeof(double));
    for (int64_t i = 0; i < n; i++) a[i] = rnd();
    return a;
}

static void conv_case(conv_t p)
{
    const int Ho = (p.H + 2 * p.ph - p.Kh) / p.sh + 1, Wo = (p.W + 2 * p.pw - p.Kw) / p.sw + 1;
    const int64_t nx = (int64_t)p.H * p.W * p.Cin * p.N, nw = (int64_t)p.Kh * p.Kw * p.Cout * p.Cin;
    const int64_t ny = (int64_t)Ho * Wo * p.Cout * p.N;
    double *x = rand_d(nx), *w = rand_d(nw), *g = rand_d(ny);
    double *y = xmalloc(ny * 8), *ya = xmalloc(ny * 8), *gw = xmalloc(nw * 8), *gwa = xmalloc(nw * 8);
    double *gx = xmalloc(nx * 8), *gxa = xmalloc(nx * 8);
    if (mqo_conv_fwd(&p, x, w, y, ya) || mqo_conv_wgrad(&p, g, x, gw, gwa) ||
        mqo_conv_dgrad(&p, w, g, gx, gxa))
        abort();
    /* sampled outputs: the last element of each output and a few in between */
    int32_t idx[4 * 4];
    const int32_t yd[4] = {Ho, Wo, p.Cout, p.N}, wd[4] = {p.Kh, p.Kw, p.Cout, p.Cin};
    const int32_t xd[4] = {p.H, p.W, p.Cin, p.N};
    const int32_t *dims[3] = {yd, wd, xd};
    for (int k = 0; k < 3; k++) {
        for (int s = 0; s < 4; s++)
            for (int d = 0; d < 4; d++) idx[4 * s + d] = s == 3 ? dims[k][d] - 1 : (dims[k][d] * s) / 3;
        double v[4], va[4];
        const int r = k == 0 ? mqo_conv_fwd_at(&p, x, w, idx, 4, v, va)
                    : k == 1 ? mqo_conv_wgrad_at(&p, g, x, idx, 4, v, va)
                             : mqo_conv_dgrad_at(&p, w, g, idx, 4, v, va);
        if (r) abort();
    }
    free(x); free(w); free(g); free(y); free(ya); free(gw); free(gwa); free(gx); free(gxa);
}

int main(void)
{
    for (int c = 0; c < 256; c++) {
        (void)mqo_e4m3_value(c);
        if (c < 16) (void)mqo_e2m1_value(c);
        if (c < 64) (void)mqo_e2m3_value(c);
        (void)mqo_elem_value(c & 1 ? 4 : 6, c & 15);
    }
    const float probes[] = {0.0f, 1e-30f, 0.001953125f, 0.5f, 3.0f, 6.0f, 7.5f, 448.0f, 464.0f,
                            1e30f, INFINITY, NAN};
    for (unsigned i = 0; i < sizeof probes / sizeof probes[0]; i++) {
        (void)mqo_e4m3_cast(probes[i]);
        if (isfinite(probes[i])) {
            (void)mqo_elem_rne(4, probes[i]);
            (void)mqo_elem_rne(6, probes[i]);
            (void)mqo_elem_sr(4, probes[i], 40000u);
            (void)mqo_elem_sr(6, probes[i], 0u);
        }
    }
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
    mqo_philox4x32_10(ctr, key, out);
    for (int e = 0; e < 16; e++) (void)mqo_sr_u16(0xFFFFFFFFFFFFFFFFULL, 123456789, e);
    float arr[7] = {0.1f, 1.0f, 2.5f, 6.0f, 400.0f, 500.0f, 0.0f};
    uint8_t ob[7];
    uint32_t u16[7] = {0, 1, 65535, 30000, 7, 8, 9};
    int64_t ts[7] = {0, 1, 2, 3, 4, 5, 6};
    int32_t es[7] = {0, 3, 7, 8, 15, 1, 2};
    uint32_t uo[7];
    mqo_e4m3_cast_array(arr, 7, ob);
    mqo_elem_rne_array(4, arr, 7, ob);
    mqo_elem_sr_array(6, arr, u16, 7, ob);
    mqo_sr_u16_array(42, ts, es, 7, uo);

    const int shapes[][4] = {{1, 1, 1, 1}, {2, 3, 5, 7}, {1, 2, 9, 6}, {3, 1, 4, 8}, {2, 2, 13, 3}};
    for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; s++)
        for (int fmt = 4; fmt <= 6; fmt += 2)
            for (int r = 0; r < 2; r++) {
                quant_roundtrip(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], fmt, r, 0);
                quant_roundtrip(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], fmt, r, 1);
            }

    float *a = xmalloc(3 * 5 * 4 * 7 * sizeof(float)), *b = xmalloc(3 * 5 * 4 * 7 * sizeof(float));
    for (int i = 0; i < 3 * 5 * 4 * 7; i++) a[i] = rnd();
    mqo_nchw_to_cbf(a, b, 3, 5, 4, 7);
    mqo_cbf_to_nchw(b, a, 3, 5, 4, 7);
    mqo_oihw_to_tap_major(a, b, 5, 7, 3, 4);
    mqo_tap_major_to_oihw(b, a, 5, 7, 3, 4);
    free(a); free(b);

    const conv_t convs[] = {
        {2, 3, 5, 6, 2, 3, 3, 1, 1, 0, 0}, {3, 5, 7, 9, 4, 3, 3, 2, 2, 1, 1},
        {2, 4, 6, 7, 3, 1, 1, 1, 1, 1, 1}, {1, 3, 9, 11, 5, 1, 3, 1, 2, 0, 1},
        {2, 2, 13, 14, 3, 3, 3, 3, 3, 1, 1}, {5, 6, 4, 5, 7, 3, 2, 2, 1, 1, 0},
    };
    for (unsigned c = 0; c < sizeof convs / sizeof convs[0]; c++) conv_case(convs[c]);
    printf("oracle sanitizer run: ok\n");
    return 0;
}
