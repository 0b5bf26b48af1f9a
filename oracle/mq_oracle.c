/*
 * mq_oracle.c -- plain CPU oracle for microscaling-quantized convolution (MicroQonv).
 *
 * TEST INFRASTRUCTURE. This is the slow, obviously-correct reference that the GPU library is
 * checked against. Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
 * load it. It shares no code, table or header with the GPU library.
 *
 * What it follows (the onedev.kr paper digest of "MicroQonv: Reshaping Convolution Tensors for
 * Efficient Microscaling in Training and Inference"):
 *   - section "How it works" (어떻게 동작하나): activations are stored channel-batch-first,
 *     X_{Cin,N} with, for every pixel (h,w), all channels and all batch elements contiguous;
 *   - section "How it differs" (무엇과 다른가): the 2-D matrix forms W_{fCout,Cin}
 *     (Cout x Kh*Kw*Cin) and G_{YfCout,N} (Cout x Hout*Wout*N); the three GEMMs Y = W.X',
 *     G_W = G_Y.X'^T and G_X' = W^T.G_Y; square blocks with the scale shared along sqrt(B)
 *     elements in each of the two dimensions, B = 16; the NVFP4 recipe (tensor scale
 *     T = max|X| / (max block-scale * max element), E4M3 block scale
 *     B = CastE4M3(max|X_i| / (T * max element)), E2M1 elements Round(X_i / (B * T)));
 *     round-to-nearest for weights and activations, stochastic rounding for gradients;
 *   - section "How it is used" (어떻게 쓰나): NVFP6 = the same scaling with E2M3 elements;
 *   - section "Premises and limits" (전제와 한계): stride 1 / no padding is only expository.
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - element grid rounding is round-to-nearest, ties to the even code, saturating at the
 *     largest element; CastE4M3 is round-to-nearest-even with subnormals, saturating at 448;
 *   - T, the block-scale quotient and the element quotient are fp32, evaluated exactly in the
 *     order the formulas are written, with IEEE division and no fused multiply-add;
 *   - a tensor with a NaN/Inf element gets T = NaN, every scale 0x7F (E4M3 NaN), every code 0;
 *     a tensor whose T is 0 gets every scale and code 0; a square whose scale (or whose
 *     divisor B*T) is 0 gets codes 0;
 *   - the code's sign bit is the sign bit of the input element (so -0.0 and small negatives
 *     that round to zero keep the sign);
 *   - stochastic rounding: between the two grid neighbours lo <= a < hi of a = |q|, round up
 *     iff (float)u16 < ((a-lo)/(hi-lo)) * 65536, with u16 a 16-bit slice of Philox4x32-10
 *     (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11);
 *     a >= max element saturates;
 *   - partial squares at the edge cover only real elements; padded slots hold code 0.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math, SSE math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MQO_FP4 4
#define MQO_FP6 6
#define MQO_RNE 0
#define MQO_SR 1

/* ------------------------------------------------------------------------------------------
 * Number formats, decoded straight from their bit-field definitions.
 *   E2M1: s|ee|m, exponent bias 1; ee=0 is subnormal (m * 0.5).
 *   E2M3: s|ee|mmm, exponent bias 1; ee=0 is subnormal (m / 8).
 *   E4M3 ("fn" flavour): s|eeee|mmm, bias 7; eeee=0 subnormal (m * 2^-9); s|1111|111 is NaN;
 *   there is no infinity, the largest finite value is 448.
 * ------------------------------------------------------------------------------------------ */
double mqo_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

double mqo_e2m3_value(int code)
{
    int s = (code >> 5) & 1, e = (code >> 3) & 3, m = code & 7;
    double mag = (e == 0) ? m / 8.0 : ldexp(1.0 + m / 8.0, e - 1);
    return s ? -mag : mag;
}

double mqo_e4m3_value(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

double mqo_elem_value(int fmt, int code)
{
    return fmt == MQO_FP4 ? mqo_e2m1_value(code) : mqo_e2m3_value(code);
}

static int elem_mag_count(int fmt) { return fmt == MQO_FP4 ? 8 : 32; }
static int elem_sign_bit(int fmt) { return fmt == MQO_FP4 ? 0x8 : 0x20; }

/* Largest element magnitude ("max B_ef"): 6 for E2M1, 7.5 for E2M3. */
static float elem_max(int fmt) { return fmt == MQO_FP4 ? 6.0f : 7.5f; }

/* Index of the value of v[0..n-1] (increasing, v[0] = 0) nearest to a >= 0.
 * A tie goes to the even index; a at or above v[n-1] gives n-1. */
static int nearest_even_index(const double *v, int n, double a)
{
    if (a >= v[n - 1]) return n - 1;
    int lo = 0, hi = n - 1; /* v[lo] <= a < v[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (v[mid] <= a) lo = mid; else hi = mid;
    }
    double m = 0.5 * (v[lo] + v[hi]);
    if (a < m) return lo;
    if (a > m) return hi;
    return (lo % 2 == 0) ? lo : hi;
}

/* Index i with v[i] <= a < v[i+1] (a >= 0, a < v[n-1]). */
static int floor_index(const double *v, int n, double a)
{
    int lo = 0, hi = n - 1;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (v[mid] <= a) lo = mid; else hi = mid;
    }
    return lo;
}

static double g_e4m3[127]; /* finite non-negative E4M3 values, codes 0x00..0x7E */
static double g_grid4[8];  /* E2M1 magnitudes, codes 0..7 */
static double g_grid6[32]; /* E2M3 magnitudes, codes 0..31 */
static int g_tables_ready = 0;

static void init_tables(void)
{
    if (g_tables_ready) return;
    for (int c = 0; c < 127; c++) g_e4m3[c] = mqo_e4m3_value(c);
    for (int c = 0; c < 8; c++) g_grid4[c] = mqo_e2m1_value(c);
    for (int c = 0; c < 32; c++) g_grid6[c] = mqo_e2m3_value(c);
    g_tables_ready = 1;
}

static const double *elem_grid(int fmt) { return fmt == MQO_FP4 ? g_grid4 : g_grid6; }

/* CastE4M3 of a non-negative fp32 value: nearest, ties to even, saturating at 448 (0x7E). */
int mqo_e4m3_cast(float s)
{
    init_tables();
    if (isnan(s)) return 0x7F;
    if (s >= 448.0f) return 0x7E;
    return nearest_even_index(g_e4m3, 127, (double)s);
}

/* Round-to-nearest-even of |q| onto the element grid; returns the magnitude code. */
int mqo_elem_rne(int fmt, float a)
{
    init_tables();
    return nearest_even_index(elem_grid(fmt), elem_mag_count(fmt), (double)a);
}

/* Stochastic rounding of a = |q| between its grid neighbours with a 16-bit uniform u16. */
int mqo_elem_sr(int fmt, float a, uint32_t u16)
{
    init_tables();
    const double *v = elem_grid(fmt);
    int n = elem_mag_count(fmt);
    if (a >= (float)v[n - 1]) return n - 1;
    int i = floor_index(v, n, (double)a);
    float lo = (float)v[i], hi = (float)v[i + 1];
    float frac = (a - lo) / (hi - lo); /* exact: a-lo by Sterbenz, hi-lo is a power of two */
    return ((float)u16 < frac * 65536.0f) ? i + 1 : i;
}

/* ------------------------------------------------------------------------------------------
 * Philox4x32-10 (Salmon et al., SC'11): 10 rounds of the 4x32 Philox S-box with multipliers
 * 0xD2511F53 / 0xCD9E8D57 and Weyl key increments 0x9E3779B9 / 0xBB67AE85.
 * ------------------------------------------------------------------------------------------ */
void mqo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; round++) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 16-bit uniform used for element e (0..15) of square t under a given seed.
 * Counter j = 2t + e/8 (two Philox calls per square), key = the 64-bit seed; element e takes
 * the (e%2)-th 16-bit half of output word (e%8)/2. */
uint32_t mqo_sr_u16(uint64_t seed, int64_t t, int e)
{
    uint64_t j = 2 * (uint64_t)t + (uint64_t)(e >> 3);
    uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    mqo_philox4x32_10(ctr, key, r);
    return (r[(e & 7) >> 1] >> (16 * (e & 1))) & 0xFFFFu;
}

/* ------------------------------------------------------------------------------------------
 * Quantization of a 4-D tensor [O0][O1][R][S] (S fastest) with 4x4 squares over (R,S).
 * Square index t = ((o0*O1 + o1)*R4 + r/4)*S4 + s/4, element e = (r%4)*4 + s%4,
 * R4 = ceil(R/4), S4 = ceil(S/4). codes[16*t + e] holds one code per byte (padded slots 0).
 * ------------------------------------------------------------------------------------------ */
int64_t mqo_num_squares(int O0, int O1, int R, int S)
{
    return (int64_t)O0 * O1 * ((R + 3) / 4) * ((S + 3) / 4);
}

int mqo_quantize(const float *src, int O0, int O1, int R, int S, int fmt, int rnd,
                 uint64_t seed, uint8_t *codes, uint8_t *scales, float *tscale)
{
    if (fmt != MQO_FP4 && fmt != MQO_FP6) return 1;
    if (rnd != MQO_RNE && rnd != MQO_SR) return 1;
    if (O0 < 1 || O1 < 1 || R < 1 || S < 1) return 1;
    init_tables();
    const int R4 = (R + 3) / 4, S4 = (S + 3) / 4;
    const int64_t nsq = mqo_num_squares(O0, O1, R, S);
    const int64_t nel = (int64_t)O0 * O1 * R * S;
    memset(codes, 0, (size_t)nsq * 16);
    memset(scales, 0, (size_t)nsq);

    /* Tensor amax over the real elements. */
    int nonfinite = 0;
    float amax = 0.0f;
    for (int64_t i = 0; i < nel; i++) {
        float a = fabsf(src[i]);
        if (!isfinite(a)) nonfinite = 1;
        else if (a > amax) amax = a;
    }
    if (nonfinite) {
        uint32_t nan_bits = 0x7FC00000u;
        memcpy(tscale, &nan_bits, 4);
        memset(scales, 0x7F, (size_t)nsq);
        return 0;
    }
    const float emax = elem_max(fmt);
    /* Tensor scale: amax / (max E4M3 value * max element value). */
    const float T = amax / (448.0f * emax);
    *tscale = T;
    if (T == 0.0f) return 0;
    const float TE = T * emax;
    const double *grid = elem_grid(fmt);
    const int nmag = elem_mag_count(fmt), sbit = elem_sign_bit(fmt);

    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nsq; t++) {
        int64_t plane = t / ((int64_t)R4 * S4); /* o0*O1 + o1 */
        int r4 = (int)((t / S4) % R4), s4 = (int)(t % S4);
        /* Square max over real elements. */
        float bmax = 0.0f;
        for (int i = 0; i < 4; i++)
            for (int j = 0; j < 4; j++) {
                int r = 4 * r4 + i, s = 4 * s4 + j;
                if (r >= R || s >= S) continue;
                float a = fabsf(src[(plane * R + r) * S + s]);
                if (a > bmax) bmax = a;
            }
        /* Block scale B = CastE4M3(bmax / (T * emax)). */
        float sq = bmax / TE;
        int bcode = mqo_e4m3_cast(sq);
        scales[t] = (uint8_t)bcode;
        float B = (float)mqo_e4m3_value(bcode);
        float D = B * T;
        if (bcode == 0 || D == 0.0f) continue;
        for (int i = 0; i < 4; i++)
            for (int j = 0; j < 4; j++) {
                int r = 4 * r4 + i, s = 4 * s4 + j;
                if (r >= R || s >= S) continue;
                int e = 4 * i + j;
                float x = src[(plane * R + r) * S + s];
                float q = x / D; /* element quotient X_i / (B * T) */
                float a = fabsf(q);
                int mag;
                if (rnd == MQO_RNE) mag = nearest_even_index(grid, nmag, (double)a);
                else mag = mqo_elem_sr(fmt, a, mqo_sr_u16(seed, t, e));
                codes[16 * t + e] = (uint8_t)(mag | (signbit(x) ? sbit : 0));
            }
    }
    return 0;
}

/* Bytes of the packed code stream: 8 (FP4) or 12 (FP6) per square. */
int64_t mqo_packed_bytes(int64_t nsq, int fmt) { return nsq * (fmt == MQO_FP4 ? 8 : 12); }

/* Pack one-code-per-byte squares into the library's stream. FP4: element e of square t is the
 * (e%2 ? high : low) nibble of byte 8t + e/2. FP6: element e is bits [6e, 6e+6) of the
 * little-endian 96-bit word of square t (bytes 12t .. 12t+11). */
void mqo_pack(const uint8_t *codes, int64_t nsq, int fmt, uint8_t *out)
{
    int64_t nb = mqo_packed_bytes(nsq, fmt);
    memset(out, 0, (size_t)nb);
    for (int64_t t = 0; t < nsq; t++)
        for (int e = 0; e < 16; e++) {
            unsigned c = codes[16 * t + e];
            if (fmt == MQO_FP4) {
                out[8 * t + e / 2] |= (uint8_t)((c & 0xF) << (4 * (e % 2)));
            } else {
                for (int b = 0; b < 6; b++) {
                    int bit = 6 * e + b;
                    if ((c >> b) & 1) out[12 * t + bit / 8] |= (uint8_t)(1u << (bit % 8));
                }
            }
        }
}

/* Inverse of mqo_pack. */
void mqo_unpack(const uint8_t *packed, int64_t nsq, int fmt, uint8_t *codes)
{
    for (int64_t t = 0; t < nsq; t++)
        for (int e = 0; e < 16; e++) {
            unsigned c = 0;
            if (fmt == MQO_FP4) {
                c = (packed[8 * t + e / 2] >> (4 * (e % 2))) & 0xF;
            } else {
                for (int b = 0; b < 6; b++) {
                    int bit = 6 * e + b;
                    c |= (unsigned)((packed[12 * t + bit / 8] >> (bit % 8)) & 1) << b;
                }
            }
            codes[16 * t + e] = (uint8_t)c;
        }
}

/* Dequantize to double: value = element(code) * E4M3(scale) * T, over the real elements,
 * written densely as [O0][O1][R][S]. Exact in double. */
void mqo_dequant(const uint8_t *codes, const uint8_t *scales, float T, int O0, int O1, int R,
                 int S, int fmt, double *out)
{
    const int R4 = (R + 3) / 4, S4 = (S + 3) / 4;
    for (int64_t plane = 0; plane < (int64_t)O0 * O1; plane++)
        for (int r = 0; r < R; r++)
            for (int s = 0; s < S; s++) {
                int64_t t = (plane * R4 + r / 4) * S4 + s / 4;
                int e = (r % 4) * 4 + s % 4;
                double v = mqo_elem_value(fmt, codes[16 * t + e]);
                out[(plane * R + r) * S + s] = v * mqo_e4m3_value(scales[t]) * (double)T;
            }
}

/* ------------------------------------------------------------------------------------------
 * Layouts. Channel-batch-first activations: [H][W][C][N] (N fastest inside a pixel).
 * Weights as 2-D W_{fCout,Cin}: stored [Kh][Kw][Cout][Cin], i.e. one Cout x Cin square-tiled
 * matrix per tap.
 * ------------------------------------------------------------------------------------------ */
void mqo_nchw_to_cbf(const float *src, float *dst, int N, int C, int H, int W)
{
    for (int n = 0; n < N; n++)
        for (int c = 0; c < C; c++)
            for (int h = 0; h < H; h++)
                for (int w = 0; w < W; w++)
                    dst[(((int64_t)h * W + w) * C + c) * N + n] =
                        src[(((int64_t)n * C + c) * H + h) * W + w];
}

void mqo_cbf_to_nchw(const float *src, float *dst, int N, int C, int H, int W)
{
    for (int n = 0; n < N; n++)
        for (int c = 0; c < C; c++)
            for (int h = 0; h < H; h++)
                for (int w = 0; w < W; w++)
                    dst[(((int64_t)n * C + c) * H + h) * W + w] =
                        src[(((int64_t)h * W + w) * C + c) * N + n];
}

void mqo_oihw_to_tap_major(const float *src, float *dst, int Cout, int Cin, int Kh, int Kw)
{
    for (int co = 0; co < Cout; co++)
        for (int ci = 0; ci < Cin; ci++)
            for (int kh = 0; kh < Kh; kh++)
                for (int kw = 0; kw < Kw; kw++)
                    dst[(((int64_t)kh * Kw + kw) * Cout + co) * Cin + ci] =
                        src[(((int64_t)co * Cin + ci) * Kh + kh) * Kw + kw];
}

void mqo_tap_major_to_oihw(const float *src, float *dst, int Cout, int Cin, int Kh, int Kw)
{
    for (int co = 0; co < Cout; co++)
        for (int ci = 0; ci < Cin; ci++)
            for (int kh = 0; kh < Kh; kh++)
                for (int kw = 0; kw < Kw; kw++)
                    dst[(((int64_t)co * Cin + ci) * Kh + kh) * Kw + kw] =
                        src[(((int64_t)kh * Kw + kw) * Cout + co) * Cin + ci];
}

/* ------------------------------------------------------------------------------------------
 * The three GEMMs on the 2-D forms, with an explicit im2col matrix.
 *   X'[k][m]   k = (kh*Kw + kw)*Cin + ci,  m = (ho*Wo + wo)*N + n
 *              = X[ho*sh - ph + kh][wo*sw - pw + kw][ci][n], 0 outside the input
 *   W2[co][k]  = W[kh][kw][co][ci]          (W_{fCout,Cin})
 *   G2[co][m]  = G[ho][wo][co][n]           (G_{YfCout,N})
 *   Y2  = W2 . X'        -> Y[ho][wo][co][n]
 *   GW2 = G2 . X'^T      -> G_W[kh][kw][co][ci]
 *   GX' = W2^T . G2, then col2im: G_X[h][w][ci][n] = sum of GX'[k][m] over the (k, m) that
 *         im2col maps to (h, w, ci, n).
 * Every output also gets A = the same sum over |terms| (the parity tolerance's scale).
 * ------------------------------------------------------------------------------------------ */
typedef struct {
    int32_t N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw;
} mqo_conv;

static int conv_ho(const mqo_conv *p) { return (p->H + 2 * p->ph - p->Kh) / p->sh + 1; }
static int conv_wo(const mqo_conv *p) { return (p->W + 2 * p->pw - p->Kw) / p->sw + 1; }

int mqo_conv_valid(const mqo_conv *p)
{
    if (p->N < 1 || p->Cin < 1 || p->H < 1 || p->W < 1 || p->Cout < 1) return 0;
    if (p->Kh < 1 || p->Kw < 1 || p->sh < 1 || p->sw < 1 || p->ph < 0 || p->pw < 0) return 0;
    if (p->H + 2 * p->ph < p->Kh || p->W + 2 * p->pw < p->Kw) return 0;
    return 1;
}

static double im2col_elem(const mqo_conv *p, const double *x, int64_t k, int64_t m)
{
    const int Wo = conv_wo(p);
    int ci = (int)(k % p->Cin), kw = (int)((k / p->Cin) % p->Kw), kh = (int)(k / ((int64_t)p->Cin * p->Kw));
    int n = (int)(m % p->N), wo = (int)((m / p->N) % Wo), ho = (int)(m / ((int64_t)p->N * Wo));
    int h = ho * p->sh - p->ph + kh, w = wo * p->sw - p->pw + kw;
    if (h < 0 || h >= p->H || w < 0 || w >= p->W) return 0.0;
    return x[(((int64_t)h * p->W + w) * p->Cin + ci) * p->N + n];
}

static double *build_im2col(const mqo_conv *p, const double *x, int64_t K, int64_t M)
{
    double *xc = (double *)malloc(sizeof(double) * (size_t)K * (size_t)M);
    if (!xc) return NULL;
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; k++)
        for (int64_t m = 0; m < M; m++) xc[k * M + m] = im2col_elem(p, x, k, m);
    return xc;
}

static double *build_w2(const mqo_conv *p, const double *w, int64_t K)
{
    double *w2 = (double *)malloc(sizeof(double) * (size_t)p->Cout * (size_t)K);
    if (!w2) return NULL;
    for (int co = 0; co < p->Cout; co++)
        for (int64_t k = 0; k < K; k++) {
            int ci = (int)(k % p->Cin), tap = (int)(k / p->Cin);
            w2[co * K + k] = w[((int64_t)tap * p->Cout + co) * p->Cin + ci];
        }
    return w2;
}

static double *build_g2(const mqo_conv *p, const double *g, int64_t M)
{
    double *g2 = (double *)malloc(sizeof(double) * (size_t)p->Cout * (size_t)M);
    if (!g2) return NULL;
    for (int co = 0; co < p->Cout; co++)
        for (int64_t m = 0; m < M; m++) {
            int64_t n = m % p->N, pix = m / p->N;
            g2[co * M + m] = g[(pix * p->Cout + co) * p->N + n];
        }
    return g2;
}

/* x: [H][W][Cin][N], w: [Kh][Kw][Cout][Cin] -> y, yabs: [Ho][Wo][Cout][N] */
int mqo_conv_fwd(const mqo_conv *p, const double *x, const double *w, double *y, double *yabs)
{
    if (!mqo_conv_valid(p)) return 1;
    const int64_t K = (int64_t)p->Kh * p->Kw * p->Cin, M = (int64_t)conv_ho(p) * conv_wo(p) * p->N;
    double *xc = build_im2col(p, x, K, M), *w2 = build_w2(p, w, K);
    double *y2 = (double *)calloc((size_t)p->Cout * (size_t)M, sizeof(double));
    double *a2 = (double *)calloc((size_t)p->Cout * (size_t)M, sizeof(double));
    int rc = 0;
    if (!xc || !w2 || !y2 || !a2) { rc = 2; goto done; }
    #pragma omp parallel for schedule(static)
    for (int co = 0; co < p->Cout; co++)
        for (int64_t k = 0; k < K; k++) {
            double wv = w2[co * K + k];
            const double *xr = xc + k * M;
            double *yr = y2 + co * M, *ar = a2 + co * M;
            for (int64_t m = 0; m < M; m++) {
                yr[m] += wv * xr[m];
                ar[m] += fabs(wv * xr[m]);
            }
        }
    for (int co = 0; co < p->Cout; co++)
        for (int64_t m = 0; m < M; m++) {
            int64_t n = m % p->N, pix = m / p->N;
            y[(pix * p->Cout + co) * p->N + n] = y2[co * M + m];
            yabs[(pix * p->Cout + co) * p->N + n] = a2[co * M + m];
        }
done:
    free(xc); free(w2); free(y2); free(a2);
    return rc;
}

/* g: [Ho][Wo][Cout][N], x: [H][W][Cin][N] -> gw, gwabs: [Kh][Kw][Cout][Cin] */
int mqo_conv_wgrad(const mqo_conv *p, const double *g, const double *x, double *gw, double *gwabs)
{
    if (!mqo_conv_valid(p)) return 1;
    const int64_t K = (int64_t)p->Kh * p->Kw * p->Cin, M = (int64_t)conv_ho(p) * conv_wo(p) * p->N;
    double *xc = build_im2col(p, x, K, M), *g2 = build_g2(p, g, M);
    int rc = 0;
    if (!xc || !g2) { rc = 2; goto done; }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int co = 0; co < p->Cout; co++)
        for (int64_t k = 0; k < K; k++) {
            const double *gr = g2 + co * M, *xr = xc + k * M;
            double s = 0.0, sa = 0.0;
            for (int64_t m = 0; m < M; m++) {
                s += gr[m] * xr[m];
                sa += fabs(gr[m] * xr[m]);
            }
            int ci = (int)(k % p->Cin), tap = (int)(k / p->Cin);
            gw[((int64_t)tap * p->Cout + co) * p->Cin + ci] = s;
            gwabs[((int64_t)tap * p->Cout + co) * p->Cin + ci] = sa;
        }
done:
    free(xc); free(g2);
    return rc;
}

/* w: [Kh][Kw][Cout][Cin], g: [Ho][Wo][Cout][N] -> gx, gxabs: [H][W][Cin][N] */
int mqo_conv_dgrad(const mqo_conv *p, const double *w, const double *g, double *gx, double *gxabs)
{
    if (!mqo_conv_valid(p)) return 1;
    const int Ho = conv_ho(p), Wo = conv_wo(p);
    const int64_t K = (int64_t)p->Kh * p->Kw * p->Cin, M = (int64_t)Ho * Wo * p->N;
    double *w2 = build_w2(p, w, K), *g2 = build_g2(p, g, M);
    double *gc = (double *)calloc((size_t)K * (size_t)M, sizeof(double));
    double *ac = (double *)calloc((size_t)K * (size_t)M, sizeof(double));
    int rc = 0;
    if (!w2 || !g2 || !gc || !ac) { rc = 2; goto done; }
    /* GX' = W2^T . G2 */
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; k++)
        for (int co = 0; co < p->Cout; co++) {
            double wv = w2[co * K + k];
            const double *gr = g2 + co * M;
            double *out = gc + k * M, *aout = ac + k * M;
            for (int64_t m = 0; m < M; m++) {
                out[m] += wv * gr[m];
                aout[m] += fabs(wv * gr[m]);
            }
        }
    /* col2im */
    const int64_t nx = (int64_t)p->H * p->W * p->Cin * p->N;
    memset(gx, 0, sizeof(double) * (size_t)nx);
    memset(gxabs, 0, sizeof(double) * (size_t)nx);
    for (int64_t k = 0; k < K; k++)
        for (int64_t m = 0; m < M; m++) {
            int ci = (int)(k % p->Cin), kw = (int)((k / p->Cin) % p->Kw), kh = (int)(k / ((int64_t)p->Cin * p->Kw));
            int n = (int)(m % p->N), wo = (int)((m / p->N) % Wo), ho = (int)(m / ((int64_t)p->N * Wo));
            int h = ho * p->sh - p->ph + kh, ww = wo * p->sw - p->pw + kw;
            if (h < 0 || h >= p->H || ww < 0 || ww >= p->W) continue;
            int64_t idx = (((int64_t)h * p->W + ww) * p->Cin + ci) * p->N + n;
            gx[idx] += gc[k * M + m];
            gxabs[idx] += ac[k * M + m];
        }
done:
    free(w2); free(g2); free(gc); free(ac);
    return rc;
}

/* ------------------------------------------------------------------------------------------
 * The same sums, one requested output element at a time (for full-size layers whose explicit
 * im2col would be too large to build). The summation order matches the full routines above,
 * so the results are bit-identical to them.
 * ------------------------------------------------------------------------------------------ */
/* idx[4*i..] = (ho, wo, co, n) */
int mqo_conv_fwd_at(const mqo_conv *p, const double *x, const double *w, const int32_t *idx,
                    int64_t ns, double *y, double *yabs)
{
    if (!mqo_conv_valid(p)) return 1;
    const int Wo = conv_wo(p);
    const int64_t K = (int64_t)p->Kh * p->Kw * p->Cin;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < ns; i++) {
        int ho = idx[4 * i], wo = idx[4 * i + 1], co = idx[4 * i + 2], n = idx[4 * i + 3];
        int64_t m = ((int64_t)ho * Wo + wo) * p->N + n;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; k++) {
            int ci = (int)(k % p->Cin), tap = (int)(k / p->Cin);
            double wv = w[((int64_t)tap * p->Cout + co) * p->Cin + ci];
            double xv = im2col_elem(p, x, k, m);
            s += wv * xv;
            sa += fabs(wv * xv);
        }
        y[i] = s;
        yabs[i] = sa;
    }
    return 0;
}

/* idx[4*i..] = (kh, kw, co, ci) */
int mqo_conv_wgrad_at(const mqo_conv *p, const double *g, const double *x, const int32_t *idx,
                      int64_t ns, double *gw, double *gwabs)
{
    if (!mqo_conv_valid(p)) return 1;
    const int64_t M = (int64_t)conv_ho(p) * conv_wo(p) * p->N;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < ns; i++) {
        int kh = idx[4 * i], kw = idx[4 * i + 1], co = idx[4 * i + 2], ci = idx[4 * i + 3];
        int64_t k = ((int64_t)kh * p->Kw + kw) * p->Cin + ci;
        double s = 0.0, sa = 0.0;
        for (int64_t m = 0; m < M; m++) {
            int64_t n = m % p->N, pix = m / p->N;
            double gv = g[(pix * p->Cout + co) * p->N + n];
            double xv = im2col_elem(p, x, k, m);
            s += gv * xv;
            sa += fabs(gv * xv);
        }
        gw[i] = s;
        gwabs[i] = sa;
    }
    return 0;
}

/* idx[4*i..] = (h, w, ci, n) */
int mqo_conv_dgrad_at(const mqo_conv *p, const double *w, const double *g, const int32_t *idx,
                      int64_t ns, double *gx, double *gxabs)
{
    if (!mqo_conv_valid(p)) return 1;
    const int Ho = conv_ho(p), Wo = conv_wo(p);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < ns; i++) {
        int h = idx[4 * i], ww = idx[4 * i + 1], ci = idx[4 * i + 2], n = idx[4 * i + 3];
        double s = 0.0, sa = 0.0;
        /* increasing k = (kh, kw, ci): the order col2im visits this element in */
        for (int kh = 0; kh < p->Kh; kh++)
            for (int kw = 0; kw < p->Kw; kw++) {
                int th = h + p->ph - kh, tw = ww + p->pw - kw;
                if (th < 0 || tw < 0 || th % p->sh || tw % p->sw) continue;
                int ho = th / p->sh, wo = tw / p->sw;
                if (ho >= Ho || wo >= Wo) continue;
                double v = 0.0, va = 0.0;
                for (int co = 0; co < p->Cout; co++) {
                    double wv = w[(((int64_t)kh * p->Kw + kw) * p->Cout + co) * p->Cin + ci];
                    double gv = g[(((int64_t)ho * Wo + wo) * p->Cout + co) * p->N + n];
                    v += wv * gv;
                    va += fabs(wv * gv);
                }
                s += v;
                sa += va;
            }
        gx[i] = s;
        gxabs[i] = sa;
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------
 * Element-wise array forms of the casts (for exhaustive checks from the test-suite).
 * ------------------------------------------------------------------------------------------ */
void mqo_e4m3_cast_array(const float *s, int64_t n, uint8_t *out)
{
    init_tables();
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)mqo_e4m3_cast(s[i]);
}

void mqo_elem_rne_array(int fmt, const float *a, int64_t n, uint8_t *out)
{
    init_tables();
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)mqo_elem_rne(fmt, a[i]);
}

void mqo_elem_sr_array(int fmt, const float *a, const uint32_t *u16, int64_t n, uint8_t *out)
{
    init_tables();
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)mqo_elem_sr(fmt, a[i], u16[i]);
}

void mqo_sr_u16_array(uint64_t seed, const int64_t *t, const int32_t *e, int64_t n, uint32_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = mqo_sr_u16(seed, t[i], e[i]);
}
