/*
 * oracle_sanitize.c -- drives every entry of the C oracle (oracle/nl_oracle.c)
 * over exact-size heap buffers so that an AddressSanitizer / UBSan build of
 * the oracle reports any out-of-bounds access, overflow or undefined shift.
 * Test infrastructure: built and run by tests/test_oracle_sanitize.py with
 * gcc only (no GPU code).  Exit status 0 = every call returned and every
 * output is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int nlo_block_size(int n);
void nlo_fwht_b(double *v, int n, int b);
void nlo_fwht(double *v, int n);
double nlo_half_to_double(uint16_t h);
double nlo_bf16_to_double(uint16_t b);
void nlo_dequant_row(int d_in, int bits, int verify, const uint8_t *bc, const uint16_t *bs,
                     const uint8_t *rc, const uint16_t *rs, const float *levels, int r, double *w);
void nlo_rotate_input(int d_in, const int8_t *sign_in, const uint16_t *x, int T, double *xr);
int nlo_forward_rows(int d_out, int d_in, int bits, int verify, const uint8_t *bc, const uint16_t *bs,
                     const uint8_t *rc, const uint16_t *rs, const float *levels, const int8_t *si,
                     const int8_t *so, const uint16_t *x, int T, int row0, int row1, double *y);
void nlo_decode(int d_in, int bits, const uint8_t *bc, const uint8_t *rc, int row0, int nrows,
                uint8_t *bi, int8_t *rq);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    /* splitmix64: byte noise for buffers, not part of any computation checked */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static void *alloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) exit(3); return p; }
static void fill_bytes(uint8_t *p, size_t n) { for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)next_u32(); }

/* finite fp16 / bf16 bit patterns, every exponent but the all-ones one */
static uint16_t finite_half(void) { uint16_t h = (uint16_t)next_u32(); return (h & 0x7C00) == 0x7C00 ? h & 0xBFFF : h; }
static uint16_t finite_bf16(void) { uint16_t h = (uint16_t)next_u32(); return (h & 0x7F80) == 0x7F80 ? h & 0xBFFF : h; }

static int check_finite(const double *v, size_t n, const char *what)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) { fprintf(stderr, "%s: non-finite at %zu\n", what, i); return 1; }
    return 0;
}

static int run_case(int d_out, int d_in, int bits, int T, int two_sided)
{
    const int G = (d_in + 127) / 128;
    const size_t nb = (size_t)d_out * G * 32, nr = (size_t)d_out * G * 16 * (size_t)(bits ? bits : 1);
    const size_t ns = (size_t)d_out * G;
    uint8_t *bc = alloc(nb), *rc = bits ? alloc(nr) : NULL;
    uint16_t *bs = alloc(ns * 2), *rs = bits ? alloc(ns * 2) : NULL;
    int8_t *si = alloc((size_t)d_in), *so = two_sided ? alloc((size_t)d_out) : NULL;
    uint16_t *x = alloc((size_t)T * d_in * 2);
    float *lev = alloc(4 * sizeof(float));
    double *y = alloc((size_t)T * d_out * sizeof(double));
    double *w = alloc((size_t)d_in * sizeof(double));
    uint8_t *bi = alloc((size_t)d_out * d_in);
    int8_t *rq = alloc((size_t)d_out * d_in);
    int bad = 0;

    fill_bytes(bc, nb);
    if (rc) fill_bytes(rc, nr);
    for (size_t i = 0; i < ns; ++i) { bs[i] = finite_half() & 0x3FFF; if (rs) rs[i] = finite_half() & 0x3FFF; }
    for (int k = 0; k < d_in; ++k) si[k] = (next_u32() & 1) ? 1 : -1;
    if (so) for (int r = 0; r < d_out; ++r) so[r] = (next_u32() & 1) ? 1 : -1;
    for (size_t i = 0; i < (size_t)T * d_in; ++i) x[i] = finite_bf16() & 0xDFFF;  /* |x| < 2^65 */
    lev[0] = -1.5f; lev[1] = -0.45f; lev[2] = 0.45f; lev[3] = 1.5f;

    for (int verify = 0; verify <= (bits ? 1 : 0); ++verify) {
        if (nlo_forward_rows(d_out, d_in, bits, verify, bc, bs, rc, rs, lev, si, so, x, T, 0, d_out, y)) {
            fprintf(stderr, "forward_rows rejected %d x %d\n", d_out, d_in);
            bad = 1;
        }
        bad |= check_finite(y, (size_t)T * d_out, "forward");
        /* a row subset: whole output blocks in the two-sided form */
        int b = two_sided ? nlo_block_size(d_out) : 1;
        int r0 = d_out >= 2 * b ? b : 0, r1 = d_out;
        if (nlo_forward_rows(d_out, d_in, bits, verify, bc, bs, rc, rs, lev, si, so, x, T, r0, r1, y)) bad = 1;
        bad |= check_finite(y, (size_t)T * (r1 - r0), "forward rows");
        nlo_dequant_row(d_in, bits, verify, bc, bs, rc, rs, lev, d_out - 1, w);
        bad |= check_finite(w, (size_t)d_in, "dequant_row");
    }
    nlo_decode(d_in, bits, bc, rc, 0, d_out, bi, bits ? rq : NULL);
    for (size_t i = 0; i < (size_t)d_out * d_in; ++i) if (bi[i] > 3) bad = 1;
    /* bad arguments are rejected, not read */
    if (nlo_forward_rows(d_out, d_in, bits, 0, bc, bs, rc, rs, lev, si, so, x, T, 0, d_out + 1, y) != -1) bad = 1;
    if (T == 0 && nlo_forward_rows(d_out, d_in, bits, 0, bc, bs, rc, rs, lev, si, so, x, 0, 0, d_out, y) != 0) bad = 1;

    free(bc); free(rc); free(bs); free(rs); free(si); free(so); free(x); free(lev); free(y); free(w);
    free(bi); free(rq);
    if (bad) fprintf(stderr, "case %d x %d bits %d T %d two %d failed\n", d_out, d_in, bits, T, two_sided);
    return bad;
}

int main(void)
{
    int bad = 0;
    /* fwht over every power-of-two block up to 4096, ragged counts of blocks */
    for (int b = 1; b <= 4096; b *= 2) {
        int n = 3 * b;
        double *v = alloc((size_t)n * sizeof(double));
        for (int i = 0; i < n; ++i) v[i] = (double)(int)(next_u32() % 2001) - 1000.0;
        nlo_fwht_b(v, n, b);
        nlo_fwht(v, n);
        bad |= check_finite(v, (size_t)n, "fwht");
        free(v);
    }
    for (uint32_t h = 0; h < 65536; ++h) { (void)nlo_half_to_double((uint16_t)h); (void)nlo_bf16_to_double((uint16_t)h); }
    for (int n = -3; n <= 20000; n += 7) (void)nlo_block_size(n);
    static const int shapes[][5] = {
        /* d_out, d_in, bits, T, two-sided */
        {8, 8, 8, 1, 1},      {24, 200, 7, 3, 1},  {12, 384, 8, 5, 0},  {96, 1000, 6, 2, 0},
        {256, 128, 6, 4, 1},  {64, 4096, 6, 1, 0}, {33, 130, 0, 2, 0},  {4096, 64, 8, 2, 1},
        {5, 127, 7, 0, 0},
    };
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        bad |= run_case(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4]);
    printf("oracle sanitize: %s\n", bad ? "FAILED" : "ok");
    return bad;
}
