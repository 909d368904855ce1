/*
 * nl_oracle.c -- plain fp64 CPU oracle of the bit-nested quantized linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes follows the forum post "bit-nested" POC recipe (page 1 of
 * the source pages):
 *   section 1  randomized Hadamard transform: Sylvester H_b normalised by
 *              1/sqrt(b), block-diagonal with b = largest power of two that
 *              divides n, capped at 4096; x' = H_i S_i x, y = S_o H_o y~.
 *   section 2  2-bit base: 2 bit-planes + one fp16 scale per (row, 128-group),
 *              code -> one of 4 Lloyd-Max levels times the scale.
 *   section 3  residual: b-bit integers on an evenly spaced grid centred on 0, times one fp16
 *              scale per (row, 128-group), in the same rotated basis.
 *   section 4  verifier forward for one Linear: y~ = (Q_base + Q_resid) x',
 *              draft forward = the same without the residual term.
 * Readings where the page is silent (bit order of the planes and fields,
 * code -> level order, output rotation optional) are the canonical storage
 * format described in synth/__init__.py.
 *
 * Everything is evaluated in double precision: codes are decoded exactly,
 * fp16 scales and bf16 activations are widened exactly, the FWHT and the dot
 * products are fp64 with sequential sums.  Loops over output rows run under
 * OpenMP; each row's sum is sequential, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define NLO_GROUP 128

/* POC section 1, "Block size": the largest power of two dividing n, capped
 * at 4096 (n = 4096 -> 4096, 8192 -> 4096, 15360 -> 1024, 3840 -> 256). */
int nlo_block_size(int n)
{
    if (n <= 0) return 0;
    int b = 1;
    while ((n % (b * 2)) == 0 && b * 2 <= 4096) b *= 2;
    return b;
}

/* In-place block-diagonal normalised Sylvester-Hadamard transform of v[0..n)
 * with blocks of b (b a power of two dividing n).  POC section 1: H starts as
 * [1] and doubles as [[H, H], [H, -H]]; the butterfly (a, c) -> (a + c, a - c)
 * over strides 1, 2, 4, ... applies that matrix in its natural (Sylvester)
 * order, then each block is divided by sqrt(b). */
void nlo_fwht_b(double *v, int n, int b)
{
    double inv = 1.0 / sqrt((double)b);
    for (int base = 0; base + b <= n; base += b) {
        double *w = v + base;
        for (int h = 1; h < b; h *= 2) {
            for (int i = 0; i < b; i += 2 * h) {
                for (int j = i; j < i + h; ++j) {
                    double a = w[j], c = w[j + h];
                    w[j] = a + c;
                    w[j + h] = a - c;
                }
            }
        }
        for (int j = 0; j < b; ++j) w[j] *= inv;
    }
}

/* The rotation of a length-n vector with the block size rule above. */
void nlo_fwht(double *v, int n) { nlo_fwht_b(v, n, nlo_block_size(n)); }

/* IEEE binary16 bit pattern -> double (exact). */
double nlo_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                  /* zero / subnormal */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m | 0x400), e - 25);
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> double (exact): the top half of an fp32. */
double nlo_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int nlo_groups(int d_in) { return (d_in + NLO_GROUP - 1) / NLO_GROUP; }

/* POC section 2 storage: code of weight (r, k) from the two bit-planes of
 * its group (plane 0 = bit 0, plane 1 = bit 1, LSB first). */
int nlo_base_code(const uint8_t *base_codes, int d_in, int r, int k)
{
    int G = nlo_groups(d_in);
    const uint8_t *grp = base_codes + ((size_t)r * G + k / NLO_GROUP) * 32;
    int j = k % NLO_GROUP;
    int b0 = (grp[j >> 3] >> (j & 7)) & 1;
    int b1 = (grp[16 + (j >> 3)] >> (j & 7)) & 1;
    return b0 | (b1 << 1);
}

/* POC section 3: b-bit two's-complement residual code of weight (r, k),
 * field j of the group at bits [j*b, j*b + b) of its little-endian bit
 * string, sign-extended. */
int nlo_resid_code(const uint8_t *resid_codes, int d_in, int bits, int r, int k)
{
    int G = nlo_groups(d_in);
    const uint8_t *grp = resid_codes + ((size_t)r * G + k / NLO_GROUP) * (16 * bits);
    int j = k % NLO_GROUP;
    int v = 0;
    for (int t = 0; t < bits; ++t) {
        int bit = j * bits + t;
        v |= ((grp[bit >> 3] >> (bit & 7)) & 1) << t;
    }
    if (v & (1 << (bits - 1))) v -= (1 << bits);
    return v;
}

/* Dequantised rotated-basis row r of W~ (POC sections 2-3):
 *   W~[r,k] = levels[c] * s_base[r,g] (+ q * s_resid[r,g] in verify mode). */
void nlo_dequant_row(int d_in, int bits, int verify,
                     const uint8_t *base_codes, const uint16_t *base_scales,
                     const uint8_t *resid_codes, const uint16_t *resid_scales,
                     const float *levels, int r, double *w)
{
    int G = nlo_groups(d_in);
    for (int k = 0; k < d_in; ++k) {
        int g = k / NLO_GROUP;
        double sb = nlo_half_to_double(base_scales[(size_t)r * G + g]);
        double v = (double)levels[nlo_base_code(base_codes, d_in, r, k)] * sb;
        if (verify) {
            double sr = nlo_half_to_double(resid_scales[(size_t)r * G + g]);
            v += (double)nlo_resid_code(resid_codes, d_in, bits, r, k) * sr;
        }
        w[k] = v;
    }
}

/* Input rotation of POC section 1/4: x' = H_i (S_i x), x given as bf16.
 * xr is [T][d_in]. */
void nlo_rotate_input(int d_in, const int8_t *sign_in, const uint16_t *x_bf16,
                      int T, double *xr)
{
    for (int t = 0; t < T; ++t) {
        double *v = xr + (size_t)t * d_in;
        for (int k = 0; k < d_in; ++k)
            v[k] = (double)sign_in[k] * nlo_bf16_to_double(x_bf16[(size_t)t * d_in + k]);
        nlo_fwht(v, d_in);
    }
}

/* The forward of one nested Linear for rows [row0, row1) (POC section 4):
 *   x'  = H_i S_i x
 *   y~  = W~ x'           (W~ in verify mode includes the residual)
 *   y   = S_o H_o y~      (only when sign_out != NULL; then [row0, row1)
 *                          must be whole output blocks)
 * y is [T][row1 - row0].  verify = 0 is the draft forward.  Returns 0, or
 * -1 on bad arguments. */
int nlo_forward_rows(int d_out, int d_in, int bits, int verify,
                     const uint8_t *base_codes, const uint16_t *base_scales,
                     const uint8_t *resid_codes, const uint16_t *resid_scales,
                     const float *levels, const int8_t *sign_in, const int8_t *sign_out,
                     const uint16_t *x_bf16, int T, int row0, int row1, double *y)
{
    if (d_out <= 0 || d_in <= 0 || T < 0 || row0 < 0 || row1 > d_out || row0 > row1) return -1;
    if (verify && (bits < 2 || bits > 8 || !resid_codes || !resid_scales)) return -1;
    int nr = row1 - row0;
    if (sign_out) {
        int b = nlo_block_size(d_out);
        if (row0 % b || nr % b) return -1;
    }
    if (T == 0 || nr == 0) return 0;
    double *xr = (double *)malloc(sizeof(double) * (size_t)T * d_in);
    if (!xr) return -1;
    nlo_rotate_input(d_in, sign_in, x_bf16, T, xr);

    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)d_in);
        if (!w) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(static)
            for (int r = row0; r < row1; ++r) {
                nlo_dequant_row(d_in, bits, verify, base_codes, base_scales,
                                resid_codes, resid_scales, levels, r, w);
                for (int t = 0; t < T; ++t) {
                    const double *xt = xr + (size_t)t * d_in;
                    double s = 0.0;
                    for (int k = 0; k < d_in; ++k) s += w[k] * xt[k];
                    y[(size_t)t * nr + (r - row0)] = s;
                }
            }
            free(w);
        }
    }
    free(xr);
    if (err) return -1;
    if (sign_out) {
        int b = nlo_block_size(d_out);
        for (int t = 0; t < T; ++t) {
            double *v = y + (size_t)t * nr;
            nlo_fwht_b(v, nr, b);
            for (int r = 0; r < nr; ++r) v[r] *= (double)sign_out[row0 + r];
        }
    }
    return 0;
}

int nlo_forward(int d_out, int d_in, int bits, int verify,
                const uint8_t *base_codes, const uint16_t *base_scales,
                const uint8_t *resid_codes, const uint16_t *resid_scales,
                const float *levels, const int8_t *sign_in, const int8_t *sign_out,
                const uint16_t *x_bf16, int T, double *y)
{
    return nlo_forward_rows(d_out, d_in, bits, verify, base_codes, base_scales,
                            resid_codes, resid_scales, levels, sign_in, sign_out,
                            x_bf16, T, 0, d_out, y);
}

/* Decode every code of rows [row0, row0 + nrows): base index (0..3) and the
 * sign-extended residual integer, [nrows][d_in] each. */
void nlo_decode(int d_in, int bits, const uint8_t *base_codes, const uint8_t *resid_codes,
                int row0, int nrows, uint8_t *base_idx, int8_t *resid)
{
    for (int r = 0; r < nrows; ++r)
        for (int k = 0; k < d_in; ++k) {
            base_idx[(size_t)r * d_in + k] = (uint8_t)nlo_base_code(base_codes, d_in, row0 + r, k);
            if (resid && resid_codes)
                resid[(size_t)r * d_in + k] =
                    (int8_t)nlo_resid_code(resid_codes, d_in, bits, row0 + r, k);
        }
}

/* Threads the OpenMP loops use (reported with the CPU baseline timing). */
#ifdef _OPENMP
#include <omp.h>
int nlo_num_threads(void) { return omp_get_max_threads(); }
#else
int nlo_num_threads(void) { return 1; }
#endif
