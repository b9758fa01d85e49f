/*
 * tb_oracle.c -- plain scalar CPU oracle for the ternary-weight int8 FFN path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The HIP library never
 * includes, links or calls it, and it shares no source with the HIP path.
 *
 * What it computes (sources, cited by page title and section):
 *   - "perf(bonsai): decode and small packed batches read the FFN from a
 *     ternary copy through a dp4a GEMV" (sparkinfer PR #1154), Summary and
 *     commit message. A Hadamard rotation emits one int8 activation copy,
 *     which gate and up share. A dp4a GEMV takes that copy against the stored
 *     ternary blocks. Block scales are folded per block. Packed steps of up to
 *     8 rows give each row exactly the result it gets alone.
 *   - bonsai-edge-serve README, model list and "kernels/" section. The
 *     ternary format stores groups of 128 weights. The sign variant stores
 *     1 bit per weight. A low-bit GEMV is bit-exact against a scalar
 *     reference.
 * The pages print no formula. Where they are silent, the plain reading below
 * is taken; each reading is listed in the design notes.
 *
 * Precision. The rotation and the quantiser decide integer codes, so they run
 * in fp32 with one IEEE rounding per operation, in the fixed order written
 * below. Build with -ffp-contract=off so that no multiply-add is fused.
 * Everything after the integer dot products (scale fold, SiLU, h) runs in
 * double.
 *
 * Formats (the plain reading of "128 weights per block plus one fp16 scale"):
 *   ternary: codes uint8[n][k/128][32]. Weight i of a row is byte i>>2,
 *            bits 2*(i&3)..+1, least significant first. Code 0 -> 0,
 *            1 -> +1, 2 -> -1, and 3 (never drawn) -> 0.
 *   sign:    codes uint8[n][k/128][16]. Weight i is bit i&7 of byte i>>3.
 *            1 -> +1, 0 -> -1.
 *   scales:  uint16[n][k/128], IEEE binary16 bit patterns.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define TBO_BLOCK 128
#define TBO_FMT_TERNARY2 0
#define TBO_FMT_SIGN1 1

int tbo_version(void) { return 1; }

/* ---- IEEE binary16 -> double, read field by field -------------------------- */
double tbo_half_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: (f/1024) * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* ---- Walsh-Hadamard transform of one 128-block, unnormalised ----------------
 * Butterfly stages with span h = 1, 2, 4, ..., 64, in that order. Each pair
 * (i, i+h) with bit h of i clear becomes (a+b, a-b) in fp32. The result is
 * H v, where H[i][j] = (-1)^popcount(i & j) is the natural-order Sylvester
 * matrix. */
void tbo_fwht128(float *v)
{
    for (int h = 1; h < TBO_BLOCK; h <<= 1)
        for (int i = 0; i < TBO_BLOCK; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

/* dq unit: the int8 step of a block whose rotated maximum is 1, in the
 * orthonormal basis H/sqrt(128): 1 / (127 * sqrt(128)), rounded once to fp32. */
float tbo_dq_unit(void) { return (float)(1.0 / (127.0 * sqrt(128.0))); }

/* ---- Rotate + absmax int8 quantise, per row and 128-block -------------------
 * u = H x_block (fp32), amax = max |u|. If amax is 0, q = 0 and dq = 0.
 * Otherwise inv = 127/amax (fp32 division), q = rint(u * inv) with ties to
 * even, clamped to [-127, 127], and dq = amax * dq_unit. Then q * dq
 * approximates (H / sqrt(128)) x_block. Returns 0, or -1 on a bad shape. */
int tbo_rotate_quant(const float *x, int m, int k, int8_t *q, float *dq)
{
    if (m < 0 || k < 0 || k % TBO_BLOCK)
        return -1;
    const int nb = k / TBO_BLOCK;
    const float unit = tbo_dq_unit();
    for (int r = 0; r < m; ++r)
        for (int b = 0; b < nb; ++b) {
            float u[TBO_BLOCK];
            memcpy(u, x + (size_t)r * k + (size_t)b * TBO_BLOCK, sizeof u);
            tbo_fwht128(u);
            float amax = 0.0f;
            for (int i = 0; i < TBO_BLOCK; ++i) {
                float a = fabsf(u[i]);
                if (a > amax)
                    amax = a;
            }
            int8_t *qb = q + (size_t)r * k + (size_t)b * TBO_BLOCK;
            if (amax == 0.0f) {
                memset(qb, 0, TBO_BLOCK);
                dq[(size_t)r * nb + b] = 0.0f;
                continue;
            }
            const float inv = 127.0f / amax;
            for (int i = 0; i < TBO_BLOCK; ++i) {
                float t = rintf(u[i] * inv);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
                qb[i] = (int8_t)t;
            }
            dq[(size_t)r * nb + b] = amax * unit;
        }
    return 0;
}

/* ---- Weight decode ------------------------------------------------------- */
static size_t row_bytes(int fmt, int k)
{
    return fmt == TBO_FMT_TERNARY2 ? (size_t)k / 4 : (size_t)k / 8;
}

int tbo_weight(const uint8_t *row, int fmt, int i)
{
    if (fmt == TBO_FMT_TERNARY2) {
        int c = (row[i >> 2] >> (2 * (i & 3))) & 3;
        return (c & 1) - (c >> 1);
    }
    return ((row[i >> 3] >> (i & 7)) & 1) ? 1 : -1;
}

/* ---- Per-block integer dot sums: isum[r][n][b] = sum_i t[n][128b+i] * q[r][128b+i] */
int tbo_block_sums(const uint8_t *codes, int fmt, int n, int k, const int8_t *q, int m,
                   int32_t *isum)
{
    if (k % TBO_BLOCK || (fmt != TBO_FMT_TERNARY2 && fmt != TBO_FMT_SIGN1))
        return -1;
    const int nb = k / TBO_BLOCK;
    const size_t rb = row_bytes(fmt, k);
    for (int j = 0; j < n; ++j) {
        const uint8_t *row = codes + (size_t)j * rb;
        for (int b = 0; b < nb; ++b) {
            int t[TBO_BLOCK];
            for (int i = 0; i < TBO_BLOCK; ++i)
                t[i] = tbo_weight(row, fmt, b * TBO_BLOCK + i);
            for (int r = 0; r < m; ++r) {
                const int8_t *qb = q + (size_t)r * k + (size_t)b * TBO_BLOCK;
                int32_t s = 0;
                for (int i = 0; i < TBO_BLOCK; ++i)
                    s += t[i] * qb[i];
                isum[((size_t)r * n + j) * nb + b] = s;
            }
        }
    }
    return 0;
}

/* ---- GEMV with per-block fold -----------------------------------------------
 * y[r][j] = sum_b s[j][b] * dq[r][b] * isum[r][j][b], with every term and the
 * sum in double. sabs[r][j] = sum_b |term|, which sets the tolerance scale.
 * rows: a list of nrows output rows to compute, or NULL for all n rows (then
 * nrows is ignored). Outputs are indexed [r][slot], slot being the position in
 * rows, or the row itself. */
int tbo_gemv_rows(const uint8_t *codes, const uint16_t *scales, int fmt, int n, int k,
                  const int8_t *q, const float *dq, int m, const int32_t *rows, int nrows,
                  double *y, double *sabs)
{
    if (k % TBO_BLOCK || (fmt != TBO_FMT_TERNARY2 && fmt != TBO_FMT_SIGN1))
        return -1;
    const int nb = k / TBO_BLOCK;
    const size_t rb = row_bytes(fmt, k);
    const int count = rows ? nrows : n;
    for (int slot = 0; slot < count; ++slot) {
        const int j = rows ? rows[slot] : slot;
        if (j < 0 || j >= n)
            return -1;
        const uint8_t *row = codes + (size_t)j * rb;
        for (int r = 0; r < m; ++r) {
            y[(size_t)r * count + slot] = 0.0;
            if (sabs)
                sabs[(size_t)r * count + slot] = 0.0;
        }
        for (int b = 0; b < nb; ++b) {
            int t[TBO_BLOCK];
            for (int i = 0; i < TBO_BLOCK; ++i)
                t[i] = tbo_weight(row, fmt, b * TBO_BLOCK + i);
            const double s = tbo_half_to_double(scales[(size_t)j * nb + b]);
            for (int r = 0; r < m; ++r) {
                const int8_t *qb = q + (size_t)r * k + (size_t)b * TBO_BLOCK;
                int32_t isum = 0;
                for (int i = 0; i < TBO_BLOCK; ++i)
                    isum += t[i] * qb[i];
                const double term = s * (double)dq[(size_t)r * nb + b] * (double)isum;
                y[(size_t)r * count + slot] += term;
                if (sabs)
                    sabs[(size_t)r * count + slot] += fabs(term);
            }
        }
    }
    return 0;
}

int tbo_gemv(const uint8_t *codes, const uint16_t *scales, int fmt, int n, int k,
             const int8_t *q, const float *dq, int m, double *y, double *sabs)
{
    return tbo_gemv_rows(codes, scales, fmt, n, k, q, dq, m, NULL, 0, y, sabs);
}

/* ---- The same GEMV from the weights before packing --------------------------
 * Takes the per-weight codes (uint8 [n][k]: ternary 0/1/2, or sign bits 0/1)
 * and the scales already widened to fp32 (float [n][nb]), so no bit unpacking
 * and no binary16 decode happen here. Writes isum[r][j][b] and y[r][j]. */
int tbo_gemv_unpacked(const uint8_t *wcodes, const float *scales_f32, int fmt, int n, int k,
                      const int8_t *q, const float *dq, int m, int32_t *isum, double *y)
{
    if (k % TBO_BLOCK || (fmt != TBO_FMT_TERNARY2 && fmt != TBO_FMT_SIGN1))
        return -1;
    static const int ternary_value[4] = {0, 1, -1, 0};
    const int nb = k / TBO_BLOCK;
    for (int r = 0; r < m; ++r)
        for (int j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                int32_t s = 0;
                for (int i = 0; i < TBO_BLOCK; ++i) {
                    const int c = wcodes[(size_t)j * k + (size_t)b * TBO_BLOCK + i];
                    const int t = fmt == TBO_FMT_TERNARY2 ? ternary_value[c & 3] : (c ? 1 : -1);
                    s += t * q[(size_t)r * k + (size_t)b * TBO_BLOCK + i];
                }
                isum[((size_t)r * n + j) * nb + b] = s;
                acc += (double)scales_f32[(size_t)j * nb + b] * (double)dq[(size_t)r * nb + b] *
                       (double)s;
            }
            y[(size_t)r * n + j] = acc;
        }
    return 0;
}

/* ---- SiLU gate ------------------------------------------------------------ */
double tbo_silu(double z) { return z / (1.0 + exp(-z)); }

/* gate and up read the same int8 copy (q, dq). Outputs, each [m][n] doubles:
 * g, u, h = silu(g) * u, and sg, su, the sums of |term| of g and u. */
int tbo_gateup_silu(const uint8_t *gcodes, const uint16_t *gscales,
                    const uint8_t *ucodes, const uint16_t *uscales, int fmt, int n, int k,
                    const int8_t *q, const float *dq, int m,
                    double *g, double *u, double *h, double *sg, double *su)
{
    int rc = tbo_gemv(gcodes, gscales, fmt, n, k, q, dq, m, g, sg);
    if (rc)
        return rc;
    rc = tbo_gemv(ucodes, uscales, fmt, n, k, q, dq, m, u, su);
    if (rc)
        return rc;
    for (size_t i = 0; i < (size_t)m * n; ++i)
        h[i] = tbo_silu(g[i]) * u[i];
    return 0;
}

/* Down stage: quantise the fp32 hidden rows h[m][k] exactly like x, then the
 * GEMV. Writes qh[m][k], dqh[m][k/128], y[r][slot] and sabs[r][slot] (rows as
 * in tbo_gemv_rows). */
int tbo_ffn_down_rows(const uint8_t *dcodes, const uint16_t *dscales, int fmt, int n, int k,
                      const float *h, int m, int8_t *qh, float *dqh,
                      const int32_t *rows, int nrows, double *y, double *sabs)
{
    int rc = tbo_rotate_quant(h, m, k, qh, dqh);
    if (rc)
        return rc;
    return tbo_gemv_rows(dcodes, dscales, fmt, n, k, qh, dqh, m, rows, nrows, y, sabs);
}
