/*
 * Drives every function of the CPU oracle (oracle/rmsnorm_oracle.c) over
 * small shapes, both dtypes, rounded and unrounded outputs, the degenerate
 * cases (no rows, one column, zero rows of data, non-finite values) and its
 * argument checks, on buffers of exactly the size each call may touch.  Built
 * with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers_cpu.py: any read or write past a buffer, and any
 * undefined operation, ends the program with an error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's entry points (it has no header of its own) */
uint16_t oracle_round_bf16(double v);
uint8_t oracle_round_e4m3(double v);
float oracle_round_f32(double v);
void oracle_round_bf16_n(const double *v, uint16_t *out, int64_t n);
void oracle_round_f32_n(const double *v, float *out, int64_t n);
int oracle_rmsnorm_fwd(const void *x, const void *w, void *out, int64_t rows, int64_t hidden, float eps,
                       int dtype, int out_dtype);
int oracle_rmsnorm_residual_fwd(const void *x, const void *residual, const void *w, void *h_out, void *out,
                                int64_t rows, int64_t hidden, float eps, int dtype, int out_dtype);
int oracle_rmsnorm_dynamic_quant_fwd(const void *x, const void *residual, const void *w, void *h_out,
                                     void *q_out, float *scale_out, int64_t rows, int64_t hidden, float eps,
                                     int dtype, int qtype);
int oracle_rmsnorm_bwd(const void *x, const void *w, const void *dy, void *dx, void *dw, int64_t rows,
                       int64_t hidden, float eps, int dtype, int out_dtype);
int oracle_layernorm_fwd(const void *x, const void *gamma, const void *beta, void *out, int64_t rows,
                         int64_t hidden, float eps, int dtype, int out_dtype);
int oracle_kv_rmsnorm_rope_cache(const void *kv, const void *gamma, const float *cos_t, const float *sin_t,
                                 const int32_t *positions, const int64_t *slots, void *norm_cache,
                                 void *rope_cache, int64_t tokens, int64_t heads, int64_t norm_dim,
                                 int64_t rope_dim, int64_t max_pos, int64_t num_slots, float eps, int rope_style,
                                 int dtype, int out_dtype);

enum { F32 = 0, BF16 = 1, F64 = 2 };

static int failures = 0;
static uint64_t state = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* splitmix64 -> [-2, 2) */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / 9007199254740992.0 * 4.0 - 2.0;
}

static size_t esize(int dtype) { return dtype == F32 ? 4 : dtype == BF16 ? 2 : 8; }

/* n elements of the dtype, exactly n * size bytes (at least one byte) */
static void *fill(int dtype, int64_t n) {
    void *p = malloc(n > 0 ? (size_t)n * esize(dtype) : 1);
    int64_t i;
    for (i = 0; i < n; ++i) {
        double v = uniform();
        if (dtype == F32)
            ((float *)p)[i] = (float)v;
        else
            ((uint16_t *)p)[i] = oracle_round_bf16(v);
    }
    return p;
}

static void *out_buf(int dtype, int64_t n) { return malloc(n > 0 ? (size_t)n * esize(dtype) : 1); }

static void expect(const char *what, int got, int want) {
    if (got != want) {
        printf("FAIL %s: %d (want %d)\n", what, got, want);
        ++failures;
    }
}

static void norms(int dtype, int out_dtype, int64_t rows, int64_t hidden) {
    const int64_t n = rows * hidden;
    void *x = fill(dtype, n), *r = fill(dtype, n), *w = fill(dtype, hidden), *b = fill(dtype, hidden);
    void *dy = fill(dtype, n);
    void *y = out_buf(out_dtype, n), *h = out_buf(dtype, n), *dx = out_buf(out_dtype, n);
    void *dw = out_buf(out_dtype, hidden);
    uint8_t *q = malloc(n > 0 ? (size_t)n : 1);
    float *s = malloc(rows > 0 ? (size_t)rows * 4 : 1);
    expect("fwd", oracle_rmsnorm_fwd(x, w, y, rows, hidden, 1e-5f, dtype, out_dtype), 0);
    expect("residual", oracle_rmsnorm_residual_fwd(x, r, w, h, y, rows, hidden, 1e-5f, dtype, out_dtype), 0);
    expect("bwd", oracle_rmsnorm_bwd(x, w, dy, dx, dw, rows, hidden, 1e-5f, dtype, out_dtype), 0);
    expect("bwd dx only", oracle_rmsnorm_bwd(x, w, dy, dx, NULL, rows, hidden, 0.25f, dtype, out_dtype), 0);
    expect("bwd dw only", oracle_rmsnorm_bwd(x, w, dy, NULL, dw, rows, hidden, 0.25f, dtype, out_dtype), 0);
    expect("ln", oracle_layernorm_fwd(x, w, b, y, rows, hidden, 1e-5f, dtype, out_dtype), 0);
    expect("ln no beta", oracle_layernorm_fwd(x, w, NULL, y, rows, hidden, 1e-5f, dtype, out_dtype), 0);
    if (out_dtype != F64) {
        int qt;
        for (qt = 0; qt < 2; ++qt) {
            expect("quant", oracle_rmsnorm_dynamic_quant_fwd(x, NULL, w, NULL, q, s, rows, hidden, 1e-5f, dtype, qt),
                   0);
            expect("quant fused",
                   oracle_rmsnorm_dynamic_quant_fwd(x, r, w, h, q, s, rows, hidden, 1e-5f, dtype, qt), 0);
        }
    }
    /* a zero row (eps > 0 and eps = 0) and a row with a non-finite value */
    if (rows > 0) {
        memset(x, 0, (size_t)hidden * esize(dtype));
        expect("fwd zero row", oracle_rmsnorm_fwd(x, w, y, 1, hidden, 1e-5f, dtype, out_dtype), 0);
        expect("fwd zero row eps 0", oracle_rmsnorm_fwd(x, w, y, 1, hidden, 0.0f, dtype, out_dtype), 0);
        if (dtype == F32)
            ((float *)x)[0] = INFINITY;
        else
            ((uint16_t *)x)[0] = 0x7F80;
        expect("fwd inf", oracle_rmsnorm_fwd(x, w, y, 1, hidden, 1e-5f, dtype, out_dtype), 0);
        expect("ln inf", oracle_layernorm_fwd(x, w, b, y, 1, hidden, 1e-5f, dtype, out_dtype), 0);
        if (out_dtype != F64)
            expect("quant inf", oracle_rmsnorm_dynamic_quant_fwd(x, NULL, w, NULL, q, s, 1, hidden, 1e-5f, dtype, 1),
                   0);
    }
    free(x), free(r), free(w), free(b), free(dy), free(y), free(h), free(dx), free(dw), free(q), free(s);
}

static void kv(int dtype, int out_dtype, int64_t tokens, int64_t heads, int64_t dn, int64_t dr, int style) {
    const int64_t d = dn + dr, max_pos = 16, slots_n = tokens + 3;
    void *x = fill(dtype, tokens * heads * d), *g = fill(dtype, dn);
    float *c = malloc((size_t)(max_pos * (dr / 2) > 0 ? max_pos * (dr / 2) : 1) * 4);
    float *sn = malloc((size_t)(max_pos * (dr / 2) > 0 ? max_pos * (dr / 2) : 1) * 4);
    int32_t *pos = malloc((size_t)(tokens > 0 ? tokens : 1) * 4);
    int64_t *slot = malloc((size_t)(tokens > 0 ? tokens : 1) * 8);
    void *nc = out_buf(out_dtype, slots_n * heads * dn), *rc = out_buf(out_dtype, slots_n * heads * (dr ? dr : 1));
    int64_t i;
    for (i = 0; i < max_pos * (dr / 2); ++i) {
        c[i] = (float)cos(0.1 * (double)i);
        sn[i] = (float)sin(0.1 * (double)i);
    }
    for (i = 0; i < tokens; ++i) {
        pos[i] = (int32_t)(i % 5 == 4 ? max_pos : i % max_pos); /* one in five out of range */
        slot[i] = i % 7 == 6 ? -1 : (i * 3) % slots_n;          /* and some padding tokens */
    }
    expect("kv", oracle_kv_rmsnorm_rope_cache(x, g, c, sn, pos, slot, nc, rc, tokens, heads, dn, dr, max_pos, slots_n,
                                              1e-6f, style, dtype, out_dtype),
           0);
    free(x), free(g), free(c), free(sn), free(pos), free(slot), free(nc), free(rc);
}

int main(void) {
    static const int64_t rows[] = {0, 1, 3, 7};
    static const int64_t hidden[] = {1, 3, 8, 64, 129, 1000};
    static const double specials[] = {0.0, -0.0, 1e-45, 1e-40, 3.4e38, 3.5e38, 1e300, 448.0, 465.0, 1e-9};
    int dt, od, s;
    size_t i, j;
    for (dt = F32; dt <= BF16; ++dt)
        for (od = 0; od < 2; ++od)
            for (i = 0; i < sizeof rows / sizeof rows[0]; ++i)
                for (j = 0; j < sizeof hidden / sizeof hidden[0]; ++j) norms(dt, od ? F64 : dt, rows[i], hidden[j]);
    for (dt = F32; dt <= BF16; ++dt)
        for (od = 0; od < 2; ++od)
            for (s = 0; s < 2; ++s) {
                kv(dt, od ? F64 : dt, 9, 2, 64, 16, s);
                kv(dt, od ? F64 : dt, 5, 1, 8, 0, s);
                kv(dt, od ? F64 : dt, 0, 1, 8, 2, s);
            }
    for (i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        double v = specials[i];
        uint16_t b[2];
        float f[2];
        double two[2];
        two[0] = v, two[1] = -v;
        (void)oracle_round_bf16(v), (void)oracle_round_e4m3(v), (void)oracle_round_f32(v);
        (void)oracle_round_e4m3(-v);
        oracle_round_bf16_n(two, b, 2);
        oracle_round_f32_n(two, f, 2);
    }
    (void)oracle_round_bf16(NAN), (void)oracle_round_e4m3(NAN), (void)oracle_round_bf16(-INFINITY);
    (void)oracle_round_e4m3(INFINITY);
    /* argument checks: each returns -1 without touching its buffers */
    expect("fwd bad rows", oracle_rmsnorm_fwd(NULL, NULL, NULL, -1, 4, 1e-5f, F32, F32), -1);
    expect("fwd bad hidden", oracle_rmsnorm_fwd(NULL, NULL, NULL, 1, 0, 1e-5f, F32, F32), -1);
    expect("fwd bad dtype", oracle_rmsnorm_fwd(NULL, NULL, NULL, 1, 4, 1e-5f, 7, 7), -1);
    expect("quant bad qtype", oracle_rmsnorm_dynamic_quant_fwd(NULL, NULL, NULL, NULL, NULL, NULL, 1, 4, 1e-5f, F32, 9),
           -1);
    expect("kv odd rope", oracle_kv_rmsnorm_rope_cache(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 8, 3, 4, 4,
                                                       1e-6f, 0, F32, F32),
           -1);
    printf("oracle sanitizer run: %d failures\n", failures);
    return failures != 0;
}
