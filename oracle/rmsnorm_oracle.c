/*
 * RMSNorm reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite (tests/), __graft_entry__.smoke() and the CPU-baseline
 * leg of bench.py may load or call this code.  The product path (the HIP
 * library under memory_bound_rmsnorm_amd/) never links, imports or falls back
 * to it, and the two share no code, header, table or constant.
 *
 * What it computes (plain definition, fp64 throughout, one rounding per
 * output element):
 *
 *   y_j = x_j * rsqrt(mean_j(x_j^2) + eps) * w_j
 *
 *   - formula, eps inside the root, mean = sum / hidden:
 *       xserv "phase 4: transformer core kernels", csrc/normalization/rmsnorm.cu
 *       (header comment) and docs/04-transformer-kernels.md, "Kernel 设计细节 /
 *       RMSNorm" (rms = sqrt(sum(x^2)/hidden_size + eps); y = x / rms * gamma);
 *       the CPU reference `cpu_rmsnorm` in crates/xserv-kernels/tests/ops_test.rs.
 *   - accumulate and scale at high precision, round once at write-back, never
 *       before the weight multiply: gollamago README, "RMSNorm 优化（TileLang）".
 *   - eps arrives as a 32-bit float and gamma has the dtype of x:
 *       xserv crates/xserv-kernels/src/rmsnorm.rs (the `eps: f32` argument and
 *       the dtype-equality assertion).
 *
 *   Fused variant (residual add, then RMSNorm of the sum): the Add that precedes
 *   RmsNorm is folded into the same pass to cut data movement -- TileLang
 *   tutorial ch. 02 "从 PyTorch 到 kernel", section 4.2 (CANN
 *   aclnnAddRmsNormDynamicQuant).  Reading taken here: h = round(x + residual)
 *   is written back in the tensor dtype and the *rounded* h is what gets
 *   normalised, i.e. the result equals an unfused add followed by RMSNorm.
 *
 *   LayerNorm (oracle_layernorm_fwd): mean, centred variance, one rounding.
 *
 *   Backward (dx and dweight for an upstream gradient dy): the plain
 *   derivative of the forward above, in fp64, each output rounded once; dweight
 *   sums over all rows in ascending row order.  See oracle_rmsnorm_bwd.
 *
 * Readings of points the pages leave open:
 *   - rounding is IEEE round-to-nearest, ties to even, directly from fp64 to
 *     the output type (no intermediate fp32 for bf16);
 *   - sum of squares runs over j = 0..hidden-1 in ascending order in fp64;
 *   - NaN/Inf inputs propagate as IEEE arithmetic dictates.
 *
 * dtype codes (private to this file): 0 = float32, 1 = bfloat16 (stored as the
 * upper 16 bits of the float32 pattern).  The normalised outputs can also be
 * written unrounded (out_dtype 2 = float64): the exact-up-to-fp64 value before
 * the one rounding, which is what a comparison needs to tell a correctly
 * rounded result from a truncated or doubly rounded one.  Every other output
 * (the fused residual sum h, which the norm itself consumes rounded, and the
 * quantised codes) is always rounded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2 /* output only: the value before rounding */
#define ORACLE_QUANT_INT8 0
#define ORACLE_QUANT_FP8_E4M3 1

/* Exact widening of one stored element to double. */
static double load_elem(const void *base, int64_t i, int dtype) {
    float f;
    if (dtype == ORACLE_F32) {
        memcpy(&f, (const char *)base + 4 * i, 4);
    } else {
        uint16_t b;
        uint32_t u;
        memcpy(&b, (const char *)base + 2 * i, 2);
        u = (uint32_t)b << 16;
        memcpy(&f, &u, 4);
    }
    return (double)f;
}

/*
 * Round a double to bfloat16 (8 significant bits, exponent range of float32),
 * nearest-even, in a single step.
 *
 * For finite non-zero v with |v| in [2^E, 2^(E+1)), the bf16 grid spacing is
 * 2^(E-7); below the smallest normal (E < -126) the spacing stays 2^-133.
 * |v| / spacing is computed exactly (division by a power of two), rounded to
 * an integer with nearbyint() under the default round-to-nearest-even mode,
 * and scaled back, which again is exact.  A result beyond the largest finite
 * bf16 value overflows to infinity, as IEEE rounding to nearest does.
 */
uint16_t oracle_round_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a, spacing, m;
    int e2;
    float f;
    uint32_t u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(v)) return (uint16_t)(sign | 0x7F80u);
    if (v == 0.0) return sign;
    a = fabs(v);
    (void)frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    e2 -= 1;                      /* now a in [2^e2, 2^(e2+1)) */
    if (e2 < -126) e2 = -126;
    spacing = ldexp(1.0, e2 - 7);
    m = nearbyint(a / spacing) * spacing;
    /* largest finite bf16 is (2 - 2^-7) * 2^127 */
    if (m > ldexp(255.0, 120)) return (uint16_t)(sign | 0x7F80u);
    f = (float)m;                 /* exact: m has at most 8 significant bits */
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

/*
 * Round a double to fp8 e4m3fn (1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, largest finite value 448), nearest-even, with
 * finite values beyond 448 saturating to +-448.  Same construction as the bf16
 * rounding: spacing 2^(E-3) for |v| in [2^E, 2^(E+1)), 2^-9 below the
 * smallest normal 2^-6.  Returns the 8-bit code (sign in bit 7).
 */
uint8_t oracle_round_e4m3(double v) {
    uint8_t sign = signbit(v) ? 0x80u : 0u;
    double a, spacing, m;
    int e2, code;
    if (isnan(v)) return (uint8_t)(sign | 0x7Fu);
    a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) a = 448.0;
    (void)frexp(a, &e2);
    e2 -= 1;
    if (e2 < -6) e2 = -6;
    spacing = ldexp(1.0, e2 - 3);
    m = nearbyint(a / spacing) * spacing;
    if (m > 448.0) m = 448.0;
    if (m < ldexp(1.0, -6)) {
        code = (int)(m * 512.0);            /* subnormal: m = code * 2^-9 */
    } else {
        (void)frexp(m, &e2);                /* m = f * 2^e2, f in [0.5, 1) */
        e2 -= 1;                            /* m in [2^e2, 2^(e2+1)) */
        code = ((e2 + 7) << 3) | (int)(ldexp(m, -e2) * 8.0 - 8.0);
    }
    return (uint8_t)(sign | code);
}

/* Round a double to float32, nearest-even (the C conversion under the default
 * floating-point environment). */
float oracle_round_f32(double v) { return (float)v; }

/* The two roundings above over arrays (for comparisons against unrounded
 * values). */
void oracle_round_bf16_n(const double *v, uint16_t *out, int64_t n) {
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = oracle_round_bf16(v[i]);
}

void oracle_round_f32_n(const double *v, float *out, int64_t n) {
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = oracle_round_f32(v[i]);
}

/* An output type is the input type or, for the normalised outputs, float64. */
static int bad_types(int dtype, int out_dtype) {
    return (dtype != ORACLE_F32 && dtype != ORACLE_BF16) || (out_dtype != dtype && out_dtype != ORACLE_F64);
}

static void store_elem(void *base, int64_t i, double v, int dtype) {
    if (dtype == ORACLE_F64) {
        memcpy((char *)base + 8 * i, &v, 8);
    } else if (dtype == ORACLE_F32) {
        float f = oracle_round_f32(v);
        memcpy((char *)base + 4 * i, &f, 4);
    } else {
        uint16_t b = oracle_round_bf16(v);
        memcpy((char *)base + 2 * i, &b, 2);
    }
}

/* Normalise one row already widened to double: v[0..hidden) -> out row. */
static void normalise_row(const double *v, const void *w, void *out, int64_t out_off,
                          int64_t hidden, float eps, int dtype, int out_dtype) {
    double s = 0.0, mean, r;
    int64_t j;
    for (j = 0; j < hidden; ++j) s += v[j] * v[j];
    mean = s / (double)hidden;
    r = 1.0 / sqrt(mean + (double)eps);
    for (j = 0; j < hidden; ++j)
        store_elem(out, out_off + j, v[j] * r * load_elem(w, j, dtype), out_dtype);
}

/*
 * out[i, :] = RMSNorm(x[i, :]) for i < rows; row-major, contiguous.  out has
 * the dtype of x, or float64 (unrounded) when out_dtype is ORACLE_F64.
 * Returns 0 on success, -1 on a bad argument or allocation failure.
 */
int oracle_rmsnorm_fwd(const void *x, const void *w, void *out, int64_t rows, int64_t hidden,
                       float eps, int dtype, int out_dtype) {
    double *v;
    int64_t i, j;
    if (rows < 0 || hidden <= 0 || bad_types(dtype, out_dtype)) return -1;
    v = (double *)malloc(sizeof(double) * (size_t)hidden);
    if (!v) return -1;
    for (i = 0; i < rows; ++i) {
        for (j = 0; j < hidden; ++j) v[j] = load_elem(x, i * hidden + j, dtype);
        normalise_row(v, w, out, i * hidden, hidden, eps, dtype, out_dtype);
    }
    free(v);
    return 0;
}

/*
 * h[i, :] = round(x[i, :] + residual[i, :]) and out[i, :] = RMSNorm(h[i, :]).
 * The sum is formed in fp64, rounded once to the dtype and written to h_out;
 * the rounded value is what the norm sees.  out_dtype applies to out only.
 */
int oracle_rmsnorm_residual_fwd(const void *x, const void *residual, const void *w, void *h_out,
                                void *out, int64_t rows, int64_t hidden, float eps, int dtype, int out_dtype) {
    double *v;
    int64_t i, j;
    if (rows < 0 || hidden <= 0 || bad_types(dtype, out_dtype)) return -1;
    v = (double *)malloc(sizeof(double) * (size_t)hidden);
    if (!v) return -1;
    for (i = 0; i < rows; ++i) {
        for (j = 0; j < hidden; ++j) {
            int64_t k = i * hidden + j;
            double sum = load_elem(x, k, dtype) + load_elem(residual, k, dtype);
            store_elem(h_out, k, sum, dtype);
            v[j] = load_elem(h_out, k, dtype);
        }
        normalise_row(v, w, out, i * hidden, hidden, eps, dtype, out_dtype);
    }
    free(v);
    return 0;
}

/*
 * Dynamic per-row (per-token) symmetric quantisation of the RMSNorm output,
 * optionally after the residual add -- the Add + RmsNorm + DynamicQuant fusion
 * named in the TileLang tutorial ch. 02, section 4.2 (CANN
 * aclnnAddRmsNormDynamicQuant).  The pages give no formula for DynamicQuant;
 * the reading taken is the plain per-token absmax scheme:
 *
 *   y_j     = v_j * r * w_j               (fp64, never rounded to the dtype)
 *   scale   = max_j |y_j| / Q             (Q = 127 for int8, 448 for e4m3fn)
 *   q_j     = round(y_j / scale)          (nearest-even; int8 clamped to
 *                                          [-127, 127], e4m3fn saturating)
 *
 * and a row whose y is all zero gets scale 0 and codes 0.  v is x, or the
 * rounded h = x + residual when residual is given (h is then written to
 * h_out as in oracle_rmsnorm_residual_fwd).  scale_out receives the scale
 * rounded to float32; the codes use the fp64 scale.
 */
int oracle_rmsnorm_dynamic_quant_fwd(const void *x, const void *residual, const void *w, void *h_out,
                                     void *q_out, float *scale_out, int64_t rows, int64_t hidden,
                                     float eps, int dtype, int qtype) {
    double *v, *y;
    int64_t i, j;
    if (rows < 0 || hidden <= 0 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    if (qtype != ORACLE_QUANT_INT8 && qtype != ORACLE_QUANT_FP8_E4M3) return -1;
    if ((residual == NULL) != (h_out == NULL)) return -1;
    v = (double *)malloc(sizeof(double) * (size_t)hidden);
    y = (double *)malloc(sizeof(double) * (size_t)hidden);
    if (!v || !y) {
        free(v);
        free(y);
        return -1;
    }
    for (i = 0; i < rows; ++i) {
        double s = 0.0, r, amax = 0.0, scale, qmax = qtype == ORACLE_QUANT_INT8 ? 127.0 : 448.0;
        for (j = 0; j < hidden; ++j) {
            int64_t k = i * hidden + j;
            if (residual) {
                store_elem(h_out, k, load_elem(x, k, dtype) + load_elem(residual, k, dtype), dtype);
                v[j] = load_elem(h_out, k, dtype);
            } else {
                v[j] = load_elem(x, k, dtype);
            }
        }
        for (j = 0; j < hidden; ++j) s += v[j] * v[j];
        r = 1.0 / sqrt(s / (double)hidden + (double)eps);
        for (j = 0; j < hidden; ++j) {
            y[j] = v[j] * r * load_elem(w, j, dtype);
            if (fabs(y[j]) > amax) amax = fabs(y[j]);
        }
        scale = amax / qmax;
        scale_out[i] = (float)scale;
        for (j = 0; j < hidden; ++j) {
            double t = amax > 0.0 ? y[j] / scale : 0.0;
            if (qtype == ORACLE_QUANT_INT8) {
                double c = nearbyint(t);
                if (c > 127.0) c = 127.0;
                if (c < -127.0) c = -127.0;
                ((int8_t *)q_out)[i * hidden + j] = (int8_t)c;
            } else {
                ((uint8_t *)q_out)[i * hidden + j] = oracle_round_e4m3(t);
            }
        }
    }
    free(v);
    free(y);
    return 0;
}

/*
 * Backward of y = x * r * w (r = 1/sqrt(sum_k x_k^2 / H + eps)) for an
 * upstream gradient dy -- the norm backward of a training step, which the
 * TileLang tutorial ch. 02, section 1.1(b), describes as mirroring the
 * forward layer by layer.  The pages give no formula; this is the plain
 * derivative, written out in fp64:
 *
 *   dr/dx_k = -r^3 x_k / H, so with c = sum_j dy_j w_j x_j
 *   dx_k    = r dy_k w_k - x_k r^3 c / H
 *   dw_j    = sum_i dy_ij x_ij r_i        (over all rows, fp64)
 *
 * dx and dw are each rounded once to the dtype (or written unrounded when
 * out_dtype is ORACLE_F64).  Either may be NULL (not wanted); the other is
 * unaffected.
 */
int oracle_rmsnorm_bwd(const void *x, const void *w, const void *dy, void *dx, void *dw, int64_t rows,
                       int64_t hidden, float eps, int dtype, int out_dtype) {
    double *acc = NULL;
    int64_t i, j;
    if (rows < 0 || hidden <= 0 || bad_types(dtype, out_dtype)) return -1;
    if (dw) {
        acc = (double *)calloc((size_t)hidden, sizeof(double));
        if (!acc) return -1;
    }
    for (i = 0; i < rows; ++i) {
        double s = 0.0, c = 0.0, r;
        for (j = 0; j < hidden; ++j) {
            double v = load_elem(x, i * hidden + j, dtype);
            s += v * v;
            c += load_elem(dy, i * hidden + j, dtype) * load_elem(w, j, dtype) * v;
        }
        r = 1.0 / sqrt(s / (double)hidden + (double)eps);
        for (j = 0; j < hidden; ++j) {
            double v = load_elem(x, i * hidden + j, dtype);
            double g = load_elem(dy, i * hidden + j, dtype);
            if (dx)
                store_elem(dx, i * hidden + j, r * g * load_elem(w, j, dtype) - v * r * r * r * c / (double)hidden,
                           out_dtype);
            if (acc) acc[j] += g * v * r;
        }
    }
    if (acc) {
        for (j = 0; j < hidden; ++j) store_elem(dw, j, acc[j], out_dtype);
        free(acc);
    }
    return 0;
}

/*
 * LayerNorm, the sibling norm on the same pages: per row,
 *
 *   y_j = gamma_j * (x_j - mu) / sqrt(var + eps) + beta_j,
 *   mu = sum_j x_j / H,  var = sum_j (x_j - mu)^2 / H   (biased, divisor H)
 *
 * (xserv "phase 4: transformer core kernels", csrc/normalization/layernorm.cu
 * header comment and docs/04-transformer-kernels.md "LayerNorm"; the CPU
 * reference cpu_layernorm in crates/xserv-kernels/tests/ops_test.rs divides the
 * centred sum of squares by hidden).  Plain two-pass definition in fp64: the
 * mean first, then the centred squares, then one rounding per output (none
 * when out_dtype is ORACLE_F64).  beta may be NULL (no bias).
 */
int oracle_layernorm_fwd(const void *x, const void *gamma, const void *beta, void *out, int64_t rows,
                         int64_t hidden, float eps, int dtype, int out_dtype) {
    int64_t i, j;
    if (rows < 0 || hidden <= 0 || bad_types(dtype, out_dtype)) return -1;
    for (i = 0; i < rows; ++i) {
        double s = 0.0, q = 0.0, mu, inv;
        for (j = 0; j < hidden; ++j) s += load_elem(x, i * hidden + j, dtype);
        mu = s / (double)hidden;
        for (j = 0; j < hidden; ++j) {
            double d = load_elem(x, i * hidden + j, dtype) - mu;
            q += d * d;
        }
        inv = 1.0 / sqrt(q / (double)hidden + (double)eps);
        for (j = 0; j < hidden; ++j) {
            double v = load_elem(gamma, j, dtype) * (load_elem(x, i * hidden + j, dtype) - mu) * inv;
            if (beta) v += load_elem(beta, j, dtype);
            store_elem(out, i * hidden + j, v, out_dtype);
        }
    }
    return 0;
}

/*
 * KV RMSNorm + RoPE + cache scatter: the fused KV-cache maintenance operator
 * the TileLang tutorial ch. 02 (sections 1.2 and 4.2) cites from CANN
 * (aclnnKvRmsNormRopeCache): the tail axis of kv is split, the left part goes
 * through RMSNorm, the right part through RoPE, and the two results are
 * scattered into two caches.  Readings (the pages give no more):
 *   kv [tokens, heads, norm_dim + rope_dim]; left part norm_dim wide, right
 *   part rope_dim wide (even);
 *   left: y = x * rsqrt(mean(x^2) + eps) * gamma, gamma [norm_dim];
 *   right: RoPE as the xserv rope.cu kernel (phase 4): each pair (a, b) at
 *   position p becomes (a*cos - b*sin, a*sin + b*cos) with cos/sin read from
 *   fp32 tables [max_pos, rope_dim/2] at row p; pairs are adjacent elements
 *   (2i, 2i+1) when rope_style is 1 (xserv) or the two halves (i, i + rope/2)
 *   when it is 0 (the split-head form of the gollamago README, "RoPE");
 *   scatter: token t writes both results at cache row slots[t] (caches
 *   [num_slots, heads, norm_dim] and [num_slots, heads, rope_dim]); a token
 *   whose slot or position is out of range (negative included) writes nothing.
 * fp64 arithmetic, one rounding per output element (none when out_dtype is
 * ORACLE_F64: both caches are then float64).
 */
int oracle_kv_rmsnorm_rope_cache(const void *kv, const void *gamma, const float *cos_t, const float *sin_t,
                                 const int32_t *positions, const int64_t *slots, void *norm_cache,
                                 void *rope_cache, int64_t tokens, int64_t heads, int64_t norm_dim,
                                 int64_t rope_dim, int64_t max_pos, int64_t num_slots, float eps, int rope_style,
                                 int dtype, int out_dtype) {
    int64_t t, h, j, d = norm_dim + rope_dim, half = rope_dim / 2;
    if (tokens < 0 || heads <= 0 || norm_dim <= 0 || rope_dim < 0 || rope_dim % 2 != 0 || max_pos < 0 ||
        num_slots < 0 || bad_types(dtype, out_dtype) || (rope_style != 0 && rope_style != 1))
        return -1;
    for (t = 0; t < tokens; ++t) {
        const int64_t slot = slots[t];
        const int64_t pos = positions[t];
        if (slot < 0 || slot >= num_slots || pos < 0 || pos >= max_pos) continue;
        for (h = 0; h < heads; ++h) {
            const int64_t in = (t * heads + h) * d;
            double s = 0.0, r;
            for (j = 0; j < norm_dim; ++j) {
                double v = load_elem(kv, in + j, dtype);
                s += v * v;
            }
            r = 1.0 / sqrt(s / (double)norm_dim + (double)eps);
            for (j = 0; j < norm_dim; ++j)
                store_elem(norm_cache, (slot * heads + h) * norm_dim + j,
                           load_elem(kv, in + j, dtype) * r * load_elem(gamma, j, dtype), out_dtype);
            for (j = 0; j < half; ++j) {
                const int64_t ia = rope_style ? 2 * j : j, ib = rope_style ? 2 * j + 1 : j + half;
                const double a = load_elem(kv, in + norm_dim + ia, dtype);
                const double b = load_elem(kv, in + norm_dim + ib, dtype);
                const double c = (double)cos_t[pos * half + j], sn = (double)sin_t[pos * half + j];
                const int64_t out = (slot * heads + h) * rope_dim;
                store_elem(rope_cache, out + ia, a * c - b * sn, out_dtype);
                store_elem(rope_cache, out + ib, a * sn + b * c, out_dtype);
            }
        }
    }
    return 0;
}
