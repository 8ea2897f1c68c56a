/*
 * Argument validation and launch-shape choice of the C-ABI library on a
 * machine with no GPU, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer on its host code (tests/test_sanitizers_cpu.py):
 *   - every entry point's automatic choice over widths 1 .. 2^20 (the KV
 *     operator: norm widths 1 .. 1100 with several rotated widths), both
 *     alignments, several row counts and both dtypes must pass validation
 *     and fail only at the launch itself (RMSNORM_ERR_RUNTIME: no device);
 *   - forced configurations over the whole range of every field, valid or
 *     not, and extreme sizes must be answered with a status, never with an
 *     out-of-bounds table read, an integer overflow or a crash.
 * The device addresses are fake and 64 GiB apart; nothing is ever launched.
 */
#include <stdint.h>
#include <stdio.h>

#include "rmsnorm.h"

static int failures = 0;

#define BASE 0x700000000000ull
#define AT(i) ((void*)(uintptr_t)(BASE + ((uint64_t)(i) << 36)))

static void expect_launch(const char* what, rmsnorm_status_t s, int64_t rows, int64_t hidden, int dtype, int off) {
    if (s != RMSNORM_ERR_RUNTIME) {
        if (failures < 20)
            printf("FAIL %s rows %lld hidden %lld dtype %d offset %d: status %d\n", what, (long long)rows,
                   (long long)hidden, dtype, off, (int)s);
        ++failures;
    }
}

static void expect_status(const char* what, rmsnorm_status_t s) {
    if (s != RMSNORM_ERR_INVALID_ARG && s != RMSNORM_ERR_RUNTIME && s != RMSNORM_OK) {
        if (failures < 20) printf("FAIL %s: status %d\n", what, (int)s);
        ++failures;
    }
}

static void automatic(void) {
    static const int64_t rows_list[] = {1, 300, 1024, 4096, 12289};
    int64_t hidden;
    size_t r;
    int dt, o;
    for (r = 0; r < sizeof rows_list / sizeof rows_list[0]; ++r)
        for (dt = 0; dt < 2; ++dt)
            for (o = 0; o < 2; ++o)
                for (hidden = 1; hidden <= (1 << 20); hidden += hidden < 2048 ? 1 : hidden < 32768 ? 61 : 4093) {
                    const int64_t rows = rows_list[r];
                    const int off = o ? (dt ? 2 : 4) : 0;
                    const rmsnorm_dtype_t d = (rmsnorm_dtype_t)dt;
                    size_t ws = 0;
                    expect_launch("fwd", rmsnorm_fwd((char*)AT(0) + off, AT(1), (char*)AT(2) + off, rows, hidden, 1e-5f,
                                                     d, NULL),
                                  rows, hidden, dt, off);
                    expect_launch("residual", rmsnorm_residual_fwd((char*)AT(0) + off, (char*)AT(3) + off, AT(1),
                                                                   (char*)AT(4) + off, (char*)AT(2) + off, rows,
                                                                   hidden, 1e-5f, d, NULL),
                                  rows, hidden, dt, off);
                    expect_launch("quant", rmsnorm_dynamic_quant_fwd((char*)AT(0) + off, NULL, AT(1), NULL, AT(5),
                                                                     (float*)AT(6), rows, hidden, 1e-5f, d,
                                                                     RMSNORM_QUANT_INT8, NULL),
                                  rows, hidden, dt, off);
                    expect_launch("quant fused",
                                  rmsnorm_dynamic_quant_fwd((char*)AT(0) + off, (char*)AT(3) + off, AT(1),
                                                            (char*)AT(4) + off, AT(5), (float*)AT(6), rows, hidden,
                                                            1e-5f, d, RMSNORM_QUANT_FP8_E4M3, NULL),
                                  rows, hidden, dt, off);
                    expect_launch("bwd dx", rmsnorm_bwd((char*)AT(0) + off, AT(1), (char*)AT(3) + off,
                                                        (char*)AT(2) + off, NULL, rows, hidden, 1e-5f, d, NULL, 0,
                                                        NULL),
                                  rows, hidden, dt, off);
                    if (rmsnorm_bwd_workspace_size(rows, hidden, d, NULL, &ws) != RMSNORM_OK) ++failures;
                    expect_launch("bwd dx dw", rmsnorm_bwd((char*)AT(0) + off, AT(1), (char*)AT(3) + off,
                                                           (char*)AT(2) + off, AT(7), rows, hidden, 1e-5f, d, AT(8),
                                                           ws, NULL),
                                  rows, hidden, dt, off);
                    expect_launch("ln", layernorm_fwd((char*)AT(0) + off, AT(1), AT(9), (char*)AT(2) + off, rows,
                                                      hidden, 1e-5f, d, NULL),
                                  rows, hidden, dt, off);
                }
}

static void automatic_kv(void) {
    static const int64_t rope[] = {0, 2, 16, 64, 128};
    int64_t dn, h;
    size_t r;
    int dt, style, o;
    for (dt = 0; dt < 2; ++dt)
        for (o = 0; o < 2; ++o)
            for (style = 0; style < 2; ++style)
                for (r = 0; r < sizeof rope / sizeof rope[0]; ++r)
                    for (h = 1; h <= 8; h *= 8)
                        for (dn = 1; dn <= 1100; ++dn) {
                            const int off = o ? (dt ? 2 : 4) : 0;
                            expect_launch("kv", kv_rmsnorm_rope_cache((char*)AT(0) + off, AT(1), (const float*)AT(2),
                                                                      (const float*)AT(3), (const int32_t*)AT(4),
                                                                      (const int64_t*)AT(5), (char*)AT(6) + off,
                                                                      (char*)AT(7) + off, 300, h, dn, rope[r], 4096,
                                                                      512, 1e-6f, style, (rmsnorm_dtype_t)dt, NULL),
                                          dn, rope[r], dt, off);
                        }
}

static void forced(void) {
    static const int64_t shapes[][2] = {{8, 1}, {8, 7}, {8, 64}, {8, 2048}, {8, 2049}, {8, 8192}, {3, 81920},
                                        {2, 131072}, {5, 163840}};
    /* rows_per_block, max_blocks, lanes_per_row, weight_lds */
    static const int32_t rest[][4] = {{1, 0, 0, 0},  {2, 0, 0, 0},   {4, 2, 0, 0},   {1, 0, 16, 0},
                                      {8, 0, 8, 0},  {1, 0, 0, 1},   {4, 0, 0, 1},   {-1, -1, -1, -1},
                                      {0, 0, 12, 2}, {9, 3, 64, 0},  {16, 0, 32, 0}, {64, 0, 8, 0}};
    size_t s, k;
    int32_t path, wpr, per;
    int dt;
    for (s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (dt = 0; dt < 2; ++dt)
            for (path = -1; path <= 6; ++path)
                for (wpr = -1; wpr <= 17; ++wpr)
                    for (per = -1; per <= 17; per += (per < 11 ? 1 : 3))
                        for (k = 0; k < sizeof rest / sizeof rest[0]; ++k) {
                            const rmsnorm_config_t c = {path, wpr, per, rest[k][0], rest[k][1], rest[k][2], rest[k][3]};
                            const int64_t rows = shapes[s][0], hidden = shapes[s][1];
                            const rmsnorm_dtype_t d = (rmsnorm_dtype_t)dt;
                            size_t ws = 0;
                            expect_status("fwd_ex", rmsnorm_fwd_ex(AT(0), AT(1), AT(2), rows, hidden, 1e-5f, d, &c,
                                                                   NULL));
                            expect_status("residual_ex", rmsnorm_residual_fwd_ex(AT(0), AT(3), AT(1), AT(4), AT(2),
                                                                                 rows, hidden, 1e-5f, d, &c, NULL));
                            expect_status("quant_ex",
                                          rmsnorm_dynamic_quant_fwd_ex(AT(0), NULL, AT(1), NULL, AT(5), (float*)AT(6),
                                                                       rows, hidden, 1e-5f, d, RMSNORM_QUANT_INT8, &c,
                                                                       NULL));
                            (void)rmsnorm_bwd_workspace_size(rows, hidden, d, &c, &ws);
                            expect_status("bwd_ex", rmsnorm_bwd_ex(AT(0), AT(1), AT(3), AT(2), AT(7), rows, hidden,
                                                                   1e-5f, d, AT(8), 1u << 30, &c, NULL));
                            expect_status("ln_ex", layernorm_fwd_ex(AT(0), AT(1), AT(9), AT(2), rows, hidden, 1e-5f, d,
                                                                    &c, NULL));
                            expect_status("kv_ex", kv_rmsnorm_rope_cache_ex(
                                                       AT(0), AT(1), (const float*)AT(2), (const float*)AT(3),
                                                       (const int32_t*)AT(4), (const int64_t*)AT(5), AT(6), AT(7),
                                                       rows, 1, hidden > 64 ? 64 : hidden + hidden % 2, 16, 64,
                                                       rows + 2, 1e-6f, 1, d, &c, NULL));
                        }
}

static void extremes(void) {
    static const int64_t big[] = {INT64_MAX, INT64_MAX / 2, (int64_t)1 << 62, (int64_t)1 << 40, (int64_t)1 << 31,
                                  ((int64_t)1 << 31) - 1, -1, 0};
    rmsnorm_config_t c;
    size_t i, j, ws;
    for (i = 0; i < sizeof big / sizeof big[0]; ++i)
        for (j = 0; j < sizeof big / sizeof big[0]; ++j) {
            const int64_t r = big[i], h = big[j];
            expect_status("fwd big", rmsnorm_fwd(AT(0), AT(1), AT(2), r, h, 1e-5f, RMSNORM_DTYPE_BF16, NULL));
            expect_status("residual big", rmsnorm_residual_fwd(AT(0), AT(3), AT(1), AT(4), AT(2), r, h, 1e-5f,
                                                               RMSNORM_DTYPE_F32, NULL));
            expect_status("quant big", rmsnorm_dynamic_quant_fwd(AT(0), NULL, AT(1), NULL, AT(5), (float*)AT(6), r, h,
                                                                 1e-5f, RMSNORM_DTYPE_BF16, RMSNORM_QUANT_INT8, NULL));
            expect_status("bwd big", rmsnorm_bwd(AT(0), AT(1), AT(3), AT(2), AT(7), r, h, 1e-5f, RMSNORM_DTYPE_BF16,
                                                 AT(8), 1u << 30, NULL));
            expect_status("ln big", layernorm_fwd(AT(0), AT(1), NULL, AT(2), r, h, 1e-5f, RMSNORM_DTYPE_BF16, NULL));
            expect_status("kv big", kv_rmsnorm_rope_cache(AT(0), AT(1), (const float*)AT(2), (const float*)AT(3),
                                                          (const int32_t*)AT(4), (const int64_t*)AT(5), AT(6), AT(7),
                                                          r, h, h, 64, r, r, 1e-6f, 0, RMSNORM_DTYPE_BF16, NULL));
            expect_status("select", rmsnorm_select_config(r, h, RMSNORM_DTYPE_BF16, 1, 1, &c));
            expect_status("select quant", rmsnorm_select_quant_config(r, h, RMSNORM_DTYPE_F32, 0, 1, &c));
            expect_status("select bwd", rmsnorm_select_bwd_config(r, h, RMSNORM_DTYPE_BF16, 1, &c));
            expect_status("select ln", layernorm_select_config(r, h, RMSNORM_DTYPE_BF16, 0, &c));
            expect_status("select kv", kv_select_config(r, h, h, 64, 1, RMSNORM_DTYPE_BF16, 1, &c));
            expect_status("workspace", rmsnorm_bwd_workspace_size(r, h, RMSNORM_DTYPE_BF16, NULL, &ws));
        }
}

int main(void) {
    automatic();
    automatic_kv();
    forced();
    extremes();
    printf("abi sanitizer run: %d failures\n", failures);
    return failures != 0;
}
