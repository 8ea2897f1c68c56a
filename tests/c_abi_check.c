/*
 * A plain C11 caller of the library's C ABI, built and run by
 * tests/test_c_abi_cpu.py on a machine without a GPU.  It exercises only the
 * entry points and argument checks that make no HIP call: status strings,
 * configuration queries, the workspace query, size / pointer / dtype
 * validation and the rows == 0 early return.  Each line printed is
 * "name value" for the test to compare; the exit status is the number of
 * failed checks.
 */
#include <stdio.h>
#include <string.h>

#include "hbm_copy.h"
#include "rmsnorm.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
    printf("%s %d\n", what, got);
    if (got != want) {
        fprintf(stderr, "FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

int main(void) {
    const rmsnorm_status_t all[] = {RMSNORM_OK, RMSNORM_ERR_INVALID_ARG, RMSNORM_ERR_UNSUPPORTED_DTYPE,
                                    RMSNORM_ERR_RUNTIME};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) {
        const char* s = rmsnorm_status_string(all[i]);
        expect("status_string_nonempty", s != NULL && strlen(s) > 0, 1);
    }

    /* automatic configurations of the stated shapes (no HIP call) */
    rmsnorm_config_t c;
    memset(&c, 0, sizeof c);
    expect("select_fwd", rmsnorm_select_config(16384, 8192, RMSNORM_DTYPE_BF16, 1, 0, &c), RMSNORM_OK);
    expect("fwd_path", c.path, RMSNORM_PATH_VECTOR);
    expect("fwd_waves_per_row", c.waves_per_row, 8);
    expect("fwd_items_per_lane", c.items_per_lane, 2);
    expect("select_fwd_null_cfg", rmsnorm_select_config(4, 64, RMSNORM_DTYPE_BF16, 1, 0, NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("select_quant", rmsnorm_select_quant_config(16384, 8192, RMSNORM_DTYPE_BF16, 1, 0, &c), RMSNORM_OK);
    expect("quant_path", c.path, RMSNORM_PATH_VECTOR);
    expect("select_bwd", rmsnorm_select_bwd_config(16384, 8192, RMSNORM_DTYPE_BF16, 1, &c), RMSNORM_OK);
    expect("bwd_max_blocks", c.max_blocks, 512);
    /* odd widths: full vectors at the row's own alignment plus a tail */
    expect("select_quant_odd", rmsnorm_select_quant_config(16384, 8191, RMSNORM_DTYPE_BF16, 1, 0, &c), RMSNORM_OK);
    expect("quant_odd_path", c.path, RMSNORM_PATH_VECTOR_ANY);
    expect("select_bwd_odd", rmsnorm_select_bwd_config(16384, 8191, RMSNORM_DTYPE_BF16, 1, &c), RMSNORM_OK);
    expect("bwd_odd_path", c.path, RMSNORM_PATH_VECTOR_ANY);
    expect("bwd_odd_rows_per_block", c.rows_per_block, 1);
    expect("select_ln", layernorm_select_config(8192, 4096, RMSNORM_DTYPE_BF16, 1, &c), RMSNORM_OK);
    expect("ln_weight_lds", c.weight_lds, 1);
    expect("select_kv", kv_select_config(16384, 1, 512, 64, 1, RMSNORM_DTYPE_BF16, 1, &c), RMSNORM_OK);
    expect("kv_lanes_per_row", c.lanes_per_row, 32);
    expect("kv_items_per_lane", c.items_per_lane, 2);

    /* workspace of the backward: min(ceil(rows / rows_per_block), partials) * round_up(hidden, 64) * 4 */
    size_t ws = 0;
    expect("bwd_workspace", rmsnorm_bwd_workspace_size(16384, 8192, RMSNORM_DTYPE_BF16, NULL, &ws), RMSNORM_OK);
    expect("bwd_workspace_mib", (int)(ws >> 20), 16);
    expect("bwd_workspace_null", rmsnorm_bwd_workspace_size(16384, 8192, RMSNORM_DTYPE_BF16, NULL, NULL),
           RMSNORM_ERR_INVALID_ARG);

    /* validation before any HIP call */
    expect("fwd_rows0", rmsnorm_fwd(NULL, NULL, NULL, 0, 64, 1e-5f, RMSNORM_DTYPE_BF16, NULL), RMSNORM_OK);
    expect("fwd_null", rmsnorm_fwd(NULL, NULL, NULL, 4, 64, 1e-5f, RMSNORM_DTYPE_BF16, NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("fwd_neg_rows", rmsnorm_fwd(NULL, NULL, NULL, -1, 64, 1e-5f, RMSNORM_DTYPE_BF16, NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("fwd_neg_eps", rmsnorm_fwd(NULL, NULL, NULL, 4, 64, -1.f, RMSNORM_DTYPE_BF16, NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("fwd_dtype", rmsnorm_fwd(NULL, NULL, NULL, 4, 64, 1e-5f, (rmsnorm_dtype_t)7, NULL),
           RMSNORM_ERR_UNSUPPORTED_DTYPE);
    expect("residual_null", rmsnorm_residual_fwd(NULL, NULL, NULL, NULL, NULL, 4, 64, 1e-5f, RMSNORM_DTYPE_F32,
                                                 NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("quant_qtype", rmsnorm_dynamic_quant_fwd(NULL, NULL, NULL, NULL, NULL, NULL, -1, 16, 1e-5f,
                                                    RMSNORM_DTYPE_BF16, (rmsnorm_quant_t)7, NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("bwd_null", rmsnorm_bwd(NULL, NULL, NULL, NULL, NULL, 4, 64, 1e-5f, RMSNORM_DTYPE_BF16, NULL, 0, NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("ln_rows0", layernorm_fwd(NULL, NULL, NULL, NULL, 0, 64, 1e-5f, RMSNORM_DTYPE_BF16, NULL), RMSNORM_OK);
    expect("ln_null", layernorm_fwd(NULL, NULL, NULL, NULL, 4, 64, 1e-5f, RMSNORM_DTYPE_BF16, NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("kv_tokens0", kv_rmsnorm_rope_cache(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 1, 512, 64, 16,
                                               16, 1e-6f, 1, RMSNORM_DTYPE_BF16, NULL),
           RMSNORM_OK);
    expect("kv_odd_rope", kv_rmsnorm_rope_cache(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 4, 1, 512, 63, 16,
                                                16, 1e-6f, 1, RMSNORM_DTYPE_BF16, NULL),
           RMSNORM_ERR_INVALID_ARG);
    expect("kv_ex_tokens0", kv_rmsnorm_rope_cache_ex(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 1, 512, 64,
                                                     16, 16, 1e-6f, 1, RMSNORM_DTYPE_BF16, &c, NULL),
           RMSNORM_OK);
    expect("copy_null", hbm_copy(NULL, NULL, 16, 0, NULL) != 0, 1);
    return failures;
}
