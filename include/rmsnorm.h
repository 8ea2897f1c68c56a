/*
 * rmsnorm.h -- C ABI of librmsnorm.so, row-wise RMSNorm for AMD Instinct
 * MI355X (gfx950).
 *
 * Operation (per row of a row-major [rows, hidden] tensor):
 *
 *     y_j = x_j * rsqrt(sum_k x_k^2 / hidden + eps) * weight_j
 *
 * eps sits inside the root and the mean divides by hidden (xserv "phase 4:
 * transformer core kernels", csrc/normalization/rmsnorm.cu header comment and
 * docs/04-transformer-kernels.md, "Kernel 设计细节 / RMSNorm").  The sum of
 * squares, the inverse root and both products are evaluated in fp32 and each
 * output is rounded to the tensor dtype exactly once, nearest-even, after the
 * weight multiply (gollamago README, "RMSNorm 优化（TileLang）": one global
 * read and one global write per row, fp32 accumulation and scaling, rounding
 * only at write-back).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers (HIP device memory, e.g. torch CUDA-tensor
 *     storage).  The caller owns every buffer; the library allocates nothing
 *     and keeps no per-call state.  Only the backward's weight gradient needs
 *     scratch memory, which the caller passes in as a workspace (or, with
 *     rmsnorm_bwd_noalloc, the library's fixed per-GPU scratch array).
 *   - Tensors are contiguous and row-major; weight is [hidden]; all tensors
 *     share one dtype.  Any element-aligned address is accepted.  With every
 *     pointer 16-byte aligned and hidden * dtype_size a multiple of 16, rows
 *     move as aligned 16-byte vectors; otherwise a row of at least one vector
 *     moves as 16-byte vectors at its own alignment plus its last few
 *     elements one by one (see RMSNORM_PATH_VECTOR_ANY for the one read
 *     outside a row: two bytes in the same 4-byte word as its first element),
 *     and a narrower row one element per access.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     work and return without synchronising; results are ready when the stream
 *     reaches that point.
 *   - Every INVALID_ARG / UNSUPPORTED_DTYPE return happens before any HIP call,
 *     so nothing is enqueued on error.  rows == 0 returns RMSNORM_OK without
 *     touching the GPU.
 *   - An output may alias an input exactly (out == x, residual_out ==
 *     residual, residual_out == x, ...): every element is read before it is
 *     overwritten, and only by the thread that writes it.  Any other overlap
 *     of an output with another buffer -- a partial overlap, weight, or the
 *     other output -- is rejected with INVALID_ARG.
 *   - For equal inputs, shapes and configuration the results are bitwise
 *     reproducible (fixed reduction order, no atomics).
 *
 * Status codes and the export convention follow the Intro-ops operator
 * runtime's public C header (include/operator_runtime/api.h: SUCCESS,
 * INVALID_ARG, UNSUPPORTED_DTYPE, RUNTIME; default visibility + extern "C").
 */
#ifndef MBR_RMSNORM_H
#define MBR_RMSNORM_H

#include <stddef.h>
#include <stdint.h>

#define RMSNORM_API __attribute__((visibility("default")))

/* The enums below are 32-bit integers at the boundary.  C++ sees them with a
 * fixed int32_t underlying type, so any 32-bit value a caller passes is a
 * value of the type (rejected by validation when unknown) rather than an
 * out-of-range enum, whose mere load C++ leaves undefined. */
#ifdef __cplusplus
#define RMSNORM_ENUM_BASE : int32_t
#else
#define RMSNORM_ENUM_BASE
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum RMSNORM_ENUM_BASE {
    RMSNORM_OK = 0,
    RMSNORM_ERR_INVALID_ARG = 1,       /* null pointer, bad size, bad eps, bad overlap, bad config */
    RMSNORM_ERR_UNSUPPORTED_DTYPE = 2, /* dtype not one of rmsnorm_dtype_t */
    RMSNORM_ERR_RUNTIME = 3            /* the HIP launch reported an error */
} rmsnorm_status_t;

typedef enum RMSNORM_ENUM_BASE {
    RMSNORM_DTYPE_F32 = 0, /* IEEE binary32 */
    RMSNORM_DTYPE_BF16 = 1 /* bfloat16: upper 16 bits of a binary32 */
} rmsnorm_dtype_t;

/*
 * rmsnorm_fwd: out[i, :] = RMSNorm(x[i, :]) * weight for 0 <= i < rows.
 *
 *   x       [rows, hidden] input, read once.
 *   weight  [hidden] scale (gamma), same dtype as x.
 *   out     [rows, hidden] output; may be x itself (in place).
 *   rows    >= 0 (0: no-op).
 *   hidden  >= 1, <= 2^31 - 1, and rows * hidden * dtype_size must fit in int64.
 *   eps     finite and >= 0 (passed as a 32-bit float, as the xserv FFI
 *           wrapper crates/xserv-kernels/src/rmsnorm.rs does).
 *   dtype   RMSNORM_DTYPE_F32 or RMSNORM_DTYPE_BF16.
 *   stream  hipStream_t or NULL.
 * Returns RMSNORM_OK once the kernel is enqueued.
 */
RMSNORM_API rmsnorm_status_t rmsnorm_fwd(const void* x, const void* weight, void* out,
                                         int64_t rows, int64_t hidden, float eps,
                                         rmsnorm_dtype_t dtype, void* stream);

/*
 * rmsnorm_residual_fwd: fused residual add + RMSNorm, one pass over the rows.
 *
 *   residual_out[i, :] = round(x[i, :] + residual[i, :])      (h, stored)
 *   out[i, :]          = RMSNorm(residual_out[i, :]) * weight  (norm of the ROUNDED h)
 *
 * Folding the Add that precedes RmsNorm into the same kernel to cut data
 * movement follows the fusion example in the TileLang tutorial ch. 02
 * "从 PyTorch 到 kernel", section 4.2 (CANN aclnnAddRmsNormDynamicQuant).
 * The sum is formed in fp32 and rounded once (exact for bf16 operands), so h
 * equals the unfused x + residual bit for bit and out equals rmsnorm_fwd(h).
 *
 *   x, residual   [rows, hidden] inputs, each read once.
 *   weight        [hidden].
 *   residual_out  [rows, hidden] h; may be x or residual itself.
 *   out           [rows, hidden] normalised h; may be x or residual, never
 *                 residual_out.
 * Other arguments and errors as rmsnorm_fwd.
 */
RMSNORM_API rmsnorm_status_t rmsnorm_residual_fwd(const void* x, const void* residual,
                                                  const void* weight, void* residual_out,
                                                  void* out, int64_t rows, int64_t hidden,
                                                  float eps, rmsnorm_dtype_t dtype,
                                                  void* stream);

/* Static, human-readable name of a status code (never NULL). */
RMSNORM_API const char* rmsnorm_status_string(rmsnorm_status_t status);

/* ------------------------------------------------------------------------
 * Launch configurations.  rmsnorm_fwd / rmsnorm_residual_fwd pick one from
 * (rows, hidden, dtype, alignment) by a fixed rule; the calls below expose
 * that choice and let a caller (tests, tuning sweeps) force another one.
 * Every configuration computes the same function; different configurations
 * may differ in the last bit through the fp32 reduction order.
 * ---------------------------------------------------------------------- */

typedef enum RMSNORM_ENUM_BASE {
    RMSNORM_PATH_AUTO = 0,     /* let the library choose (the other fields are ignored) */
    RMSNORM_PATH_VECTOR = 1,   /* row in VGPRs, 16-byte loads/stores; needs 16-byte alignment */
    RMSNORM_PATH_ELEMENT = 2,  /* row in VGPRs, one element per access; any alignment */
    RMSNORM_PATH_TWO_PASS = 3, /* row too large for registers and LDS, or an unaligned row too
                                  large for registers: second read of x (and residual) */
    RMSNORM_PATH_VECTOR_ANY = 4, /* rmsnorm_fwd_ex / rmsnorm_residual_fwd_ex /
                                   rmsnorm_dynamic_quant_fwd_ex / rmsnorm_bwd_ex /
                                   layernorm_fwd_ex: any width of at least one
                                   vector and any element alignment; the row's full
                                   16-byte vectors at whatever alignment it has, then its last
                                   hidden % (16 / size) elements one by one; rows_per_block 1.
                                   bf16 normalised output: a row that starts 2 bytes past a
                                   4-byte boundary moves as the row one element earlier
                                   (when x, out, residual and h share their offset modulo 4
                                   and the configuration covers hidden + 1 elements); the
                                   two bytes before the row, in the same 4-byte word, are
                                   then read but never written */
    RMSNORM_PATH_VECTOR_LDS = 5 /* rmsnorm_fwd_ex / rmsnorm_residual_fwd_ex: rows wider than
                                   the register path holds, still read once: 1024 lanes
                                   (waves_per_row 16, rows_per_block 1), items_per_lane
                                   vectors per lane in VGPRs (10 plain; 6 or 7 fused), the
                                   row's remaining vectors staged in LDS, at most 162816
                                   bytes of them; needs 16-byte alignment */
} rmsnorm_path_t;

typedef struct {
    int32_t path;           /* rmsnorm_path_t */
    int32_t waves_per_row;  /* 64-lane waves cooperating on one row: 1, 2, 4, 8 or 16 */
    int32_t items_per_lane; /* VECTOR: 16-byte vectors per lane.  Built for
                               rmsnorm_fwd_ex: 1-8, and 10 at 16 waves per row;
                               rmsnorm_residual_fwd_ex: 1-5, 1-6 at 16 waves.
                               VECTOR_ANY: vectors per lane, 1-5; at 16 waves 1-6
                               (1-4 fused).  ELEMENT: elements per lane; only rows
                               narrower than one 16-byte vector take this path, so
                               only 1 element with waves_per_row 1 is built.  The
                               other entry points state their own built sets;
                               VECTOR_LDS: vectors per lane held in VGPRs (see above);
                               TWO_PASS: ignored (0) */
    int32_t rows_per_block; /* rows per workgroup; 64 * waves_per_row * rows_per_block <= 512
                               (1024 when waves_per_row == 16); TWO_PASS: must be 1 */
    int32_t max_blocks;     /* >= 0; 0: one workgroup per group of rows_per_block rows;
                               n > 0: at most n workgroups, each looping over row groups */
    int32_t lanes_per_row;  /* 0: 64 * waves_per_row (whole waves).  VECTOR path of every
                               entry point with a configuration: 8, 16 or 32 lanes per row with
                               waves_per_row 1 and items_per_lane 1 or 2, several rows
                               sharing a wave; lanes_per_row * rows_per_block must then be
                               a multiple of 64 and at most 512 */
    int32_t weight_lds;     /* 0 or 1.  1: VECTOR path with whole-wave rows only; each
                               workgroup copies the weight into LDS once (hidden * size
                               bytes, at most 159 KiB) and its rows take it from there
                               instead of from global memory.  The results are bitwise the
                               same either way.  layernorm_fwd_ex: gamma and beta staged
                               the same way.  Must be 0 for rmsnorm_bwd_ex */
} rmsnorm_config_t;

/*
 * Fill *cfg with the configuration rmsnorm_fwd / rmsnorm_residual_fwd would use
 * for this shape.  vector_aligned != 0 states that every pointer will be
 * 16-byte aligned.  INVALID_ARG for cfg == NULL or bad sizes; no HIP call.
 */
RMSNORM_API rmsnorm_status_t rmsnorm_select_config(int64_t rows, int64_t hidden,
                                                   rmsnorm_dtype_t dtype,
                                                   int32_t vector_aligned, int32_t fused,
                                                   rmsnorm_config_t* cfg);

/*
 * As rmsnorm_fwd / rmsnorm_residual_fwd with an explicit configuration
 * (cfg == NULL or cfg->path == RMSNORM_PATH_AUTO: automatic choice).
 * INVALID_ARG if the configuration is not built, cannot cover hidden, or
 * needs an alignment the pointers do not have.
 */
RMSNORM_API rmsnorm_status_t rmsnorm_fwd_ex(const void* x, const void* weight, void* out,
                                            int64_t rows, int64_t hidden, float eps,
                                            rmsnorm_dtype_t dtype, const rmsnorm_config_t* cfg,
                                            void* stream);

RMSNORM_API rmsnorm_status_t rmsnorm_residual_fwd_ex(const void* x, const void* residual,
                                                     const void* weight, void* residual_out,
                                                     void* out, int64_t rows, int64_t hidden,
                                                     float eps, rmsnorm_dtype_t dtype,
                                                     const rmsnorm_config_t* cfg, void* stream);

/* ------------------------------------------------------------------------
 * RMSNorm with dynamic per-row quantisation of its output.
 * ---------------------------------------------------------------------- */

typedef enum RMSNORM_ENUM_BASE {
    RMSNORM_QUANT_INT8 = 0,     /* signed 8-bit codes in [-127, 127], Q = 127 */
    RMSNORM_QUANT_FP8_E4M3 = 1  /* OCP fp8 e4m3fn codes (bias 7, max 448, no inf), Q = 448 */
} rmsnorm_quant_t;

/*
 * rmsnorm_dynamic_quant_fwd: (residual add +) RMSNorm + per-row symmetric
 * dynamic quantisation, one pass over the rows -- the Add + RmsNorm +
 * DynamicQuant fusion the TileLang tutorial ch. 02, section 4.2, cites from
 * CANN (aclnnAddRmsNormDynamicQuant) as a way to cut data movement.  The pages
 * give no quantiser formula; this library implements the plain per-token one:
 *
 *   v         = x, or h = round(x + residual) (written to residual_out)
 *   y_j       = v_j * rsqrt(sum_k v_k^2 / hidden + eps) * weight_j   (fp32, never rounded)
 *   scale_out[i] = max_j |y_j| / Q
 *   q_out[i, j]  = round(y_j / scale_out[i])   nearest-even; int8 clamped to
 *                                              [-127, 127], fp8 saturating at +-448
 *
 * A row with max_j |y_j| == 0 gets scale 0 and all-zero codes.  The root
 * cancels from y_j / scale, so the codes are evaluated as
 * (v_j * weight_j) * (Q / max_k |v_k * weight_k|); they can differ from a
 * higher-precision evaluation only where y_j / scale lies within float32
 * rounding of a tie between two codes.
 *
 *   x, weight      as rmsnorm_fwd (dtype bf16 or f32).
 *   residual       [rows, hidden] or NULL (no add); residual_out is NULL exactly
 *                  when residual is; it may alias x or residual exactly.
 *   q_out          [rows, hidden] bytes: int8 or e4m3fn codes, row-major.
 *   scale_out      [rows] float32, 4-byte aligned.
 *   qtype          rmsnorm_quant_t; anything else -> RMSNORM_ERR_UNSUPPORTED_DTYPE.
 * q_out and scale_out may not overlap any other buffer or each other.  The
 * 16-byte vector path additionally needs q_out 16-byte aligned; otherwise (or
 * for widths that are not whole vectors) the any-alignment path writes the
 * codes at any byte offset.  Other rules and errors as rmsnorm_fwd.
 */
RMSNORM_API rmsnorm_status_t rmsnorm_dynamic_quant_fwd(const void* x, const void* residual,
                                                      const void* weight, void* residual_out,
                                                      void* q_out, float* scale_out, int64_t rows,
                                                      int64_t hidden, float eps, rmsnorm_dtype_t dtype,
                                                      rmsnorm_quant_t qtype, void* stream);

/* As rmsnorm_dynamic_quant_fwd with an explicit launch configuration; the
 * quantised kernels are built for 1-5 vectors per lane, 1-4 with 16 waves per
 * row (VECTOR and VECTOR_ANY), and ELEMENT 1 element with waves_per_row 1. */
RMSNORM_API rmsnorm_status_t rmsnorm_dynamic_quant_fwd_ex(const void* x, const void* residual,
                                                         const void* weight, void* residual_out,
                                                         void* q_out, float* scale_out, int64_t rows,
                                                         int64_t hidden, float eps,
                                                         rmsnorm_dtype_t dtype, rmsnorm_quant_t qtype,
                                                         const rmsnorm_config_t* cfg, void* stream);

/* The configuration rmsnorm_dynamic_quant_fwd would use (as rmsnorm_select_config). */
RMSNORM_API rmsnorm_status_t rmsnorm_select_quant_config(int64_t rows, int64_t hidden,
                                                         rmsnorm_dtype_t dtype,
                                                         int32_t vector_aligned, int32_t fused,
                                                         rmsnorm_config_t* cfg);

/*
 * Backward.  For y = RMSNorm(x) * weight and an upstream gradient dy, the
 * norm backward of a training step's backward stage (TileLang tutorial ch. 02,
 * "从 PyTorch 到 kernel", section 1.1(b); the pages give no formula, this is
 * the plain derivative), per row with r = rsqrt(sum_k x_k^2 / hidden + eps):
 *
 *     dx_k      = r * (dy_k * weight_k - x_k * r^2 * c / hidden),
 *                 c = sum_j dy_j * weight_j * x_j
 *     dweight_j = sum_i dy_ij * x_ij * r_i          (over all rows)
 *
 * evaluated in fp32 and rounded once to the tensor dtype.  dweight is reduced
 * across rows in two fixed-order stages (per-workgroup fp32 partial rows in
 * the workspace, then a column sum), so results are bitwise reproducible for
 * equal inputs, shape and configuration; no atomics.  Workspace handling
 * follows the create / query-workspace / execute pattern of the Intro-ops
 * operator runtime's public C header (include/operator_runtime/api.h).
 *
 * rmsnorm_bwd:
 *   x, weight  the forward's inputs ([rows, hidden], [hidden]).
 *   dy         [rows, hidden] upstream gradient, same dtype.
 *   dx         [rows, hidden] output; may be x or dy itself (exactly), must
 *              not touch weight or partially overlap x or dy.
 *   dweight    [hidden] output, or NULL when the weight gradient is not
 *              wanted (then workspace is ignored).  Overwritten, not
 *              accumulated into.  Overlaps nothing.  With rows == 0 it is
 *              set to zero and the other pointers are not used.
 *   workspace  device memory of at least rmsnorm_bwd_workspace_size() bytes,
 *              16-byte aligned, overlapping nothing; contents on entry are
 *              irrelevant and are clobbered.  May be NULL when the size is 0.
 *              The same workspace must not be in use by another call that
 *              may run concurrently (another stream).
 *   workspace_bytes  its size; smaller than needed is INVALID_ARG.
 *   rows, hidden, eps, dtype, stream: as rmsnorm_fwd.
 * Enqueues one kernel for dx (and the partial rows), plus one for dweight.
 */
RMSNORM_API rmsnorm_status_t rmsnorm_bwd(const void* x, const void* weight, const void* dy, void* dx,
                                         void* dweight, int64_t rows, int64_t hidden, float eps,
                                         rmsnorm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* rmsnorm_bwd with a launch configuration (NULL or path AUTO = automatic).
 * rows_per_block > 1 is accepted on path VECTOR only (64 * waves_per_row *
 * rows_per_block threads within the limit of rmsnorm_config_t; with dweight,
 * hidden * 4 bytes of LDS at most 159 KiB): the rows of a workgroup's slots then
 * share one partial dweight row.  max_blocks caps the grid and is the number
 * of partial dweight rows (0 = no cap).  lanes_per_row 8, 16 or 32 (rows of at
 * most 2 * lanes_per_row vectors; waves_per_row 1, items_per_lane 1 or 2;
 * lanes_per_row * rows_per_block a multiple of 64, at most 512): several rows
 * per wave, each taking one row slot; with dweight and more than one wave per
 * workgroup, hidden * 4 bytes of LDS, at most 159 KiB.  Built: VECTOR 1-8
 * vectors per lane with one wave per row, 1-6 with 2-8 waves, 1-4 with 16;
 * VECTOR_ANY 1-6, 1-3 with 16 waves; ELEMENT 1 element with waves_per_row 1. */
RMSNORM_API rmsnorm_status_t rmsnorm_bwd_ex(const void* x, const void* weight, const void* dy, void* dx,
                                            void* dweight, int64_t rows, int64_t hidden, float eps,
                                            rmsnorm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                            const rmsnorm_config_t* cfg, void* stream);

/* rmsnorm_bwd for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc: no
 * workspace argument, and no allocation inside.  The partial dweight rows live
 * in a 16 MiB array the library holds in device memory (one per GPU, kept
 * until the process ends).  Arguments and results as rmsnorm_bwd; the launch
 * configuration is rmsnorm_bwd's automatic choice, with the number of partial
 * dweight rows capped at what the array holds, 16 MiB / (round_up(hidden, 64)
 * * 4) (512 rows at hidden 8192): below the cap the results equal
 * rmsnorm_bwd's bitwise, above it only the dweight summation order differs.
 * hidden above 4194304 with dweight is INVALID_ARG (one partial row would not
 * fit).  Runs on the current device (the stream must belong to it); the
 * array's address is looked up there on the first call (RUNTIME if HIP
 * fails).  Every call on one GPU shares that GPU's array: calls that may run
 * at the same time on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  Nothing in the array needs clearing between
 * calls: each call writes every partial row it reads. */
RMSNORM_API rmsnorm_status_t rmsnorm_bwd_noalloc(const void* x, const void* weight, const void* dy, void* dx,
                                                 void* dweight, int64_t rows, int64_t hidden, float eps,
                                                 rmsnorm_dtype_t dtype, void* stream);

/* Bytes of workspace rmsnorm_bwd (cfg NULL or AUTO: any pointer alignment) or
 * rmsnorm_bwd_ex with cfg needs to produce dweight:
 * min(ceil(rows / rows_per_block), max_blocks) * round_up(hidden, 64) * 4.
 * No HIP call. */
RMSNORM_API rmsnorm_status_t rmsnorm_bwd_workspace_size(int64_t rows, int64_t hidden, rmsnorm_dtype_t dtype,
                                                        const rmsnorm_config_t* cfg, size_t* bytes);

/* The configuration rmsnorm_bwd would choose (max_blocks = its partial-row
 * cap).  No HIP call. */
RMSNORM_API rmsnorm_status_t rmsnorm_select_bwd_config(int64_t rows, int64_t hidden, rmsnorm_dtype_t dtype,
                                                       int32_t vector_aligned, rmsnorm_config_t* cfg);

/*
 * LayerNorm, the sibling norm on the same pages (xserv "phase 4: transformer
 * core kernels", csrc/normalization/layernorm.cu header comment and
 * docs/04-transformer-kernels.md "LayerNorm"), per row:
 *
 *     y_j = gamma_j * (x_j - mu) * rsqrt(var + eps) + beta_j,
 *     mu = sum_j x_j / hidden,  var = sum_j (x_j - mu)^2 / hidden
 *
 * (biased variance, as the pages' CPU reference).  The mean is reduced first
 * and the centred squares after it, from the row held in registers (no
 * E[x^2] - mu^2 cancellation, no extra memory pass), in fp32; each output is
 * rounded once after the affine step.
 *
 *   x       [rows, hidden] input, read once (three times for rows wider than
 *           the register path covers).
 *   gamma   [hidden], same dtype.
 *   beta    [hidden], same dtype, or NULL for no bias.
 *   out     [rows, hidden]; may be x itself, must not touch gamma or beta.
 *   rows, hidden, eps, dtype, stream: as rmsnorm_fwd.
 */
RMSNORM_API rmsnorm_status_t layernorm_fwd(const void* x, const void* gamma, const void* beta, void* out,
                                           int64_t rows, int64_t hidden, float eps, rmsnorm_dtype_t dtype,
                                           void* stream);

/* layernorm_fwd with a launch configuration (NULL or path AUTO = automatic;
 * path TWO_PASS selects the three-pass wide-row kernel).  weight_lds (gamma
 * and beta staged in LDS once per workgroup, hidden * size bytes each, at most
 * 159 KiB together) is taken on path VECTOR only; rows_per_block > 1 requires
 * it (the row slots share that copy), with 64 * waves_per_row *
 * rows_per_block within the limit of rmsnorm_config_t.  lanes_per_row 8, 16
 * or 32 (weight_lds 0): several rows per wave, each taking one row slot and
 * holding its gamma / beta slice in registers.  Built: VECTOR and VECTOR_ANY
 * 1-8 vectors per lane (16 waves per row: 1-4 and 1-3); ELEMENT 1 element with
 * waves_per_row 1. */
RMSNORM_API rmsnorm_status_t layernorm_fwd_ex(const void* x, const void* gamma, const void* beta, void* out,
                                              int64_t rows, int64_t hidden, float eps, rmsnorm_dtype_t dtype,
                                              const rmsnorm_config_t* cfg, void* stream);

/* The configuration layernorm_fwd would choose.  No HIP call. */
RMSNORM_API rmsnorm_status_t layernorm_select_config(int64_t rows, int64_t hidden, rmsnorm_dtype_t dtype,
                                                     int32_t vector_aligned, rmsnorm_config_t* cfg);

/*
 * KV RMSNorm + RoPE + cache scatter: the fused KV-cache maintenance operator
 * the TileLang tutorial ch. 02 ("从 PyTorch 到 kernel", sections 1.2 and 4.2)
 * cites from CANN (aclnnKvRmsNormRopeCache).  For every token t and head h,
 * the row kv[t, h, :] is split along its tail axis:
 *
 *   kv[t, h, 0 : norm_dim]             -> RMSNorm (eps, gamma, as rmsnorm_fwd)
 *                                          -> norm_cache[slots[t], h, :]
 *   kv[t, h, norm_dim : norm_dim+rope] -> RoPE at position positions[t]
 *                                          -> rope_cache[slots[t], h, :]
 *
 * RoPE as xserv's rope.cu (phase 4): a pair (a, b) becomes
 * (a*cos - b*sin, a*sin + b*cos) with cos = cos_table[p, i], sin =
 * sin_table[p, i]; the pairs are adjacent elements (2i, 2i+1) with rope_style 1
 * or the two halves (i, i + rope_dim/2) with rope_style 0.  fp32 math, one
 * rounding per output element.
 *
 *   kv          [tokens, heads, norm_dim + rope_dim], dtype.
 *   gamma       [norm_dim], dtype.
 *   cos_table, sin_table  [max_pos, rope_dim/2] float32 (may be NULL when
 *               rope_dim is 0).
 *   positions   [tokens] int32;  slots [tokens] int64: the cache row of each
 *               token (for a paged cache, block_table[seq][pos / block_size] *
 *               block_size + pos % block_size).  A token whose slot is not in
 *               [0, num_slots) or whose position is not in [0, max_pos)
 *               writes nothing (padding); slots must be distinct within a call
 *               (two tokens with one slot race).
 *   norm_cache  [num_slots, heads, norm_dim], dtype; only the rows named by
 *               valid slots are written.
 *   rope_cache  [num_slots, heads, rope_dim], dtype; same (may be NULL when
 *               rope_dim is 0).
 *   heads >= 1, norm_dim >= 1, rope_dim >= 0 and even; eps as rmsnorm_fwd;
 *   rope_style 0 or 1.  The caches must not overlap each other or any input.
 * 16-byte vector accesses are used when every buffer is 16-byte aligned,
 * norm_dim is a multiple of the vector width, rope_dim a multiple of it
 * (pairs) or of twice it (halves), and the rotated part fits in 64 lanes;
 * otherwise an element kernel runs.  tokens == 0 returns RMSNORM_OK without
 * touching the GPU.
 */
RMSNORM_API rmsnorm_status_t kv_rmsnorm_rope_cache(const void* kv, const void* gamma, const float* cos_table,
                                                   const float* sin_table, const int32_t* positions,
                                                   const int64_t* slots, void* norm_cache, void* rope_cache,
                                                   int64_t tokens, int64_t heads, int64_t norm_dim,
                                                   int64_t rope_dim, int64_t max_pos, int64_t num_slots, float eps,
                                                   int32_t rope_style, rmsnorm_dtype_t dtype, void* stream);

/* kv_rmsnorm_rope_cache with a launch configuration (NULL or path AUTO =
 * automatic).  path VECTOR (16-byte aligned buffers and a vector shape as
 * above): lanes_per_row 0 (a whole wave per row) with items_per_lane 1, 2, 4
 * or 8 norm vectors per lane, or lanes_per_row 16 or 32 (several rows per
 * wave) with items_per_lane 1 or 2; the rotated part must fit the row's
 * lanes.  path ELEMENT: the element kernel (lanes_per_row 0).  waves_per_row
 * and rows_per_block must be 1, max_blocks and weight_lds 0.  INVALID_ARG
 * otherwise; the results do not depend on the configuration beyond the
 * rounding of the row sum. */
RMSNORM_API rmsnorm_status_t kv_rmsnorm_rope_cache_ex(const void* kv, const void* gamma, const float* cos_table,
                                                      const float* sin_table, const int32_t* positions,
                                                      const int64_t* slots, void* norm_cache, void* rope_cache,
                                                      int64_t tokens, int64_t heads, int64_t norm_dim,
                                                      int64_t rope_dim, int64_t max_pos, int64_t num_slots,
                                                      float eps, int32_t rope_style, rmsnorm_dtype_t dtype,
                                                      const rmsnorm_config_t* cfg, void* stream);

/* The configuration kv_rmsnorm_rope_cache would use for this shape
 * (vector_aligned != 0: every buffer will be 16-byte aligned).  INVALID_ARG
 * for cfg == NULL or bad sizes; no HIP call. */
RMSNORM_API rmsnorm_status_t kv_select_config(int64_t tokens, int64_t heads, int64_t norm_dim, int64_t rope_dim,
                                              int32_t rope_style, rmsnorm_dtype_t dtype, int32_t vector_aligned,
                                              rmsnorm_config_t* cfg);

#ifdef __cplusplus
}
#endif

#endif /* MBR_RMSNORM_H */
