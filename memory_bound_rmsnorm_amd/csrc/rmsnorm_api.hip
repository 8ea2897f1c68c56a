// C ABI of librmsnorm.so: argument validation, launch-configuration choice
// and kernel launch.  Declarations and the contract are in include/rmsnorm.h.
//
// Every INVALID_ARG / UNSUPPORTED_DTYPE path returns before the first HIP
// call, so a rejected call enqueues nothing.  Launches go onto the caller's
// stream and are not waited for (the xserv FFI wrapper synchronises the device
// after each launch; the gollamago README measures launch plus host sync at
// about 0.1 ms, the same order as the operator itself, so this library never
// synchronises).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/rmsnorm.h"
#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace {

constexpr int64_t kVectorBytes = 16;
// Largest grid launched in one call; bigger jobs loop inside the kernel.
constexpr int64_t kMaxGrid = int64_t(1) << 20;

struct Problem {
    const void* x;
    const void* res;
    const void* w;
    void* h;
    void* out;
    int64_t rows;
    int64_t hidden;
    float eps;
    int dtype;  // 0 f32, 1 bf16
    bool fused;
    int qt;        // 0: normalised output; 1: int8 codes; 2: fp8 e4m3fn codes
    float* scale;  // quantised forms: per-row scales
};

int elem_size(int dtype) { return dtype == RMSNORM_DTYPE_F32 ? 4 : 2; }
int vec_elems(int dtype) { return dtype == RMSNORM_DTYPE_F32 ? 4 : 8; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int index_of(const int* list, int n, int v) {
    for (int i = 0; i < n; ++i)
        if (list[i] == v) return i;
    return -1;
}

// Smallest built value >= want, or -1.
int round_up_in(const int* list, int n, int64_t want) {
    for (int i = 0; i < n; ++i)
        if (list[i] >= want) return list[i];
    return -1;
}

bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + static_cast<uintptr_t>(nb) && pb < pa + static_cast<uintptr_t>(na);
}

// An output may coincide exactly with an input; any other contact is an error.
bool output_vs_input_ok(const void* o, const void* i, int64_t n) { return o == i || !ranges_overlap(o, n, i, n); }

rmsnorm_status_t validate_sizes(int64_t rows, int64_t hidden, float eps, int dtype) {
    if (rows < 0 || hidden <= 0 || hidden > INT32_MAX) return RMSNORM_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || isinf(eps)) return RMSNORM_ERR_INVALID_ARG;  // rejects NaN too
    if (dtype != RMSNORM_DTYPE_F32 && dtype != RMSNORM_DTYPE_BF16) return RMSNORM_ERR_UNSUPPORTED_DTYPE;
    if (rows > 0 && rows > INT64_MAX / hidden / elem_size(dtype)) return RMSNORM_ERR_INVALID_ARG;
    return RMSNORM_OK;
}

rmsnorm_status_t validate_pointers(const Problem& p) {
    const int es = elem_size(p.dtype);
    if (!p.x || !p.w || !p.out) return RMSNORM_ERR_INVALID_ARG;
    if (p.fused && (!p.res || !p.h)) return RMSNORM_ERR_INVALID_ARG;
    const void* ptrs[] = {p.x, p.w, p.res, p.h};
    for (const void* q : ptrs)
        if (q && reinterpret_cast<uintptr_t>(q) % es != 0) return RMSNORM_ERR_INVALID_ARG;
    const int64_t nb = p.rows * p.hidden * es;  // no overflow: checked in validate_sizes
    const int64_t wb = p.hidden * es;
    if (p.qt != 0) {
        // codes (one byte per element) and scales touch nothing else at all
        const int64_t qb = p.rows * p.hidden, sb = p.rows * 4;
        if (!p.scale || reinterpret_cast<uintptr_t>(p.scale) % 4 != 0) return RMSNORM_ERR_INVALID_ARG;
        const void* others[] = {p.x, p.w, p.res, p.h};
        const int64_t sizes[] = {nb, wb, nb, nb};
        for (int i = 0; i < 4; ++i) {
            if (!others[i]) continue;
            if (ranges_overlap(p.out, qb, others[i], sizes[i]) || ranges_overlap(p.scale, sb, others[i], sizes[i]))
                return RMSNORM_ERR_INVALID_ARG;
        }
        if (ranges_overlap(p.out, qb, p.scale, sb)) return RMSNORM_ERR_INVALID_ARG;
        if (p.fused) {
            if (ranges_overlap(p.h, nb, p.w, wb)) return RMSNORM_ERR_INVALID_ARG;
            if (!output_vs_input_ok(p.h, p.x, nb) || !output_vs_input_ok(p.h, p.res, nb)) return RMSNORM_ERR_INVALID_ARG;
        }
        return RMSNORM_OK;
    }
    if (reinterpret_cast<uintptr_t>(p.out) % es != 0) return RMSNORM_ERR_INVALID_ARG;
    if (ranges_overlap(p.out, nb, p.w, wb)) return RMSNORM_ERR_INVALID_ARG;
    if (!output_vs_input_ok(p.out, p.x, nb)) return RMSNORM_ERR_INVALID_ARG;
    if (p.fused) {
        if (ranges_overlap(p.h, nb, p.w, wb)) return RMSNORM_ERR_INVALID_ARG;
        if (ranges_overlap(p.h, nb, p.out, nb)) return RMSNORM_ERR_INVALID_ARG;
        if (!output_vs_input_ok(p.h, p.x, nb) || !output_vs_input_ok(p.h, p.res, nb) ||
            !output_vs_input_ok(p.out, p.res, nb))
            return RMSNORM_ERR_INVALID_ARG;
    }
    return RMSNORM_OK;
}

bool vector_aligned(const Problem& p) {
    if ((p.hidden * elem_size(p.dtype)) % kVectorBytes != 0) return false;
    const void* ptrs[] = {p.x, p.w, p.out, p.res, p.h};
    for (const void* q : ptrs)
        if (q && reinterpret_cast<uintptr_t>(q) % kVectorBytes != 0) return false;
    return true;  // codes: a 16-byte-aligned base keeps every row's 8- (4-) byte stores aligned
}

// The automatic choice, from launch-shape sweeps on MI355X.  Vector path:
// spread a row over the fewest waves (one row per workgroup) that keep at most
// two 16-byte vectors of it per lane (three for the fused form, whose lanes
// then keep the weight resident) -- many short waves keep more requests in
// flight than a few long ones; e.g. bf16 hidden 8192 runs as 8 waves x 2
// vectors, the fused bf16 hidden 5120 as 4 waves x 3.  The quantised forms
// store half as many bytes per vector and hold the weight anyway; they run
// fastest with up to four (five fused) vectors per lane: 4 x 4 for hidden
// 8192, 2 x 5 for the fused 5120.  Element path: at most 8 elements per lane.  When rows are few,
// each row gets more waves so the whole GPU has work.  Rows that no built
// register-resident configuration covers take the two-pass path.
rmsnorm_config_t choose(int64_t rows, int64_t hidden, int dtype, bool aligned, bool fused, int qt) {
    rmsnorm_config_t c = {RMSNORM_PATH_TWO_PASS, 16, 0, 1, 0};
    const bool vec = aligned && hidden % vec_elems(dtype) == 0;
    const int64_t units = vec ? hidden / vec_elems(dtype) : hidden;
    const int* list = vec ? mbr::kVplList : mbr::kEplList;
    const int nlist = vec ? mbr::kNumVpl : mbr::kNumEpl;
    const int cap = vec ? (qt ? (fused ? 5 : 4) : (fused ? 3 : 2)) : 8;
    auto fit = [&](int wpr) {
        const int per = round_up_in(list, nlist, ceil_div(units, int64_t(64) * wpr));
        if (per < 0) return -1;
        const bool built = qt ? (vec ? mbr::qvec_built(wpr, per) : mbr::qelem_built(wpr, per))
                              : (vec ? mbr::vec_built(wpr, per, fused) : mbr::elem_built(wpr, per));
        return built ? per : -1;
    };
    int wpr = 1;
    while (wpr < 16 && ceil_div(units, int64_t(64) * wpr) > cap) wpr *= 2;
    while (wpr < 16 && rows < 4096 / wpr && units >= int64_t(64) * wpr * 2) wpr *= 2;
    int per = fit(wpr);
    while (per < 0 && wpr < 16) {
        wpr *= 2;
        per = fit(wpr);
    }
    if (per < 0) return c;
    c.path = vec ? RMSNORM_PATH_VECTOR : RMSNORM_PATH_ELEMENT;
    c.waves_per_row = wpr;
    c.items_per_lane = per;
    c.rows_per_block = 1;
    c.max_blocks = 0;
    return c;
}

rmsnorm_status_t launch(const Problem& p, const rmsnorm_config_t* user, hipStream_t stream) {
    const bool aligned = vector_aligned(p);
    const rmsnorm_config_t c = (user && user->path != RMSNORM_PATH_AUTO) ? *user : choose(p.rows, p.hidden, p.dtype, aligned, p.fused, p.qt);
    const int wi = index_of(mbr::kWprList, mbr::kNumWpr, c.waves_per_row);
    if (wi < 0 || c.rows_per_block < 1 || c.max_blocks < 0) return RMSNORM_ERR_INVALID_ARG;
    const int64_t lanes_per_row = int64_t(64) * c.waves_per_row;

    mbr::RowArgs a;
    a.x = p.x;
    a.res = p.res;
    a.w = p.w;
    a.h = p.h;
    a.out = p.out;
    a.rows = p.rows;
    a.rows_per_block = c.rows_per_block;
    a.hidden_f = static_cast<float>(p.hidden);
    a.eps = p.eps;
    a.scale = p.scale;

    const void* fn = nullptr;
    int64_t threads = 0;
    switch (c.path) {
        case RMSNORM_PATH_VECTOR: {
            if (!aligned || p.hidden % vec_elems(p.dtype) != 0) return RMSNORM_ERR_INVALID_ARG;
            const int vi = index_of(mbr::kVplList, mbr::kNumVpl, c.items_per_lane);
            const int64_t nvec = p.hidden / vec_elems(p.dtype);
            if (vi < 0 || lanes_per_row * c.items_per_lane < nvec) return RMSNORM_ERR_INVALID_ARG;
            threads = lanes_per_row * c.rows_per_block;
            if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            const bool masked = lanes_per_row * c.items_per_lane != nvec;
            fn = p.qt ? mbr::qvec_kernel(p.dtype, p.qt, p.fused, masked, wi, vi)
                      : mbr::vec_kernel(p.dtype, p.fused, masked, wi, vi);
            a.units = static_cast<int32_t>(nvec);
            break;
        }
        case RMSNORM_PATH_ELEMENT: {
            const int ei = index_of(mbr::kEplList, mbr::kNumEpl, c.items_per_lane);
            if (ei < 0 || lanes_per_row * c.items_per_lane < p.hidden) return RMSNORM_ERR_INVALID_ARG;
            threads = lanes_per_row * c.rows_per_block;
            if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            fn = p.qt ? mbr::qelem_kernel(p.dtype, p.qt, p.fused, wi, ei) : mbr::elem_kernel(p.dtype, p.fused, wi, ei);
            a.units = static_cast<int32_t>(p.hidden);
            break;
        }
        case RMSNORM_PATH_TWO_PASS: {
            if (c.rows_per_block != 1) return RMSNORM_ERR_INVALID_ARG;
            const bool vec = aligned && p.hidden % vec_elems(p.dtype) == 0;
            threads = lanes_per_row;
            fn = p.qt ? mbr::qtwopass_kernel(p.dtype, p.qt, p.fused, vec) : mbr::twopass_kernel(p.dtype, p.fused, vec);
            a.units = static_cast<int32_t>(vec ? p.hidden / vec_elems(p.dtype) : p.hidden);
            break;
        }
        default:
            return RMSNORM_ERR_INVALID_ARG;
    }
    if (!fn) return RMSNORM_ERR_INVALID_ARG;
    a.n_groups = ceil_div(p.rows, c.rows_per_block);
    int64_t grid = a.n_groups < kMaxGrid ? a.n_groups : kMaxGrid;
    if (c.max_blocks > 0 && grid > c.max_blocks) grid = c.max_blocks;

    if (p.rows == 0) return RMSNORM_OK;
    void* args[] = {&a};
    hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(static_cast<unsigned>(threads)),
                                   args, 0, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // do not leave a sticky error for the caller's next HIP call
        return RMSNORM_ERR_RUNTIME;
    }
    return RMSNORM_OK;
}

rmsnorm_status_t run(const Problem& p, const rmsnorm_config_t* cfg, void* stream) {
    rmsnorm_status_t s = validate_sizes(p.rows, p.hidden, p.eps, p.dtype);
    if (s != RMSNORM_OK) return s;
    if (p.rows == 0) return RMSNORM_OK;
    s = validate_pointers(p);
    if (s != RMSNORM_OK) return s;
    return launch(p, cfg, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

RMSNORM_API rmsnorm_status_t rmsnorm_fwd(const void* x, const void* weight, void* out, int64_t rows,
                                         int64_t hidden, float eps, rmsnorm_dtype_t dtype, void* stream) {
    return rmsnorm_fwd_ex(x, weight, out, rows, hidden, eps, dtype, nullptr, stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_residual_fwd(const void* x, const void* residual, const void* weight,
                                                  void* residual_out, void* out, int64_t rows, int64_t hidden,
                                                  float eps, rmsnorm_dtype_t dtype, void* stream) {
    return rmsnorm_residual_fwd_ex(x, residual, weight, residual_out, out, rows, hidden, eps, dtype, nullptr,
                                   stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_fwd_ex(const void* x, const void* weight, void* out, int64_t rows,
                                            int64_t hidden, float eps, rmsnorm_dtype_t dtype,
                                            const rmsnorm_config_t* cfg, void* stream) {
    Problem p = {x, nullptr, weight, nullptr, out, rows, hidden, eps, static_cast<int>(dtype), false, 0, nullptr};
    return run(p, cfg, stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_residual_fwd_ex(const void* x, const void* residual, const void* weight,
                                                     void* residual_out, void* out, int64_t rows, int64_t hidden,
                                                     float eps, rmsnorm_dtype_t dtype,
                                                     const rmsnorm_config_t* cfg, void* stream) {
    Problem p = {x, residual, weight, residual_out, out, rows, hidden, eps, static_cast<int>(dtype), true, 0, nullptr};
    return run(p, cfg, stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_select_config(int64_t rows, int64_t hidden, rmsnorm_dtype_t dtype,
                                                   int32_t vector_aligned_flag, int32_t fused,
                                                   rmsnorm_config_t* cfg) {
    if (!cfg) return RMSNORM_ERR_INVALID_ARG;
    rmsnorm_status_t s = validate_sizes(rows, hidden, 0.0f, static_cast<int>(dtype));
    if (s != RMSNORM_OK) return s;
    *cfg = choose(rows, hidden, static_cast<int>(dtype), vector_aligned_flag != 0, fused != 0, 0);
    return RMSNORM_OK;
}

RMSNORM_API rmsnorm_status_t rmsnorm_dynamic_quant_fwd_ex(const void* x, const void* residual, const void* weight,
                                                         void* residual_out, void* q_out, float* scale_out,
                                                         int64_t rows, int64_t hidden, float eps,
                                                         rmsnorm_dtype_t dtype, rmsnorm_quant_t qtype,
                                                         const rmsnorm_config_t* cfg, void* stream) {
    if (qtype != RMSNORM_QUANT_INT8 && qtype != RMSNORM_QUANT_FP8_E4M3) {
        const rmsnorm_status_t s = validate_sizes(rows, hidden, eps, static_cast<int>(dtype));
        return s != RMSNORM_OK ? s : RMSNORM_ERR_UNSUPPORTED_DTYPE;
    }
    if ((residual == nullptr) != (residual_out == nullptr)) return RMSNORM_ERR_INVALID_ARG;
    if (rows > INT64_MAX / 4) return RMSNORM_ERR_INVALID_ARG;  // the scale vector's byte size must fit
    Problem p = {x, residual, weight, residual_out, q_out, rows, hidden, eps, static_cast<int>(dtype),
                 residual != nullptr, qtype == RMSNORM_QUANT_INT8 ? 1 : 2, scale_out};
    return run(p, cfg, stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_dynamic_quant_fwd(const void* x, const void* residual, const void* weight,
                                                      void* residual_out, void* q_out, float* scale_out,
                                                      int64_t rows, int64_t hidden, float eps, rmsnorm_dtype_t dtype,
                                                      rmsnorm_quant_t qtype, void* stream) {
    return rmsnorm_dynamic_quant_fwd_ex(x, residual, weight, residual_out, q_out, scale_out, rows, hidden, eps, dtype,
                                        qtype, nullptr, stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_select_quant_config(int64_t rows, int64_t hidden, rmsnorm_dtype_t dtype,
                                                         int32_t vector_aligned_flag, int32_t fused,
                                                         rmsnorm_config_t* cfg) {
    if (!cfg) return RMSNORM_ERR_INVALID_ARG;
    rmsnorm_status_t s = validate_sizes(rows, hidden, 0.0f, static_cast<int>(dtype));
    if (s != RMSNORM_OK) return s;
    *cfg = choose(rows, hidden, static_cast<int>(dtype), vector_aligned_flag != 0, fused != 0, 1);
    return RMSNORM_OK;
}

RMSNORM_API const char* rmsnorm_status_string(rmsnorm_status_t status) {
    switch (status) {
        case RMSNORM_OK:
            return "RMSNORM_OK";
        case RMSNORM_ERR_INVALID_ARG:
            return "RMSNORM_ERR_INVALID_ARG: invalid argument (pointer, size, eps, overlap or configuration)";
        case RMSNORM_ERR_UNSUPPORTED_DTYPE:
            return "RMSNORM_ERR_UNSUPPORTED_DTYPE: dtype must be RMSNORM_DTYPE_F32 or RMSNORM_DTYPE_BF16";
        case RMSNORM_ERR_RUNTIME:
            return "RMSNORM_ERR_RUNTIME: the HIP runtime reported an error at launch";
    }
    return "unknown rmsnorm status";
}

}  // extern "C"
