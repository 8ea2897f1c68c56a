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

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <math.h>
#include <mutex>
#include <stdint.h>

#include "../../include/rmsnorm.h"
#include "kv_kernels.hpp"
#include "layernorm_kernels.hpp"
#include "rmsnorm_bwd_kernels.hpp"
#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace {

constexpr int64_t kVectorBytes = 16;
// Largest grid launched in one call; bigger jobs loop inside the kernel.
constexpr int64_t kMaxGrid = int64_t(1) << 20;
// Most dynamic LDS a workgroup may take for a staged weight (gamma and beta
// for LayerNorm) or the backward's slot combine: a gfx950 workgroup can take
// 160 KiB (the device reports 163840 bytes per block), less 1 KiB kept for
// the kernels' own row totals.
constexpr size_t kWeightLdsMax = 160 * 1024 - 1024;
// The LayerNorm automatic choice stages gamma and beta only within the window
// its sweeps covered (60 KiB together).
constexpr size_t kLnStageAutoMax = 60 * 1024;
// Workgroup size when rows narrower than half a wave share waves: one wave.
// Sweeps on MI355X (HIP-graph timing): bf16 [262144, 128] runs in 23.3 us as
// 16 lanes x 1 vector x 4 rows per 64-lane workgroup, against 62.8 us with a
// whole wave per row; [524288, 64] 23.7 against 115 us; [131072, 256]
// 23.3 against 36.3 us; 128- to 512-lane workgroups were 1-6 % slower.
constexpr int kSubwaveThreads = 64;

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

// Whether the any-alignment path's shifted frame can apply: bf16, and x (and
// residual, h, and a normalised out; codes have no alignment) at the same
// offset modulo 4 bytes, so that every row's tensors share it; some row must
// start 2 bytes past a 4-byte boundary (an odd width, or a base there).
bool shifted_frame(const Problem& p) {
    if (p.dtype != RMSNORM_DTYPE_BF16) return false;
    const uintptr_t m = reinterpret_cast<uintptr_t>(p.x) & 3;
    if (!p.qt && (reinterpret_cast<uintptr_t>(p.out) & 3) != m) return false;
    if (p.fused && ((reinterpret_cast<uintptr_t>(p.res) & 3) != m || (reinterpret_cast<uintptr_t>(p.h) & 3) != m))
        return false;
    return m != 0 || p.hidden % 2 != 0;
}

// Vectors per lane the register + LDS path holds in registers for a row of
// nvec vectors, or 0 when the row does not fit it: the register part must
// leave at least one vector for LDS, and the rest must fit the LDS limit.
int stage_rv(int64_t nvec, bool fused) {
    const int64_t lds_vectors = mbr::kStageLdsMax / kVectorBytes;
    int rv = 0;
    if (!fused) {
        rv = mbr::kStageRvPlain;
    } else {
        for (int v : mbr::kStageRvFused)  // ascending: the most registers that leave a staged part
            if (nvec > int64_t(mbr::kStageLanes) * v) rv = v;
    }
    if (rv == 0) return 0;
    const int64_t staged = nvec - int64_t(mbr::kStageLanes) * rv;
    return staged >= 1 && staged <= lds_vectors ? rv : 0;
}

// The automatic choice, from launch-shape sweeps on MI355X.  Vector path:
// spread a row over the fewest waves (one row per workgroup) that keep at most
// two 16-byte vectors of it per lane (four for the fused form, whose lanes
// then keep the weight resident) -- many short waves keep more requests in
// flight than a few long ones; e.g. bf16 hidden 8192 runs as 8 waves x 2
// vectors, the fused bf16 hidden 5120 as 4 waves x 3 and 8192 as 4 x 4
// (fused [12289, 8192]: 128.5 us against 132.3 as 8 x 2).  The quantised forms
// store half as many bytes per vector and hold the weight anyway; they run
// fastest with up to four (five fused) vectors per lane: 4 x 4 for hidden
// 8192, 2 x 5 for the fused 5120.  Element path (rows narrower than one
// vector): one wave, one element per lane.  When rows are few,
// each row gets more waves so the whole GPU has work.  Rows that no built
// register-resident configuration covers take the two-pass path.
rmsnorm_config_t choose(int64_t rows, int64_t hidden, int dtype, bool aligned, bool fused, int qt) {
    rmsnorm_config_t c = {RMSNORM_PATH_TWO_PASS, 16, 0, 1, 0, 0, 0};
    const bool vec = aligned && hidden % vec_elems(dtype) == 0;
    // any other width or alignment: full vectors at the row's own alignment
    // plus a tail of single elements (every form)
    const bool any = !vec && hidden >= vec_elems(dtype);
    // the any-alignment path's shifted frame (bf16 rows that start 2 bytes
    // past a 4-byte boundary) moves one more element per row
    const int64_t frame_extra = any && dtype == RMSNORM_DTYPE_BF16 ? 1 : 0;
    const int64_t units = vec || any ? (hidden + frame_extra) / vec_elems(dtype) : hidden;
    const int* list = vec ? mbr::kVplList : any ? mbr::kAnyVplList : mbr::kEplList;
    const int nlist = vec ? mbr::kNumVpl : any ? mbr::kNumAnyVpl : mbr::kNumEpl;
    const int cap = vec || any ? (qt ? (fused ? 5 : 4) : (fused ? 4 : 2)) : 8;
    auto fit = [&](int wpr) {
        const int per = round_up_in(list, nlist, ceil_div(units, int64_t(64) * wpr));
        if (per < 0) return -1;
        const bool built = qt ? (vec ? mbr::qvec_built(wpr, per)
                                 : any ? mbr::qany_built(wpr, per)
                                       : mbr::qelem_built(wpr, per))
                         : vec ? mbr::vec_built(wpr, per, fused)
                         : any ? mbr::any_built(wpr, per, fused)
                               : mbr::elem_built(wpr, per);
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
    if (per < 0) {
        // Wider than every register configuration.  Aligned rows that fit
        // 1024 lanes' registers plus LDS are still read once (register + LDS
        // path); the rest take two passes.
        if (vec && !qt) {
            const int rv = stage_rv(units, fused);
            if (rv > 0) {
                c.path = RMSNORM_PATH_VECTOR_LDS;
                c.waves_per_row = 16;
                c.items_per_lane = rv;
            }
        }
        return c;
    }
    if ((vec || any) && !qt && rows >= 1024 && (!fused || rows < 4096) && int64_t(64) * wpr * per > units) {
        // rows the cap leaves padded (bf16 hidden 3072, 5120, 6144; fused
        // 5120 below 4096 rows): the fewest idle lanes with at most five
        // vectors per lane, ties kept as chosen.  Sweeps on MI355X: [8192,
        // 5120] 2 x 5 28.6 us against 31.6 as 8 x 2, [4096, 6144] 4 x 3 18.3
        // against 19.5, fused [1024, 5120] 2 x 5 7.6 against 9.0 as 4 x 3.
        int64_t pad = int64_t(64) * wpr * per - units;
        for (int w = 1; w <= 16; w *= 2) {
            const int v = fit(w);
            if (v < 0 || v > 5) continue;
            const int64_t q = int64_t(64) * w * v - units;
            if (q < pad) {
                pad = q;
                wpr = w;
                per = v;
            }
        }
    }
    c.path = vec ? RMSNORM_PATH_VECTOR : any ? RMSNORM_PATH_VECTOR_ANY : RMSNORM_PATH_ELEMENT;
    c.waves_per_row = wpr;
    c.items_per_lane = per;
    c.rows_per_block = 1;
    c.max_blocks = 0;
    if (vec && !fused && !qt && units >= 384 && units * kVectorBytes <= int64_t(kWeightLdsMax)) {
        // A plain job that fits one residency round (3072 to 4096 waves of
        // rows at up to eight vectors per lane): four rows per workgroup
        // (two at two waves a row) sharing one LDS copy of the weight, which
        // leaves each lane 6-8 fewer global loads.  Sweeps on MI355X: bf16
        // [2048, 8192] 11.7 us against 13.8, [2048, 5120] 7.5 against 10.1,
        // [4096, 3072] 9.1 against 11.2; no gain outside that window.
        int w1 = 1;
        while (ceil_div(units, int64_t(64) * w1) > 8) w1 *= 2;
        const int v1 = fit(w1);
        if (v1 > 0 && rows * w1 >= 3072 && rows * w1 <= 4096 && w1 <= 2) {
            c.waves_per_row = w1;
            c.items_per_lane = v1;
            c.rows_per_block = 4;
            c.weight_lds = 1;
        }
    }
    if (vec && !fused && !qt && units <= mbr::kLprList[mbr::kNumLpr - 1]) {
        // a plain row narrower than half a wave: the smallest lane group that
        // holds it with one vector per lane, one wave per workgroup
        const int lpr = round_up_in(mbr::kLprList, mbr::kNumLpr, units);
        const int64_t per_wave = 64 / lpr;  // rows sharing one wave
        c.lanes_per_row = lpr;
        c.items_per_lane = 1;
        c.rows_per_block = static_cast<int32_t>(
            std::min<int64_t>(kSubwaveThreads / lpr, std::max<int64_t>(per_wave, ceil_div(rows, per_wave) * per_wave)));
    } else if (vec && units <= 2 * mbr::kLprList[mbr::kNumLpr - 1] && (fused || qt || units % 64 != 0)) {
        // Fused and quantised rows of at most 64 vectors, and plain ones of
        // 33..63 (a whole wave would leave lanes idle): the smallest lane group
        // that holds the row with at most two vectors per lane, two waves per
        // workgroup (one while there would be under 256 workgroups).  HIP-graph
        // sweeps on MI355X, against one wave per row or one vector per lane:
        // int8 [262144, 128] 19.6-20.3 us against 25.6, int8 [65536, 512] 20.0-20.3
        // against 26.8, fused [262144, 128] 44.9 against 46.9, plain
        // [65536, 384] 18.9 against 22.1.
        int lpr = 0;
        for (int i = 0; i < mbr::kNumLpr && !lpr; ++i)
            if (ceil_div(units, int64_t(mbr::kLprList[i])) <= 2) lpr = mbr::kLprList[i];
        int rpb = 128 / lpr;
        if (rows < int64_t(rpb) * 256) rpb = 64 / lpr;
        c.waves_per_row = 1;
        c.items_per_lane = static_cast<int>(ceil_div(units, int64_t(lpr)));
        c.rows_per_block = rpb;
        c.lanes_per_row = lpr;
    }
    return c;
}

rmsnorm_status_t launch(const Problem& p, const rmsnorm_config_t* user, hipStream_t stream) {
    const bool aligned = vector_aligned(p);
    const rmsnorm_config_t c = (user && user->path != RMSNORM_PATH_AUTO) ? *user : choose(p.rows, p.hidden, p.dtype, aligned, p.fused, p.qt);
    const int wi = index_of(mbr::kWprList, mbr::kNumWpr, c.waves_per_row);
    if (wi < 0 || c.rows_per_block < 1 || c.max_blocks < 0) return RMSNORM_ERR_INVALID_ARG;
    if (c.weight_lds != 0 && c.weight_lds != 1) return RMSNORM_ERR_INVALID_ARG;
    const bool whole = c.lanes_per_row == 0 || c.lanes_per_row == 64 * c.waves_per_row;
    if (c.weight_lds && (c.path != RMSNORM_PATH_VECTOR || !whole)) return RMSNORM_ERR_INVALID_ARG;
    const int64_t lanes_per_row = whole ? int64_t(64) * c.waves_per_row : c.lanes_per_row;

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
    a.w_lds = c.weight_lds;
    a.tail = 0;
    a.frame = 0;
    size_t lds_bytes = 0;

    const void* fn = nullptr;
    int64_t threads = 0;
    switch (c.path) {
        case RMSNORM_PATH_VECTOR: {
            if (!aligned || p.hidden % vec_elems(p.dtype) != 0) return RMSNORM_ERR_INVALID_ARG;
            const int64_t nvec = p.hidden / vec_elems(p.dtype);
            if (!whole) {  // several rows per wave, lanes_per_row lanes each
                const int li = index_of(mbr::kLprList, mbr::kNumLpr, c.lanes_per_row);
                const int vi = index_of(mbr::kSwVplList, mbr::kNumSwVpl, c.items_per_lane);
                if (c.waves_per_row != 1 || li < 0 || vi < 0 || lanes_per_row * c.items_per_lane < nvec)
                    return RMSNORM_ERR_INVALID_ARG;
                threads = lanes_per_row * c.rows_per_block;
                if (threads % 64 != 0 || threads > mbr::max_threads_for(1)) return RMSNORM_ERR_INVALID_ARG;
                fn = mbr::subwave_kernel(p.dtype, p.fused, p.qt, lanes_per_row * c.items_per_lane != nvec, li, vi);
                a.units = static_cast<int32_t>(nvec);
                break;
            }
            const int vi = index_of(mbr::kVplList, mbr::kNumVpl, c.items_per_lane);
            if (vi < 0 || lanes_per_row * c.items_per_lane < nvec) return RMSNORM_ERR_INVALID_ARG;
            threads = lanes_per_row * c.rows_per_block;
            if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            const bool masked = lanes_per_row * c.items_per_lane != nvec;
            fn = p.qt ? mbr::qvec_kernel(p.dtype, p.qt, p.fused, masked, wi, vi)
                      : mbr::vec_kernel(p.dtype, p.fused, masked, wi, vi);
            a.units = static_cast<int32_t>(nvec);
            if (c.weight_lds) {
                lds_bytes = static_cast<size_t>(nvec) * kVectorBytes;
                if (lds_bytes > kWeightLdsMax) return RMSNORM_ERR_INVALID_ARG;
            }
            break;
        }
        case RMSNORM_PATH_VECTOR_ANY: {
            if (!whole || c.rows_per_block != 1 || c.weight_lds) return RMSNORM_ERR_INVALID_ARG;
            const int64_t nvec = p.hidden / vec_elems(p.dtype);
            const int vi = index_of(mbr::kAnyVplList, mbr::kNumAnyVpl, c.items_per_lane);
            if (nvec < 1 || vi < 0 || lanes_per_row * c.items_per_lane < nvec) return RMSNORM_ERR_INVALID_ARG;
            threads = lanes_per_row;
            if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            // bf16 rows that start 2 bytes past a 4-byte boundary move in the
            // shifted frame (one more element per row) when every row tensor
            // shares that offset and the configuration covers the longer row
            a.frame = shifted_frame(p) && lanes_per_row * c.items_per_lane >= (p.hidden + 1) / vec_elems(p.dtype);
            const bool masked = a.frame || lanes_per_row * c.items_per_lane != nvec;
            fn = p.qt ? mbr::qany_kernel(p.dtype, p.qt, p.fused, masked, wi, vi)
                      : mbr::any_kernel(p.dtype, p.fused, masked, wi, vi);
            a.units = static_cast<int32_t>(nvec);
            a.tail = static_cast<int32_t>(p.hidden - nvec * vec_elems(p.dtype));
            break;
        }
        case RMSNORM_PATH_ELEMENT: {
            if (!whole) return RMSNORM_ERR_INVALID_ARG;
            const int ei = index_of(mbr::kEplList, mbr::kNumEpl, c.items_per_lane);
            if (ei < 0 || lanes_per_row * c.items_per_lane < p.hidden) return RMSNORM_ERR_INVALID_ARG;
            threads = lanes_per_row * c.rows_per_block;
            if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            fn = p.qt ? mbr::qelem_kernel(p.dtype, p.qt, p.fused, wi, ei) : mbr::elem_kernel(p.dtype, p.fused, wi, ei);
            a.units = static_cast<int32_t>(p.hidden);
            break;
        }
        case RMSNORM_PATH_VECTOR_LDS: {
            if (!aligned || p.hidden % vec_elems(p.dtype) != 0 || p.qt) return RMSNORM_ERR_INVALID_ARG;
            if (c.waves_per_row != 16 || !whole || c.rows_per_block != 1 || c.weight_lds) return RMSNORM_ERR_INVALID_ARG;
            const int64_t nvec = p.hidden / vec_elems(p.dtype);
            const int64_t staged = nvec - int64_t(mbr::kStageLanes) * c.items_per_lane;
            if (staged < 1 || staged * kVectorBytes > mbr::kStageLdsMax) return RMSNORM_ERR_INVALID_ARG;
            fn = mbr::stage_kernel(p.dtype, p.fused, c.items_per_lane);
            threads = mbr::kStageLanes;
            lds_bytes = static_cast<size_t>(staged * kVectorBytes);
            a.units = static_cast<int32_t>(nvec);
            break;
        }
        case RMSNORM_PATH_TWO_PASS: {
            if (c.rows_per_block != 1 || !whole) return RMSNORM_ERR_INVALID_ARG;
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
                                   args, lds_bytes, stream);
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

// ---------------------------------------------------------------- backward

struct BwdProblem {
    const void* x;
    const void* w;
    const void* dy;
    void* dx;
    void* dw;  // nullptr: dweight not wanted
    int64_t rows;
    int64_t hidden;
    float eps;
    int dtype;
    void* ws;
    size_t ws_bytes;
};

// Floats per partial dweight row: hidden rounded up to 64 (256-byte rows).
int64_t bwd_ld(int64_t hidden) { return (hidden + 63) / 64 * 64; }

// Grid cap of the backward walk with few rows and on the element and two-pass
// paths: 512 workgroups (two per CU on MI355X).  Fixed, not read from the
// device, so that a shape's results (and its workspace size) are the same on
// any GPU.
constexpr int64_t kBwdGrid = 512;

// LDS the backward vector kernel may take for combining its row slots' sums
// (the 160 KiB a gfx950 workgroup can take, less 1 KiB for its row totals).
constexpr size_t kBwdCombineLds = 160 * 1024 - 1024;

// Partial dweight rows (= workgroups of the walk) for a configuration: one per
// group of rows_per_block rows, at most max_blocks.
int64_t bwd_partials(int64_t rows, const rmsnorm_config_t& c) {
    const int64_t cap = c.max_blocks > 0 ? c.max_blocks : kMaxGrid;
    const int64_t groups = ceil_div(rows, int64_t(c.rows_per_block > 0 ? c.rows_per_block : 1));
    return groups < cap ? groups : cap;
}

bool bwd_vector_aligned(const BwdProblem& p) {
    if ((p.hidden * elem_size(p.dtype)) % kVectorBytes != 0) return false;
    const void* ptrs[] = {p.x, p.w, p.dy, p.dx};
    for (const void* q : ptrs)
        if (reinterpret_cast<uintptr_t>(q) % kVectorBytes != 0) return false;
    return true;
}

// Vector path (sweeps on MI355X over bf16 / fp32, hidden 1024..8192, rows
// 1024..16384), by the number of rows:
//   * fewer than 1024: one row per workgroup, spread over more waves (up to
//     2048 waves in all);
//   * 1024 .. 8191, rows of at most 512 vectors: one wave per row holding the
//     whole row (up to eight vectors per lane), four row slots per workgroup
//     (eight for rows of at most 128 vectors) and 256 workgroups: few partial
//     dweight rows, and every lane's loads in flight at once;
//   * otherwise: the waves per row that leave the fewest lanes past the row
//     end with at most six vectors per lane, ties going to four vectors per
//     lane (bf16 hidden 5120: 2 waves x 5, not 4 x 3 with a sixth of the
//     lanes idle, 9% faster); workgroups of four waves filled with row
//     slots; 512 workgroups.
// Narrow rows (at most 64 vectors, from 1024 rows): the smallest lane group
// of 8, 16 or 32 that holds the row with at most two vectors per lane,
// several rows per wave; workgroups of four waves (eight with one vector per
// lane), fewer row slots while there would be under 256 groups of rows; 512
// workgroups.  bf16 [262144, 128]: 37.7 us against 151.7 with a wave per row.
// Element path (rows narrower than one vector): one wave, one element per
// lane.
rmsnorm_config_t choose_bwd(int64_t rows, int64_t hidden, int dtype, bool aligned) {
    rmsnorm_config_t c = {RMSNORM_PATH_TWO_PASS, 16, 0, 1, static_cast<int32_t>(kBwdGrid), 0, 0};
    const bool vec = aligned && hidden % vec_elems(dtype) == 0;
    // any other width or alignment: full vectors at the row's own alignment
    // plus a tail of single elements, one row per workgroup
    const bool any = !vec && hidden >= vec_elems(dtype);
    const bool vlike = vec || any;
    const int64_t units = vlike ? hidden / vec_elems(dtype) : hidden;
    const int* list = vlike ? mbr::kBwdVplList : mbr::kBwdEplList;
    const int nlist = vlike ? mbr::kNumBwdVpl : mbr::kNumBwdEpl;
    // The any-alignment kernel takes one row per workgroup: below 12288 rows it
    // runs fastest with at most two vectors per lane and more waves per row.
    // Sweeps on MI355X (bf16, 512 workgroups): [4096, 4097] 4 x 2 27.5 us
    // against 29.5 as 2 x 4, [4096, 2049] 2 x 2 19.4 against 22.6 as 1 x 4;
    // from 12288 rows on the balanced rule below holds ([12289, 5121] 2 x 5
    // 88.8 us, [16384, 8191] 4 x 4 179.6; the element kernel 114.2 and 179.0).
    const bool any_short = any && rows < 12288;
    const int cap = vlike ? (any_short ? 2 : 4) : 8;
    const bool few = rows < 1024;
    if (vec && !few && units <= 64) {
        int lpr = 0;
        for (int i = 0; i < mbr::kNumLpr && !lpr; ++i)
            if (ceil_div(units, int64_t(mbr::kLprList[i])) <= 2) lpr = mbr::kLprList[i];
        const int vpl = static_cast<int>(ceil_div(units, int64_t(lpr)));
        int rpb = (vpl == 1 ? 512 : 256) / lpr;
        while (rpb > 64 / lpr && rows < int64_t(rpb) * 256) rpb /= 2;
        c.path = RMSNORM_PATH_VECTOR;
        c.waves_per_row = 1;
        c.items_per_lane = vpl;
        c.rows_per_block = rpb;
        c.max_blocks = 512;
        c.lanes_per_row = lpr;
        return c;
    }
    auto fit = [&](int wpr) {
        const int per = round_up_in(list, nlist, ceil_div(units, int64_t(64) * wpr));
        if (per < 0) return -1;
        const bool built = vec ? mbr::bwd_vec_built(wpr, per) : !any || mbr::bwd_any_built(wpr, per);
        return built ? per : -1;
    };
    const bool whole_row = vec && !few && rows < 8192 && units <= 512;
    const bool balanced = vlike && !few && !whole_row && !any_short;
    int wpr = 1;
    if (balanced) {
        int64_t best_pad = -1;
        int best_v = 0;
        for (int w = 1; w <= 16; w *= 2) {
            const int v = fit(w);
            if (v < 0 || v > 6) continue;
            const int64_t pad = int64_t(64) * w * v - units;
            if (best_pad < 0 || pad < best_pad || (pad == best_pad && std::abs(v - 4) < std::abs(best_v - 4))) {
                wpr = w;
                best_pad = pad;
                best_v = v;
            }
        }
    } else if (!whole_row) {
        while (wpr < 16 && ceil_div(units, int64_t(64) * wpr) > cap) wpr *= 2;
        while (!vlike && wpr < 4 && units >= int64_t(64) * wpr * 2) wpr *= 2;
        while (wpr < 16 && rows < 2048 / wpr && units >= int64_t(64) * wpr * 2) wpr *= 2;
    }
    int per = fit(wpr);
    while (per < 0 && wpr < 16) {
        wpr *= 2;
        per = fit(wpr);
    }
    if (per < 0) return c;
    c.path = vec ? RMSNORM_PATH_VECTOR : any ? RMSNORM_PATH_VECTOR_ANY : RMSNORM_PATH_ELEMENT;
    c.waves_per_row = wpr;
    c.items_per_lane = per;
    if (whole_row) {
        c.rows_per_block = units <= 128 ? 8 : 4;
        c.max_blocks = 256;
    } else if (balanced) {
        c.rows_per_block = wpr < 4 && vec ? 4 / wpr : 1;
        c.max_blocks = 512;
    }
    return c;
}

// Workspace bytes a configuration needs (0 without dweight or rows).
int64_t bwd_workspace_need(int64_t rows, int64_t hidden, const rmsnorm_config_t& c) {
    return bwd_partials(rows, c) * bwd_ld(hidden) * 4;
}

rmsnorm_status_t validate_bwd_pointers(const BwdProblem& p, int64_t ws_need) {
    const int es = elem_size(p.dtype);
    if (!p.x || !p.w || !p.dy || !p.dx) return RMSNORM_ERR_INVALID_ARG;
    const void* ptrs[] = {p.x, p.w, p.dy, p.dx, p.dw};
    for (const void* q : ptrs)
        if (q && reinterpret_cast<uintptr_t>(q) % es != 0) return RMSNORM_ERR_INVALID_ARG;
    const int64_t nb = p.rows * p.hidden * es;
    const int64_t wb = p.hidden * es;
    if (!output_vs_input_ok(p.dx, p.x, nb) || !output_vs_input_ok(p.dx, p.dy, nb)) return RMSNORM_ERR_INVALID_ARG;
    if (ranges_overlap(p.dx, nb, p.w, wb)) return RMSNORM_ERR_INVALID_ARG;
    if (!p.dw) return RMSNORM_OK;
    const void* others[] = {p.x, p.w, p.dy, p.dx};
    const int64_t sizes[] = {nb, wb, nb, nb};
    for (int i = 0; i < 4; ++i)
        if (ranges_overlap(p.dw, wb, others[i], sizes[i])) return RMSNORM_ERR_INVALID_ARG;
    if (ws_need == 0) return RMSNORM_OK;
    if (!p.ws || reinterpret_cast<uintptr_t>(p.ws) % kVectorBytes != 0) return RMSNORM_ERR_INVALID_ARG;
    if (p.ws_bytes < static_cast<uint64_t>(ws_need)) return RMSNORM_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i)
        if (ranges_overlap(p.ws, ws_need, others[i], sizes[i])) return RMSNORM_ERR_INVALID_ARG;
    if (ranges_overlap(p.ws, ws_need, p.dw, wb)) return RMSNORM_ERR_INVALID_ARG;
    return RMSNORM_OK;
}

rmsnorm_status_t launch_checked(const void* fn, int64_t grid, int64_t threads, void* arg, hipStream_t stream,
                                size_t lds_bytes = 0) {
    void* args[] = {arg};
    const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(static_cast<unsigned>(threads)),
                                         args, lds_bytes, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return RMSNORM_ERR_RUNTIME;
    }
    return RMSNORM_OK;
}

rmsnorm_status_t run_bwd(const BwdProblem& p, const rmsnorm_config_t* user, void* stream_arg) {
    rmsnorm_status_t s = validate_sizes(p.rows, p.hidden, p.eps, p.dtype);
    if (s != RMSNORM_OK) return s;
    const bool aligned = p.x && p.w && p.dy && p.dx && bwd_vector_aligned(p);
    const rmsnorm_config_t c =
        (user && user->path != RMSNORM_PATH_AUTO) ? *user : choose_bwd(p.rows, p.hidden, p.dtype, aligned);
    const int wi = index_of(mbr::kWprList, mbr::kNumWpr, c.waves_per_row);
    if (wi < 0 || c.rows_per_block < 1 || c.max_blocks < 0) return RMSNORM_ERR_INVALID_ARG;
    if (c.rows_per_block > 1 && c.path != RMSNORM_PATH_VECTOR) return RMSNORM_ERR_INVALID_ARG;
    if (c.weight_lds != 0) return RMSNORM_ERR_INVALID_ARG;
    const bool whole = c.lanes_per_row == 0 || c.lanes_per_row == 64 * c.waves_per_row;
    if (!whole && c.path != RMSNORM_PATH_VECTOR) return RMSNORM_ERR_INVALID_ARG;
    const bool dw = p.dw != nullptr;
    const int64_t ws_need = dw ? bwd_workspace_need(p.rows, p.hidden, c) : 0;
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    if (p.rows == 0) {
        // nothing to differentiate: dx is empty and dweight is zero
        if (!dw) return RMSNORM_OK;
        if (reinterpret_cast<uintptr_t>(p.dw) % elem_size(p.dtype) != 0) return RMSNORM_ERR_INVALID_ARG;
        mbr::DwArgs d = {nullptr, p.dw, bwd_ld(p.hidden), 0, static_cast<int32_t>(p.hidden)};
        return launch_checked(mbr::bwd_dw_kernel(p.dtype), ceil_div(d.ld, mbr::kDwCols), mbr::kDwThreads, &d, stream);
    }
    s = validate_bwd_pointers(p, ws_need);
    if (s != RMSNORM_OK) return s;

    const int64_t lanes = whole ? int64_t(64) * c.waves_per_row : c.lanes_per_row;
    mbr::BwdArgs a;
    a.x = p.x;
    a.w = p.w;
    a.dy = p.dy;
    a.dx = p.dx;
    a.part = static_cast<float*>(p.ws);
    a.rows = p.rows;
    a.rows_per_block = c.rows_per_block;
    a.n_groups = ceil_div(p.rows, int64_t(c.rows_per_block));
    a.ld = bwd_ld(p.hidden);
    a.inv_hidden = static_cast<float>(1.0 / static_cast<double>(p.hidden));
    a.eps = p.eps;
    a.tail = 0;
    const void* fn = nullptr;
    const int64_t threads = lanes * c.rows_per_block;
    size_t lds = 0;
    switch (c.path) {
        case RMSNORM_PATH_VECTOR: {
            if (!aligned || p.hidden % vec_elems(p.dtype) != 0) return RMSNORM_ERR_INVALID_ARG;
            const int vi = index_of(mbr::kBwdVplList, mbr::kNumBwdVpl, c.items_per_lane);
            const int64_t nvec = p.hidden / vec_elems(p.dtype);
            const bool masked = lanes * c.items_per_lane != nvec;
            if (whole) {
                if (vi < 0 || lanes * c.items_per_lane < nvec) return RMSNORM_ERR_INVALID_ARG;
                if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
                fn = mbr::bwd_vec_kernel(p.dtype, dw, masked, wi, vi);
            } else {  // several rows per wave, lanes_per_row lanes each
                const int li = index_of(mbr::kLprList, mbr::kNumLpr, c.lanes_per_row);
                const int si = index_of(mbr::kSwVplList, mbr::kNumSwVpl, c.items_per_lane);
                if (c.waves_per_row != 1 || li < 0 || si < 0 || lanes * c.items_per_lane < nvec)
                    return RMSNORM_ERR_INVALID_ARG;
                if (threads % 64 != 0 || threads > mbr::max_threads_for(1)) return RMSNORM_ERR_INVALID_ARG;
                fn = mbr::bwd_subwave_kernel(p.dtype, dw, masked, li, si);
            }
            a.units = static_cast<int32_t>(nvec);
            // several row slots (several waves, for rows narrower than a wave)
            // combine their dweight sums in LDS: hidden floats
            if (dw && (whole ? c.rows_per_block > 1 : threads > 64)) lds = static_cast<size_t>(p.hidden) * 4;
            if (lds > kBwdCombineLds) return RMSNORM_ERR_INVALID_ARG;
            break;
        }
        case RMSNORM_PATH_VECTOR_ANY: {
            if (!whole) return RMSNORM_ERR_INVALID_ARG;  // rows_per_block 1: checked above
            const int64_t nvec = p.hidden / vec_elems(p.dtype);
            const int vi = index_of(mbr::kBwdVplList, mbr::kNumBwdVpl, c.items_per_lane);
            if (nvec < 1 || vi < 0 || lanes * c.items_per_lane < nvec) return RMSNORM_ERR_INVALID_ARG;
            if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            fn = mbr::bwd_any_kernel(p.dtype, dw, lanes * c.items_per_lane != nvec, wi, vi);
            a.units = static_cast<int32_t>(nvec);
            a.tail = static_cast<int32_t>(p.hidden - nvec * vec_elems(p.dtype));
            break;
        }
        case RMSNORM_PATH_ELEMENT: {
            const int ei = index_of(mbr::kBwdEplList, mbr::kNumBwdEpl, c.items_per_lane);
            if (ei < 0 || lanes * c.items_per_lane < p.hidden) return RMSNORM_ERR_INVALID_ARG;
            if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            fn = mbr::bwd_elem_kernel(p.dtype, dw, wi, ei);
            a.units = static_cast<int32_t>(p.hidden);
            break;
        }
        case RMSNORM_PATH_TWO_PASS: {
            const bool vec = aligned && p.hidden % vec_elems(p.dtype) == 0;
            fn = mbr::bwd_twopass_kernel(p.dtype, dw, vec);
            a.units = static_cast<int32_t>(vec ? p.hidden / vec_elems(p.dtype) : p.hidden);
            break;
        }
        default:
            return RMSNORM_ERR_INVALID_ARG;
    }
    if (!fn) return RMSNORM_ERR_INVALID_ARG;
    const int64_t grid = bwd_partials(p.rows, c);
    s = launch_checked(fn, grid, threads, &a, stream, lds);
    if (s != RMSNORM_OK) return s;
    if (dw) {
        mbr::DwArgs d;
        d.part = static_cast<const float*>(p.ws);
        d.dw = p.dw;
        d.ld = a.ld;
        d.n_part = static_cast<int32_t>(grid);
        d.hidden = static_cast<int32_t>(p.hidden);
        s = launch_checked(mbr::bwd_dw_kernel(p.dtype), ceil_div(a.ld, mbr::kDwCols), mbr::kDwThreads, &d, stream);
    }
    return s;
}

// ---------------------------------------------------------------- allocation-free backward

// The allocation-free backward keeps its partial dweight rows in this fixed
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy (16 MiB) until the process ends.  In host code the name
// is only a host-side stand-in: the array's device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of the scratch array, looked up on its first use with
// the device current; nullptr if HIP reports an error.
float* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    float* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
            (void)hipGetLastError();
            return nullptr;
        }
        p = static_cast<float*>(q);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

rmsnorm_status_t run_bwd_noalloc(BwdProblem p, void* stream) {
    rmsnorm_status_t s = validate_sizes(p.rows, p.hidden, p.eps, p.dtype);
    if (s != RMSNORM_OK) return s;
    if (p.rows == 0) return run_bwd(p, nullptr, stream);  // dweight zeroed, no partial rows
    const bool aligned = p.x && p.w && p.dy && p.dx && bwd_vector_aligned(p);
    rmsnorm_config_t c = choose_bwd(p.rows, p.hidden, p.dtype, aligned);
    if (p.dw) {
        // as many partial rows as the scratch array holds, at most the
        // automatic choice's (then the results equal rmsnorm_bwd's bitwise)
        const int64_t cap = static_cast<int64_t>(kScratchBytes) / (bwd_ld(p.hidden) * 4);
        if (cap < 1) return RMSNORM_ERR_INVALID_ARG;
        if (bwd_partials(p.rows, c) > cap) c.max_blocks = static_cast<int32_t>(cap);
    }
    s = validate_bwd_pointers(p, 0);  // every argument error before the first HIP call
    if (s != RMSNORM_OK) return s;
    if (p.dw) {
        float* ws = scratch_on_current_device();
        if (!ws) return RMSNORM_ERR_RUNTIME;
        p.ws = ws;
        p.ws_bytes = kScratchBytes;
    }
    return run_bwd(p, &c, stream);
}

// ---------------------------------------------------------------- LayerNorm

struct LnProblem {
    const void* x;
    const void* g;
    const void* b;  // nullptr: no bias
    void* out;
    int64_t rows;
    int64_t hidden;
    float eps;
    int dtype;
};

bool ln_vector_aligned(const LnProblem& p) {
    if ((p.hidden * elem_size(p.dtype)) % kVectorBytes != 0) return false;
    const void* ptrs[] = {p.x, p.g, p.b, p.out};
    for (const void* q : ptrs)
        if (q && reinterpret_cast<uintptr_t>(q) % kVectorBytes != 0) return false;
    return true;
}

// Each LayerNorm row needs two workgroup reductions, so rows take as few
// waves as registers allow: up to eight 16-byte vectors (or elements) per lane,
// more waves per row only when rows are few; one row per workgroup, uncapped
// grid.  Sweeps on MI355X with per-row gamma/beta loads, bf16 [8192, 4096]:
// 1 wave x 8 vectors 25.9 us, 2 x 4 26.1, 4 x 2 28.3, 8 x 1 31.8.  Wide rows
// with enough of them then move to row slots sharing gamma/beta in LDS
// (below).  Rows beyond every built register configuration take the
// multi-pass path.  Narrow rows (at most 64 vectors, from 1024 rows) share
// waves in lane groups of 8, 16 or 32 with at most two vectors per lane:
// workgroups of four waves and an uncapped grid, or eight waves and 1024
// workgroups with one vector per lane; fewer row slots while there would be
// under 256 groups of rows.  HIP-graph sweeps on MI355X: bf16 [262144, 128]
// 23.2 us against 70.4 with a wave per row, [131072, 256] 23.2 against 40.1,
// [262144, 64] 14.4 against 68.2.
rmsnorm_config_t choose_ln(int64_t rows, int64_t hidden, int dtype, bool aligned) {
    rmsnorm_config_t c = {RMSNORM_PATH_TWO_PASS, 16, 0, 1, 0, 0, 0};
    const bool vec = aligned && hidden % vec_elems(dtype) == 0;
    // any other width or alignment: full vectors at the row's own alignment,
    // then a tail of single elements
    const bool any = !vec && hidden >= vec_elems(dtype);
    const int64_t units = vec || any ? hidden / vec_elems(dtype) : hidden;
    if (vec && units <= 64 && rows >= 1024) {
        int lpr = 0;
        for (int i = 0; i < mbr::kNumLpr && !lpr; ++i)
            if (ceil_div(units, int64_t(mbr::kLprList[i])) <= 2) lpr = mbr::kLprList[i];
        const int vpl = static_cast<int>(ceil_div(units, int64_t(lpr)));
        int rpb = (vpl == 1 ? 512 : 256) / lpr;
        while (rpb > 64 / lpr && rows < int64_t(rpb) * 256) rpb /= 2;
        c.path = RMSNORM_PATH_VECTOR;
        c.waves_per_row = 1;
        c.items_per_lane = vpl;
        c.rows_per_block = rpb;
        c.max_blocks = vpl == 1 ? 1024 : 0;
        c.lanes_per_row = lpr;
        return c;
    }
    const int* list = vec ? mbr::kLnVplList : any ? mbr::kAnyVplList : mbr::kLnEplList;
    const int nlist = vec ? mbr::kNumLnVpl : any ? mbr::kNumAnyVpl : mbr::kNumLnEpl;
    const int cap = 8;
    auto fit = [&](int wpr) {
        const int per = round_up_in(list, nlist, ceil_div(units, int64_t(64) * wpr));
        if (per < 0) return -1;
        return (vec ? mbr::ln_vec_built(wpr, per) : !any || mbr::ln_any_built(wpr, per)) ? per : -1;
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
    c.path = vec ? RMSNORM_PATH_VECTOR : any ? RMSNORM_PATH_VECTOR_ANY : RMSNORM_PATH_ELEMENT;
    c.waves_per_row = wpr;
    c.items_per_lane = per;
    // Rows of 384 vectors or more, gamma and beta fitting LDS (sized for a
    // beta): row slots sharing one LDS copy of them.  From 4096 rows, the
    // waves per row with the fewest idle lanes at up to five vectors per lane
    // (ties: closest to four) and 512-lane workgroups; at 2048..4095 rows of
    // more than 512 vectors, two waves per row and four slots, so that the
    // job is one round of workgroups.  Sweeps on MI355X (HIP-graph timing,
    // bf16 with beta): [8192, 4096] 25.0 us as 2 x 4 x 4 slots against 26.4,
    // [4096, 4096] 12.5 against 14.5, [4096, 8192] 25.7 (4 x 4 x 2) against
    // 28.8, [2048, 8192] 11.9 (2 x 8 x 4) against 16.5.
    if (vec && units >= 384 && units * kVectorBytes * 2 <= int64_t(kLnStageAutoMax)) {
        int w = 0, v = 0;
        if (rows >= 4096) {
            int64_t best_pad = -1;
            for (int ww = 1; ww <= 16; ww *= 2) {
                const int vv = fit(ww);
                if (vv < 0 || vv > 5) continue;
                const int64_t pad = int64_t(64) * ww * vv - units;
                if (best_pad < 0 || pad < best_pad || (pad == best_pad && std::abs(vv - 4) < std::abs(v - 4))) {
                    best_pad = pad;
                    w = ww;
                    v = vv;
                }
            }
        } else if (rows >= 2048 && units > 512) {
            w = 2;
            v = fit(2);
        }
        if (w > 0 && v > 0 && w <= 8) {
            c.waves_per_row = w;
            c.items_per_lane = v;
            c.rows_per_block = 512 / (64 * w);
            c.weight_lds = 1;
        }
    }
    return c;
}

rmsnorm_status_t validate_ln_pointers(const LnProblem& p) {
    const int es = elem_size(p.dtype);
    if (!p.x || !p.g || !p.out) return RMSNORM_ERR_INVALID_ARG;
    const void* ptrs[] = {p.x, p.g, p.b, p.out};
    for (const void* q : ptrs)
        if (q && reinterpret_cast<uintptr_t>(q) % es != 0) return RMSNORM_ERR_INVALID_ARG;
    const int64_t nb = p.rows * p.hidden * es;
    const int64_t wb = p.hidden * es;
    if (!output_vs_input_ok(p.out, p.x, nb)) return RMSNORM_ERR_INVALID_ARG;
    if (ranges_overlap(p.out, nb, p.g, wb)) return RMSNORM_ERR_INVALID_ARG;
    if (p.b && ranges_overlap(p.out, nb, p.b, wb)) return RMSNORM_ERR_INVALID_ARG;
    return RMSNORM_OK;
}

rmsnorm_status_t run_ln(const LnProblem& p, const rmsnorm_config_t* user, void* stream) {
    rmsnorm_status_t s = validate_sizes(p.rows, p.hidden, p.eps, p.dtype);
    if (s != RMSNORM_OK) return s;
    if (p.rows == 0) return RMSNORM_OK;
    s = validate_ln_pointers(p);
    if (s != RMSNORM_OK) return s;
    const bool aligned = ln_vector_aligned(p);
    const rmsnorm_config_t c =
        (user && user->path != RMSNORM_PATH_AUTO) ? *user : choose_ln(p.rows, p.hidden, p.dtype, aligned);
    const int wi = index_of(mbr::kWprList, mbr::kNumWpr, c.waves_per_row);
    if (wi < 0 || c.rows_per_block < 1 || c.max_blocks < 0) return RMSNORM_ERR_INVALID_ARG;
    if (c.weight_lds != 0 && c.weight_lds != 1) return RMSNORM_ERR_INVALID_ARG;
    const bool whole = c.lanes_per_row == 0 || c.lanes_per_row == 64 * c.waves_per_row;
    if ((c.rows_per_block != 1 || c.weight_lds || !whole) && c.path != RMSNORM_PATH_VECTOR)
        return RMSNORM_ERR_INVALID_ARG;
    // whole-wave slots share the LDS copy; sub-wave rows keep gamma / beta per lane
    if (whole ? c.rows_per_block != 1 && !c.weight_lds : c.weight_lds != 0) return RMSNORM_ERR_INVALID_ARG;
    const int64_t lanes = whole ? int64_t(64) * c.waves_per_row : c.lanes_per_row;
    const int64_t threads = lanes * c.rows_per_block;
    mbr::LnArgs a;
    a.x = p.x;
    a.g = p.g;
    a.b = p.b;
    a.out = p.out;
    a.rows = p.rows;
    a.rows_per_block = c.rows_per_block;
    a.n_groups = ceil_div(p.rows, int64_t(c.rows_per_block));
    a.hidden_f = static_cast<float>(p.hidden);
    a.eps = p.eps;
    a.tail = 0;
    const void* fn = nullptr;
    size_t lds = 0;
    switch (c.path) {
        case RMSNORM_PATH_VECTOR: {
            if (!aligned || p.hidden % vec_elems(p.dtype) != 0) return RMSNORM_ERR_INVALID_ARG;
            const int vi = index_of(mbr::kLnVplList, mbr::kNumLnVpl, c.items_per_lane);
            const int64_t nvec = p.hidden / vec_elems(p.dtype);
            const bool masked = lanes * c.items_per_lane != nvec;
            if (whole) {
                if (vi < 0 || lanes * c.items_per_lane < nvec) return RMSNORM_ERR_INVALID_ARG;
                if (threads > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
                fn = mbr::ln_vec_kernel_ptr(p.dtype, masked, c.weight_lds != 0, wi, vi);
            } else {  // several rows per wave, lanes_per_row lanes each
                const int li = index_of(mbr::kLprList, mbr::kNumLpr, c.lanes_per_row);
                const int si = index_of(mbr::kSwVplList, mbr::kNumSwVpl, c.items_per_lane);
                if (c.waves_per_row != 1 || li < 0 || si < 0 || lanes * c.items_per_lane < nvec)
                    return RMSNORM_ERR_INVALID_ARG;
                if (threads % 64 != 0 || threads > mbr::max_threads_for(1)) return RMSNORM_ERR_INVALID_ARG;
                fn = mbr::ln_subwave_kernel_ptr(p.dtype, masked, li, si);
            }
            a.units = static_cast<int32_t>(nvec);
            if (c.weight_lds) {
                lds = static_cast<size_t>(nvec) * kVectorBytes * (p.b ? 2 : 1);
                if (lds > kWeightLdsMax) return RMSNORM_ERR_INVALID_ARG;
            }
            break;
        }
        case RMSNORM_PATH_VECTOR_ANY: {
            if (!whole || c.rows_per_block != 1 || c.weight_lds) return RMSNORM_ERR_INVALID_ARG;
            const int64_t nvec = p.hidden / vec_elems(p.dtype);
            const int vi = index_of(mbr::kAnyVplList, mbr::kNumAnyVpl, c.items_per_lane);
            if (nvec < 1 || vi < 0 || lanes * c.items_per_lane < nvec) return RMSNORM_ERR_INVALID_ARG;
            if (lanes > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            fn = mbr::ln_any_kernel_ptr(p.dtype, lanes * c.items_per_lane != nvec, wi, vi);
            a.units = static_cast<int32_t>(nvec);
            a.tail = static_cast<int32_t>(p.hidden - nvec * vec_elems(p.dtype));
            break;
        }
        case RMSNORM_PATH_ELEMENT: {
            const int ei = index_of(mbr::kLnEplList, mbr::kNumLnEpl, c.items_per_lane);
            if (ei < 0 || lanes * c.items_per_lane < p.hidden) return RMSNORM_ERR_INVALID_ARG;
            if (lanes > mbr::max_threads_for(c.waves_per_row)) return RMSNORM_ERR_INVALID_ARG;
            fn = mbr::ln_elem_kernel_ptr(p.dtype, wi, ei);
            a.units = static_cast<int32_t>(p.hidden);
            break;
        }
        case RMSNORM_PATH_TWO_PASS: {
            const bool vec = aligned && p.hidden % vec_elems(p.dtype) == 0;
            fn = mbr::ln_multipass_kernel_ptr(p.dtype, vec);
            a.units = static_cast<int32_t>(vec ? p.hidden / vec_elems(p.dtype) : p.hidden);
            break;
        }
        default:
            return RMSNORM_ERR_INVALID_ARG;
    }
    if (!fn) return RMSNORM_ERR_INVALID_ARG;
    int64_t grid = a.n_groups < kMaxGrid ? a.n_groups : kMaxGrid;
    if (c.max_blocks > 0 && grid > c.max_blocks) grid = c.max_blocks;
    return launch_checked(fn, grid, threads, &a, static_cast<hipStream_t>(stream), lds);
}

// ---------------------------------------------------------------- KV RMSNorm + RoPE + cache

struct KvProblem {
    const void* kv;
    const void* gamma;
    const float* cos_t;
    const float* sin_t;
    const int32_t* pos;
    const int64_t* slots;
    void* nc;
    void* rc;
    int64_t tokens;
    int64_t heads;
    int64_t dn;
    int64_t dr;
    int64_t max_pos;
    int64_t num_slots;
    float eps;
    int style;
    int dtype;
};

bool fits(int64_t a, int64_t b, int64_t c, int64_t d) {  // a * b * c * d <= INT64_MAX, all >= 0
    if (a == 0 || b == 0 || c == 0 || d == 0) return true;
    return a <= INT64_MAX / b && a * b <= INT64_MAX / c && a * b * c <= INT64_MAX / d;
}

rmsnorm_status_t validate_kv(const KvProblem& p) {
    if (p.tokens < 0 || p.heads < 1 || p.heads > INT32_MAX || p.dn < 1 || p.dr < 0 || p.dr % 2 != 0 ||
        p.dn + p.dr > INT32_MAX || p.max_pos < 0 || p.num_slots < 0)
        return RMSNORM_ERR_INVALID_ARG;
    if (!(p.eps >= 0.0f) || isinf(p.eps) || (p.style != 0 && p.style != 1)) return RMSNORM_ERR_INVALID_ARG;
    if (p.dtype != RMSNORM_DTYPE_F32 && p.dtype != RMSNORM_DTYPE_BF16) return RMSNORM_ERR_UNSUPPORTED_DTYPE;
    const int64_t es = elem_size(p.dtype);
    if (!fits(p.tokens, p.heads, p.dn + p.dr, es) || !fits(p.num_slots, p.heads, p.dn + p.dr, es) ||
        !fits(p.max_pos, p.dr, 4, 1))
        return RMSNORM_ERR_INVALID_ARG;
    return RMSNORM_OK;
}

rmsnorm_status_t validate_kv_pointers(const KvProblem& p) {
    const int es = elem_size(p.dtype);
    if (!p.kv || !p.gamma || !p.pos || !p.slots || !p.nc) return RMSNORM_ERR_INVALID_ARG;
    if (p.dr > 0 && (!p.cos_t || !p.sin_t || !p.rc)) return RMSNORM_ERR_INVALID_ARG;
    const void* ptrs[] = {p.kv, p.gamma, p.nc, p.rc};
    for (const void* q : ptrs)
        if (q && reinterpret_cast<uintptr_t>(q) % es != 0) return RMSNORM_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(p.pos) % 4 || reinterpret_cast<uintptr_t>(p.slots) % 8 ||
        reinterpret_cast<uintptr_t>(p.cos_t) % 4 || reinterpret_cast<uintptr_t>(p.sin_t) % 4)
        return RMSNORM_ERR_INVALID_ARG;
    const int64_t d = p.dn + p.dr;
    const int64_t ncb = p.num_slots * p.heads * p.dn * es, rcb = p.num_slots * p.heads * p.dr * es;
    const int64_t tb = p.max_pos * (p.dr / 2) * 4;
    const void* in[] = {p.kv, p.gamma, p.cos_t, p.sin_t, p.pos, p.slots};
    const int64_t insz[] = {p.tokens * p.heads * d * es, p.dn * es, tb, tb, p.tokens * 4, p.tokens * 8};
    for (int i = 0; i < 6; ++i) {
        if (!in[i]) continue;
        if (ranges_overlap(p.nc, ncb, in[i], insz[i]) || ranges_overlap(p.rc, rcb, in[i], insz[i]))
            return RMSNORM_ERR_INVALID_ARG;
    }
    if (p.rc && ranges_overlap(p.nc, ncb, p.rc, rcb)) return RMSNORM_ERR_INVALID_ARG;
    return RMSNORM_OK;
}

bool kv_aligned(const KvProblem& p) {
    const void* ptrs[] = {p.kv, p.gamma, p.nc, p.rc, p.cos_t, p.sin_t};
    for (const void* q : ptrs)
        if (q && reinterpret_cast<uintptr_t>(q) % kVectorBytes != 0) return false;
    return true;
}

// Lanes with rotary work per row, or -1 when the shape cannot take 16-byte
// vectors: these must never straddle the split or a rope pair group, and
// table rows need 16-byte (8-byte for fp32 adjacent pairs) aligned per-lane
// entries.
int64_t kv_rope_lanes(int64_t dn, int64_t dr, int style, int dtype) {
    const int v = vec_elems(dtype);
    const int64_t unit = style == 1 ? v : 2 * v;
    if (dn % v != 0 || dr % unit != 0) return -1;
    return style == 1 ? dr / v : dr / (2 * v);
}

// Automatic KV launch configuration.  Path VECTOR: the smallest lane group
// of 8, 16 or 32 that holds the norm part with at most two vectors per lane
// and the rotated part, several rows per wave; else a whole wave per row
// with up to 8 norm vectors per lane and the rotated part in at most 64
// lanes.  Otherwise ELEMENT.  HIP-graph sweeps on MI355X: the bf16 prefill
// (16384 rows of 512 + 64) 9.2 us as 32 lanes x 2 against 11.0 with a wave
// per row; 16384 tokens x 8 heads of 128 + 64, 19.5 us as 8 lanes x 2
// against 21.1 as 16 x 1 and 53.9 with a wave per row.
rmsnorm_config_t choose_kv(int64_t dn, int64_t dr, int style, int dtype, bool aligned) {
    rmsnorm_config_t c = {RMSNORM_PATH_ELEMENT, 1, 0, 1, 0, 0, 0};
    const int64_t rope_lanes = kv_rope_lanes(dn, dr, style, dtype);
    if (!aligned || rope_lanes < 0 || rope_lanes > 64) return c;
    const int64_t nv = dn / vec_elems(dtype);
    for (int i = 0; i < mbr::kNumKvLpr; ++i) {
        const int lpr = mbr::kKvLprList[i];
        if (ceil_div(nv, int64_t(lpr)) <= 2 && rope_lanes <= lpr) {
            c.path = RMSNORM_PATH_VECTOR;
            c.items_per_lane = static_cast<int32_t>(ceil_div(nv, int64_t(lpr)));
            c.lanes_per_row = lpr;
            return c;
        }
    }
    for (int i = 0; i < mbr::kNumKvVpl; ++i) {
        if (int64_t(64) * mbr::kKvVplList[i] >= nv) {
            c.path = RMSNORM_PATH_VECTOR;
            c.items_per_lane = mbr::kKvVplList[i];
            return c;
        }
    }
    return c;
}

rmsnorm_status_t run_kv(const KvProblem& p, const rmsnorm_config_t* user, void* stream) {
    rmsnorm_status_t s = validate_kv(p);
    if (s != RMSNORM_OK) return s;
    if (p.tokens == 0) return RMSNORM_OK;
    s = validate_kv_pointers(p);
    if (s != RMSNORM_OK) return s;
    const bool aligned = kv_aligned(p);
    const rmsnorm_config_t c = (user && user->path != RMSNORM_PATH_AUTO)
                                   ? *user
                                   : choose_kv(p.dn, p.dr, p.style, p.dtype, aligned);
    if (c.waves_per_row != 1 || c.rows_per_block != 1 || c.max_blocks != 0 || c.weight_lds != 0)
        return RMSNORM_ERR_INVALID_ARG;
    const bool whole = c.lanes_per_row == 0 || c.lanes_per_row == 64;
    mbr::KvArgs a;
    a.kv = p.kv;
    a.gamma = p.gamma;
    a.cos_t = p.cos_t;
    a.sin_t = p.sin_t;
    a.pos = p.pos;
    a.slots = p.slots;
    a.nc = p.nc;
    a.rc = p.rc;
    a.rows = p.tokens * p.heads;
    a.max_pos = p.max_pos;
    a.num_slots = p.num_slots;
    a.heads = static_cast<int32_t>(p.heads);
    a.norm_dim = static_cast<int32_t>(p.dn);
    a.rope_dim = static_cast<int32_t>(p.dr);
    a.norm_dim_f = static_cast<float>(p.dn);
    a.eps = p.eps;
    const void* fn = nullptr;
    int64_t rows_per_wave = 1;
    if (c.path == RMSNORM_PATH_VECTOR) {
        const int64_t rope_lanes = kv_rope_lanes(p.dn, p.dr, p.style, p.dtype);
        const int64_t lanes = whole ? 64 : c.lanes_per_row;
        const int64_t nv = p.dn / vec_elems(p.dtype);
        if (!aligned || rope_lanes < 0 || rope_lanes > lanes || lanes * c.items_per_lane < nv)
            return RMSNORM_ERR_INVALID_ARG;
        const bool masked = lanes * c.items_per_lane != nv;
        if (whole) {
            const int vi = index_of(mbr::kKvVplList, mbr::kNumKvVpl, c.items_per_lane);
            if (vi < 0) return RMSNORM_ERR_INVALID_ARG;
            fn = mbr::kv_vec_kernel_ptr(p.dtype, p.style, masked, vi);
        } else {
            const int li = index_of(mbr::kKvLprList, mbr::kNumKvLpr, c.lanes_per_row);
            const int vi = index_of(mbr::kKvSwVplList, mbr::kNumKvSwVpl, c.items_per_lane);
            if (li < 0 || vi < 0) return RMSNORM_ERR_INVALID_ARG;
            fn = mbr::kv_subwave_kernel_ptr(p.dtype, p.style, masked, li, vi);
            rows_per_wave = 64 / c.lanes_per_row;
        }
    } else if (c.path == RMSNORM_PATH_ELEMENT) {
        if (!whole) return RMSNORM_ERR_INVALID_ARG;
        fn = mbr::kv_elem_kernel_ptr(p.dtype, p.style);
    }
    if (!fn) return RMSNORM_ERR_INVALID_ARG;
    // Four waves per workgroup.  Sweeps on MI355X (bf16 prefill, 16384 rows
    // of 512 + 64, one row per wave): two or eight waves per workgroup within
    // noise; two or four rows per wave one after another, all loaded before
    // any is reduced, slower (13.4 us against 12.1), since fewer waves are in
    // flight.
    constexpr int64_t kWavesPerBlock = 4;
    int64_t grid = ceil_div(a.rows, kWavesPerBlock * rows_per_wave);
    if (grid > kMaxGrid) grid = kMaxGrid;
    return launch_checked(fn, grid, 64 * kWavesPerBlock, &a, static_cast<hipStream_t>(stream));
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

RMSNORM_API rmsnorm_status_t rmsnorm_bwd_ex(const void* x, const void* weight, const void* dy, void* dx,
                                            void* dweight, int64_t rows, int64_t hidden, float eps,
                                            rmsnorm_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                            const rmsnorm_config_t* cfg, void* stream) {
    const BwdProblem p = {x, weight, dy, dx, dweight, rows, hidden, eps, static_cast<int>(dtype), workspace,
                          workspace_bytes};
    return run_bwd(p, cfg, stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_bwd(const void* x, const void* weight, const void* dy, void* dx, void* dweight,
                                         int64_t rows, int64_t hidden, float eps, rmsnorm_dtype_t dtype,
                                         void* workspace, size_t workspace_bytes, void* stream) {
    return rmsnorm_bwd_ex(x, weight, dy, dx, dweight, rows, hidden, eps, dtype, workspace, workspace_bytes, nullptr,
                          stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_bwd_noalloc(const void* x, const void* weight, const void* dy, void* dx,
                                                 void* dweight, int64_t rows, int64_t hidden, float eps,
                                                 rmsnorm_dtype_t dtype, void* stream) {
    const BwdProblem p = {x, weight, dy, dx, dweight, rows, hidden, eps, static_cast<int>(dtype), nullptr, 0};
    return run_bwd_noalloc(p, stream);
}

RMSNORM_API rmsnorm_status_t rmsnorm_bwd_workspace_size(int64_t rows, int64_t hidden, rmsnorm_dtype_t dtype,
                                                        const rmsnorm_config_t* cfg, size_t* bytes) {
    if (!bytes) return RMSNORM_ERR_INVALID_ARG;
    const rmsnorm_status_t s = validate_sizes(rows, hidden, 0.0f, static_cast<int>(dtype));
    if (s != RMSNORM_OK) return s;
    int64_t need;
    if (cfg && cfg->path != RMSNORM_PATH_AUTO) {
        if (cfg->max_blocks < 0) return RMSNORM_ERR_INVALID_ARG;
        need = bwd_workspace_need(rows, hidden, *cfg);
    } else {
        const int d = static_cast<int>(dtype);
        const int64_t a = bwd_workspace_need(rows, hidden, choose_bwd(rows, hidden, d, true));
        const int64_t b = bwd_workspace_need(rows, hidden, choose_bwd(rows, hidden, d, false));
        need = a > b ? a : b;
    }
    *bytes = static_cast<size_t>(need);
    return RMSNORM_OK;
}

RMSNORM_API rmsnorm_status_t rmsnorm_select_bwd_config(int64_t rows, int64_t hidden, rmsnorm_dtype_t dtype,
                                                       int32_t vector_aligned_flag, rmsnorm_config_t* cfg) {
    if (!cfg) return RMSNORM_ERR_INVALID_ARG;
    const rmsnorm_status_t s = validate_sizes(rows, hidden, 0.0f, static_cast<int>(dtype));
    if (s != RMSNORM_OK) return s;
    *cfg = choose_bwd(rows, hidden, static_cast<int>(dtype), vector_aligned_flag != 0);
    return RMSNORM_OK;
}

RMSNORM_API rmsnorm_status_t layernorm_fwd_ex(const void* x, const void* gamma, const void* beta, void* out,
                                              int64_t rows, int64_t hidden, float eps, rmsnorm_dtype_t dtype,
                                              const rmsnorm_config_t* cfg, void* stream) {
    const LnProblem p = {x, gamma, beta, out, rows, hidden, eps, static_cast<int>(dtype)};
    return run_ln(p, cfg, stream);
}

RMSNORM_API rmsnorm_status_t layernorm_fwd(const void* x, const void* gamma, const void* beta, void* out,
                                           int64_t rows, int64_t hidden, float eps, rmsnorm_dtype_t dtype,
                                           void* stream) {
    return layernorm_fwd_ex(x, gamma, beta, out, rows, hidden, eps, dtype, nullptr, stream);
}

RMSNORM_API rmsnorm_status_t layernorm_select_config(int64_t rows, int64_t hidden, rmsnorm_dtype_t dtype,
                                                     int32_t vector_aligned_flag, rmsnorm_config_t* cfg) {
    if (!cfg) return RMSNORM_ERR_INVALID_ARG;
    const rmsnorm_status_t s = validate_sizes(rows, hidden, 0.0f, static_cast<int>(dtype));
    if (s != RMSNORM_OK) return s;
    *cfg = choose_ln(rows, hidden, static_cast<int>(dtype), vector_aligned_flag != 0);
    return RMSNORM_OK;
}

RMSNORM_API rmsnorm_status_t kv_rmsnorm_rope_cache(const void* kv, const void* gamma, const float* cos_table,
                                                   const float* sin_table, const int32_t* positions,
                                                   const int64_t* slots, void* norm_cache, void* rope_cache,
                                                   int64_t tokens, int64_t heads, int64_t norm_dim,
                                                   int64_t rope_dim, int64_t max_pos, int64_t num_slots, float eps,
                                                   int32_t rope_style, rmsnorm_dtype_t dtype, void* stream) {
    return kv_rmsnorm_rope_cache_ex(kv, gamma, cos_table, sin_table, positions, slots, norm_cache, rope_cache, tokens,
                                    heads, norm_dim, rope_dim, max_pos, num_slots, eps, rope_style, dtype, nullptr,
                                    stream);
}

RMSNORM_API rmsnorm_status_t kv_rmsnorm_rope_cache_ex(const void* kv, const void* gamma, const float* cos_table,
                                                      const float* sin_table, const int32_t* positions,
                                                      const int64_t* slots, void* norm_cache, void* rope_cache,
                                                      int64_t tokens, int64_t heads, int64_t norm_dim,
                                                      int64_t rope_dim, int64_t max_pos, int64_t num_slots,
                                                      float eps, int32_t rope_style, rmsnorm_dtype_t dtype,
                                                      const rmsnorm_config_t* cfg, void* stream) {
    const KvProblem p = {kv,       gamma,     cos_table, sin_table, positions, slots,
                         norm_cache, rope_cache, tokens, heads,     norm_dim,  rope_dim,
                         max_pos,  num_slots, eps,       rope_style, static_cast<int>(dtype)};
    return run_kv(p, cfg, stream);
}

RMSNORM_API rmsnorm_status_t kv_select_config(int64_t tokens, int64_t heads, int64_t norm_dim, int64_t rope_dim,
                                              int32_t rope_style, rmsnorm_dtype_t dtype,
                                              int32_t vector_aligned_flag, rmsnorm_config_t* cfg) {
    if (!cfg) return RMSNORM_ERR_INVALID_ARG;
    const KvProblem p = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, tokens, heads,
                         norm_dim, rope_dim, 0, 0, 0.0f, rope_style, static_cast<int>(dtype)};
    const rmsnorm_status_t s = validate_kv(p);
    if (s != RMSNORM_OK) return s;
    *cfg = choose_kv(norm_dim, rope_dim, rope_style, static_cast<int>(dtype), vector_aligned_flag != 0);
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
