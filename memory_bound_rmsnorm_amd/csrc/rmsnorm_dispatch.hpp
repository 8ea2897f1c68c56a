// Kernel tables shared by the instantiation units and the C-ABI layer.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mbr {

// Built configurations: the ones the automatic choices (forward, quantised,
// backward, LayerNorm) can pick, plus one sweep set -- the plain forward
// vector kernels at every waves-per-row below 16 with up to 8 vectors per
// lane -- for launch-shape sweeps of the hot path through the _ex entry
// points.  A lane of a 1024-lane workgroup has 128 VGPRs, of a narrower one
// 256; nothing is built that would spill.
//
// Vector path: waves per row x 16-byte vectors per lane.  Below 16 waves the
// choice keeps at most 5 vectors per lane (plain rows up to 8 when four rows
// share an LDS copy of the weight); 16 waves take what registers allow.
constexpr int kWprList[] = {1, 2, 4, 8, 16};
constexpr int kVplList[] = {1, 2, 3, 4, 5, 6, 7, 8, 10};
constexpr int kEplList[] = {1, 2, 4, 8, 16};
constexpr int kNumWpr = sizeof(kWprList) / sizeof(int);
constexpr int kNumVpl = sizeof(kVplList) / sizeof(int);
constexpr int kNumEpl = sizeof(kEplList) / sizeof(int);

constexpr int max_threads_for(int wpr) { return wpr == 16 ? 1024 : 512; }

constexpr bool vec_built(int wpr, int vpl, bool fused) {
    return fused ? vpl <= (wpr < 16 ? 5 : 6) : vpl <= (wpr < 16 ? 8 : 10);
}
// Element path: only rows narrower than one 16-byte vector take it, as one
// wave with one element per lane.
constexpr bool elem_built(int wpr, int epl) { return wpr == 1 && epl == 1; }
// Quantised forms (int8 / fp8 codes plus a per-row scale) also hold the weight
// slice; the choice keeps at most 5 vectors per lane (4 at 16 waves).
constexpr bool qvec_built(int wpr, int vpl) { return vpl <= (wpr < 16 ? 5 : 4); }
constexpr bool qelem_built(int wpr, int epl) { return elem_built(wpr, epl); }

// Any-alignment vector path (rows of any width at any element alignment):
// full 16-byte vectors per lane, plus a tail of single elements.
constexpr int kAnyVplList[] = {1, 2, 3, 4, 5, 6, 7, 8};
constexpr int kNumAnyVpl = sizeof(kAnyVplList) / sizeof(int);
constexpr bool any_built(int wpr, int vpl, bool fused) { return vpl <= (wpr < 16 ? 5 : fused ? 4 : 6); }
// Its quantised forms hold the weight slice as well, as on the vector path.
constexpr bool qany_built(int wpr, int vpl) { return vpl <= (wpr < 16 ? 5 : 4); }

// Host-side kernel handles (addresses of the __global__ stubs), or nullptr.
// dtype: 0 = f32, 1 = bf16.
const void* vec_kernel(int dtype, bool fused, bool masked, int wpr_index, int vpl_index);
const void* elem_kernel(int dtype, bool fused, int wpr_index, int epl_index);
const void* twopass_kernel(int dtype, bool fused, bool vec);

const void* any_kernel(int dtype, bool fused, bool masked, int wpr_index, int vpl_index);

// Register + LDS path (rows wider than the register configurations): vectors
// per lane held in VGPRs, the rest of the row staged in dynamic LDS of at
// most kStageLdsMax bytes (160 KiB per gfx950 workgroup, less 1 KiB for the
// kernel's own row totals).
constexpr int kStageRvPlain = 10;
constexpr int kStageRvFused[] = {6, 7};
constexpr int kStageLanes = 1024;
constexpr long kStageLdsMax = 160 * 1024 - 1024;
const void* stage_kernel(int dtype, bool fused, int rv);

// Quantised forms; qt: 1 = int8, 2 = fp8 e4m3fn.
const void* qvec_kernel(int dtype, int qt, bool fused, bool masked, int wpr_index, int vpl_index);
const void* qany_kernel(int dtype, int qt, bool fused, bool masked, int wpr_index, int vpl_index);
const void* qelem_kernel(int dtype, int qt, bool fused, int wpr_index, int epl_index);
const void* qtwopass_kernel(int dtype, int qt, bool fused, bool vec);
const void* qvec_kernel_bf16(int qt, bool fused, bool masked, int wi, int vi);
const void* qvec_kernel_f32(int qt, bool fused, bool masked, int wi, int vi);

// Rows narrower than a wave: LPR lanes per row (a row per lane group), one or
// two 16-byte vectors per lane; every form (plain, fused, quantised).
constexpr int kLprList[] = {8, 16, 32};
constexpr int kSwVplList[] = {1, 2};
constexpr int kNumLpr = sizeof(kLprList) / sizeof(int);
constexpr int kNumSwVpl = sizeof(kSwVplList) / sizeof(int);
// qt: 0 = normalised output, 1 = int8, 2 = fp8 e4m3fn.
const void* subwave_kernel(int dtype, bool fused, int qt, bool masked, int lpr_index, int vpl_index);

// Backward (dx, and dweight through per-workgroup partial rows): the lane
// holds x, dy and the weight slice (plus fp32 column sums when dweight is
// wanted), so the vector path carries at most 8 vectors per lane (4 in a
// 1024-lane workgroup); the element path, as in the forward, only takes rows
// narrower than one vector.
constexpr int kBwdVplList[] = {1, 2, 3, 4, 5, 6, 7, 8};
constexpr int kBwdEplList[] = {1, 2, 4, 8};
constexpr int kNumBwdVpl = sizeof(kBwdVplList) / sizeof(int);
constexpr int kNumBwdEpl = sizeof(kBwdEplList) / sizeof(int);
// One wave holds a whole row of up to 8 vectors; the balanced rule keeps at
// most 6 per lane.
constexpr bool bwd_vec_built(int wpr, int vpl) { return vpl <= (wpr == 1 ? 8 : wpr < 16 ? 6 : 4); }
constexpr bool bwd_elem_built(int wpr, int epl) { return wpr == 1 && epl == 1; }

const void* bwd_vec_kernel(int dtype, bool dw, bool masked, int wpr_index, int vpl_index);
const void* bwd_elem_kernel(int dtype, bool dw, int wpr_index, int epl_index);
// Any width and element alignment, in vectors (kBwdVplList); it also holds
// its tail values, so 16 waves per row take at most 3 vectors per lane.
constexpr bool bwd_any_built(int wpr, int vpl) { return vpl <= (wpr < 16 ? 6 : 3); }
const void* bwd_any_kernel(int dtype, bool dw, bool masked, int wpr_index, int vpl_index);
// Backward vector kernel with rows narrower than a wave (kLprList lanes per
// row, kSwVplList vectors per lane, one wave per row slot group).
const void* bwd_subwave_kernel(int dtype, bool dw, bool masked, int lpr_index, int vpl_index);
const void* bwd_twopass_kernel(int dtype, bool dw, bool vec);
const void* bwd_dw_kernel(int dtype);

// LayerNorm: the row and the per-vector gamma / beta live in registers; up to
// 8 vectors per lane (4 in a 1024-lane workgroup, whose lanes have 128 VGPRs)
// are built spill-free; wider rows take the multi-pass path, rows narrower
// than one vector the one-element-per-lane kernel.
constexpr int kLnVplList[] = {1, 2, 3, 4, 5, 6, 7, 8};
constexpr bool ln_vec_built(int wpr, int vpl) { return wpr < 16 || vpl <= 4; }
constexpr int kLnEplList[] = {1, 2, 4, 8};
constexpr bool ln_elem_built(int wpr, int epl) { return wpr == 1 && epl == 1; }
constexpr int kNumLnVpl = sizeof(kLnVplList) / sizeof(int);
constexpr int kNumLnEpl = sizeof(kLnEplList) / sizeof(int);

const void* ln_vec_kernel_ptr(int dtype, bool masked, bool gamma_beta_lds, int wpr_index, int vpl_index);
// LayerNorm vector kernel with rows narrower than a wave (kLprList lanes per
// row, kSwVplList vectors per lane, per-lane gamma / beta).
const void* ln_subwave_kernel_ptr(int dtype, bool masked, int lpr_index, int vpl_index);
// LayerNorm at any width and element alignment, in vectors (kAnyVplList);
// x, gamma and beta are live together, so a 1024-lane workgroup takes 3.
constexpr bool ln_any_built(int wpr, int vpl) { return wpr < 16 || vpl <= 3; }
const void* ln_any_kernel_ptr(int dtype, bool masked, int wpr_index, int vpl_index);
const void* ln_elem_kernel_ptr(int dtype, int wpr_index, int epl_index);
const void* ln_multipass_kernel_ptr(int dtype, bool vec);

// KV RMSNorm + RoPE + cache: one wave per row; the norm part in 1, 2, 4 or 8
// 16-byte vectors per lane (index 0..3), rope style 0 (halves) or 1 (pairs).
constexpr int kKvVplList[] = {1, 2, 4, 8};
constexpr int kNumKvVpl = sizeof(kKvVplList) / sizeof(int);
// Rows narrower than a wave: lanes per row, and norm vectors per lane.
constexpr int kKvLprList[] = {8, 16, 32};
constexpr int kNumKvLpr = sizeof(kKvLprList) / sizeof(int);
constexpr int kKvSwVplList[] = {1, 2};
constexpr int kNumKvSwVpl = sizeof(kKvSwVplList) / sizeof(int);
const void* kv_vec_kernel_ptr(int dtype, int style, bool masked, int vpl_index);
const void* kv_subwave_kernel_ptr(int dtype, int style, bool masked, int lpr_index, int vpl_index);
const void* kv_elem_kernel_ptr(int dtype, int style);

// Per-unit getters defined in the instantiation files.
const void* vec_kernel_bf16(bool fused, bool masked, int wi, int vi);
const void* vec_kernel_f32(bool fused, bool masked, int wi, int vi);

}  // namespace mbr
