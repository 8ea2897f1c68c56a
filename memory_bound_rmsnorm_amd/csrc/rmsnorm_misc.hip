// Instantiations of the element-path and two-pass kernels, and the lookup
// functions the C-ABI layer uses.
#include <utility>

#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace mbr {
namespace {

template <class E, int WPR, int EPL, bool FUSED>
const void* elem_ptr() {
    if constexpr (elem_built(WPR, EPL))
        return reinterpret_cast<const void*>(&rms_elem_kernel<E, WPR, EPL, FUSED>);
    else
        return nullptr;
}

template <class E, bool FUSED, size_t... I>
const void* const* elem_table(std::index_sequence<I...>) {
    static const void* const table[] = {elem_ptr<E, kWprList[I / kNumEpl], kEplList[I % kNumEpl], FUSED>()...};
    return table;
}

}  // namespace

const void* vec_kernel(int dtype, bool fused, bool masked, int wi, int vi) {
    return dtype == 1 ? vec_kernel_bf16(fused, masked, wi, vi) : vec_kernel_f32(fused, masked, wi, vi);
}

const void* elem_kernel(int dtype, bool fused, int wi, int ei) {
    using Seq = std::make_index_sequence<kNumWpr * kNumEpl>;
    if (wi < 0 || wi >= kNumWpr || ei < 0 || ei >= kNumEpl) return nullptr;
    const void* const* t;
    if (dtype == 1)
        t = fused ? elem_table<Bf16, true>(Seq{}) : elem_table<Bf16, false>(Seq{});
    else
        t = fused ? elem_table<F32, true>(Seq{}) : elem_table<F32, false>(Seq{});
    return t[wi * kNumEpl + ei];
}

const void* stage_kernel(int dtype, bool fused, int rv) {
    // chunk of staged vectors per lane through registers: the largest that
    // stays spill-free at 128 VGPRs (1024-lane workgroups)
    if (!fused) {
        if (rv != kStageRvPlain) return nullptr;
        return dtype == 1 ? reinterpret_cast<const void*>(&rms_stage_kernel<Bf16, 10, 10, false>)
                          : reinterpret_cast<const void*>(&rms_stage_kernel<F32, 10, 10, false>);
    }
    if (rv == 6)
        return dtype == 1 ? reinterpret_cast<const void*>(&rms_stage_kernel<Bf16, 6, 5, true>)
                          : reinterpret_cast<const void*>(&rms_stage_kernel<F32, 6, 5, true>);
    if (rv == 7)
        return dtype == 1 ? reinterpret_cast<const void*>(&rms_stage_kernel<Bf16, 7, 4, true>)
                          : reinterpret_cast<const void*>(&rms_stage_kernel<F32, 7, 4, true>);
    return nullptr;
}

const void* twopass_kernel(int dtype, bool fused, bool vec) {
    if (dtype == 1) {
        if (vec) return fused ? reinterpret_cast<const void*>(&rms_twopass_kernel<Bf16, true, true>)
                              : reinterpret_cast<const void*>(&rms_twopass_kernel<Bf16, true, false>);
        return fused ? reinterpret_cast<const void*>(&rms_twopass_kernel<Bf16, false, true>)
                     : reinterpret_cast<const void*>(&rms_twopass_kernel<Bf16, false, false>);
    }
    if (vec) return fused ? reinterpret_cast<const void*>(&rms_twopass_kernel<F32, true, true>)
                          : reinterpret_cast<const void*>(&rms_twopass_kernel<F32, true, false>);
    return fused ? reinterpret_cast<const void*>(&rms_twopass_kernel<F32, false, true>)
                 : reinterpret_cast<const void*>(&rms_twopass_kernel<F32, false, false>);
}

}  // namespace mbr
