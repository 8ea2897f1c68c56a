// Instantiations of the element-path and two-pass kernels in their quantised
// forms, and the quantised-kernel lookup functions.
#include <utility>

#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace mbr {
namespace {

template <class E, int WPR, int EPL, bool FUSED, int QT>
const void* qelem_ptr() {
    if constexpr (qelem_built(WPR, EPL))
        return reinterpret_cast<const void*>(&rms_elem_kernel<E, WPR, EPL, FUSED, QT>);
    else
        return nullptr;
}

template <class E, bool FUSED, int QT, size_t... I>
const void* const* qelem_table(std::index_sequence<I...>) {
    static const void* const table[] = {qelem_ptr<E, kWprList[I / kNumEpl], kEplList[I % kNumEpl], FUSED, QT>()...};
    return table;
}

template <class E, int QT>
const void* qelem_lookup(bool fused, int i) {
    using Seq = std::make_index_sequence<kNumWpr * kNumEpl>;
    return (fused ? qelem_table<E, true, QT>(Seq{}) : qelem_table<E, false, QT>(Seq{}))[i];
}

template <class E, int QT>
const void* qtwopass_lookup(bool fused, bool vec) {
    if (vec) return fused ? reinterpret_cast<const void*>(&rms_twopass_kernel<E, true, true, QT>)
                          : reinterpret_cast<const void*>(&rms_twopass_kernel<E, true, false, QT>);
    return fused ? reinterpret_cast<const void*>(&rms_twopass_kernel<E, false, true, QT>)
                 : reinterpret_cast<const void*>(&rms_twopass_kernel<E, false, false, QT>);
}

}  // namespace

const void* qvec_kernel(int dtype, int qt, bool fused, bool masked, int wi, int vi) {
    return dtype == 1 ? qvec_kernel_bf16(qt, fused, masked, wi, vi) : qvec_kernel_f32(qt, fused, masked, wi, vi);
}

const void* qelem_kernel(int dtype, int qt, bool fused, int wi, int ei) {
    if (wi < 0 || wi >= kNumWpr || ei < 0 || ei >= kNumEpl || (qt != 1 && qt != 2)) return nullptr;
    const int i = wi * kNumEpl + ei;
    if (dtype == 1) return qt == 1 ? qelem_lookup<Bf16, 1>(fused, i) : qelem_lookup<Bf16, 2>(fused, i);
    return qt == 1 ? qelem_lookup<F32, 1>(fused, i) : qelem_lookup<F32, 2>(fused, i);
}

const void* qtwopass_kernel(int dtype, int qt, bool fused, bool vec) {
    if (qt != 1 && qt != 2) return nullptr;
    if (dtype == 1) return qt == 1 ? qtwopass_lookup<Bf16, 1>(fused, vec) : qtwopass_lookup<Bf16, 2>(fused, vec);
    return qt == 1 ? qtwopass_lookup<F32, 1>(fused, vec) : qtwopass_lookup<F32, 2>(fused, vec);
}

}  // namespace mbr
