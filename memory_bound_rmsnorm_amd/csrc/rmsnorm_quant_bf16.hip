// Instantiations of the vector-path kernel in its quantised forms for bf16
// input: int8 and fp8 e4m3fn codes, plain and fused, exact and masked, every
// built (waves per row, vectors per lane) pair.
#include <utility>

#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace mbr {
namespace {

template <int WPR, int VPL, bool MASKED, bool FUSED, int QT>
const void* qvec_ptr() {
    if constexpr (qvec_built(WPR, VPL))
        return reinterpret_cast<const void*>(&rms_vec_kernel<Bf16, WPR, VPL, MASKED, FUSED, QT>);
    else
        return nullptr;
}

template <int QT, bool FUSED, bool MASKED, size_t... I>
const void* const* qvec_table(std::index_sequence<I...>) {
    static const void* const table[] = {qvec_ptr<kWprList[I / kNumVpl], kVplList[I % kNumVpl], MASKED, FUSED, QT>()...};
    return table;
}

template <int QT>
const void* const* pick(bool fused, bool masked) {
    using Seq = std::make_index_sequence<kNumWpr * kNumVpl>;
    return fused ? (masked ? qvec_table<QT, true, true>(Seq{}) : qvec_table<QT, true, false>(Seq{}))
                 : (masked ? qvec_table<QT, false, true>(Seq{}) : qvec_table<QT, false, false>(Seq{}));
}

}  // namespace

const void* qvec_kernel_bf16(int qt, bool fused, bool masked, int wi, int vi) {
    if (wi < 0 || wi >= kNumWpr || vi < 0 || vi >= kNumVpl) return nullptr;
    if (qt == 1) return pick<1>(fused, masked)[wi * kNumVpl + vi];
    if (qt == 2) return pick<2>(fused, masked)[wi * kNumVpl + vi];
    return nullptr;
}

}  // namespace mbr
