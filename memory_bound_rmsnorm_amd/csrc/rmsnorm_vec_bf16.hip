// Instantiations of the vector-path kernel for bf16: every built
// (waves per row, vectors per lane) pair, plain and fused, exact and masked.
#include <utility>

#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace mbr {
namespace {

template <int WPR, int VPL, bool MASKED, bool FUSED>
const void* vec_ptr() {
    if constexpr (vec_built(WPR, VPL, FUSED))
        return reinterpret_cast<const void*>(&rms_vec_kernel<Bf16, WPR, VPL, MASKED, FUSED>);
    else
        return nullptr;
}

template <bool FUSED, bool MASKED, size_t... I>
const void* const* vec_table(std::index_sequence<I...>) {
    static const void* const table[] = {vec_ptr<kWprList[I / kNumVpl], kVplList[I % kNumVpl], MASKED, FUSED>()...};
    return table;
}

}  // namespace

const void* vec_kernel_bf16(bool fused, bool masked, int wi, int vi) {
    using Seq = std::make_index_sequence<kNumWpr * kNumVpl>;
    if (wi < 0 || wi >= kNumWpr || vi < 0 || vi >= kNumVpl) return nullptr;
    const void* const* t = fused ? (masked ? vec_table<true, true>(Seq{}) : vec_table<true, false>(Seq{}))
                                 : (masked ? vec_table<false, true>(Seq{}) : vec_table<false, false>(Seq{}));
    return t[wi * kNumVpl + vi];
}

}  // namespace mbr
