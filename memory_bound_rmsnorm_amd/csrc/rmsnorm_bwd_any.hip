// Instantiations of the any-alignment backward kernel (rows of any width at
// any element alignment; dx with or without the dweight partial rows), bf16
// and fp32.
#include <utility>

#include "rmsnorm_bwd_kernels.hpp"
#include "rmsnorm_dispatch.hpp"

namespace mbr {
namespace {

template <class E, int WPR, int VPL, bool MASKED, bool DW>
const void* bany_ptr() {
    if constexpr (bwd_any_built(WPR, VPL))
        return reinterpret_cast<const void*>(&rms_bwd_any_kernel<E, WPR, VPL, MASKED, DW>);
    else
        return nullptr;
}

template <class E, bool DW, bool MASKED, size_t... I>
const void* const* bany_table(std::index_sequence<I...>) {
    static const void* const table[] = {
        bany_ptr<E, kWprList[I / kNumBwdVpl], kBwdVplList[I % kNumBwdVpl], MASKED, DW>()...};
    return table;
}

template <class E, size_t... I>
const void* const* bany_tables(bool dw, bool masked, std::index_sequence<I...> s) {
    return dw ? (masked ? bany_table<E, true, true>(s) : bany_table<E, true, false>(s))
              : (masked ? bany_table<E, false, true>(s) : bany_table<E, false, false>(s));
}

}  // namespace

const void* bwd_any_kernel(int dtype, bool dw, bool masked, int wi, int vi) {
    using Seq = std::make_index_sequence<kNumWpr * kNumBwdVpl>;
    if (wi < 0 || wi >= kNumWpr || vi < 0 || vi >= kNumBwdVpl) return nullptr;
    const void* const* t = dtype == 1 ? bany_tables<Bf16>(dw, masked, Seq{}) : bany_tables<F32>(dw, masked, Seq{});
    return t[wi * kNumBwdVpl + vi];
}

}  // namespace mbr
