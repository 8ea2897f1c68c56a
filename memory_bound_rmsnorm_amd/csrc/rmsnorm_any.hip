// Instantiations of the any-alignment vector kernel (rows of any width at any
// element alignment, plain and fused), bf16 and fp32.
#include <utility>

#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace mbr {
namespace {

template <class E, int WPR, int VPL, bool MASKED, bool FUSED>
const void* any_ptr() {
    if constexpr (any_built(WPR, VPL, FUSED))
        return reinterpret_cast<const void*>(&rms_any_kernel<E, WPR, VPL, MASKED, FUSED>);
    else
        return nullptr;
}

template <class E, bool FUSED, bool MASKED, size_t... I>
const void* const* any_table(std::index_sequence<I...>) {
    static const void* const table[] = {
        any_ptr<E, kWprList[I / kNumAnyVpl], kAnyVplList[I % kNumAnyVpl], MASKED, FUSED>()...};
    return table;
}

template <class E, size_t... I>
const void* const* any_tables(bool fused, bool masked, std::index_sequence<I...> s) {
    return fused ? (masked ? any_table<E, true, true>(s) : any_table<E, true, false>(s))
                 : (masked ? any_table<E, false, true>(s) : any_table<E, false, false>(s));
}

}  // namespace

const void* any_kernel(int dtype, bool fused, bool masked, int wi, int vi) {
    using Seq = std::make_index_sequence<kNumWpr * kNumAnyVpl>;
    if (wi < 0 || wi >= kNumWpr || vi < 0 || vi >= kNumAnyVpl) return nullptr;
    const void* const* t = dtype == 1 ? any_tables<Bf16>(fused, masked, Seq{}) : any_tables<F32>(fused, masked, Seq{});
    return t[wi * kNumAnyVpl + vi];
}

}  // namespace mbr
