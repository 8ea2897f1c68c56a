// Instantiations of the any-alignment vector kernel for the quantised forms
// (int8 and fp8 e4m3fn codes plus one fp32 scale per row; plain and fused),
// bf16 and fp32 inputs.
#include <utility>

#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace mbr {
namespace {

template <class E, int QT, int WPR, int VPL, bool MASKED, bool FUSED>
const void* qany_ptr() {
    if constexpr (qany_built(WPR, VPL))
        return reinterpret_cast<const void*>(&rms_any_kernel<E, WPR, VPL, MASKED, FUSED, QT>);
    else
        return nullptr;
}

template <class E, int QT, bool FUSED, bool MASKED, size_t... I>
const void* const* qany_table(std::index_sequence<I...>) {
    static const void* const table[] = {
        qany_ptr<E, QT, kWprList[I / kNumAnyVpl], kAnyVplList[I % kNumAnyVpl], MASKED, FUSED>()...};
    return table;
}

template <class E, int QT, size_t... I>
const void* const* qany_tables(bool fused, bool masked, std::index_sequence<I...> s) {
    return fused ? (masked ? qany_table<E, QT, true, true>(s) : qany_table<E, QT, true, false>(s))
                 : (masked ? qany_table<E, QT, false, true>(s) : qany_table<E, QT, false, false>(s));
}

template <class E, size_t... I>
const void* const* qany_tables_qt(int qt, bool fused, bool masked, std::index_sequence<I...> s) {
    return qt == 1 ? qany_tables<E, 1>(fused, masked, s) : qany_tables<E, 2>(fused, masked, s);
}

}  // namespace

const void* qany_kernel(int dtype, int qt, bool fused, bool masked, int wi, int vi) {
    using Seq = std::make_index_sequence<kNumWpr * kNumAnyVpl>;
    if ((qt != 1 && qt != 2) || wi < 0 || wi >= kNumWpr || vi < 0 || vi >= kNumAnyVpl) return nullptr;
    const void* const* t = dtype == 1 ? qany_tables_qt<Bf16>(qt, fused, masked, Seq{})
                                      : qany_tables_qt<F32>(qt, fused, masked, Seq{});
    return t[wi * kNumAnyVpl + vi];
}

}  // namespace mbr
