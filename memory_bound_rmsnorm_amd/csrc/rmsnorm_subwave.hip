// Instantiations of the vector kernel with rows narrower than a wave
// (8, 16 or 32 lanes per row, one or two 16-byte vectors per lane), for every
// form: plain, fused residual, and the int8 / fp8 quantised outputs.
#include <utility>

#include "rmsnorm_dispatch.hpp"
#include "rmsnorm_kernels.hpp"

namespace mbr {
namespace {

template <class E, bool FUSED, int QT, bool MASKED, size_t... I>
const void* const* sw_table(std::index_sequence<I...>) {
    static const void* const table[] = {reinterpret_cast<const void*>(
        &rms_vec_kernel<E, 1, kSwVplList[I % kNumSwVpl], MASKED, FUSED, QT, kLprList[I / kNumSwVpl]>)...};
    return table;
}

template <class E, bool FUSED, int QT>
const void* const* sw_tables(bool masked) {
    using Seq = std::make_index_sequence<kNumLpr * kNumSwVpl>;
    return masked ? sw_table<E, FUSED, QT, true>(Seq{}) : sw_table<E, FUSED, QT, false>(Seq{});
}

template <class E>
const void* const* sw_for(bool fused, int qt, bool masked) {
    if (fused) {
        if (qt == 1) return sw_tables<E, true, 1>(masked);
        if (qt == 2) return sw_tables<E, true, 2>(masked);
        return sw_tables<E, true, 0>(masked);
    }
    if (qt == 1) return sw_tables<E, false, 1>(masked);
    if (qt == 2) return sw_tables<E, false, 2>(masked);
    return sw_tables<E, false, 0>(masked);
}

}  // namespace

const void* subwave_kernel(int dtype, bool fused, int qt, bool masked, int li, int vi) {
    if (li < 0 || li >= kNumLpr || vi < 0 || vi >= kNumSwVpl || qt < 0 || qt > 2) return nullptr;
    const void* const* t = dtype == 1 ? sw_for<Bf16>(fused, qt, masked) : sw_for<F32>(fused, qt, masked);
    return t[li * kNumSwVpl + vi];
}

}  // namespace mbr
