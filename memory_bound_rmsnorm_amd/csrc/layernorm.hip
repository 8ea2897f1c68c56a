// Instantiations of the LayerNorm kernels and their lookup functions.
#include <utility>

#include "layernorm_kernels.hpp"
#include "rmsnorm_dispatch.hpp"

namespace mbr {
namespace {

template <class E, int WPR, int VPL, bool MASKED, bool GBL>
const void* lvec_ptr() {
    if constexpr (ln_vec_built(WPR, VPL))
        return reinterpret_cast<const void*>(&ln_vec_kernel<E, WPR, VPL, MASKED, GBL>);
    else
        return nullptr;
}

template <class E, bool MASKED, bool GBL, size_t... I>
const void* const* lvec_table(std::index_sequence<I...>) {
    static const void* const table[] = {
        lvec_ptr<E, kWprList[I / kNumLnVpl], kLnVplList[I % kNumLnVpl], MASKED, GBL>()...};
    return table;
}

template <class E, size_t... I>
const void* const* lvec_table_for(bool masked, bool gbl, std::index_sequence<I...> seq) {
    if (gbl) return masked ? lvec_table<E, true, true>(seq) : lvec_table<E, false, true>(seq);
    return masked ? lvec_table<E, true, false>(seq) : lvec_table<E, false, false>(seq);
}

template <class E, bool MASKED, size_t... I>
const void* const* lsub_table(std::index_sequence<I...>) {
    static const void* const table[] = {reinterpret_cast<const void*>(
        &ln_vec_kernel<E, 1, kSwVplList[I % kNumSwVpl], MASKED, false, kLprList[I / kNumSwVpl]>)...};
    return table;
}

template <class E, int WPR, int VPL, bool MASKED>
const void* lany_ptr() {
    if constexpr (ln_any_built(WPR, VPL))
        return reinterpret_cast<const void*>(&ln_any_kernel<E, WPR, VPL, MASKED>);
    else
        return nullptr;
}

template <class E, bool MASKED, size_t... I>
const void* const* lany_table(std::index_sequence<I...>) {
    static const void* const table[] = {lany_ptr<E, kWprList[I / kNumAnyVpl], kAnyVplList[I % kNumAnyVpl], MASKED>()...};
    return table;
}

template <class E, int WPR, int EPL>
const void* lelem_ptr() {
    if constexpr (ln_elem_built(WPR, EPL))
        return reinterpret_cast<const void*>(&ln_elem_kernel<E, WPR, EPL>);
    else
        return nullptr;
}

template <class E, size_t... I>
const void* const* lelem_table(std::index_sequence<I...>) {
    static const void* const table[] = {lelem_ptr<E, kWprList[I / kNumLnEpl], kLnEplList[I % kNumLnEpl]>()...};
    return table;
}

}  // namespace

const void* ln_vec_kernel_ptr(int dtype, bool masked, bool gamma_beta_lds, int wi, int vi) {
    using Seq = std::make_index_sequence<kNumWpr * kNumLnVpl>;
    if (wi < 0 || wi >= kNumWpr || vi < 0 || vi >= kNumLnVpl) return nullptr;
    const void* const* t = dtype == 1 ? lvec_table_for<Bf16>(masked, gamma_beta_lds, Seq{})
                                      : lvec_table_for<F32>(masked, gamma_beta_lds, Seq{});
    return t[wi * kNumLnVpl + vi];
}

const void* ln_subwave_kernel_ptr(int dtype, bool masked, int li, int vi) {
    using Seq = std::make_index_sequence<kNumLpr * kNumSwVpl>;
    if (li < 0 || li >= kNumLpr || vi < 0 || vi >= kNumSwVpl) return nullptr;
    const void* const* t = dtype == 1 ? (masked ? lsub_table<Bf16, true>(Seq{}) : lsub_table<Bf16, false>(Seq{}))
                                      : (masked ? lsub_table<F32, true>(Seq{}) : lsub_table<F32, false>(Seq{}));
    return t[li * kNumSwVpl + vi];
}

const void* ln_any_kernel_ptr(int dtype, bool masked, int wi, int vi) {
    using Seq = std::make_index_sequence<kNumWpr * kNumAnyVpl>;
    if (wi < 0 || wi >= kNumWpr || vi < 0 || vi >= kNumAnyVpl) return nullptr;
    const void* const* t = dtype == 1 ? (masked ? lany_table<Bf16, true>(Seq{}) : lany_table<Bf16, false>(Seq{}))
                                      : (masked ? lany_table<F32, true>(Seq{}) : lany_table<F32, false>(Seq{}));
    return t[wi * kNumAnyVpl + vi];
}

const void* ln_elem_kernel_ptr(int dtype, int wi, int ei) {
    using Seq = std::make_index_sequence<kNumWpr * kNumLnEpl>;
    if (wi < 0 || wi >= kNumWpr || ei < 0 || ei >= kNumLnEpl) return nullptr;
    const void* const* t = dtype == 1 ? lelem_table<Bf16>(Seq{}) : lelem_table<F32>(Seq{});
    return t[wi * kNumLnEpl + ei];
}

const void* ln_multipass_kernel_ptr(int dtype, bool vec) {
    if (dtype == 1)
        return vec ? reinterpret_cast<const void*>(&ln_multipass_kernel<Bf16, true>)
                   : reinterpret_cast<const void*>(&ln_multipass_kernel<Bf16, false>);
    return vec ? reinterpret_cast<const void*>(&ln_multipass_kernel<F32, true>)
               : reinterpret_cast<const void*>(&ln_multipass_kernel<F32, false>);
}

}  // namespace mbr
