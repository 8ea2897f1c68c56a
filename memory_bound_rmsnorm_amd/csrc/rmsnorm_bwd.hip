// Instantiations of the backward kernels (vector, element, two-pass, and the
// dweight column reduction) and their lookup functions.
#include <utility>

#include "rmsnorm_bwd_kernels.hpp"
#include "rmsnorm_dispatch.hpp"

namespace mbr {
namespace {

template <class E, int WPR, int VPL, bool MASKED, bool DW>
const void* bvec_ptr() {
    if constexpr (bwd_vec_built(WPR, VPL))
        return reinterpret_cast<const void*>(&rms_bwd_vec_kernel<E, WPR, VPL, MASKED, DW>);
    else
        return nullptr;
}

template <class E, bool MASKED, bool DW, size_t... I>
const void* const* bvec_table(std::index_sequence<I...>) {
    static const void* const table[] = {
        bvec_ptr<E, kWprList[I / kNumBwdVpl], kBwdVplList[I % kNumBwdVpl], MASKED, DW>()...};
    return table;
}

template <class E, size_t... I>
const void* const* bvec_tables(bool masked, bool dw, std::index_sequence<I...> s) {
    return masked ? (dw ? bvec_table<E, true, true>(s) : bvec_table<E, true, false>(s))
                  : (dw ? bvec_table<E, false, true>(s) : bvec_table<E, false, false>(s));
}

template <class E, bool MASKED, bool DW, size_t... I>
const void* const* bsub_table(std::index_sequence<I...>) {
    static const void* const table[] = {reinterpret_cast<const void*>(
        &rms_bwd_vec_kernel<E, 1, kSwVplList[I % kNumSwVpl], MASKED, DW, kLprList[I / kNumSwVpl]>)...};
    return table;
}

template <class E, size_t... I>
const void* const* bsub_tables(bool masked, bool dw, std::index_sequence<I...> s) {
    return masked ? (dw ? bsub_table<E, true, true>(s) : bsub_table<E, true, false>(s))
                  : (dw ? bsub_table<E, false, true>(s) : bsub_table<E, false, false>(s));
}

template <class E, int WPR, int EPL, bool DW>
const void* belem_ptr() {
    if constexpr (bwd_elem_built(WPR, EPL))
        return reinterpret_cast<const void*>(&rms_bwd_elem_kernel<E, WPR, EPL, DW>);
    else
        return nullptr;
}

template <class E, bool DW, size_t... I>
const void* const* belem_table(std::index_sequence<I...>) {
    static const void* const table[] = {belem_ptr<E, kWprList[I / kNumBwdEpl], kBwdEplList[I % kNumBwdEpl], DW>()...};
    return table;
}

template <class E>
const void* btwopass(bool vec, bool dw) {
    if (vec) return dw ? reinterpret_cast<const void*>(&rms_bwd_twopass_kernel<E, true, true>)
                       : reinterpret_cast<const void*>(&rms_bwd_twopass_kernel<E, true, false>);
    return dw ? reinterpret_cast<const void*>(&rms_bwd_twopass_kernel<E, false, true>)
              : reinterpret_cast<const void*>(&rms_bwd_twopass_kernel<E, false, false>);
}

}  // namespace

const void* bwd_vec_kernel(int dtype, bool dw, bool masked, int wi, int vi) {
    using Seq = std::make_index_sequence<kNumWpr * kNumBwdVpl>;
    if (wi < 0 || wi >= kNumWpr || vi < 0 || vi >= kNumBwdVpl) return nullptr;
    const void* const* t = dtype == 1 ? bvec_tables<Bf16>(masked, dw, Seq{}) : bvec_tables<F32>(masked, dw, Seq{});
    return t[wi * kNumBwdVpl + vi];
}

const void* bwd_subwave_kernel(int dtype, bool dw, bool masked, int li, int vi) {
    using Seq = std::make_index_sequence<kNumLpr * kNumSwVpl>;
    if (li < 0 || li >= kNumLpr || vi < 0 || vi >= kNumSwVpl) return nullptr;
    const void* const* t = dtype == 1 ? bsub_tables<Bf16>(masked, dw, Seq{}) : bsub_tables<F32>(masked, dw, Seq{});
    return t[li * kNumSwVpl + vi];
}

const void* bwd_elem_kernel(int dtype, bool dw, int wi, int ei) {
    using Seq = std::make_index_sequence<kNumWpr * kNumBwdEpl>;
    if (wi < 0 || wi >= kNumWpr || ei < 0 || ei >= kNumBwdEpl) return nullptr;
    const void* const* t;
    if (dtype == 1)
        t = dw ? belem_table<Bf16, true>(Seq{}) : belem_table<Bf16, false>(Seq{});
    else
        t = dw ? belem_table<F32, true>(Seq{}) : belem_table<F32, false>(Seq{});
    return t[wi * kNumBwdEpl + ei];
}

const void* bwd_twopass_kernel(int dtype, bool dw, bool vec) {
    return dtype == 1 ? btwopass<Bf16>(vec, dw) : btwopass<F32>(vec, dw);
}

const void* bwd_dw_kernel(int dtype) {
    return dtype == 1 ? reinterpret_cast<const void*>(&rms_bwd_dw_kernel<Bf16>)
                      : reinterpret_cast<const void*>(&rms_bwd_dw_kernel<F32>);
}

}  // namespace mbr
