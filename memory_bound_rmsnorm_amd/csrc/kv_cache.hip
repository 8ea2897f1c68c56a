// Instantiations of the KV RMSNorm + RoPE + cache kernels and their lookup.
#include "kv_kernels.hpp"
#include "rmsnorm_dispatch.hpp"

namespace mbr {
namespace {

template <class E, int NVPL, int STYLE>
const void* kv_vec_ptr(bool masked) {
    return masked ? reinterpret_cast<const void*>(&kv_vec_kernel<E, NVPL, true, STYLE>)
                  : reinterpret_cast<const void*>(&kv_vec_kernel<E, NVPL, false, STYLE>);
}

template <class E, int STYLE>
const void* kv_vec_for(int vi, bool masked) {
    switch (vi) {
        case 0: return kv_vec_ptr<E, 1, STYLE>(masked);
        case 1: return kv_vec_ptr<E, 2, STYLE>(masked);
        case 2: return kv_vec_ptr<E, 4, STYLE>(masked);
        case 3: return kv_vec_ptr<E, 8, STYLE>(masked);
        default: return nullptr;
    }
}

template <class E, int STYLE, int LPR>
const void* kv_sub_for(int vi, bool masked) {
    switch (vi) {
        case 0: return masked ? reinterpret_cast<const void*>(&kv_vec_kernel<E, 1, true, STYLE, LPR>)
                              : reinterpret_cast<const void*>(&kv_vec_kernel<E, 1, false, STYLE, LPR>);
        case 1: return masked ? reinterpret_cast<const void*>(&kv_vec_kernel<E, 2, true, STYLE, LPR>)
                              : reinterpret_cast<const void*>(&kv_vec_kernel<E, 2, false, STYLE, LPR>);
        default: return nullptr;
    }
}

template <class E, int STYLE>
const void* kv_sub_lpr(int li, int vi, bool masked) {
    switch (li) {
        case 0: return kv_sub_for<E, STYLE, 8>(vi, masked);
        case 1: return kv_sub_for<E, STYLE, 16>(vi, masked);
        case 2: return kv_sub_for<E, STYLE, 32>(vi, masked);
        default: return nullptr;
    }
}

}  // namespace

const void* kv_subwave_kernel_ptr(int dtype, int style, bool masked, int li, int vi) {
    if (dtype == 1) return style ? kv_sub_lpr<Bf16, 1>(li, vi, masked) : kv_sub_lpr<Bf16, 0>(li, vi, masked);
    return style ? kv_sub_lpr<F32, 1>(li, vi, masked) : kv_sub_lpr<F32, 0>(li, vi, masked);
}

const void* kv_vec_kernel_ptr(int dtype, int style, bool masked, int vi) {
    if (dtype == 1) return style ? kv_vec_for<Bf16, 1>(vi, masked) : kv_vec_for<Bf16, 0>(vi, masked);
    return style ? kv_vec_for<F32, 1>(vi, masked) : kv_vec_for<F32, 0>(vi, masked);
}

const void* kv_elem_kernel_ptr(int dtype, int style) {
    if (dtype == 1)
        return style ? reinterpret_cast<const void*>(&kv_elem_kernel<Bf16, 1>)
                     : reinterpret_cast<const void*>(&kv_elem_kernel<Bf16, 0>);
    return style ? reinterpret_cast<const void*>(&kv_elem_kernel<F32, 1>)
                 : reinterpret_cast<const void*>(&kv_elem_kernel<F32, 0>);
}

}  // namespace mbr
