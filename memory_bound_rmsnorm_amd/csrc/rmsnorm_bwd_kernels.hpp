// RMSNorm backward kernels for gfx950 (CDNA4, wave64).
//
// For y = x * r * w with r = rsqrt(sum_k x_k^2 / H + eps) and an upstream
// gradient dy, the derivative (the norm backward of a training step's backward
// stage, TileLang tutorial ch. 02, section 1.1(b); the pages give no formula,
// this is the plain one) is
//
//   dx_k = r * (dy_k * w_k - x_k * r^2 * c / H),   c = sum_j dy_j * w_j * x_j
//   dw_j = sum_i dy_ij * x_ij * r_i
//
// dx is another row pass: the row of x and dy lives in registers, the two row
// sums (x^2 and dy*w*x) go through the same lane -> wave -> workgroup
// reduction as the forward (one barrier per row), and dx is written once.
//
// dw is the first reduction across rows.  It is done in two deterministic
// stages without atomics: a capped grid walks the rows (workgroup b takes rows
// b, b + G, b + 2G, ...) and every lane keeps fp32 sums for its own columns,
// which stay fixed from row to row; at the end each workgroup writes one
// partial row of fp32 sums into a caller-provided workspace, and
// rms_bwd_dw_kernel adds the G partial rows per column in a fixed order and
// rounds once.  Both stages are HBM-bound streams; nothing is a contraction.
#pragma once

#include "rmsnorm_kernels.hpp"

namespace mbr {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct BwdArgs {
    const void* x;
    const void* w;
    const void* dy;
    void* dx;
    float* part;     // DW: [gridDim.x][ld] fp32 partial dweight rows
    int64_t rows;
    int64_t n_groups;        // ceil(rows / rows_per_block)
    int64_t ld;              // floats per partial row (a multiple of 64, >= hidden)
    int32_t units;           // per row: 16-byte vectors (vector path) or elements
    int32_t rows_per_block;  // vector path: rows a workgroup works on at once
    float inv_hidden;        // 1 / hidden rounded once on the host (exact for powers of two):
                             // the row sums multiply by it instead of dividing
    float eps;
    int32_t tail;            // any-alignment path: elements after the row's full vectors
};

struct DwArgs {
    const float* part;  // [n_part][ld]
    void* dw;           // [hidden], tensor dtype
    int64_t ld;
    int32_t n_part;
    int32_t hidden;
};

// Row totals of both sums, identical bits in every lane of the row; the row
// occupies waves slot*WPR .. slot*WPR + WPR - 1 of the workgroup.  Every wave
// of the workgroup reaches the barrier once per call.
template <int WPR>
__device__ __forceinline__ void row_sums(float& ss, float& cc, float (&ps)[2][16], float (&pc)[2][16], int it,
                                         int wave, int slot = 0) {
    ss = wave_sum(ss);
    cc = wave_sum(cc);
    if constexpr (WPR > 1) {
        if ((threadIdx.x & 63) == 0) {
            ps[it & 1][wave] = ss;
            pc[it & 1][wave] = cc;
        }
        __syncthreads();
        ss = 0.f;
        cc = 0.f;
#pragma unroll
        for (int i = 0; i < WPR; ++i) {
            ss += ps[it & 1][slot * WPR + i];
            cc += pc[it & 1][slot * WPR + i];
        }
    }
}

// Sum over the 64 / L lanes of a wave that hold the same position in their
// aligned L-lane groups (L = 8, 16 or 32).  row_ror:8 pairs lane i with lane
// i ^ 8 inside each 16-lane row, and the two permlane swaps pair lanes i ^ 16
// and i ^ 32; both partners add the same two values, so every lane returns
// the same bits as its partners.
template <int L>
__device__ __forceinline__ float across_groups_sum(float v) {
    static_assert(L == 8 || L == 16 || L == 32, "group width");
    if constexpr (L == 8) v += dpp_mov<0x128>(v);
    if constexpr (L <= 16) {
        auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Makes the compiler treat a packed vector as redefined here (no instruction
// is emitted), so values widened from it before this point are recomputed
// after it instead of being held: a row's x, dy and w then stay packed across
// the reduction (12 VGPRs per bf16 vector instead of 24 widened fp32 ones).
__device__ __forceinline__ void repack(u32x4& v) { asm volatile("" : "+v"(v)); }

// Where the row kernel needs it: the widened values would otherwise spill
// (8 vectors per lane, or 4 and more in a 1024-lane workgroup, 128 VGPRs).
// Elsewhere holding them saves a third of the widening work (the 4 x 4 kernel:
// 633 -> 569 VALU instructions per row, 156 VGPRs, still 3 waves per SIMD
// against the 2 its 512-workgroup grid keeps resident): bf16 [4096, 2048]
// 16.0 -> 15.7 us, fp32 [16384, 2048] 69.2 -> 67.7, [16384, 8192] 134.9 ->
// 134.5.  With it the 1 x 8 kernel keeps [2048, 4096] at 18.6 us (22.2 spilling).
template <int WPR, int VPL>
constexpr bool kBwdRepack = VPL >= 8 || (WPR == 16 && VPL >= 4);

// One partial row: V consecutive fp32 sums per 16-byte input vector.
__device__ __forceinline__ void store_partial(float* p, const float* acc, Bf16) {
    f32x4 a = {acc[0], acc[1], acc[2], acc[3]}, b = {acc[4], acc[5], acc[6], acc[7]};
    reinterpret_cast<f32x4*>(p)[0] = a;
    reinterpret_cast<f32x4*>(p)[1] = b;
}
__device__ __forceinline__ void store_partial(float* p, const float* acc, F32) {
    f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
    reinterpret_cast<f32x4*>(p)[0] = a;
}

// Vector path: WPR waves per row, VPL 16-byte vectors per lane, lane l of a
// row owning vectors l, l + 64*WPR, ... of both x and dy; the weight slice
// stays in registers for the whole walk.  A workgroup holds rows_per_block
// row slots; in each step of its walk slot s takes row group*rows_per_block +
// s.  With several slots, the slots' dweight sums are combined in LDS, in slot
// order, into the workgroup's single partial row: fewer partial rows for the
// same number of waves in flight.  (A conditional next-row prefetch measured
// the same as none: the compiler waits for every load after the branch.)
//
// LPR < 64 (with WPR 1): rows narrower than a wave share it, each row owning
// an aligned group of LPR lanes (8, 16 or 32) and being one row slot; the row
// sums are group sums with no LDS and no barrier.  A wave's groups add their
// dweight sums among themselves first, and the LDS combine then runs over
// waves instead of slots.
template <class E, int WPR, int VPL, bool MASKED, bool DW, int LPR = 64>
__global__ void __launch_bounds__(max_threads<WPR>()) rms_bwd_vec_kernel(const BwdArgs a) {
    static_assert(LPR == 64 || WPR == 1, "sub-wave rows use one wave");
    constexpr int LANES = LPR < 64 ? LPR : 64 * WPR;
    constexpr int V = E::kVec;
    const int wave = wave_id();
    const int slot = LPR < 64 ? static_cast<int>(threadIdx.x) / LPR : wave / WPR;
    const int lane = static_cast<int>(threadIdx.x) - slot * LANES;
    const int nvec = a.units;
    const int rpb = a.rows_per_block;
    __shared__ float ps[2][16], pc[2][16];

    // Byte offset of a lane's k-th vector within a row: unsigned 32-bit, so
    // that accesses take a wave-uniform 64-bit row base in SGPRs plus one
    // VGPR offset instead of a 64-bit VGPR address per vector.
    auto voff = [&](int k) {
        const int v = k * LANES + lane;
        return static_cast<unsigned>(MASKED ? (v < nvec ? v : nvec - 1) : v) * 16u;
    };
    auto at = [](const void* base, unsigned off) {
        return reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + off);
    };
    auto in_row = [&](int k) { return !MASKED || k * LANES + lane < nvec; };
    const int64_t row_bytes = static_cast<int64_t>(nvec) * 16;

    u32x4 wv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) wv[k] = load_keep(at(a.w, voff(k)));
    float acc[DW ? VPL * V : 1];
    if constexpr (DW) {
#pragma unroll
        for (int i = 0; i < VPL * V; ++i) acc[i] = 0.f;
    }

    int it = 0;
    for (int64_t grp = blockIdx.x; grp < a.n_groups; grp += gridDim.x, ++it) {
        const int64_t row = grp * rpb + slot;
        const bool valid = row < a.rows;
        u32x4 xv[VPL], gv[VPL];
        float ss = 0.f, cc = 0.f;
        // Sub-wave rows address from the group's first row (wave-uniform)
        // plus a 32-bit offset per lane group; a group past the last row
        // loads the last row again instead of branching around the loads,
        // and its sums are dropped.
        const int64_t brow = LPR < 64 ? grp * rpb : row;
        const unsigned soff = LPR < 64 ? static_cast<unsigned>(((valid ? row : a.rows - 1) - brow) * row_bytes) : 0u;
        if (LPR < 64 || valid) {
            const char* xr = static_cast<const char*>(a.x) + brow * row_bytes;
            const char* gr = static_cast<const char*>(a.dy) + brow * row_bytes;
#pragma unroll
            for (int k = 0; k < VPL; ++k) xv[k] = load_stream(at(xr, soff + voff(k)));
#pragma unroll
            for (int k = 0; k < VPL; ++k) gv[k] = load_stream(at(gr, soff + voff(k)));
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                float fx[V], fg[V], fw[V];
                widen(xv[k], fx, E{});
                widen(gv[k], fg, E{});
                widen(wv[k], fw, E{});
                float s = 0.f, c = 0.f;
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    s += fx[i] * fx[i];
                    c += (fg[i] * fw[i]) * fx[i];
                }
                ss += in_row(k) ? s : 0.f;
                cc += in_row(k) ? c : 0.f;
            }
        }
        if constexpr (LPR < 64) {
            ss = group_sum<LPR>(ss);
            cc = group_sum<LPR>(cc);
        } else {
            row_sums<WPR>(ss, cc, ps, pc, it, wave, slot);
        }
        if (!valid) continue;
        if constexpr (kBwdRepack<WPR, VPL>) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                repack(xv[k]);
                repack(gv[k]);
                repack(wv[k]);
            }
        }
        const float r = rsqrtf(mul_rn(ss, a.inv_hidden) + a.eps);
        const float k2 = mul_rn(r * r * cc, a.inv_hidden);
        char* dxr = static_cast<char*>(a.dx) + brow * row_bytes;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (!in_row(k)) continue;
            float fx[V], fg[V], fw[V], d[V];
            widen(xv[k], fx, E{});
            widen(gv[k], fg, E{});
            widen(wv[k], fw, E{});
#pragma unroll
            for (int i = 0; i < V; ++i) d[i] = r * (fg[i] * fw[i] - fx[i] * k2);
            store_stream(reinterpret_cast<u32x4*>(dxr + soff + voff(k)), narrow(d, E{}));
            if constexpr (DW) {
#pragma unroll
                for (int i = 0; i < V; ++i) acc[k * V + i] += (fg[i] * fx[i]) * r;
            }
        }
    }
    if constexpr (DW) {
        float* pr = a.part + static_cast<int64_t>(blockIdx.x) * a.ld;
        // Rows narrower than a wave: the lane groups of a wave first add their
        // sums across groups (every group ends with the same bits) and group 0
        // then stands for the wave.
        if constexpr (LPR < 64) {
#pragma unroll
            for (int i = 0; i < VPL * V; ++i) acc[i] = across_groups_sum<LPR>(acc[i]);
        }
        const int parties = LPR < 64 ? static_cast<int>(blockDim.x) / 64 : rpb;
        const int party = LPR < 64 ? wave : slot;
        const bool speaks = LPR == 64 || (threadIdx.x & 63) < LPR;
        if (parties == 1) {
            if (!speaks) return;
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                if (in_row(k)) store_partial(pr + static_cast<int64_t>(k * LANES + lane) * V, acc + k * V, E{});
            return;
        }
        // the parties add their sums into one LDS row in order, then the
        // whole workgroup writes it out
        extern __shared__ float comb[];  // nvec * V floats
        for (int s = 0; s < parties; ++s) {
            if (party == s && speaks) {
#pragma unroll
                for (int k = 0; k < VPL; ++k) {
                    if (!in_row(k)) continue;
                    float* c = comb + (k * LANES + lane) * V;
#pragma unroll
                    for (int i = 0; i < V; ++i) c[i] = s == 0 ? acc[k * V + i] : c[i] + acc[k * V + i];
                }
            }
            __syncthreads();
        }
        const int nq = nvec * V / 4;
        for (int j = static_cast<int>(threadIdx.x); j < nq; j += blockDim.x)
            reinterpret_cast<f32x4*>(pr)[j] = reinterpret_cast<const f32x4*>(comb)[j];
    }
}

// Element path: any hidden, any element alignment; lane l owns elements
// l, l + 64*WPR, ... (EPL of them).
template <class E, int WPR, int EPL, bool DW>
__global__ void __launch_bounds__(max_threads<WPR>()) rms_bwd_elem_kernel(const BwdArgs a) {
    using S = typename E::scalar;
    constexpr int LANES = 64 * WPR;
    const int wave = wave_id();
    const int lane = static_cast<int>(threadIdx.x);
    const int H = a.units;
    __shared__ float ps[2][16], pc[2][16];
    auto jdx = [&](int k) {
        const int j = k * LANES + lane;
        return j < H ? j : H - 1;
    };
    auto in_row = [&](int k) { return k * LANES + lane < H; };

    float fw[EPL], acc[DW ? EPL : 1];
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        fw[k] = widen1(static_cast<const S*>(a.w)[jdx(k)]);
        if constexpr (DW) acc[k] = 0.f;
    }
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const S* xr = static_cast<const S*>(a.x) + row * H;
        const S* gr = static_cast<const S*>(a.dy) + row * H;
        float fx[EPL], fg[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) fx[k] = widen1(xr[jdx(k)]);
#pragma unroll
        for (int k = 0; k < EPL; ++k) fg[k] = widen1(gr[jdx(k)]);
        float ss = 0.f, cc = 0.f;
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
            ss += in_row(k) ? fx[k] * fx[k] : 0.f;
            cc += in_row(k) ? (fg[k] * fw[k]) * fx[k] : 0.f;
        }
        row_sums<WPR>(ss, cc, ps, pc, it, wave);
        const float r = rsqrtf(mul_rn(ss, a.inv_hidden) + a.eps);
        const float k2 = mul_rn(r * r * cc, a.inv_hidden);
        S* dxr = static_cast<S*>(a.dx) + row * H;
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
            if (!in_row(k)) continue;
            dxr[k * LANES + lane] = narrow1(r * (fg[k] * fw[k] - fx[k] * k2), E{});
            if constexpr (DW) acc[k] += (fg[k] * fx[k]) * r;
        }
    }
    if constexpr (DW) {
        float* pr = a.part + static_cast<int64_t>(blockIdx.x) * a.ld;
#pragma unroll
        for (int k = 0; k < EPL; ++k)
            if (in_row(k)) pr[k * LANES + lane] = acc[k];
    }
}

// The any-alignment kernel also holds its tail values: it repacks from 5
// vectors per lane (3 in a 1024-lane workgroup) to stay clear of spills.
template <int WPR, int VPL>
constexpr bool kBwdAnyRepack = VPL >= 5 || (WPR == 16 && VPL >= 3);

// Any width and any element alignment, in vectors: a row of H elements is
// H / V full 16-byte vectors, moved at whatever alignment the row starts at,
// and then H % V tail elements moved one by one.  Lane l owns vectors l,
// l + 64*WPR, ... (VPL of them) and, if l < H % V, tail element l; every
// access stays inside its row.  One row per workgroup at a time; otherwise the
// vector path's sums, rounding and dweight partial rows (columns of the tail
// land in the partial row's last H % V places).
template <class E, int WPR, int VPL, bool MASKED, bool DW>
__global__ void __launch_bounds__(max_threads<WPR>()) rms_bwd_any_kernel(const BwdArgs a) {
    using S = typename E::scalar;
    constexpr int LANES = 64 * WPR;
    constexpr int V = E::kVec;
    const int wave = wave_id();
    const int lane = static_cast<int>(threadIdx.x);
    const int nvec = a.units;
    const int tail = a.tail;
    const int64_t row_bytes = (static_cast<int64_t>(nvec) * V + tail) * static_cast<int64_t>(sizeof(S));
    __shared__ float ps[2][16], pc[2][16];

    // 32-bit byte offsets within a row on a wave-uniform row base, as on the
    // vector path
    auto voff = [&](int k) {
        const int v = k * LANES + lane;
        return static_cast<unsigned>(MASKED ? (v < nvec ? v : nvec - 1) : v) * 16u;
    };
    auto in_row = [&](int k) { return !MASKED || k * LANES + lane < nvec; };
    const bool has_tail = lane < tail;
    const unsigned toff = static_cast<unsigned>((nvec * V + lane) * static_cast<int>(sizeof(S)));

    const char* wr = static_cast<const char*>(a.w);
    u32x4 wv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) wv[k] = load_keep_any(wr + voff(k));
    const float wt = has_tail ? widen1(*reinterpret_cast<const S*>(wr + toff)) : 0.f;
    float acc[DW ? VPL * V : 1], acct = 0.f;
    if constexpr (DW) {
#pragma unroll
        for (int i = 0; i < VPL * V; ++i) acc[i] = 0.f;
    }

    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const char* xr = static_cast<const char*>(a.x) + row * row_bytes;
        const char* gr = static_cast<const char*>(a.dy) + row * row_bytes;
        u32x4 xv[VPL], gv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) xv[k] = load_stream_any(xr + voff(k));
#pragma unroll
        for (int k = 0; k < VPL; ++k) gv[k] = load_stream_any(gr + voff(k));
        float xt = 0.f, gt = 0.f;
        if (has_tail) {
            xt = widen1(*reinterpret_cast<const S*>(xr + toff));
            gt = widen1(*reinterpret_cast<const S*>(gr + toff));
        }
        float ss = xt * xt, cc = (gt * wt) * xt;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float fx[V], fg[V], fw[V];
            widen(xv[k], fx, E{});
            widen(gv[k], fg, E{});
            widen(wv[k], fw, E{});
            float s = 0.f, c = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                s += fx[i] * fx[i];
                c += (fg[i] * fw[i]) * fx[i];
            }
            ss += in_row(k) ? s : 0.f;
            cc += in_row(k) ? c : 0.f;
        }
        row_sums<WPR>(ss, cc, ps, pc, it, wave);
        if constexpr (kBwdAnyRepack<WPR, VPL>) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                repack(xv[k]);
                repack(gv[k]);
                repack(wv[k]);
            }
        }
        const float r = rsqrtf(mul_rn(ss, a.inv_hidden) + a.eps);
        const float k2 = mul_rn(r * r * cc, a.inv_hidden);
        char* dxr = static_cast<char*>(a.dx) + row * row_bytes;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (!in_row(k)) continue;
            float fx[V], fg[V], fw[V], d[V];
            widen(xv[k], fx, E{});
            widen(gv[k], fg, E{});
            widen(wv[k], fw, E{});
#pragma unroll
            for (int i = 0; i < V; ++i) d[i] = r * (fg[i] * fw[i] - fx[i] * k2);
            store_stream_any(dxr + voff(k), narrow(d, E{}));
            if constexpr (DW) {
#pragma unroll
                for (int i = 0; i < V; ++i) acc[k * V + i] += (fg[i] * fx[i]) * r;
            }
        }
        if (has_tail) {
            *reinterpret_cast<S*>(dxr + toff) = narrow1(r * (gt * wt - xt * k2), E{});
            if constexpr (DW) acct += (gt * xt) * r;
        }
    }
    if constexpr (DW) {
        float* pr = a.part + static_cast<int64_t>(blockIdx.x) * a.ld;
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            if (in_row(k)) store_partial(pr + static_cast<int64_t>(k * LANES + lane) * V, acc + k * V, E{});
        if (has_tail) pr[nvec * V + lane] = acct;
    }
}

// Rows too wide for registers: 1024 lanes stride over the row twice.  Pass 1
// reads x, dy and w for the two sums; pass 2 reads them again and writes dx.
// A thread's columns are the same in every row, so its dweight sums live in
// its own slots of the workgroup's partial row (written on the first row,
// read-modify-written after; no other thread touches them).  Exact aliasing of
// dx with x or dy stays safe: each element is read and then written by the
// same thread.
template <class E, bool VEC, bool DW>
__global__ void __launch_bounds__(1024) rms_bwd_twopass_kernel(const BwdArgs a) {
    using S = typename E::scalar;
    constexpr int V = E::kVec;
    const int wave = wave_id();
    const int nwaves = static_cast<int>(blockDim.x) >> 6;
    const int n = a.units;
    __shared__ float ps[2][16], pc[2][16];
    float* const pr = DW ? a.part + static_cast<int64_t>(blockIdx.x) * a.ld : nullptr;

    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const int64_t base = row * n;
        float ss = 0.f, cc = 0.f;
        for (int j = threadIdx.x; j < n; j += blockDim.x) {
            if constexpr (VEC) {
                float fx[V], fg[V], fw[V];
                widen(load_stream(static_cast<const u32x4*>(a.x) + base + j), fx, E{});
                widen(load_stream(static_cast<const u32x4*>(a.dy) + base + j), fg, E{});
                widen(load_keep(static_cast<const u32x4*>(a.w) + j), fw, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    ss += fx[i] * fx[i];
                    cc += (fg[i] * fw[i]) * fx[i];
                }
            } else {
                const float fx = widen1(static_cast<const S*>(a.x)[base + j]);
                const float fg = widen1(static_cast<const S*>(a.dy)[base + j]);
                ss += fx * fx;
                cc += (fg * widen1(static_cast<const S*>(a.w)[j])) * fx;
            }
        }
        ss = wave_sum(ss);
        cc = wave_sum(cc);
        if ((threadIdx.x & 63) == 0) {
            ps[it & 1][wave] = ss;
            pc[it & 1][wave] = cc;
        }
        __syncthreads();
        ss = 0.f;
        cc = 0.f;
        for (int i = 0; i < nwaves; ++i) {
            ss += ps[it & 1][i];
            cc += pc[it & 1][i];
        }
        const float r = rsqrtf(mul_rn(ss, a.inv_hidden) + a.eps);
        const float k2 = mul_rn(r * r * cc, a.inv_hidden);
        for (int j = threadIdx.x; j < n; j += blockDim.x) {
            if constexpr (VEC) {
                float fx[V], fg[V], fw[V], d[V];
                widen(load_stream(static_cast<const u32x4*>(a.x) + base + j), fx, E{});
                widen(load_stream(static_cast<const u32x4*>(a.dy) + base + j), fg, E{});
                widen(load_keep(static_cast<const u32x4*>(a.w) + j), fw, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) d[i] = r * (fg[i] * fw[i] - fx[i] * k2);
                store_stream(static_cast<u32x4*>(a.dx) + base + j, narrow(d, E{}));
                if constexpr (DW) {
                    f32x4* p = reinterpret_cast<f32x4*>(pr + static_cast<int64_t>(j) * V);
#pragma unroll
                    for (int q = 0; q < V / 4; ++q) {
                        f32x4 t = {(fg[4 * q] * fx[4 * q]) * r, (fg[4 * q + 1] * fx[4 * q + 1]) * r,
                                   (fg[4 * q + 2] * fx[4 * q + 2]) * r, (fg[4 * q + 3] * fx[4 * q + 3]) * r};
                        p[q] = it == 0 ? t : p[q] + t;
                    }
                }
            } else {
                const float fx = widen1(static_cast<const S*>(a.x)[base + j]);
                const float fg = widen1(static_cast<const S*>(a.dy)[base + j]);
                const float fw = widen1(static_cast<const S*>(a.w)[j]);
                static_cast<S*>(a.dx)[base + j] = narrow1(r * (fg * fw - fx * k2), E{});
                if constexpr (DW) {
                    const float t = (fg * fx) * r;
                    pr[j] = it == 0 ? t : pr[j] + t;
                }
            }
        }
    }
}

// Second stage of dweight: workgroup b sums the columns of kDwQuads column
// quads (4 fp32 columns each) over the n_part partial rows.  Thread t of the
// workgroup takes quad q = t % kDwQuads and slice s = t / kDwQuads, and adds
// partial rows s, s + S, s + 2S, ... (S = kDwSlices) of its quad in that
// order (loads issued four at a time).  The S slice sums are then combined
// by a fixed tree: a butterfly over the slices held by one wave (lane
// exchanges at distances kDwQuads, 2 kDwQuads, ..., 32), then the waves'
// totals added in wave order through LDS; the total is rounded once to the
// tensor dtype.  n_part == 0 writes zeros.  A workgroup reads 128 bytes of
// each partial row: narrower tiles measured slower on MI355X, since
// neighbouring workgroups (usually on different XCDs) then fetch the same
// cache lines.
constexpr int kDwThreads = 512;
constexpr int kDwQuads = 8;
constexpr int kDwSlices = kDwThreads / kDwQuads;
constexpr int kDwCols = 4 * kDwQuads;  // columns per workgroup
static_assert(64 % kDwCols == 0, "a workgroup's columns must not cross the end of a 64-float partial row");

__device__ __forceinline__ f32x4 shfl_xor4(f32x4 v, int m) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __shfl_xor(v[i], m);
    return r;
}

template <class E>
__global__ void __launch_bounds__(kDwThreads) rms_bwd_dw_kernel(const DwArgs a) {
    using S = typename E::scalar;
    const int q = threadIdx.x % kDwQuads;
    const int s = threadIdx.x / kDwQuads;
    const int64_t quad = static_cast<int64_t>(blockIdx.x) * kDwQuads + q;
    const f32x4* col = reinterpret_cast<const f32x4*>(a.part) + quad;
    const int64_t stride = a.ld / 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int p = s;
    for (; p + 3 * kDwSlices < a.n_part; p += 4 * kDwSlices) {
        const f32x4 v0 = col[p * stride];
        const f32x4 v1 = col[(p + kDwSlices) * stride];
        const f32x4 v2 = col[(p + 2 * kDwSlices) * stride];
        const f32x4 v3 = col[(p + 3 * kDwSlices) * stride];
        acc += v0;
        acc += v1;
        acc += v2;
        acc += v3;
    }
    for (; p < a.n_part; p += kDwSlices) acc += col[p * stride];
#pragma unroll
    for (int m = kDwQuads; m < 64; m <<= 1) acc += shfl_xor4(acc, m);
    constexpr int kWaves = kDwThreads / 64;
    __shared__ f32x4 sm[kWaves][kDwQuads];
    const int lane = threadIdx.x & 63;
    if (lane < kDwQuads) sm[threadIdx.x / 64][lane] = acc;
    __syncthreads();
    if (threadIdx.x < kDwQuads) {
        f32x4 t = sm[0][q];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t += sm[w][q];
        S* out = static_cast<S*>(a.dw);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t c = quad * 4 + i;
            if (c < a.hidden) out[c] = narrow1(t[i], E{});
        }
    }
}

}  // namespace mbr
