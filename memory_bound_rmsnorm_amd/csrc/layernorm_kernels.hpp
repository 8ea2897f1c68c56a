// LayerNorm kernels for gfx950 (CDNA4, wave64), the sibling of the RMSNorm
// path:
//
//   y_j = gamma_j * (x_j - mu) * rsqrt(var + eps) + beta_j,
//   mu = sum_j x_j / H,  var = sum_j (x_j - mu)^2 / H
//
// (xserv "phase 4: transformer core kernels", csrc/normalization/layernorm.cu
// header comment and docs/04-transformer-kernels.md "LayerNorm"; biased
// variance as in the pages' CPU reference).  The pages' kernel takes the
// variance as E[x^2] - mu^2 from one pass of sums, which cancels when |mu| is
// large against the spread.  Here the row stays in registers and the moments
// come from the corrected two-pass scheme (Chan, Golub and LeVeque, "Algorithms
// for computing the sample variance", 1983): a first reduction gives the fp32
// mean m0; a second one, from the same registers, sums both (x - m0) and
// (x - m0)^2, so that c = sum(x - m0)/H corrects m0's rounding error and
// var = sum(x - m0)^2/H - c^2 (c^2 is tiny).  The output uses (x - m0) - c.
// The error then scales with the spread of the row, not with |mu|.  The
// gamma / beta loads are issued between the two reductions so that they are in
// flight during the second one.  fp32 throughout, one rounding at write-back.
//
// Same lane -> wave (DPP + permlane) -> workgroup (one LDS slot per wave,
// fixed order) reduction as the RMSNorm kernels: bitwise identical totals in
// every lane, reproducible run to run.  HBM-bound; no contraction.
#pragma once

#include "rmsnorm_kernels.hpp"

namespace mbr {

struct LnArgs {
    const void* x;
    const void* g;  // gamma
    const void* b;  // beta, or nullptr (no bias)
    void* out;
    int64_t rows;
    int64_t n_groups;        // vector path: ceil(rows / rows_per_block)
    int32_t units;           // per row: 16-byte vectors (vector path) or elements
    int32_t rows_per_block;  // vector path: row slots per workgroup
    float hidden_f;
    float eps;
    int32_t tail;            // any-alignment vector path: elements after the full vectors (< kVec)
};

// Workgroup totals of N per-lane values: wave sums, one LDS slot per wave
// and value, one barrier, fixed-order sums of the slots.  The first call of a
// row uses slot set 0 and the second set 1; a set is written again only after
// the other set's barrier, so single buffers suffice.
// The row's waves are wave0 .. wave0 + NWAVES - 1 of the workgroup (several
// row slots share a workgroup on the vector path).
template <int NWAVES, int N>
__device__ __forceinline__ void block_sums(float (&v)[N], float (&slots)[N][16], int wave, int nwaves_rt = NWAVES,
                                           int wave0 = 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = wave_sum(v[k]);
    if (NWAVES == 1 || nwaves_rt == 1) return;
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int k = 0; k < N; ++k) slots[k][wave] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        float t = 0.f;
        if constexpr (NWAVES > 0) {
#pragma unroll
            for (int i = 0; i < NWAVES; ++i) t += slots[k][wave0 + i];
        } else {
            for (int i = 0; i < nwaves_rt; ++i) t += slots[k][i];
        }
        v[k] = t;
    }
}

// Moments of a row from the two reductions: the corrected shift c and inv.
struct LnMoments {
    float m0;   // first-pass mean
    float c;    // sum(x - m0) / H
    float inv;  // rsqrt(var + eps)
};

__device__ __forceinline__ LnMoments ln_moments(float m0, const float (&tq)[2], const LnArgs& a) {
    const float c = tq[0] / a.hidden_f;
    const float var = fmaxf(tq[1] / a.hidden_f - c * c, 0.f);
    return {m0, c, rsqrtf(var + a.eps)};
}

// Vector path: WPR waves per row, lane l of a row owning 16-byte vectors l,
// l + 64*WPR, ... (VPL of them).  MASKED: the row has fewer than 64*WPR*VPL
// vectors; loads are clamped in bounds, the extra values excluded from both
// sums, stores skipped.  GBL: the workgroup copies gamma (and beta) into LDS
// once, published by the first row barrier (or an explicit one when a row
// takes one wave), and holds rows_per_block row slots that read them from
// there: in each step of its walk slot s takes row group*rows_per_block + s
// (a slot past the last row reads the last row again and stores nothing).
// Without GBL a workgroup works on one row at a time and loads gamma and beta
// per row; the slot terms fold away at compile time.
//
// LPR < 64 (one wave, no GBL): rows narrower than a wave share it, each row
// owning an aligned group of LPR lanes (8, 16 or 32) and being one row slot;
// both reductions are group sums with no LDS and no barrier, and each lane
// loads its gamma / beta slice once for the whole walk.
template <class E, int WPR, int VPL, bool MASKED, bool GBL, int LPR = 64>
__global__ void __launch_bounds__(max_threads<WPR>()) ln_vec_kernel(const LnArgs a) {
    static_assert(LPR == 64 || (WPR == 1 && !GBL), "sub-wave rows use one wave and per-lane gamma / beta");
    constexpr bool SUB = LPR < 64;
    constexpr int LANES = SUB ? LPR : 64 * WPR;
    constexpr int V = E::kVec;
    const int wave = wave_id();
    const int slot = SUB ? static_cast<int>(threadIdx.x) / LPR : GBL ? wave / WPR : 0;
    const int lane = static_cast<int>(threadIdx.x) - slot * LANES;
    const int nvec = a.units;
    const int64_t rpb = GBL || SUB ? a.rows_per_block : 1;
    const int64_t n_groups = GBL || SUB ? a.n_groups : a.rows;
    const bool bias = a.b != nullptr;
    __shared__ float s1[1][16], s2[2][16];
    extern __shared__ u32x4 gb[];  // GBL: gamma [nvec], then beta [nvec]

    auto vidx = [&](int k) {
        const int v = k * LANES + lane;
        return MASKED ? (v < nvec ? v : nvec - 1) : v;
    };
    auto in_row = [&](int k) { return !MASKED || k * LANES + lane < nvec; };

    if constexpr (GBL) {
        // gamma and beta vectors fetched together: one round trip per step
        for (int j = static_cast<int>(threadIdx.x); j < nvec; j += static_cast<int>(blockDim.x)) {
            gb[j] = load_keep(static_cast<const u32x4*>(a.g) + j);
            if (bias) gb[nvec + j] = load_keep(static_cast<const u32x4*>(a.b) + j);
        }
        if constexpr (WPR == 1) __syncthreads();
    }

    u32x4 gs[SUB ? VPL : 1], bs[SUB ? VPL : 1];
    if constexpr (SUB) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            gs[k] = load_keep(static_cast<const u32x4*>(a.g) + vidx(k));
            if (bias) bs[k] = load_keep(static_cast<const u32x4*>(a.b) + vidx(k));
        }
    }

    for (int64_t grp = blockIdx.x; grp < n_groups; grp += gridDim.x) {
        const int64_t row = grp * rpb + slot;
        const bool valid = !(GBL || SUB) || row < a.rows;
        // sub-wave rows address from the group's first row (wave-uniform)
        // plus a per-lane-group vector offset
        const int64_t brow = SUB ? grp * rpb : valid ? row : a.rows - 1;
        const int soff = SUB ? static_cast<int>(((valid ? row : a.rows - 1) - brow) * nvec) : 0;
        const u32x4* xr = static_cast<const u32x4*>(a.x) + brow * nvec;
        u32x4 d[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) d[k] = load_stream(xr + (soff + vidx(k)));
        float s[1] = {0.f};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[V];
            widen(d[k], f, E{});
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) t += f[i];
            s[0] += in_row(k) ? t : 0.f;
        }
        if constexpr (SUB) {
            s[0] = group_sum<LPR>(s[0]);
        } else {
            block_sums<WPR>(s, s1, wave, WPR, slot * WPR);
        }
        const float m0 = s[0] / a.hidden_f;
        u32x4 gv[GBL || SUB ? 1 : VPL], bv[GBL || SUB ? 1 : VPL];
        if constexpr (!GBL && !SUB) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                gv[k] = load_keep(static_cast<const u32x4*>(a.g) + vidx(k));
                if (bias) bv[k] = load_keep(static_cast<const u32x4*>(a.b) + vidx(k));
            }
        }
        float tq[2] = {0.f, 0.f};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[V];
            widen(d[k], f, E{});
            float t = 0.f, q = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const float e = f[i] - m0;
                t += e;
                q += e * e;
            }
            tq[0] += in_row(k) ? t : 0.f;
            tq[1] += in_row(k) ? q : 0.f;
        }
        if constexpr (SUB) {
            tq[0] = group_sum<LPR>(tq[0]);
            tq[1] = group_sum<LPR>(tq[1]);
        } else {
            block_sums<WPR>(tq, s2, wave, WPR, slot * WPR);
        }
        if (!valid) continue;  // GBL or sub-wave only: a slot past the last row
        const LnMoments m = ln_moments(m0, tq, a);
        u32x4* outr = static_cast<u32x4*>(a.out) + (SUB ? brow * nvec + soff : row * nvec);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (!in_row(k)) continue;
            float f[V], fg[V], fb[V];
            widen(d[k], f, E{});
            if constexpr (GBL) {
                widen(gb[k * LANES + lane], fg, E{});
                if (bias) widen(gb[nvec + k * LANES + lane], fb, E{});
            } else if constexpr (SUB) {
                widen(gs[k], fg, E{});
                if (bias) widen(bs[k], fb, E{});
            } else {
                widen(gv[k], fg, E{});
                if (bias) widen(bv[k], fb, E{});
            }
            if (!bias) {
#pragma unroll
                for (int i = 0; i < V; ++i) fb[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < V; ++i) f[i] = fg[i] * (((f[i] - m.m0) - m.c) * m.inv) + fb[i];
            store_stream(outr + k * LANES + lane, narrow(f, E{}));
        }
    }
}

// Any width and any element alignment, in vectors: a row of H elements is
// H / V full 16-byte vectors moved at the row's own alignment (unaligned
// 16-byte accesses, as the RMSNorm any-alignment kernel), then H % V tail
// elements, tail element l owned by lane l.  One row per workgroup at a time;
// gamma and beta are read per row like the vector path's per-row loads.  The
// moments are the vector path's corrected two-pass sums, with the tail
// element added first in each lane.
template <class E, int WPR, int VPL, bool MASKED>
__global__ void __launch_bounds__(max_threads<WPR>()) ln_any_kernel(const LnArgs a) {
    using S = typename E::scalar;
    constexpr int LANES = 64 * WPR;
    constexpr int V = E::kVec;
    const int wave = wave_id();
    const int lane = static_cast<int>(threadIdx.x);
    const int nvec = a.units;
    const int tail = a.tail;
    const int64_t row_bytes = (static_cast<int64_t>(nvec) * V + tail) * static_cast<int64_t>(sizeof(S));
    const bool bias = a.b != nullptr;
    __shared__ float s1[1][16], s2[2][16];
    auto voff = [&](int k) {
        const int v = k * LANES + lane;
        return static_cast<int64_t>(MASKED ? (v < nvec ? v : nvec - 1) : v) * 16;
    };
    auto in_row = [&](int k) { return !MASKED || k * LANES + lane < nvec; };
    const bool has_tail = lane < tail;
    const int64_t toff = (static_cast<int64_t>(nvec) * V + lane) * static_cast<int64_t>(sizeof(S));
    const char* gr = static_cast<const char*>(a.g);
    const char* br = static_cast<const char*>(a.b);

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const char* xr = static_cast<const char*>(a.x) + row * row_bytes;
        u32x4 d[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) d[k] = load_stream_any(xr + voff(k));
        const float xt = has_tail ? widen1(*reinterpret_cast<const S*>(xr + toff)) : 0.f;
        float s[1] = {xt};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[V];
            widen(d[k], f, E{});
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) t += f[i];
            s[0] += in_row(k) ? t : 0.f;
        }
        block_sums<WPR>(s, s1, wave);
        const float m0 = s[0] / a.hidden_f;
        u32x4 gv[VPL], bv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            gv[k] = load_keep_any(gr + voff(k));
            if (bias) bv[k] = load_keep_any(br + voff(k));
        }
        const float et = has_tail ? xt - m0 : 0.f;
        float tq[2] = {et, et * et};
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[V];
            widen(d[k], f, E{});
            float t = 0.f, q = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const float e = f[i] - m0;
                t += e;
                q += e * e;
            }
            tq[0] += in_row(k) ? t : 0.f;
            tq[1] += in_row(k) ? q : 0.f;
        }
        block_sums<WPR>(tq, s2, wave);
        const LnMoments m = ln_moments(m0, tq, a);
        char* outr = static_cast<char*>(a.out) + row * row_bytes;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (!in_row(k)) continue;
            float f[V], fg[V], fb[V];
            widen(d[k], f, E{});
            widen(gv[k], fg, E{});
            if (bias) {
                widen(bv[k], fb, E{});
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) fb[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < V; ++i) f[i] = fg[i] * (((f[i] - m.m0) - m.c) * m.inv) + fb[i];
            store_stream_any(outr + voff(k), narrow(f, E{}));
        }
        if (has_tail) {
            const float gt = widen1(*reinterpret_cast<const S*>(gr + toff));
            const float bt = bias ? widen1(*reinterpret_cast<const S*>(br + toff)) : 0.f;
            *reinterpret_cast<S*>(outr + toff) = narrow1(gt * (((xt - m.m0) - m.c) * m.inv) + bt, E{});
        }
    }
}

// Element path: any hidden, any element alignment; lane l owns elements
// l, l + 64*WPR, ... (EPL of them).
template <class E, int WPR, int EPL>
__global__ void __launch_bounds__(max_threads<WPR>()) ln_elem_kernel(const LnArgs a) {
    using S = typename E::scalar;
    constexpr int LANES = 64 * WPR;
    const int wave = wave_id();
    const int lane = static_cast<int>(threadIdx.x);
    const int H = a.units;
    const bool bias = a.b != nullptr;
    __shared__ float s1[1][16], s2[2][16];
    auto jdx = [&](int k) {
        const int j = k * LANES + lane;
        return j < H ? j : H - 1;
    };
    auto in_row = [&](int k) { return k * LANES + lane < H; };

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const S* xr = static_cast<const S*>(a.x) + row * H;
        float f[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) f[k] = widen1(xr[jdx(k)]);
        float s[1] = {0.f};
#pragma unroll
        for (int k = 0; k < EPL; ++k) s[0] += in_row(k) ? f[k] : 0.f;
        block_sums<WPR>(s, s1, wave);
        const float m0 = s[0] / a.hidden_f;
        float fg[EPL], fb[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
            fg[k] = widen1(static_cast<const S*>(a.g)[jdx(k)]);
            fb[k] = bias ? widen1(static_cast<const S*>(a.b)[jdx(k)]) : 0.f;
        }
        float tq[2] = {0.f, 0.f};
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
            const float e = f[k] - m0;
            tq[0] += in_row(k) ? e : 0.f;
            tq[1] += in_row(k) ? e * e : 0.f;
        }
        block_sums<WPR>(tq, s2, wave);
        const LnMoments m = ln_moments(m0, tq, a);
        S* outr = static_cast<S*>(a.out) + row * H;
#pragma unroll
        for (int k = 0; k < EPL; ++k)
            if (in_row(k)) outr[k * LANES + lane] = narrow1(fg[k] * (((f[k] - m.m0) - m.c) * m.inv) + fb[k], E{});
    }
}

// Rows too wide for registers: blockDim.x lanes stride over the row three
// times (sum; centred squares; output), one row per workgroup iteration.  The
// first two passes write nothing, so exact aliasing of out with x stays safe.
template <class E, bool VEC>
__global__ void __launch_bounds__(1024) ln_multipass_kernel(const LnArgs a) {
    using S = typename E::scalar;
    constexpr int V = E::kVec;
    const int wave = wave_id();
    const int nwaves = static_cast<int>(blockDim.x) >> 6;
    const int n = a.units;
    const bool bias = a.b != nullptr;
    __shared__ float s1[1][16], s2[2][16];

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t base = row * n;
        float s[1] = {0.f};
        for (int j = threadIdx.x; j < n; j += blockDim.x) {
            if constexpr (VEC) {
                float f[V];
                widen(load_stream(static_cast<const u32x4*>(a.x) + base + j), f, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) s[0] += f[i];
            } else {
                s[0] += widen1(static_cast<const S*>(a.x)[base + j]);
            }
        }
        block_sums<0>(s, s1, wave, nwaves);
        const float m0 = s[0] / a.hidden_f;
        float tq[2] = {0.f, 0.f};
        for (int j = threadIdx.x; j < n; j += blockDim.x) {
            if constexpr (VEC) {
                float f[V];
                widen(load_stream(static_cast<const u32x4*>(a.x) + base + j), f, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const float e = f[i] - m0;
                    tq[0] += e;
                    tq[1] += e * e;
                }
            } else {
                const float e = widen1(static_cast<const S*>(a.x)[base + j]) - m0;
                tq[0] += e;
                tq[1] += e * e;
            }
        }
        block_sums<0>(tq, s2, wave, nwaves);
        const LnMoments m = ln_moments(m0, tq, a);
        for (int j = threadIdx.x; j < n; j += blockDim.x) {
            if constexpr (VEC) {
                float f[V], fg[V], fb[V];
                widen(load_stream(static_cast<const u32x4*>(a.x) + base + j), f, E{});
                widen(load_keep(static_cast<const u32x4*>(a.g) + j), fg, E{});
                if (bias) {
                    widen(load_keep(static_cast<const u32x4*>(a.b) + j), fb, E{});
                } else {
#pragma unroll
                    for (int i = 0; i < V; ++i) fb[i] = 0.f;
                }
#pragma unroll
                for (int i = 0; i < V; ++i) f[i] = fg[i] * (((f[i] - m.m0) - m.c) * m.inv) + fb[i];
                store_stream(static_cast<u32x4*>(a.out) + base + j, narrow(f, E{}));
            } else {
                const float f = widen1(static_cast<const S*>(a.x)[base + j]);
                const float fg = widen1(static_cast<const S*>(a.g)[j]);
                const float fb = bias ? widen1(static_cast<const S*>(a.b)[j]) : 0.f;
                static_cast<S*>(a.out)[base + j] = narrow1(fg * (((f - m.m0) - m.c) * m.inv) + fb, E{});
            }
        }
    }
}

}  // namespace mbr
