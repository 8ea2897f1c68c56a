// Row-wise RMSNorm kernels for gfx950 (CDNA4, wave64).
//
//   y_j = x_j * rsqrt(sum_k x_k^2 / hidden + eps) * w_j
//
// (xserv "phase 4: transformer core kernels", csrc/normalization/rmsnorm.cu
// and docs/04-transformer-kernels.md "RMSNorm"), fp32 accumulation and scaling
// with a single rounding at write-back and exactly one global read and one
// global write of every row (gollamago README, "RMSNorm 优化（TileLang）").
//
// Kernel families, all one row per group of 64*WPR lanes:
//   rms_vec_kernel      the row lives in VGPRs as packed 16-byte vectors
//                       (bf16x8 / f32x4); coalesced 16-byte loads and stores.
//   rms_any_kernel      the same at any element alignment (full vectors plus
//                       a tail of single elements; bf16 rows 2 bytes past a
//                       4-byte boundary move one element earlier, 4-byte
//                       aligned).
//   rms_elem_kernel     the row lives in VGPRs as fp32 scalars, one element per
//                       access: rows narrower than one 16-byte vector.
//   rms_stage_kernel    rows larger than the register budget of a 1024-lane
//                       workgroup: part in VGPRs, the rest staged in LDS.
//   rms_twopass_kernel  rows larger than that, or unaligned wide rows: pass 1
//                       sums squares, pass 2 re-reads x.
//
// QT != 0 selects the dynamic-quantisation form (the Add + RmsNorm +
// DynamicQuant fusion the TileLang tutorial ch. 02, section 4.2, cites from
// CANN): instead of the normalised row, each row is written as int8 (QT 1) or
// fp8 e4m3fn (QT 2) codes with one fp32 scale, scale = max|y| / Q and
// code_j = round(y_j / scale).  Because y_j = x_j * r * w_j with one r > 0 per
// row, r cancels from the codes: they are computed as (x_j * w_j) * (Q / m)
// with m = max_k |x_k * w_k|, which the lanes track in the same reduction pass
// as the sum of squares (one barrier per row, as in the plain form), and the
// scale is r * m / Q.
//
// The sum of squares is reduced lane -> wave (DPP within 16-lane rows, then
// the gfx950 permlane16/permlane32 swaps) -> workgroup (one LDS slot per wave,
// one barrier, every wave adds the slots in the same fixed order).  Every lane
// ends with bit-identical totals, so the inverse root needs no broadcast and
// results are reproducible run to run.  There is no contraction anywhere, so
// no MFMA: the kernels are bound by HBM bandwidth.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbr {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Everything a launch needs; passed by value as the kernel argument.
struct RowArgs {
    const void* x;
    const void* res;  // fused only
    const void* w;
    void* h;          // fused only: residual_out
    void* out;
    int64_t rows;
    int64_t n_groups;    // ceil(rows / rows_per_block)
    int32_t units;       // per row: 16-byte vectors (vector path) or elements
    int32_t rows_per_block;
    float hidden_f;      // hidden as fp32, the mean's divisor
    float eps;
    float* scale;        // quantised forms: one fp32 scale per row
    int32_t w_lds;       // vector path, normalised output: weight staged in LDS
    int32_t tail;        // any-alignment vector path: elements after the full vectors (< kVec)
    int32_t frame;       // any-alignment vector path, bf16, normalised output: rows that
                         // start 2 bytes past a 4-byte boundary move as the dword-aligned
                         // row one element earlier (every row tensor shares that offset)
};

// ---------------------------------------------------------------- dtypes

struct Bf16 {
    static constexpr int kVec = 8;  // elements per 16-byte vector
    using scalar = uint16_t;
};
struct F32 {
    static constexpr int kVec = 4;
    using scalar = float;
};

__device__ __forceinline__ void widen(const u32x4 v, float (&f)[8], Bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void widen(const u32x4 v, float (&f)[4], F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}

// fp32 -> bf16, nearest-even (v_cvt_pk_bf16_f32 on gfx950); low half = lo.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x4 narrow(const float (&f)[8], Bf16) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return r;
}
__device__ __forceinline__ u32x4 narrow(const float (&f)[4], F32) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    return r;
}

__device__ __forceinline__ float widen1(uint16_t b) { return __uint_as_float((unsigned)b << 16); }
__device__ __forceinline__ float widen1(float f) { return f; }
__device__ __forceinline__ uint16_t narrow1(float f, Bf16) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float narrow1(float f, F32) { return f; }

// ---------------------------------------------------------------- memory

// Streamed operands (x, residual, outputs) are touched once: non-temporal
// hints keep them from displacing the weight, which every row re-reads.
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ u32x4 load_keep(const u32x4* p) { return *p; }

// A product the compiler may not fuse into a following add (device code is
// built with contraction on): where a kernel family must give the same bits
// in every launch configuration, such a product is rounded on its own.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

// ---------------------------------------------------------------- reduction

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; every lane returns the same bits.  Each
// step adds a lane's value to its partner's with the two operands in the same
// order on both sides, so partners compute identical sums.
//   quad_perm [1,0,3,2], quad_perm [2,3,0,1]: sums over quads
//   row_half_mirror, row_mirror:              sums over 8 and 16 lanes
//   permlane16_swap:                          rows 0+1 and 2+3
//   permlane32_swap:                          lanes 0-31 + 32-63
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    {
        auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    {
        auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    return v;
}

// Sum over each aligned group of L lanes (L = 8, 16, 32 or 64): the first
// steps of wave_sum, stopped at the group width; every lane of a group returns
// the same bits.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(L == 8 || L == 16 || L == 32 || L == 64, "group width");
    if constexpr (L == 64) {
        return wave_sum(v);
    } else {
        v += dpp_mov<0xB1>(v);
        v += dpp_mov<0x4E>(v);
        v += dpp_mov<0x141>(v);
        if constexpr (L >= 16) v += dpp_mov<0x140>(v);
        if constexpr (L == 32) {
            auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
        return v;
    }
}

// Maximum over the 64 lanes of a wave, same pattern as wave_sum (fmaxf is
// commutative, so every lane returns the same bits).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    {
        auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    {
        auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    return v;
}

// Maximum over each aligned group of L lanes, as group_sum.
template <int L>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (L == 64) {
        return wave_max(v);
    } else {
        v = fmaxf(v, dpp_mov<0xB1>(v));
        v = fmaxf(v, dpp_mov<0x4E>(v));
        v = fmaxf(v, dpp_mov<0x141>(v));
        if constexpr (L >= 16) v = fmaxf(v, dpp_mov<0x140>(v));
        if constexpr (L == 32) {
            auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
        }
        return v;
    }
}

// ---------------------------------------------------------------- quantised output

template <int QT>
constexpr float quant_max() { return QT == 1 ? 127.0f : 448.0f; }

// One code from t = y / scale: int8 nearest-even clamped to [-127, 127], or
// fp8 e4m3fn nearest-even (v_cvt_pk_fp8_f32) after clamping to +-448.
template <int QT>
__device__ __forceinline__ unsigned quant_code(float t) {
    if constexpr (QT == 1) {
        const float c = fminf(fmaxf(__builtin_rintf(t), -127.0f), 127.0f);
        return static_cast<unsigned>(static_cast<int>(c)) & 0xffu;
    } else {
        const float c = fminf(fmaxf(t, -448.0f), 448.0f);
        return static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xffu;
    }
}

// Four codes packed little-endian into one dword.  int8: after the clamp,
// adding 1.5 * 2^23 rounds t to the nearest integer (ties to even, as rintf)
// and leaves it in the low mantissa bits, so the low byte of the sum's bits is
// the two's-complement code; v_perm_b32 gathers the four low bytes.  Three
// VALU operations per code fewer than rint, convert, mask and shift.
template <int QT>
__device__ __forceinline__ unsigned quant_pack4(float t0, float t1, float t2, float t3) {
    if constexpr (QT == 1) {
        constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
        const unsigned b0 = __float_as_uint(fminf(fmaxf(t0, -127.0f), 127.0f) + kRound);
        const unsigned b1 = __float_as_uint(fminf(fmaxf(t1, -127.0f), 127.0f) + kRound);
        const unsigned b2 = __float_as_uint(fminf(fmaxf(t2, -127.0f), 127.0f) + kRound);
        const unsigned b3 = __float_as_uint(fminf(fmaxf(t3, -127.0f), 127.0f) + kRound);
        // selector bytes 0-3 pick from the second operand, 4-7 from the first, 0x0c gives zero
        const unsigned lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
        const unsigned hi = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
        return lo | hi;
    } else {
        const float c0 = fminf(fmaxf(t0, -448.0f), 448.0f), c1 = fminf(fmaxf(t1, -448.0f), 448.0f);
        const float c2 = fminf(fmaxf(t2, -448.0f), 448.0f), c3 = fminf(fmaxf(t3, -448.0f), 448.0f);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
        return static_cast<unsigned>(w);
    }
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Codes of one 16-byte input vector: 8 bytes for bf16 (u32x2), 4 for fp32.
template <int QT>
__device__ __forceinline__ void store_codes(void* q_row, int v, const float (&t)[8], Bf16) {
    u32x2 c;
    c[0] = quant_pack4<QT>(t[0], t[1], t[2], t[3]);
    c[1] = quant_pack4<QT>(t[4], t[5], t[6], t[7]);
    __builtin_nontemporal_store(c, static_cast<u32x2*>(q_row) + v);
}
template <int QT>
__device__ __forceinline__ void store_codes(void* q_row, int v, const float (&t)[4], F32) {
    __builtin_nontemporal_store(quant_pack4<QT>(t[0], t[1], t[2], t[3]), static_cast<unsigned*>(q_row) + v);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Copy n 16-byte vectors from global memory into LDS with the whole
// workgroup.  Each step covers up to 4 * blockDim vectors: the number of loads
// per thread (m) is the same for every thread, so the loads go out back to
// back, and only the last one can fall past the end (then it is skipped).  The
// copy costs about one memory round trip instead of one per loop step; the
// caller places the barrier that publishes it.
__device__ __forceinline__ void stage_to_lds(const u32x4* src, u32x4* dst, int n) {
    const int t = static_cast<int>(threadIdx.x), nt = static_cast<int>(blockDim.x);
    for (int j0 = 0; j0 < n; j0 += 4 * nt) {
        const int m = min(4, (n - j0 + nt - 1) / nt);  // uniform
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + u * nt + t;
            if (u < m && j < n) v[u] = load_keep(src + j);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + u * nt + t;
            if (u < m && j < n) dst[j] = v[u];
        }
    }
}

// ---------------------------------------------------------------- vector path

template <int WPR>
constexpr int max_threads() { return WPR == 16 ? 1024 : 512; }

// The weight slice a lane needs is the same for every row.  Where registers
// allow, a workgroup loads it once, up front, so that no dependent L2 round
// trip sits between a row's reduction and its stores.  Measured on MI355X this
// pays when a lane holds three or more vectors of a row; with one or two the
// up-front weight loads only delay the row's own loads (and cost occupancy),
// so there the slice is loaded after the reduction instead.
template <int WPR, int VPL, bool FUSED>
constexpr bool weight_resident() { return VPL >= 3 && VPL <= (WPR == 16 ? 4 : 8) && (!FUSED || VPL <= 6); }
// The quantised forms need x_j * w_j before the reduction (for the row max),
// so they always hold the weight slice.
// With a capped grid each workgroup walks several row groups; when the row
// slice is small the next row's loads are issued before the current row is
// reduced and stored, so memory stays busy across the reduction.
template <int VPL, bool FUSED>
constexpr bool row_pipelined() { return VPL * (FUSED ? 2 : 1) <= 4; }

// WPR waves (64*WPR lanes) per row, VPL 16-byte vectors per lane.  Wave w of a
// row owns the row's vectors w*64*VPL .. (w+1)*64*VPL - 1 and lane l of it
// vectors w*64*VPL + l, w*64*VPL + 64 + l, ...: each wave works on a
// contiguous stretch of VPL KiB of the row, each of its load/store
// instructions on 1 KiB.  Measured on MI355X against lanes striding over the whole row
// (lane l of the row owning vectors l, l + 64*WPR, ...), bf16 [16384, 8192] as
// 8 waves x 2 vectors: 85.0 us against 86.2 in the same probe kernel.  With
// one wave per row, or one vector per lane, the two layouts coincide.
// MASKED: the row has fewer than 64*WPR*VPL vectors; loads are clamped in
// bounds (the extra values are excluded from the sum) and stores skipped.
//
// LPR < 64 (with WPR 1): rows narrower than a wave share it, each row owning
// an aligned group of LPR lanes (8, 16 or 32); the row sums are group sums,
// with no LDS and no barrier.  A bf16 row of 128 (16 vectors) then keeps all
// 64 lanes busy with 4 rows instead of leaving 48 lanes idle.
template <class E, int WPR, int VPL, bool MASKED, bool FUSED, int QT = 0, int LPR = 64>
__global__ void __launch_bounds__(max_threads<WPR>()) rms_vec_kernel(const RowArgs a) {
    static_assert(LPR == 64 || WPR == 1, "sub-wave rows use one wave");
    constexpr int LANES = LPR < 64 ? LPR : 64 * WPR;
    constexpr int V = E::kVec;
    constexpr int NR = FUSED ? VPL : 1;  // residual registers
    constexpr bool WRES = QT != 0 || weight_resident<WPR, VPL, FUSED>();
    constexpr bool PIPE = row_pipelined<VPL, FUSED>();
    const int wave = wave_id();
    const int slot = LPR < 64 ? static_cast<int>(threadIdx.x) / LPR : wave / WPR;  // row within the workgroup
    const int lane_row = static_cast<int>(threadIdx.x) - slot * LANES;
    const int nvec = a.units;
    const int64_t rpb = a.rows_per_block;
    __shared__ float part[2][16];
    __shared__ float mpart[QT ? 2 : 1][QT ? 16 : 1];

    // position of a lane's k-th vector in its row (lane groups narrower than a
    // wave: k*LPR + lane; whole waves: the wave's contiguous stretch)
    const int vbase = LPR < 64 ? lane_row : (lane_row >> 6) * (64 * VPL) + (lane_row & 63);
    auto vpos = [&](int k) { return vbase + k * (LPR < 64 ? LPR : 64); };
    auto vidx = [&](int k) {
        const int v = vpos(k);
        return MASKED ? (v < nvec ? v : nvec - 1) : v;
    };
    auto in_row = [&](int k) { return !MASKED || vpos(k) < nvec; };
    auto load_row = [&](int64_t row, u32x4 (&xv)[VPL], u32x4 (&rv)[NR]) {
        const u32x4* xr = static_cast<const u32x4*>(a.x) + row * nvec;
#pragma unroll
        for (int k = 0; k < VPL; ++k) xv[k] = load_stream(xr + vidx(k));
        if constexpr (FUSED) {
            const u32x4* rr = static_cast<const u32x4*>(a.res) + row * nvec;
#pragma unroll
            for (int k = 0; k < VPL; ++k) rv[k] = load_stream(rr + vidx(k));
        }
    };

    const u32x4* wr = static_cast<const u32x4*>(a.w);
    // w_lds: the workgroup copies the weight into LDS once (dynamic LDS of
    // units * 16 bytes) and every row slot takes its slice from there, in place
    // of per-lane global loads.  Lanes that hold the weight (WRES, and every
    // quantised form) fill their registers from LDS after a barrier; the
    // others read LDS at the output, after the first row barrier (or an
    // explicit one when rows take a single wave).
    extern __shared__ u32x4 wlds[];
    const bool use_lds = LPR == 64 && a.w_lds != 0;
    u32x4 wv[WRES ? VPL : 1];
    if (use_lds) {
        stage_to_lds(wr, wlds, nvec);
        if (WRES || WPR == 1) __syncthreads();
    }
    if constexpr (WRES) {
        // one branch around each whole block, so each path issues its loads
        // back to back
        if (use_lds) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) wv[k] = wlds[vidx(k)];
        } else {
#pragma unroll
            for (int k = 0; k < VPL; ++k) wv[k] = load_keep(wr + vidx(k));
        }
    }

    int64_t g = blockIdx.x;
    u32x4 nx[PIPE ? VPL : 1], nr[PIPE ? NR : 1];  // prefetched next row
    if constexpr (PIPE) {
        if (g < a.n_groups && g * rpb + slot < a.rows) load_row(g * rpb + slot, nx, nr);
    }
    int it = 0;
    for (; g < a.n_groups; g += gridDim.x, ++it) {
        const int64_t row = g * rpb + slot;
        const bool valid = row < a.rows;
        u32x4 d[VPL], rv[NR];
        if constexpr (PIPE) {
#pragma unroll
            for (int k = 0; k < VPL; ++k) d[k] = nx[k];
#pragma unroll
            for (int k = 0; k < NR; ++k) rv[k] = nr[k];
            const int64_t next = (g + gridDim.x) * rpb + slot;
            if (g + gridDim.x < a.n_groups && next < a.rows) load_row(next, nx, nr);
        } else {
            if (valid) load_row(row, d, rv);
        }
        float ss = 0.f, mx = 0.f;
        if (valid) {
            if constexpr (FUSED) {
                u32x4* hr = static_cast<u32x4*>(a.h) + row * nvec;
#pragma unroll
                for (int k = 0; k < VPL; ++k) {
                    float fx[V], fr[V];
                    widen(d[k], fx, E{});
                    widen(rv[k], fr, E{});
#pragma unroll
                    for (int i = 0; i < V; ++i) fx[i] += fr[i];
                    d[k] = narrow(fx, E{});  // h rounded once; the norm sees this value
                    if (in_row(k)) store_stream(hr + vpos(k), d[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                float f[V];
                widen(d[k], f, E{});
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < V; ++i) s += f[i] * f[i];
                ss += in_row(k) ? s : 0.f;
                if constexpr (QT != 0) {
                    float fw[V];
                    widen(wv[k], fw, E{});
                    float m = 0.f;
#pragma unroll
                    for (int i = 0; i < V; ++i) m = fmaxf(m, fabsf(f[i] * fw[i]));
                    mx = in_row(k) ? fmaxf(mx, m) : mx;
                }
            }
        }
        ss = group_sum<LPR>(ss);
        if constexpr (QT != 0) mx = group_max<LPR>(mx);
        if constexpr (WPR > 1) {
            if ((threadIdx.x & 63) == 0) {
                part[it & 1][wave] = ss;
                if constexpr (QT != 0) mpart[it & 1][wave] = mx;
            }
            __syncthreads();
            ss = 0.f;
#pragma unroll
            for (int i = 0; i < WPR; ++i) ss += part[it & 1][slot * WPR + i];
            if constexpr (QT != 0) {
                mx = 0.f;
#pragma unroll
                for (int i = 0; i < WPR; ++i) mx = fmaxf(mx, mpart[it & 1][slot * WPR + i]);
            }
        }
        if (valid && QT != 0) {
            const float r = rsqrtf(ss / a.hidden_f + a.eps);
            const float inv = mx > 0.f ? quant_max<QT>() / mx : 0.f;
            if (lane_row == 0) a.scale[row] = r * mx / quant_max<QT>();
            void* qr = static_cast<unsigned char*>(a.out) + row * static_cast<int64_t>(nvec) * V;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                if (!in_row(k)) continue;
                float f[V], fw[V];
                widen(d[k], f, E{});
                widen(wv[k], fw, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) f[i] = (f[i] * fw[i]) * inv;
                store_codes<QT>(qr, vpos(k), f, E{});
            }
        } else if (valid) {
            const float r = rsqrtf(ss / a.hidden_f + a.eps);
            u32x4* outr = static_cast<u32x4*>(a.out) + row * nvec;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                if (!in_row(k)) continue;
                float f[V], fw[V];
                widen(d[k], f, E{});
                if constexpr (WRES)
                    widen(wv[k], fw, E{});
                else if (use_lds)
                    widen(wlds[vpos(k)], fw, E{});
                else
                    widen(load_keep(wr + vpos(k)), fw, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) f[i] = f[i] * r * fw[i];
                store_stream(outr + vpos(k), narrow(f, E{}));
            }
        }
    }
}

// ---------------------------------------------------------------- any-alignment vector path

// A 16-byte vector at any element alignment.  The HSA ABI runs gfx950 in
// unaligned-access mode, so a global load or store of 16 bytes needs only the
// alignment of the access's own elements; the compiler then issues one
// global_load/store_dwordx4 as for an aligned vector.
typedef u32x4 u32x4_any2 __attribute__((aligned(2)));
typedef unsigned u32_any2 __attribute__((aligned(2)));

__device__ __forceinline__ u32x4 load_stream_any(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_any2*>(p));
}
__device__ __forceinline__ u32x4 load_keep_any(const char* p) { return *reinterpret_cast<const u32x4_any2*>(p); }
__device__ __forceinline__ void store_stream_any(char* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_any2*>(p));
}

// The 16 bytes of a vector at a 4-byte-aligned address except its first
// element slot (two bytes): the shifted frame's first vector, whose first slot
// lies before the row.
__device__ __forceinline__ void store_after_first_slot(char* p, u32x4 v) {
    *reinterpret_cast<uint16_t*>(p + 2) = static_cast<uint16_t>(v[0] >> 16);
    unsigned* q = reinterpret_cast<unsigned*>(p + 4);
    q[0] = v[1];
    q[1] = v[2];
    q[2] = v[3];
}

// Codes of one input vector at any byte offset: 8 bytes for bf16, 4 for fp32.
typedef u32x2 u32x2_any1 __attribute__((aligned(1)));
typedef unsigned u32_any1 __attribute__((aligned(1)));
template <int QT>
__device__ __forceinline__ void store_codes_any(char* p, const float (&t)[8], Bf16) {
    u32x2 c;
    c[0] = quant_pack4<QT>(t[0], t[1], t[2], t[3]);
    c[1] = quant_pack4<QT>(t[4], t[5], t[6], t[7]);
    __builtin_nontemporal_store(c, reinterpret_cast<u32x2_any1*>(p));
}
// The shifted frame's first vector of codes: every code but the first, whose
// slot lies before the row.
template <int QT>
__device__ __forceinline__ void store_codes_after_first(char* p, const float (&t)[8]) {
    const unsigned c0 = quant_pack4<QT>(t[0], t[1], t[2], t[3]);
    const unsigned c1 = quant_pack4<QT>(t[4], t[5], t[6], t[7]);
#pragma unroll
    for (int b = 1; b < 4; ++b) p[b] = static_cast<char>(c0 >> (8 * b));
#pragma unroll
    for (int b = 0; b < 4; ++b) p[4 + b] = static_cast<char>(c1 >> (8 * b));
}
template <int QT>
__device__ __forceinline__ void store_codes_any(char* p, const float (&t)[4], F32) {
    __builtin_nontemporal_store(quant_pack4<QT>(t[0], t[1], t[2], t[3]), reinterpret_cast<u32_any1*>(p));
}

// Rows of any width and any element alignment (every form): a row of H
// elements is H / V full 16-byte vectors, moved at whatever alignment the row
// starts at, and then H % V tail elements moved one by one.  Lane l of a row
// owns vectors l, l + 64*WPR, ... (VPL of them) and, if l < H % V, tail
// element l.  Nothing is written outside the row, nor read past a row's end
// or the tensor's.  One row per workgroup at a time; otherwise the vector
// path's reduction, rounding and output order.  The quantised forms (QT) hold
// the weight slice from the start, as on the vector path, and write their
// codes at the row's byte offset in the code tensor.
//
// Shifted frame (a.frame; bf16 normalised output, masked launches): 16-byte
// accesses 2 bytes past a 4-byte boundary run far slower on gfx950 than
// 4-byte-aligned ones, so a row that starts there is moved as the virtual row
// of H + 1 elements one slot earlier, which starts 4-byte aligned.  The
// virtual first slot is the two bytes before the row, in the same 4-byte word
// as the row's first element: it is read, zeroed, and never written.  The
// weight keeps its own alignment: each virtual vector takes the weight's own
// vector and the two elements before it, shifted up one slot in registers.
template <class E, int WPR, int VPL, bool MASKED, bool FUSED, int QT = 0>
__global__ void __launch_bounds__(max_threads<WPR>()) rms_any_kernel(const RowArgs a) {
    using S = typename E::scalar;
    constexpr int LANES = 64 * WPR;
    constexpr int V = E::kVec;
    constexpr int NR = FUSED ? VPL : 1;
    const int wave = wave_id();
    const int lane = static_cast<int>(threadIdx.x);
    constexpr bool kFrame = MASKED && sizeof(S) == 2;
    const int nvec = a.units;  // full vectors per row
    const int tail = a.tail;
    const int64_t row_elems = static_cast<int64_t>(nvec) * V + tail;
    const int64_t row_bytes = row_elems * static_cast<int64_t>(sizeof(S));
    __shared__ float part[2][16];
    __shared__ float mpart[QT ? 2 : 1][QT ? 16 : 1];

    // per row: sh = 1 in the shifted frame, nv full vectors, tl tail elements
    int sh = 0, nv = nvec, tl = tail;
    auto voff = [&](int k) {
        const int v = k * LANES + lane;
        return static_cast<int64_t>(MASKED ? (v < nv ? v : nv - 1) : v) * 16;
    };
    auto in_row = [&](int k) { return !MASKED || k * LANES + lane < nv; };
    auto toff = [&]() { return (static_cast<int64_t>(nv) * V + lane) * static_cast<int64_t>(sizeof(S)); };
    const char* wr = static_cast<const char*>(a.w);
    const int64_t wbytes = row_elems * static_cast<int64_t>(sizeof(S));
    // Weight access in the shifted frame, without branches (a load inside a
    // branch makes the compiler wait for every load in flight where the
    // branch ends).  A virtual vector takes the weight's own vector at byte
    // offset wo moved up one element behind the 4 bytes before it (0 for the
    // first).  The last virtual vector of an H = 7 (mod 8) row would take a
    // vector ending 2 bytes past the weight ("over"): the 16 bytes that end at
    // the weight's end are already its virtual vector.
    auto over_end = [&](int64_t wo) { return kFrame && wo + 16 > wbytes; };
    auto weight_vec = [&](int64_t wo) { return load_keep_any(wr + (over_end(wo) ? wbytes - 16 : wo)); };
    auto weight_before = [&](int64_t wo) {
        const unsigned b = *reinterpret_cast<const u32_any2*>(wr + (wo >= 4 ? wo - 4 : 0));
        return wo >= 4 ? b : 0u;
    };
    auto shift_weight = [&](u32x4 w, unsigned b, bool over) {
        u32x4 r;
        r[0] = __builtin_amdgcn_alignbyte(w[0], b, 2);
        r[1] = __builtin_amdgcn_alignbyte(w[1], w[0], 2);
        r[2] = __builtin_amdgcn_alignbyte(w[2], w[1], 2);
        r[3] = __builtin_amdgcn_alignbyte(w[3], w[2], 2);
        return over ? w : r;
    };

    // Quantised forms hold the weight slice from the start: its own vectors
    // (and, in the shifted frame, the 4 bytes before each and the tail weight
    // of both frames), for every vector the longer virtual row can take.
    const int nvw = kFrame && a.frame ? static_cast<int>((row_elems + 1) / V) : nvec;
    auto woff = [&](int k) {
        const int v = k * LANES + lane;
        return static_cast<int64_t>(MASKED ? (v < nvw ? v : nvw - 1) : v) * 16;
    };
    u32x4 wv[QT ? VPL : 1];
    unsigned wb[QT && kFrame ? VPL : 1];
    float wt0 = 0.f, wt1 = 0.f;
    if constexpr (QT != 0) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t wo = woff(k);
            if (!over_end(wo)) {
                wv[k] = load_keep_any(wr + wo);
            } else {
                // the weight's vector H / 8 ends 2 bytes past the weight: its
                // last element (never used) is not read
                const u32_any2* p = reinterpret_cast<const u32_any2*>(wr + wo);
                wv[k][0] = p[0];
                wv[k][1] = p[1];
                wv[k][2] = p[2];
                wv[k][3] = *reinterpret_cast<const uint16_t*>(wr + wo + 12);
            }
            if constexpr (kFrame) wb[k] = a.frame && wo >= 4 ? *reinterpret_cast<const u32_any2*>(wr + wo - 4) : 0u;
        }
        const int64_t t0 = static_cast<int64_t>(nvec) * V + lane;       // tail element, unshifted row
        const int64_t t1 = static_cast<int64_t>(nvw) * V + lane - 1;    // and in the shifted frame
        if (lane < tail) wt0 = widen1(reinterpret_cast<const S*>(wr)[t0]);
        if (kFrame && a.frame && lane < (row_elems + 1) % V) wt1 = widen1(reinterpret_cast<const S*>(wr)[t1]);
    }
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const char* xrow = static_cast<const char*>(a.x) + row * row_bytes;
        if constexpr (kFrame) {
            sh = a.frame && (reinterpret_cast<uintptr_t>(xrow) & 2) ? 1 : 0;
            nv = static_cast<int>((row_elems + sh) / V);
            tl = static_cast<int>((row_elems + sh) % V);
        }
        const int64_t back = sh * static_cast<int64_t>(sizeof(S));  // virtual row start, bytes before the row
        const bool has_tail = lane < tl;
        const char* xr = xrow - back;
        u32x4 d[VPL], rv[NR];
#pragma unroll
        for (int k = 0; k < VPL; ++k) d[k] = load_stream_any(xr + voff(k));
        if (sh && lane == 0) d[0][0] &= 0xffff0000u;  // the slot before the row
        float xt = 0.f;
        if (has_tail) xt = widen1(*reinterpret_cast<const S*>(xr + toff()));
        if constexpr (FUSED) {
            const char* rr = static_cast<const char*>(a.res) + row * row_bytes - back;
#pragma unroll
            for (int k = 0; k < VPL; ++k) rv[k] = load_stream_any(rr + voff(k));
            if (sh && lane == 0) rv[0][0] &= 0xffff0000u;
            char* hr = static_cast<char*>(a.h) + row * row_bytes - back;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                float fx[V], fr[V];
                widen(d[k], fx, E{});
                widen(rv[k], fr, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) fx[i] += fr[i];
                d[k] = narrow(fx, E{});  // h rounded once; the norm sees this value
                if (!in_row(k)) continue;
                if (k == 0 && sh && lane == 0)
                    store_after_first_slot(hr, d[k]);
                else
                    store_stream_any(hr + voff(k), d[k]);
            }
            if (has_tail) {
                const S ht = narrow1(xt + widen1(*reinterpret_cast<const S*>(rr + toff())), E{});
                *reinterpret_cast<S*>(hr + toff()) = ht;
                xt = widen1(ht);
            }
        }
        const float wt = sh ? wt1 : wt0;
        float ss = xt * xt;
        float mx = QT != 0 ? fabsf(xt * wt) : 0.f;
        auto qweight = [&](int k) {  // quantised forms: this row's weight vector k
            if constexpr (QT != 0 && kFrame) return sh ? shift_weight(wv[k], wb[k], false) : wv[k];
            return wv[k];
        };
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float f[V];
            widen(d[k], f, E{});
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) s += f[i] * f[i];
            ss += in_row(k) ? s : 0.f;
            if constexpr (QT != 0) {
                float fw[V];
                widen(qweight(k), fw, E{});
                float m = 0.f;
#pragma unroll
                for (int i = 0; i < V; ++i) m = fmaxf(m, fabsf(f[i] * fw[i]));
                mx = in_row(k) ? fmaxf(mx, m) : mx;
            }
        }
        ss = wave_sum(ss);
        if constexpr (QT != 0) mx = wave_max(mx);
        if constexpr (WPR > 1) {
            if ((threadIdx.x & 63) == 0) {
                part[it & 1][wave] = ss;
                if constexpr (QT != 0) mpart[it & 1][wave] = mx;
            }
            __syncthreads();
            ss = 0.f;
#pragma unroll
            for (int i = 0; i < WPR; ++i) ss += part[it & 1][i];
            if constexpr (QT != 0) {
                mx = 0.f;
#pragma unroll
                for (int i = 0; i < WPR; ++i) mx = fmaxf(mx, mpart[it & 1][i]);
            }
        }
        const float r = rsqrtf(ss / a.hidden_f + a.eps);
        if constexpr (QT != 0) {
            const float inv = mx > 0.f ? quant_max<QT>() / mx : 0.f;
            if (lane == 0) a.scale[row] = r * mx / quant_max<QT>();
            char* qr = static_cast<char*>(a.out) + row * row_elems - sh;  // one byte per element
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                if (!in_row(k)) continue;
                float f[V], fw[V];
                widen(d[k], f, E{});
                widen(qweight(k), fw, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) f[i] = (f[i] * fw[i]) * inv;
                if constexpr (kFrame) {
                    if (k == 0 && sh && lane == 0) {
                        store_codes_after_first<QT>(qr, f);
                        continue;
                    }
                }
                store_codes_any<QT>(qr + voff(k) / static_cast<int64_t>(sizeof(S)), f, E{});
            }
            if (has_tail) qr[static_cast<int64_t>(nv) * V + lane] = static_cast<char>(quant_code<QT>((xt * wt) * inv));
            continue;
        }
        char* outr = static_cast<char*>(a.out) + row * row_bytes - back;
        const char* wv0 = wr - back;  // the weight one element back in the shifted frame
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (!in_row(k)) continue;
            const bool first = k == 0 && sh && lane == 0;
            // shifted frame: the weight's own vector v and the last two
            // elements before it, moved up one slot in registers (both loads
            // at the weight's alignment)
            const u32x4 wa = weight_vec(voff(k));
            const u32x4 wk = sh ? shift_weight(wa, weight_before(voff(k)), over_end(voff(k))) : wa;
            float f[V], fw[V];
            widen(d[k], f, E{});
            widen(wk, fw, E{});
#pragma unroll
            for (int i = 0; i < V; ++i) f[i] = f[i] * r * fw[i];
            if (first)
                store_after_first_slot(outr, narrow(f, E{}));
            else
                store_stream_any(outr + voff(k), narrow(f, E{}));
        }
        if (has_tail) {
            const float wt = widen1(*reinterpret_cast<const S*>(wv0 + toff()));
            *reinterpret_cast<S*>(outr + toff()) = narrow1(xt * r * wt, E{});
        }
    }
}

// ---------------------------------------------------------------- element path

// One element per access; lane l of a row owns elements l, l + 64*WPR, ...
// (each wave instruction covers 64 consecutive elements).  Always masked.
template <class E, int WPR, int EPL, bool FUSED, int QT = 0>
__global__ void __launch_bounds__(max_threads<WPR>()) rms_elem_kernel(const RowArgs a) {
    using S = typename E::scalar;
    constexpr int LANES = 64 * WPR;
    const int wave = wave_id();
    const int slot = wave / WPR;
    const int lane_row = static_cast<int>(threadIdx.x) - slot * LANES;
    const int H = a.units;
    __shared__ float part[2][16];
    __shared__ float mpart[QT ? 2 : 1][QT ? 16 : 1];
    float wq[QT ? EPL : 1];  // quantised forms: this lane's weights, loaded once
    if constexpr (QT != 0) {
        const S* wr = static_cast<const S*>(a.w);
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
            const int j = k * LANES + lane_row;
            wq[k] = widen1(wr[j < H ? j : H - 1]);
        }
    }

    int it = 0;
    for (int64_t g = blockIdx.x; g < a.n_groups; g += gridDim.x, ++it) {
        const int64_t row = g * a.rows_per_block + slot;
        const bool valid = row < a.rows;
        const int64_t base = row * H;
        float d[EPL];
        float ss = 0.f, mx = 0.f;
        if (valid) {
            const S* xr = static_cast<const S*>(a.x) + base;
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                const int j = k * LANES + lane_row;
                d[k] = widen1(xr[j < H ? j : H - 1]);
            }
            if constexpr (FUSED) {
                const S* rr = static_cast<const S*>(a.res) + base;
                S* hr = static_cast<S*>(a.h) + base;
#pragma unroll
                for (int k = 0; k < EPL; ++k) {
                    const int j = k * LANES + lane_row;
                    const S hv = narrow1(d[k] + widen1(rr[j < H ? j : H - 1]), E{});
                    d[k] = widen1(hv);
                    if (j < H) hr[j] = hv;
                }
            }
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                const int j = k * LANES + lane_row;
                ss += j < H ? d[k] * d[k] : 0.f;
                if constexpr (QT != 0) mx = j < H ? fmaxf(mx, fabsf(d[k] * wq[k])) : mx;
            }
        }
        ss = wave_sum(ss);
        if constexpr (QT != 0) mx = wave_max(mx);
        if constexpr (WPR > 1) {
            if ((threadIdx.x & 63) == 0) {
                part[it & 1][wave] = ss;
                if constexpr (QT != 0) mpart[it & 1][wave] = mx;
            }
            __syncthreads();
            ss = 0.f;
#pragma unroll
            for (int i = 0; i < WPR; ++i) ss += part[it & 1][slot * WPR + i];
            if constexpr (QT != 0) {
                mx = 0.f;
#pragma unroll
                for (int i = 0; i < WPR; ++i) mx = fmaxf(mx, mpart[it & 1][slot * WPR + i]);
            }
        }
        if (valid && QT != 0) {
            const float r = rsqrtf(ss / a.hidden_f + a.eps);
            const float inv = mx > 0.f ? quant_max<QT>() / mx : 0.f;
            if (lane_row == 0) a.scale[row] = r * mx / quant_max<QT>();
            unsigned char* qr = static_cast<unsigned char*>(a.out) + base;
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                const int j = k * LANES + lane_row;
                if (j < H) qr[j] = static_cast<unsigned char>(quant_code<QT>((d[k] * wq[k]) * inv));
            }
        } else if (valid) {
            const float r = rsqrtf(ss / a.hidden_f + a.eps);
            const S* wr = static_cast<const S*>(a.w);
            S* outr = static_cast<S*>(a.out) + base;
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                const int j = k * LANES + lane_row;
                if (j < H) outr[j] = narrow1(d[k] * r * widen1(wr[j]), E{});
            }
        }
    }
}

// ---------------------------------------------------------------- register + LDS path

// Rows wider than any register-resident configuration, still read once and
// written once (the one-read-per-row point of the gollamago README, "RMSNorm
// 优化（TileLang）"): 1024 lanes per row; the first 1024 * RV vectors of the
// row stay in VGPRs as on the vector path (lane l owns vectors l, l + 1024,
// ...), and the remaining nl = units - 1024 * RV vectors are staged in
// dynamic LDS, nl * 16 bytes (up to nearly the 160 KiB a gfx950 workgroup
// can take).  Lane l stages vectors R + l, R + l + 1024, ... in LDS slots l,
// l + 1024, ...: it alone writes and reads its slots, so the staged part
// needs no barrier of its own.  The staged vectors pass through registers CH
// per lane at a time, issued right after the register part's loads; their
// squares join the same per-lane sum.  The reduction (one LDS slot per wave,
// one barrier, every wave adding the 16 slots in order) and the rounding are
// the vector path's.  Aligned rows only, one row per workgroup at a time.
template <class E, int RV, int CH, bool FUSED>
__global__ void __launch_bounds__(1024) rms_stage_kernel(const RowArgs a) {
    constexpr int LANES = 1024;
    constexpr int V = E::kVec;
    constexpr int R = LANES * RV;
    const int lane = static_cast<int>(threadIdx.x);
    const int wave = wave_id();
    const int nvec = a.units;
    const int nl = nvec - R;                     // staged vectors, > 0
    const int ml = (nl + LANES - 1) / LANES;     // staged slots per lane (uniform)
    __shared__ float part[2][16];
    extern __shared__ u32x4 stage[];
    const u32x4* wr = static_cast<const u32x4*>(a.w);

    auto add_round = [&](u32x4 xv, u32x4 rv) {  // h = round(x + residual)
        float fx[V], fr[V];
        widen(xv, fx, E{});
        widen(rv, fr, E{});
#pragma unroll
        for (int i = 0; i < V; ++i) fx[i] += fr[i];
        return narrow(fx, E{});
    };
    auto sumsq = [&](u32x4 v) {
        float f[V];
        widen(v, f, E{});
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) s += f[i] * f[i];
        return s;
    };
    auto scaled = [&](u32x4 v, u32x4 w, float r) {
        // widen the packed vector again here: without this (empty) register
        // constraint the compiler reuses the fp32 values of the sum of squares
        // and keeps them live across the barrier, twice the registers of the
        // packed row, and spills
        asm volatile("" : "+v"(v));
        float f[V], fw[V];
        widen(v, f, E{});
        widen(w, fw, E{});
#pragma unroll
        for (int i = 0; i < V; ++i) f[i] = f[i] * r * fw[i];
        return narrow(f, E{});
    };

    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const u32x4* xr = static_cast<const u32x4*>(a.x) + row * nvec;
        const u32x4* rr = static_cast<const u32x4*>(a.res) + row * nvec;  // fused only
        u32x4* hr = static_cast<u32x4*>(a.h) + row * nvec;               // fused only
        u32x4 d[RV], rv[FUSED ? RV : 1];
#pragma unroll
        for (int k = 0; k < RV; ++k) d[k] = load_stream(xr + k * LANES + lane);
        if constexpr (FUSED) {
#pragma unroll
            for (int k = 0; k < RV; ++k) rv[k] = load_stream(rr + k * LANES + lane);
        }
        float ss = 0.f;
        for (int m0 = 0; m0 < ml; m0 += CH) {
            u32x4 t[CH], tr[FUSED ? CH : 1];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int u = (m0 + c) * LANES + lane;
                if (u < nl) {
                    t[c] = load_stream(xr + R + u);
                    if constexpr (FUSED) tr[c] = load_stream(rr + R + u);
                }
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int u = (m0 + c) * LANES + lane;
                if (u < nl) {
                    if constexpr (FUSED) {
                        t[c] = add_round(t[c], tr[c]);  // h rounded once; the norm sees this value
                        store_stream(hr + R + u, t[c]);
                    }
                    ss += sumsq(t[c]);
                    stage[u] = t[c];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < RV; ++k) {
            if constexpr (FUSED) {
                d[k] = add_round(d[k], rv[k]);
                store_stream(hr + k * LANES + lane, d[k]);
            }
            ss += sumsq(d[k]);
        }
        ss = wave_sum(ss);
        if ((lane & 63) == 0) part[it & 1][wave] = ss;
        __syncthreads();
        ss = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += part[it & 1][i];
        const float r = rsqrtf(ss / a.hidden_f + a.eps);
        u32x4* outr = static_cast<u32x4*>(a.out) + row * nvec;
#pragma unroll
        for (int k = 0; k < RV; ++k)
            store_stream(outr + k * LANES + lane, scaled(d[k], load_keep(wr + k * LANES + lane), r));
        for (int m = 0; m < ml; ++m) {
            const int u = m * LANES + lane;
            if (u < nl) store_stream(outr + R + u, scaled(stage[u], load_keep(wr + R + u), r));
        }
    }
}

// ---------------------------------------------------------------- two-pass path

// One row per workgroup iteration, blockDim.x lanes striding over the row.
// Pass 1 reads x (and residual) and sums squares of x (of the rounded h);
// pass 2 reads them again, recomputes h, and writes h and y.  Pass 1 writes
// nothing, so exact input/output aliasing stays safe: every element is read
// and then written by the same thread.
template <class E, bool VEC, bool FUSED, int QT = 0>
__global__ void __launch_bounds__(1024) rms_twopass_kernel(const RowArgs a) {
    using S = typename E::scalar;
    constexpr int V = E::kVec;
    const int wave = wave_id();
    const int nwaves = static_cast<int>(blockDim.x) >> 6;
    const int n = a.units;
    __shared__ float part[2][16];
    __shared__ float mpart[QT ? 2 : 1][QT ? 16 : 1];

    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const int64_t base = row * n;
        float ss = 0.f, mx = 0.f;
        for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
            if constexpr (VEC) {
                float f[V];
                widen(load_stream(static_cast<const u32x4*>(a.x) + base + j), f, E{});
                if constexpr (FUSED) {
                    float fr[V];
                    widen(load_stream(static_cast<const u32x4*>(a.res) + base + j), fr, E{});
#pragma unroll
                    for (int i = 0; i < V; ++i) f[i] += fr[i];
                    widen(narrow(f, E{}), f, E{});
                }
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < V; ++i) s += f[i] * f[i];
                ss += s;
                if constexpr (QT != 0) {
                    float fw[V];
                    widen(load_keep(static_cast<const u32x4*>(a.w) + j), fw, E{});
#pragma unroll
                    for (int i = 0; i < V; ++i) mx = fmaxf(mx, fabsf(f[i] * fw[i]));
                }
            } else {
                float f = widen1(static_cast<const S*>(a.x)[base + j]);
                if constexpr (FUSED) f = widen1(narrow1(f + widen1(static_cast<const S*>(a.res)[base + j]), E{}));
                ss += f * f;
                if constexpr (QT != 0) mx = fmaxf(mx, fabsf(f * widen1(static_cast<const S*>(a.w)[j])));
            }
        }
        ss = wave_sum(ss);
        if constexpr (QT != 0) mx = wave_max(mx);
        if ((threadIdx.x & 63) == 0) {
            part[it & 1][wave] = ss;
            if constexpr (QT != 0) mpart[it & 1][wave] = mx;
        }
        __syncthreads();
        ss = 0.f;
        for (int i = 0; i < nwaves; ++i) ss += part[it & 1][i];
        const float r = rsqrtf(ss / a.hidden_f + a.eps);
        if constexpr (QT != 0) {
            mx = 0.f;
            for (int i = 0; i < nwaves; ++i) mx = fmaxf(mx, mpart[it & 1][i]);
            const float inv = mx > 0.f ? quant_max<QT>() / mx : 0.f;
            if (threadIdx.x == 0) a.scale[row] = r * mx / quant_max<QT>();
            for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
                if constexpr (VEC) {
                    float f[V], fw[V];
                    u32x4 xv = load_stream(static_cast<const u32x4*>(a.x) + base + j);
                    if constexpr (FUSED) {
                        float fr[V];
                        widen(xv, f, E{});
                        widen(load_stream(static_cast<const u32x4*>(a.res) + base + j), fr, E{});
#pragma unroll
                        for (int i = 0; i < V; ++i) f[i] += fr[i];
                        xv = narrow(f, E{});
                        store_stream(static_cast<u32x4*>(a.h) + base + j, xv);
                    }
                    widen(xv, f, E{});
                    widen(load_keep(static_cast<const u32x4*>(a.w) + j), fw, E{});
#pragma unroll
                    for (int i = 0; i < V; ++i) f[i] = (f[i] * fw[i]) * inv;
                    store_codes<QT>(static_cast<unsigned char*>(a.out) + base * V, static_cast<int>(j), f, E{});
                } else {
                    float f = widen1(static_cast<const S*>(a.x)[base + j]);
                    if constexpr (FUSED) {
                        const S hv = narrow1(f + widen1(static_cast<const S*>(a.res)[base + j]), E{});
                        static_cast<S*>(a.h)[base + j] = hv;
                        f = widen1(hv);
                    }
                    static_cast<unsigned char*>(a.out)[base + j] =
                        static_cast<unsigned char>(quant_code<QT>((f * widen1(static_cast<const S*>(a.w)[j])) * inv));
                }
            }
            continue;
        }
        for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
            if constexpr (VEC) {
                float f[V], fw[V];
                u32x4 xv = load_stream(static_cast<const u32x4*>(a.x) + base + j);
                if constexpr (FUSED) {
                    float fr[V];
                    widen(xv, f, E{});
                    widen(load_stream(static_cast<const u32x4*>(a.res) + base + j), fr, E{});
#pragma unroll
                    for (int i = 0; i < V; ++i) f[i] += fr[i];
                    xv = narrow(f, E{});
                    store_stream(static_cast<u32x4*>(a.h) + base + j, xv);
                }
                widen(xv, f, E{});
                widen(load_keep(static_cast<const u32x4*>(a.w) + j), fw, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) f[i] = f[i] * r * fw[i];
                store_stream(static_cast<u32x4*>(a.out) + base + j, narrow(f, E{}));
            } else {
                float f = widen1(static_cast<const S*>(a.x)[base + j]);
                if constexpr (FUSED) {
                    const S hv = narrow1(f + widen1(static_cast<const S*>(a.res)[base + j]), E{});
                    static_cast<S*>(a.h)[base + j] = hv;
                    f = widen1(hv);
                }
                static_cast<S*>(a.out)[base + j] = narrow1(f * r * widen1(static_cast<const S*>(a.w)[j]), E{});
            }
        }
    }
}

}  // namespace mbr
