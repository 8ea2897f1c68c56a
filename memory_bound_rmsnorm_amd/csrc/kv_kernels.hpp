// KV RMSNorm + RoPE + cache scatter for gfx950 (CDNA4, wave64): the fused
// KV-cache maintenance operator the TileLang tutorial ch. 02 (sections 1.2 and
// 4.2) cites from CANN (aclnnKvRmsNormRopeCache).  Each row of kv (one token,
// one head) is split along its tail axis:
//
//   left  norm_dim: y = x * rsqrt(mean(x^2) + eps) * gamma   -> norm_cache[slot]
//   right rope_dim: each pair (a, b) at the token's position p becomes
//                   (a*cos - b*sin, a*sin + b*cos), cos/sin from fp32 tables
//                   [max_pos, rope_dim/2] (xserv rope.cu, phase 4)  -> rope_cache[slot]
//
// with pairs of adjacent elements (2i, 2i+1) (STYLE 1) or of the two halves
// (i, i + rope_dim/2) (STYLE 0).  The slot is the token's cache row, as a paged
// cache's block table resolves it.  A token whose slot or position is out of
// range (negative included) writes nothing; the check is wave-uniform and
// precedes every load and store of the row, so no access can leave the
// buffers.  fp32 math, one rounding per output.
//
// One wave per row: no LDS, no barrier.  The norm part is spread over the 64
// lanes as 16-byte vectors (lane l owns vectors l, l + 64, ...); the rotated
// part is handled by the first lanes, one 16-byte vector each (adjacent pairs)
// or one vector from each half (halves), with the matching table entries
// loaded as fp32 vectors.  The op is a gather/scatter stream: HBM-bound.
#pragma once

#include "rmsnorm_kernels.hpp"

namespace mbr {

struct KvArgs {
    const void* kv;
    const void* gamma;
    const float* cos_t;
    const float* sin_t;
    const int32_t* pos;
    const int64_t* slots;
    void* nc;  // norm cache [num_slots, heads, norm_dim]
    void* rc;  // rope cache [num_slots, heads, rope_dim]
    int64_t rows;      // tokens * heads
    int64_t max_pos;
    int64_t num_slots;
    int32_t heads;
    int32_t norm_dim;  // elements
    int32_t rope_dim;  // elements (even)
    float norm_dim_f;
    float eps;
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Table entries [j0, j0 + V/2) (adjacent pairs, one vector) or [j0, j0 + V)
// (halves: V pairs across two vectors), as fp32.
template <int N>
__device__ __forceinline__ void load_table(const float* row, int j0, float (&out)[N]) {
    static_assert(N % 2 == 0, "");
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int q = 0; q < N / 4; ++q) {
            const f32x4v v = *reinterpret_cast<const f32x4v*>(row + j0 + 4 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i) out[4 * q + i] = v[i];
        }
    } else {
        typedef float f32x2v __attribute__((ext_vector_type(2)));
        const f32x2v v = *reinterpret_cast<const f32x2v*>(row + j0);
        out[0] = v[0];
        out[1] = v[1];
    }
}

// One row per wave.  The row's kv loads depend only on the row index, so
// they are issued before the token's slot and position are read; the
// range check on those (wave-uniform) then guards every table read and every
// cache store, and a skipped token's loaded values are simply dropped.
//
// LPR < 64: 64 / LPR rows share a wave, each owning an aligned group of LPR
// lanes (8, 16 or 32; the rotated part must fit them).  A group past the last
// row loads the last row again; the range check is then per group, taken
// after the group sum (which every lane of the wave joins) and before the
// stores, and a skipped group reads no table.
template <class E, int NVPL, bool MASKED, int STYLE, int LPR = 64>
__global__ void __launch_bounds__(256) kv_vec_kernel(const KvArgs a) {
    constexpr int V = E::kVec;
    constexpr int NT = STYLE == 1 ? V / 2 : V;  // table entries per rope lane
    constexpr int G = 64 / LPR;                 // rows per wave
    const int lane = static_cast<int>(threadIdx.x) & (LPR - 1);
    const int grp = G > 1 ? (static_cast<int>(threadIdx.x) & 63) / LPR : 0;
    const int nv = a.norm_dim / V;               // norm vectors per row
    const int rv = a.rope_dim / V;               // rope vectors per row
    const int d_vec = nv + rv;                   // vectors per kv row
    const int half = a.rope_dim / 2;
    const int rlanes = STYLE == 1 ? rv : rv / 2; // lanes with rope work
    const bool rope_lane = lane < rlanes;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    auto vidx = [&](int k) {
        const int v = k * LPR + lane;
        return MASKED ? (v < nv ? v : nv - 1) : v;
    };
    auto in_row = [&](int k) { return !MASKED || k * LPR + lane < nv; };

    u32x4 gv[NVPL];
#pragma unroll
    for (int k = 0; k < NVPL; ++k) gv[k] = load_keep(static_cast<const u32x4*>(a.gamma) + vidx(k));

    for (int64_t base = (static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + wave_id()) * G; base < a.rows;
         base += waves * G) {
        const int64_t row0 = base + grp;
        const bool in_rows = G == 1 || row0 < a.rows;
        const int64_t row = in_rows ? row0 : a.rows - 1;
        const u32x4* xr = static_cast<const u32x4*>(a.kv) + row * d_vec;
        u32x4 xv[NVPL], ra, rb;
#pragma unroll
        for (int k = 0; k < NVPL; ++k) xv[k] = load_stream(xr + vidx(k));
        if (rope_lane) {
            ra = load_stream(xr + nv + lane);
            if (STYLE == 0) rb = load_stream(xr + nv + rlanes + lane);
        }
        const int64_t t = row / a.heads;
        const int64_t h = row - t * a.heads;
        const int64_t slot = a.slots[t];
        const int64_t p = a.pos[t];
        const bool ok = in_rows && slot >= 0 && slot < a.num_slots && p >= 0 && p < a.max_pos;
        if constexpr (G == 1) {
            if (!ok) continue;  // wave-uniform
        }
        float ct[NT], st[NT];
        if (rope_lane && (G == 1 || ok)) {
            load_table(a.cos_t + p * half, lane * NT, ct);
            load_table(a.sin_t + p * half, lane * NT, st);
        }
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < NVPL; ++k) {
            float f[V];
            widen(xv[k], f, E{});
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) s += f[i] * f[i];
            ss += in_row(k) ? s : 0.f;
        }
        const float r = rsqrtf(group_sum<LPR>(ss) / a.norm_dim_f + a.eps);
        if constexpr (G > 1) {
            if (!ok) continue;  // per lane group, after the group sum
        }
        u32x4* ncr = static_cast<u32x4*>(a.nc) + (slot * a.heads + h) * nv;
#pragma unroll
        for (int k = 0; k < NVPL; ++k) {
            if (!in_row(k)) continue;
            float f[V], fw[V];
            widen(xv[k], f, E{});
            widen(gv[k], fw, E{});
#pragma unroll
            for (int i = 0; i < V; ++i) f[i] = f[i] * r * fw[i];
            store_stream(ncr + k * LPR + lane, narrow(f, E{}));
        }
        if (rope_lane) {
            u32x4* rcr = static_cast<u32x4*>(a.rc) + (slot * a.heads + h) * rv;
            if constexpr (STYLE == 1) {
                float f[V];
                widen(ra, f, E{});
#pragma unroll
                for (int i = 0; i < V / 2; ++i) {
                    const float x0 = f[2 * i], x1 = f[2 * i + 1];
                    f[2 * i] = x0 * ct[i] - x1 * st[i];
                    f[2 * i + 1] = x0 * st[i] + x1 * ct[i];
                }
                store_stream(rcr + lane, narrow(f, E{}));
            } else {
                float fa[V], fb[V];
                widen(ra, fa, E{});
                widen(rb, fb, E{});
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const float x0 = fa[i], x1 = fb[i];
                    fa[i] = x0 * ct[i] - x1 * st[i];
                    fb[i] = x0 * st[i] + x1 * ct[i];
                }
                store_stream(rcr + lane, narrow(fa, E{}));
                store_stream(rcr + rlanes + lane, narrow(fb, E{}));
            }
        }
    }
}

// Any shape and element alignment: one wave per row, lanes stride over the
// elements (the norm part is read twice, the second time from cache).
template <class E, int STYLE>
__global__ void __launch_bounds__(256) kv_elem_kernel(const KvArgs a) {
    using S = typename E::scalar;
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int d = a.norm_dim + a.rope_dim;
    const int half = a.rope_dim / 2;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + wave_id(); row < a.rows;
         row += waves) {
        const int64_t t = row / a.heads;
        const int64_t h = row - t * a.heads;
        const int64_t slot = a.slots[t];
        const int64_t p = a.pos[t];
        if (slot < 0 || slot >= a.num_slots || p < 0 || p >= a.max_pos) continue;  // wave-uniform
        const S* xr = static_cast<const S*>(a.kv) + row * d;
        float ss = 0.f;
        for (int j = lane; j < a.norm_dim; j += 64) {
            const float v = widen1(xr[j]);
            ss += v * v;
        }
        const float r = rsqrtf(wave_sum(ss) / a.norm_dim_f + a.eps);
        S* ncr = static_cast<S*>(a.nc) + (slot * a.heads + h) * a.norm_dim;
        for (int j = lane; j < a.norm_dim; j += 64)
            ncr[j] = narrow1(widen1(xr[j]) * r * widen1(static_cast<const S*>(a.gamma)[j]), E{});
        S* rcr = static_cast<S*>(a.rc) + (slot * a.heads + h) * a.rope_dim;
        for (int j = lane; j < half; j += 64) {
            const int ia = STYLE == 1 ? 2 * j : j, ib = STYLE == 1 ? 2 * j + 1 : j + half;
            const float x0 = widen1(xr[a.norm_dim + ia]), x1 = widen1(xr[a.norm_dim + ib]);
            const float c = a.cos_t[p * half + j], s = a.sin_t[p * half + j];
            rcr[ia] = narrow1(x0 * c - x1 * s, E{});
            rcr[ib] = narrow1(x0 * s + x1 * c, E{});
        }
    }
}

}  // namespace mbr
