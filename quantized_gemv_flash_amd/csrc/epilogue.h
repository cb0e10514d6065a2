// epilogue.h -- reductions shared by the step's epilogue kernels and by the
// GEMV prologues that stand in for them at small batch sizes.  Both callers
// run the same functions with the same thread mapping, so a value is computed
// by the same operations in the same order whichever kernel produces it (a
// sequence's result does not depend on the batch it is in).
#pragma once

#include "rra_internal.h"

namespace rra {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// silu(g) u, rounded to fp32 (never fused into a consumer's add)
__device__ __forceinline__ float swiglu1(float g, float u) {
#pragma clang fp contract(off)
    return silu(g) * u;
}

// a = sum_s p[s * stride], c = sum_s q[s * stride], in split order.
__device__ __forceinline__ void sum_splits2(const float *__restrict__ p, const float *__restrict__ q,
                                            int split, long long stride, float &a, float &c) {
    a = 0.f;
    c = 0.f;
    for (int s0 = 0; s0 < split; s0 += 8) {
        float u[8], w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const size_t off = (size_t)min(s0 + j, split - 1) * stride;
            u[j] = p[off];
            w[j] = q[off];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            a += (s0 + j < split) ? u[j] : 0.f;
            c += (s0 + j < split) ? w[j] : 0.f;
        }
    }
}

// RoPE of the pair (a, c) by (cos, sin): (a cos - c sin, a sin + c cos),
// with explicit FMAs so that every kernel computes the same bits.
__device__ __forceinline__ void rope_pair(float &a, float &c, float cs, float sn) {
    const float ra = fmaf(a, cs, -(c * sn)), rc = fmaf(a, sn, c * cs);
    a = ra;
    c = rc;
}

__device__ __forceinline__ void load8(const float *p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(float *p, const float (&v)[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// One lane's 8 columns of the residual step: v = x + acc (acc the split sum
// of the block's output, when add), sq += v^2 in column order, gv = gamma v.
__device__ __forceinline__ void resid8(float (&v)[8], const float (&acc)[8], bool add,
                                       const float (&gamma)[8], float (&gv)[8], float &sq) {
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (add) v[e] += acc[e];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sq = fmaf(v[e], v[e], sq);
        gv[e] = gamma[e] * v[e];
    }
}

// Split sum of NV 8-column vectors (p[v] .. p[v] + 8) shared by the four
// waves of a 256-thread block: lane g of every wave works on the same group,
// wave q adds planes q, q + 4, q + 8, ... (8 / NV planes in flight per
// thread), and wave 0 then adds the other waves' sums in wave order (a fixed
// order: the result does not depend on timing).  All 256 threads must call
// it (it synchronises the block); the total is valid in wave 0.  `red` is
// 3 * 64 * NV * 8 floats of shared memory.
template <int NV>
__device__ __forceinline__ void group_split_sum(const float *const (&p)[NV], bool active,
                                                int split, long long stride,
                                                float (&acc)[NV][8], float *red) {
    const int gl = threadIdx.x & 63, q = threadIdx.x >> 6;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[v][e] = 0.f;
    if (active) {
        constexpr int UN = 8 / NV;
        for (int s0 = q; s0 < split; s0 += 4 * UN) {
            float4 a[UN][NV][2];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                const size_t off = (size_t)min(s0 + 4 * u, split - 1) * stride;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    a[u][v][0] = *reinterpret_cast<const float4 *>(p[v] + off);
                    a[u][v][1] = *reinterpret_cast<const float4 *>(p[v] + off + 4);
                }
            }
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                if (s0 + 4 * u >= split) continue;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    acc[v][0] += a[u][v][0].x; acc[v][1] += a[u][v][0].y;
                    acc[v][2] += a[u][v][0].z; acc[v][3] += a[u][v][0].w;
                    acc[v][4] += a[u][v][1].x; acc[v][5] += a[u][v][1].y;
                    acc[v][6] += a[u][v][1].z; acc[v][7] += a[u][v][1].w;
                }
            }
        }
    }
    if (q > 0) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[(((q - 1) * 64 + gl) * NV + v) * 8 + e] = acc[v][e];
    }
    __syncthreads();
    if (q == 0) {
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[v][e] += red[((r * 64 + gl) * NV + v) * 8 + e];
    }
}

// [head_dim] flash_decoding_attention_into, second pass: the output of query
// head h of sequence m from its splits' partials (part_o normalised outputs,
// part_lse log-sum-exps; the first min(L, nc_max) splits hold rows):
// sum_c e^(lse_c - max) o_c / sum_c e^(lse_c - max).  One wave; lane holds
// columns lane + 64 j in acc[j].  L == 0 leaves acc at 0.  ANY: the first
// loads are clamped to the allocated splits rather than to those that hold
// rows, so they need not wait for the length; the values of splits past the
// length (stale memory) are then selected away, not multiplied by 0; L is
// then the raw length, clamped to max_len here, after the loads.
template <int HD, bool ANY = false>
__device__ __forceinline__ void fd_combine(const float *__restrict__ part_o,
                                           const float *__restrict__ part_lse, int m, int h,
                                           int nq, int nc_max, int L, int lane,
                                           float (&acc)[HD / 64], int max_len = 0) {
    constexpr int PER = HD / 64;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    if (!ANY && L <= 0) return;
    const uint32_t len_raw = (uint32_t)L;
    const float *lse = part_lse + ((size_t)m * nq + h) * nc_max;
    const float *po = part_o + ((size_t)m * nq + h) * nc_max * HD;
    // Every load that does not depend on another is issued first: this
    // lane's lse (split `lane`; up to 64 splits stay in registers and are
    // read back by shuffles) and the first 16 splits' outputs.
    const int ncl = ANY ? nc_max : min(L, nc_max);  // splits the first loads may touch
    const float l0 = lse[min(lane, ncl - 1)];
    float v0[8][PER], v1[8][PER];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            v0[j][i] = po[(size_t)min(j, ncl - 1) * HD + lane + 64 * i];
            v1[j][i] = po[(size_t)min(8 + j, ncl - 1) * HD + lane + 64 * i];
        }
    if constexpr (ANY) {
        __builtin_amdgcn_sched_barrier(0);  // the loads above go out before the length is used
        L = (int)min(len_raw, (uint32_t)max_len);
    }
    const int nc = min(L, nc_max);  // splits that had rows
    float mx = lane < nc ? l0 : -INFINITY;
    for (int c = lane + 64; c < nc; c += 64) mx = fmaxf(mx, lse[c]);
    mx = wave_max(mx);
    float wsum = lane < nc ? expf(l0 - mx) : 0.f;
    for (int c = lane + 64; c < nc; c += 64) wsum += expf(lse[c] - mx);
    wsum = wave_sum(wsum);
    // splits 8 at a time, in split order
    auto add8 = [&](int c0, const float (&v)[8][PER]) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int cj = min(c0 + j, nc - 1);
            const float lc = cj < 64 ? __shfl(l0, cj, 64) : lse[cj];
            w[j] = (c0 + j < nc) ? expf(lc - mx) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < PER; ++i)
                acc[i] = fmaf(w[j], (!ANY || c0 + j < nc) ? v[j][i] : 0.f, acc[i]);
    };
    add8(0, v0);
    if (nc > 8) add8(8, v1);
    for (int c0 = 16; c0 < nc; c0 += 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < PER; ++i)
                v0[j][i] = po[(size_t)min(c0 + j, nc - 1) * HD + lane + 64 * i];
        add8(c0, v0);
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] /= wsum;
    if constexpr (ANY)  // no early exit: the loads above must not wait for L
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] = L > 0 ? acc[j] : 0.f;
}

// (v2, i2) beats (v1, i1) if larger, or equal with a lower index.  NaN never
// wins.  The result of combining a set of candidates is the same in any order.
__device__ __forceinline__ void arg_combine(float &v1, uint32_t &i1, float v2, uint32_t i2) {
    if (v2 > v1 || (v2 == v1 && i2 < i1)) {
        v1 = v2;
        i1 = i2;
    }
}

}  // namespace
}  // namespace rra
