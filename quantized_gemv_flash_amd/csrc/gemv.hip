// gemv.hip -- weights-once dequantising batched GEMV (y = W x for M inputs).
//
// [batched_forward] forward_batched_to_token_ids: every weight block is read
// and dequantised once for all M inputs.
//
// Q8/Q4 path (gfx950 matrix cores).  One v_mfma_f32_16x16x32_f16 takes a
// 16-row x 32-column slab of W -- exactly one quantisation block per row -- and
// a 32 x 16 slab of X^T (16 sequences).  The quantised values q (Q8) or q - 8
// (Q4) are small integers, exact in fp16; the block scale is applied in fp32
// after the block's products, so W is never rounded.  X is fp32 and enters as
// x = hi + lo with hi = fp16(x), lo = fp16(x - hi): two MFMAs per slab give
// ~22 significant bits, i.e. fp32-like dot products (products are exact in the
// fp32 accumulator: 11-bit x 11-bit mantissas).
//
// Data movement.  Weights are pre-tiled (rra_repack_weight): one 16-row x KT
// tile is 1 KiB of values (each lane of a wave loads 16 contiguous bytes that
// already sit in MFMA operand order) followed by the scales, ordered the way
// the MFMA result rows land in the lanes.  A wave streams whole 1 KiB tiles
// with 128-bit loads.  The X slabs for one K tile are converted to hi/lo fp16
// once per workgroup into LDS (double-buffered) and shared by the 4 waves and
// their RPW row tiles.  Long K is split over workgroups; each split writes
// its partial sums, reduced in a fixed order later (deterministic, no atomics).
//
// F32 path: plain wave-per-row FMA GEMV (fp32 weights are only used by small
// models, where it is latency-bound).
#include "rra_internal.h"

namespace rra {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int FMT>
struct TileFmt;
template <>
struct TileFmt<RRA_Q4> {
    static constexpr int KT = 128, NB = 4, TB = 1024 + 128;
};
template <>
struct TileFmt<RRA_Q8> {
    static constexpr int KT = 64, NB = 2, TB = 1024 + 64;
};

__device__ __forceinline__ uint32_t pk_sub(uint32_t p, float c) {
    half2_t h = __builtin_bit_cast(half2_t, p);
    _Float16 ch = (_Float16)c;
    h = h - half2_t{ch, ch};
    return __builtin_bit_cast(uint32_t, h);
}

// Pairs byte0/byte1 (or byte2/byte3) of v into two fp16 values 1024 + byte.
__device__ __forceinline__ uint32_t pair_lo(uint32_t v) {
    return 0x64006400u | (v & 0xFFu) | ((v & 0xFF00u) << 8);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t v) {
    return 0x64006400u | ((v >> 16) & 0xFFu) | ((v >> 8) & 0xFF0000u);
}

// Q4: one dword = 8 nibbles of a group (byte u holds element 2u low, 2u+1 high)
// -> fp16 (q - 8) in element order [0, 2, 4, 6, 1, 3, 5, 7].
__device__ __forceinline__ half8_t dequant_q4(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    uint4 v;
    v.x = pk_sub(pair_lo(lo), 1032.f);
    v.y = pk_sub(pair_hi(lo), 1032.f);
    v.z = pk_sub(pair_lo(hi), 1032.f);
    v.w = pk_sub(pair_hi(hi), 1032.f);
    return __builtin_bit_cast(half8_t, v);
}

// Q8: two dwords = int8 elements 0..7 of a group -> fp16 q in element order.
__device__ __forceinline__ half8_t dequant_q8(uint32_t d0, uint32_t d1) {
    const uint32_t u0 = d0 ^ 0x80808080u, u1 = d1 ^ 0x80808080u;  // q + 128
    uint4 v;
    v.x = pk_sub(pair_lo(u0), 1152.f);
    v.y = pk_sub(pair_hi(u0), 1152.f);
    v.z = pk_sub(pair_lo(u1), 1152.f);
    v.w = pk_sub(pair_hi(u1), 1152.f);
    return __builtin_bit_cast(half8_t, v);
}

// Converts the X columns of K tile `kt` into MFMA B operands in LDS.
// Fragment (b, c, h) is 64 lanes x 8 fp16: lane (j = lane/16, col = lane%16)
// holds x[16c + col][kt*KT + 32b + 8j + e'] for the element order e' that the
// weight operand uses (Q4: 0,2,4,6,1,3,5,7; Q8: 0..7), h = 0 hi part, 1 lo part.
template <int FMT, int CT>
__device__ __forceinline__ void stage_x(const float *__restrict__ x, int M, int K, int kt,
                                        uint8_t *buf) {
    using F = TileFmt<FMT>;
    constexpr int MP = 16 * CT;
    constexpr int GROUPS = MP * F::KT / 8;
    for (int gi = threadIdx.x; gi < GROUPS; gi += blockDim.x) {
        const int m = gi % MP, grp = gi / MP;
        const int b = grp >> 2, j = grp & 3;
        const int k0 = kt * F::KT + 32 * b + 8 * j;
        float v[8];
        if (m < M && k0 < K) {
            const float4 a0 = *reinterpret_cast<const float4 *>(x + (size_t)m * K + k0);
            const float4 a1 = *reinterpret_cast<const float4 *>(x + (size_t)m * K + k0 + 4);
            v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
            v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
        half8_t hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int src = (FMT == RRA_Q4) ? ((e < 4) ? 2 * e : 2 * (e - 4) + 1) : e;
            const _Float16 h = (_Float16)v[src];
            hi[e] = h;
            lo[e] = (_Float16)(v[src] - (float)h);
        }
        const int c = m >> 4, ln = j * 16 + (m & 15);
        *reinterpret_cast<half8_t *>(buf + ((b * CT + c) * 2 + 0) * 1024 + ln * 16) = hi;
        *reinterpret_cast<half8_t *>(buf + ((b * CT + c) * 2 + 1) * 1024 + ln * 16) = lo;
    }
}

// Grid (row blocks of 4*RPW*16 rows, K splits); 256 threads = 4 waves; wave w
// owns row tiles [(blockIdx.x*4 + w)*RPW, +RPW).  Writes out[split][m][n].
template <int FMT, int CT, int RPW>
__global__ __launch_bounds__(256) void gemv_q_kernel(const uint8_t *__restrict__ wt,
                                                     const float *__restrict__ x,
                                                     float *__restrict__ out, int M, int N, int K,
                                                     int nkt, int kt_per_split,
                                                     long long split_stride) {
    using F = TileFmt<FMT>;
    constexpr int NB = F::NB, TB = F::TB;
    constexpr int FRAG = NB * CT * 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][FRAG * 1024];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int n_rt = (N + 15) >> 4;
    const int rt0 = (blockIdx.x * 4 + wave) * RPW;
    const int kt_begin = blockIdx.y * kt_per_split;
    const int kt_end = min(nkt, kt_begin + kt_per_split);

    floatx4 acc[RPW][CT];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[r][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int kt = kt_begin; kt < kt_end; ++kt) {
        uint8_t *buf = lds[(kt - kt_begin) & 1];
        stage_x<FMT, CT>(x, M, K, kt, buf);
        __syncthreads();

        half8_t B[NB][CT][2];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    B[b][c][h] = *reinterpret_cast<const half8_t *>(
                        buf + ((b * CT + c) * 2 + h) * 1024 + lane * 16);

#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int rt = rt0 + r;
            if (rt >= n_rt) continue;
            const uint8_t *tile = wt + ((size_t)rt * nkt + kt) * TB;
            const uint4 qv = *reinterpret_cast<const uint4 *>(tile + lane * 16);
            const uint32_t qd[4] = {qv.x, qv.y, qv.z, qv.w};
            // Scales of result rows 4g+i, blocks b of this tile: index i*NB + b.
            _Float16 sh[4 * NB];
            if (FMT == RRA_Q4) {
                const uint4 s0 = *reinterpret_cast<const uint4 *>(tile + 1024 + 32 * g);
                const uint4 s1 = *reinterpret_cast<const uint4 *>(tile + 1024 + 32 * g + 16);
                const half8_t h0 = __builtin_bit_cast(half8_t, s0);
                const half8_t h1 = __builtin_bit_cast(half8_t, s1);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sh[e] = h0[e];
                    sh[8 + e] = h1[e];
                }
            } else {
                const uint4 s0 = *reinterpret_cast<const uint4 *>(tile + 1024 + 16 * g);
                const half8_t h0 = __builtin_bit_cast(half8_t, s0);
#pragma unroll
                for (int e = 0; e < 8; ++e) sh[e] = h0[e];
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const half8_t a = (FMT == RRA_Q4) ? dequant_q4(qd[b])
                                                  : dequant_q8(qd[2 * b], qd[2 * b + 1]);
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    floatx4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        a, B[b][c][0], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, B[b][c][1], t, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[r][c][i] = fmaf((float)sh[i * NB + b], t[i], acc[r][c][i]);
                }
            }
        }
    }

    // Result layout of a 16x16 MFMA: lane holds rows 4g..4g+3 of column lane%16.
    float *o = out + (size_t)blockIdx.y * split_stride;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int rt = rt0 + r;
        if (rt >= n_rt) continue;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const int m = 16 * c + (lane & 15);
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = rt * 16 + 4 * g + i;
                if (row < N) o[(size_t)m * N + row] = acc[r][c][i];
            }
        }
    }
}

// fp32 weights: one wave per output row, lanes stride K, all M inputs.
__global__ __launch_bounds__(256) void gemv_f32_kernel(const float *__restrict__ w,
                                                       const float *__restrict__ x,
                                                       float *__restrict__ out, int M, int N,
                                                       int K) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= N) return;
    float acc[RRA_M_MAX];
#pragma unroll
    for (int m = 0; m < RRA_M_MAX; ++m) acc[m] = 0.f;
    const float *wr = w + (size_t)row * K;
    for (int k = lane; k < K; k += 64) {
        const float wv = wr[k];
#pragma unroll
        for (int m = 0; m < RRA_M_MAX; ++m)
            if (m < M) acc[m] = fmaf(wv, x[(size_t)m * K + k], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < RRA_M_MAX; ++m) {
        if (m < M) {
            float v = acc[m];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) out[(size_t)m * N + row] = v;
        }
    }
}

__global__ void reduce_splits_kernel(const float *__restrict__ part, int split,
                                     long long split_stride, float *__restrict__ y,
                                     long long total) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    float v = part[i];
    for (int s = 1; s < split; ++s) v += part[(size_t)s * split_stride + i];
    y[i] = v;
}

// ------------------------------------------------------------------ repack
// Tile (rt, kt), lane (r = lane%16, j = lane/16): 16 bytes = for each block b
// of the tile the j-th 4 (Q4) or 8 (Q8) bytes of row 16rt + r.  Scales: entry
// (g, i, b) = scale of row 16rt + 4g + i, block b, at index (g*4 + i)*NB + b.
template <int FMT>
__global__ void repack_kernel(const uint8_t *__restrict__ q, const uint16_t *__restrict__ scale,
                              uint8_t *__restrict__ tiled, int N, int K, int nkt) {
    using F = TileFmt<FMT>;
    const long long tile = blockIdx.x;
    const int lane = threadIdx.x;
    const int rt = (int)(tile / nkt), kt = (int)(tile % nkt);
    uint8_t *dst = tiled + tile * F::TB;
    const int nblk = K / 32;
    const int r = lane & 15, j = lane >> 4;
    const int row = rt * 16 + r;
    uint32_t d[4];
    if (FMT == RRA_Q4) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int blk = kt * 4 + b;
            d[b] = (row < N && blk < nblk)
                       ? *reinterpret_cast<const uint32_t *>(q + (size_t)row * (K / 2) + blk * 16 + 4 * j)
                       : 0x88888888u;
        }
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int blk = kt * 2 + b;
            const bool ok = row < N && blk < nblk;
            const uint8_t *src = q + (size_t)row * K + blk * 32 + 8 * j;
            d[2 * b] = ok ? *reinterpret_cast<const uint32_t *>(src) : 0u;
            d[2 * b + 1] = ok ? *reinterpret_cast<const uint32_t *>(src + 4) : 0u;
        }
    }
    *reinterpret_cast<uint4 *>(dst + lane * 16) = uint4{d[0], d[1], d[2], d[3]};
    constexpr int NS = 16 * F::NB;
    if (lane < NS) {
        const int e = lane;
        const int b = e % F::NB, gi = e / F::NB;  // gi = g*4 + i
        const int srow = rt * 16 + gi;            // 4g + i == gi
        const int blk = kt * F::NB + b;
        reinterpret_cast<uint16_t *>(dst + 1024)[e] =
            (srow < N && blk < nblk) ? scale[(size_t)srow * nblk + blk] : (uint16_t)0;
    }
}

template <int FMT>
__global__ void unpack_kernel(const uint8_t *__restrict__ tiled, uint8_t *__restrict__ q,
                              uint16_t *__restrict__ scale, int N, int K, int nkt) {
    using F = TileFmt<FMT>;
    const long long tile = blockIdx.x;
    const int lane = threadIdx.x;
    const int rt = (int)(tile / nkt), kt = (int)(tile % nkt);
    const uint8_t *src = tiled + tile * F::TB;
    const int nblk = K / 32;
    const int r = lane & 15, j = lane >> 4;
    const int row = rt * 16 + r;
    const uint4 v = *reinterpret_cast<const uint4 *>(src + lane * 16);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    if (FMT == RRA_Q4) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int blk = kt * 4 + b;
            if (row < N && blk < nblk)
                *reinterpret_cast<uint32_t *>(q + (size_t)row * (K / 2) + blk * 16 + 4 * j) = d[b];
        }
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int blk = kt * 2 + b;
            if (row < N && blk < nblk) {
                uint8_t *dst = q + (size_t)row * K + blk * 32 + 8 * j;
                *reinterpret_cast<uint32_t *>(dst) = d[2 * b];
                *reinterpret_cast<uint32_t *>(dst + 4) = d[2 * b + 1];
            }
        }
    }
    constexpr int NS = 16 * F::NB;
    if (lane < NS) {
        const int e = lane;
        const int b = e % F::NB, gi = e / F::NB;
        const int srow = rt * 16 + gi;
        const int blk = kt * F::NB + b;
        if (srow < N && blk < nblk)
            scale[(size_t)srow * nblk + blk] = reinterpret_cast<const uint16_t *>(src + 1024)[e];
    }
}

template <int FMT, int CT, int RPW>
rra_status launch_q(const rra_weight &w, const GemvPlan &p, const float *x, int m, float *out,
                    size_t stride, hipStream_t s) {
    const int n_rt = (int)cdiv(w.n, 16);
    const int nkt = (int)cdiv(w.k, TileFmt<FMT>::KT);
    dim3 grid((unsigned)cdiv(n_rt, 4 * RPW), (unsigned)p.split);
    hipLaunchKernelGGL((gemv_q_kernel<FMT, CT, RPW>), grid, dim3(256), 0, s,
                       static_cast<const uint8_t *>(w.data), x, out, m, (int)w.n, (int)w.k, nkt,
                       p.kt_per_split, (long long)stride);
    return check_launch("gemv_q_kernel");
}

template <int FMT>
rra_status launch_fmt(const rra_weight &w, const GemvPlan &p, const float *x, int m, float *out,
                      size_t stride, hipStream_t s) {
    if (m <= 16) {
        if (p.rpw >= 4) return launch_q<FMT, 1, 4>(w, p, x, m, out, stride, s);
        if (p.rpw == 2) return launch_q<FMT, 1, 2>(w, p, x, m, out, stride, s);
        return launch_q<FMT, 1, 1>(w, p, x, m, out, stride, s);
    }
    if (p.rpw >= 4) return launch_q<FMT, 2, 4>(w, p, x, m, out, stride, s);
    if (p.rpw == 2) return launch_q<FMT, 2, 2>(w, p, x, m, out, stride, s);
    return launch_q<FMT, 2, 1>(w, p, x, m, out, stride, s);
}

}  // namespace

GemvPlan gemv_plan(const rra_weight &w, int m) {
    GemvPlan p;
    if (w.fmt == RRA_F32) return p;
    const int n_rt = (int)cdiv(w.n, 16);
    const int nkt = (int)cdiv(w.k, tile_k(w.fmt));
    p.rpw = (m > 16) ? 4 : 2;
    while (p.rpw > 1 && cdiv(n_rt, 4 * p.rpw) < 64) p.rpw >>= 1;
    const int n_rb = (int)cdiv(n_rt, 4 * p.rpw);
    const int target = 512;  // about two 256-thread groups per compute unit
    int split = (int)std::max<int64_t>(1, std::min<int64_t>(nkt, cdiv(target, n_rb)));
    split = std::min(split, std::max(1, nkt / 2));  // at least 2 K tiles per split
    p.kt_per_split = (int)cdiv(nkt, split);
    p.split = (int)cdiv(nkt, p.kt_per_split);
    return p;
}

rra_status launch_gemv(const rra_weight &w, const GemvPlan &p, const float *x, int m, float *out,
                       size_t stride, hipStream_t s) {
    if (w.fmt == RRA_F32) {
        dim3 grid((unsigned)cdiv(w.n, 4));
        hipLaunchKernelGGL(gemv_f32_kernel, grid, dim3(256), 0, s,
                           static_cast<const float *>(w.data), x, out, m, (int)w.n, (int)w.k);
        return check_launch("gemv_f32_kernel");
    }
    if (w.fmt == RRA_Q4) return launch_fmt<RRA_Q4>(w, p, x, m, out, stride, s);
    return launch_fmt<RRA_Q8>(w, p, x, m, out, stride, s);
}

rra_status launch_reduce_splits(const float *part, int split, size_t split_stride, float *y,
                                int m, int n, hipStream_t s) {
    const long long total = (long long)m * n;
    hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s,
                       part, split, (long long)split_stride, y, total);
    return check_launch("reduce_splits_kernel");
}

}  // namespace rra

using namespace rra;

extern "C" size_t rra_tiled_bytes(int32_t fmt, int64_t n, int64_t k) {
    if ((fmt != RRA_Q4 && fmt != RRA_Q8) || n <= 0 || k <= 0 || k % 32) return 0;
    return (size_t)cdiv(n, 16) * (size_t)cdiv(k, tile_k(fmt)) * (size_t)tile_bytes(fmt);
}

extern "C" rra_status rra_repack_weight(const rra_weight *planar, void *tiled, size_t tiled_bytes,
                                        rra_weight *out, hipStream_t s) {
    clear_error();
    if (!planar || !tiled || !out) return fail(RRA_EINVAL, "rra_repack_weight: null argument");
    if (planar->fmt != RRA_Q4 && planar->fmt != RRA_Q8)
        return fail(RRA_EINVAL, "rra_repack_weight: only Q8/Q4 weights are tiled");
    if (planar->layout != RRA_PLANAR)
        return fail(RRA_EINVAL, "rra_repack_weight: input must be planar");
    RRA_TRY(validate_weight(planar, "rra_repack_weight", false));
    const size_t need = rra_tiled_bytes(planar->fmt, planar->n, planar->k);
    if (tiled_bytes < need)
        return fail(RRA_EINVAL, "rra_repack_weight: buffer has %zu bytes, needs %zu", tiled_bytes,
                    need);
    const int nkt = (int)cdiv(planar->k, tile_k(planar->fmt));
    const long long tiles = cdiv(planar->n, 16) * (long long)nkt;
    auto q = static_cast<const uint8_t *>(planar->data);
    auto dst = static_cast<uint8_t *>(tiled);
    if (planar->fmt == RRA_Q4)
        hipLaunchKernelGGL(repack_kernel<RRA_Q4>, dim3((unsigned)tiles), dim3(64), 0, s, q,
                           planar->scale, dst, (int)planar->n, (int)planar->k, nkt);
    else
        hipLaunchKernelGGL(repack_kernel<RRA_Q8>, dim3((unsigned)tiles), dim3(64), 0, s, q,
                           planar->scale, dst, (int)planar->n, (int)planar->k, nkt);
    RRA_TRY(check_launch("repack_kernel"));
    *out = *planar;
    out->layout = RRA_TILED;
    out->data = tiled;
    out->scale = nullptr;
    return RRA_OK;
}

extern "C" rra_status rra_unpack_weight(const rra_weight *tiled, void *data, uint16_t *scale,
                                        hipStream_t s) {
    clear_error();
    if (!tiled || !data || !scale) return fail(RRA_EINVAL, "rra_unpack_weight: null argument");
    if ((tiled->fmt != RRA_Q4 && tiled->fmt != RRA_Q8) || tiled->layout != RRA_TILED)
        return fail(RRA_EINVAL, "rra_unpack_weight: input must be a tiled Q8/Q4 weight");
    RRA_TRY(validate_weight(tiled, "rra_unpack_weight", true));
    const int nkt = (int)cdiv(tiled->k, tile_k(tiled->fmt));
    const long long tiles = cdiv(tiled->n, 16) * (long long)nkt;
    auto src = static_cast<const uint8_t *>(tiled->data);
    auto q = static_cast<uint8_t *>(data);
    if (tiled->fmt == RRA_Q4)
        hipLaunchKernelGGL(unpack_kernel<RRA_Q4>, dim3((unsigned)tiles), dim3(64), 0, s, src, q,
                           scale, (int)tiled->n, (int)tiled->k, nkt);
    else
        hipLaunchKernelGGL(unpack_kernel<RRA_Q8>, dim3((unsigned)tiles), dim3(64), 0, s, src, q,
                           scale, (int)tiled->n, (int)tiled->k, nkt);
    return check_launch("unpack_kernel");
}

extern "C" size_t rra_batched_gemv_workspace_bytes(const rra_weight *w, int32_t m) {
    if (!w || m < 1 || m > RRA_M_MAX || w->n <= 0) return 0;
    const GemvPlan p = gemv_plan(*w, m);
    return p.split > 1 ? (size_t)p.split * (size_t)m * (size_t)w->n * sizeof(float) : 0;
}

extern "C" rra_status rra_batched_gemv(const rra_weight *w, const float *x, float *y, int32_t m,
                                       void *ws, size_t ws_bytes, hipStream_t s) {
    clear_error();
    if (!w || !x || !y) return fail(RRA_EINVAL, "rra_batched_gemv: null argument");
    if (m < 1 || m > RRA_M_MAX) return fail(RRA_EINVAL, "rra_batched_gemv: m=%d not in 1..32", m);
    RRA_TRY(validate_weight(w, "rra_batched_gemv", true));
    GemvPlan p = gemv_plan(*w, m);
    if (!ws || p.split == 1) {
        // No scratch: one pass over the whole K range per row block.
        const int nkt = w->fmt == RRA_F32 ? 1 : (int)cdiv(w->k, tile_k(w->fmt));
        p.split = 1;
        p.kt_per_split = nkt;
        return launch_gemv(*w, p, x, m, y, 0, s);
    }
    const size_t need = rra_batched_gemv_workspace_bytes(w, m);
    if (ws_bytes < need)
        return fail(RRA_ENOTINIT, "rra_batched_gemv: workspace has %zu bytes, needs %zu", ws_bytes,
                    need);
    float *part = static_cast<float *>(ws);
    const size_t stride = (size_t)m * (size_t)w->n;
    RRA_TRY(launch_gemv(*w, p, x, m, part, stride, s));
    return launch_reduce_splits(part, p.split, stride, y, m, (int)w->n, s);
}
