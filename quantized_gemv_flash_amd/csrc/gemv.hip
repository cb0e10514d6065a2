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
// the MFMA result rows land in the lanes.  The activations arrive already
// split into the hi/lo operand image (frag.h), written once by the kernel that
// produced them; a workgroup copies its share of the image and of the scales
// into LDS with LDS-DMA (global_load_lds: no registers, no conversion).  Long K
// is split over workgroups; each split writes its partial sums, reduced in a
// fixed order later (deterministic, no atomics).
//
// F32 path: plain wave-per-row FMA GEMV (fp32 weights are only used by small
// models, where it is latency-bound).
#include "frag.h"
#include "rra_internal.h"

namespace rra {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
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

// Component i (a compile-time constant after unrolling) of a 128-bit value.
__device__ __forceinline__ uint32_t u32_at(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Two fp16 values 1024 + byte from bytes 0,1 (pair_lo) or 2,3 (pair_hi) of v:
// one v_perm_b32 against 0x64 bytes (fp16 0x64XX = 1024 + XX for XX < 256).
// v_perm_b32 selector bytes 0-3 pick bytes of its second operand, 4-7 of its
// first.
__device__ __forceinline__ uint32_t pair_lo(uint32_t v) {
    return __builtin_amdgcn_perm(v, 0x64646464u, 0x00050004u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t v) {
    return __builtin_amdgcn_perm(v, 0x64646464u, 0x00070006u);
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

// 16 bytes of global memory -> LDS at `lds` + 16 * lane (LDS-DMA).  `lds` must
// be the same for the whole wave.
__device__ __forceinline__ void dma16(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// Waits until at most N vector-memory instructions of this wave are in
// flight (s_waitcnt vmcnt(N); expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Grid (row blocks of 64*RPW rows, K splits); 256 threads = 4 waves; wave w
// owns row tiles [(blockIdx.x*4 + w)*RPW, +RPW).  The split's K tiles are
// processed KTW at a time ("chunks") in a software pipeline; iteration c:
//   1. LDS-DMA of chunk c+1's activation image and scales into the other LDS
//      buffer;
//   2. loads of chunk c+2's quantised values into registers (a ring of 3);
//   3. dequantise + MFMA + block scale of chunk c (registers + LDS);
//   4. wait for step 1 only (vector memory ops retire in issue order, so this
//      never waits for step 2), barrier.
// Each chunk of weights thus has two compute periods to arrive.  Outputs are
// multiplied by inv[m] (RMSNorm, when nrm.ss is set) and written to
// out[split][m][n] (split_stride floats apart).
template <int FMT, int CT, int RPW, int KTW>
__global__ __launch_bounds__(256) void gemv_q_kernel(const uint8_t *__restrict__ wt,
                                                     const uint8_t *__restrict__ ximg,
                                                     float *__restrict__ out, int M, int N, int K,
                                                     int nkt, int kt_per_split,
                                                     long long split_stride, NormIn nrm) {
    using F = TileFmt<FMT>;
    constexpr int NB = F::NB, TB = F::TB, MP = 16 * CT;
    constexpr int FRAG = NB * CT * 2;              // 1 KiB image fragments per K tile
    constexpr int SB = TB - 1024;                  // scale bytes per tile
    constexpr int SCH = 4 * RPW * KTW * SB / 16;   // 16-byte scale pieces per chunk
    constexpr int SCW = (SCH + 63) / 64;           // DMA wave-instructions for them
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][KTW][FRAG * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t sl[2][SCW * 1024];
    __shared__ float inv_s[MP];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_rt = (N + 15) >> 4;
    const int rt_wg = blockIdx.x * 4 * RPW;  // first row tile of the workgroup
    const int rt0 = rt_wg + wave * RPW;
    const int kt_begin = blockIdx.y * kt_per_split;
    const int kt_end = min(nkt, kt_begin + kt_per_split);
    const int nch = (kt_end - kt_begin + KTW - 1) / KTW;

    if (tid < MP) {
        float inv = 1.f;
        if (nrm.ss) {
            float sq = 0.f;
            if (tid < M)
                for (int p = 0; p < nrm.nparts; ++p) sq += nrm.ss[tid * nrm.nparts + p];
            inv = 1.0f / sqrtf(sq / (float)K + nrm.eps);
        }
        inv_s[tid] = inv;
    }

    // K tiles of a chunk past the split end reuse the last valid tile's data
    // (finite) with its quantised values replaced by zeros.
    auto stage = [&](int c, int buf) {
        const int kt0 = kt_begin + c * KTW;
        for (int f = wave; f < KTW * FRAG; f += 4) {
            const int t = f / FRAG, fr = f - t * FRAG;
            const int kt = min(kt0 + t, kt_end - 1);
            dma16(ximg + ((size_t)kt * FRAG + fr) * 1024 + lane * 16, xs[buf][t] + fr * 1024);
        }
        for (int i = wave; i < SCW; i += 4) {  // scale piece e -> (row tile, K tile, piece)
            const int e = min(i * 64 + lane, SCH - 1);
            const int piece = e % (SB / 16), tt = (e / (SB / 16)) % KTW, rr = e / (SB / 16) / KTW;
            const int rt = min(rt_wg + rr, n_rt - 1), kt = min(kt0 + tt, kt_end - 1);
            dma16(wt + ((size_t)rt * nkt + kt) * TB + 1024 + piece * 16, sl[buf] + i * 1024);
        }
    };
    auto issue = [&](uint4 (&q)[KTW][RPW], int c) {
        const int kt0 = kt_begin + c * KTW;
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int rt = min(rt0 + r, n_rt - 1), kt = min(kt0 + t, kt_end - 1);
                const uint4 v = *reinterpret_cast<const uint4 *>(
                    wt + ((size_t)rt * nkt + kt) * TB + lane * 16);
                // past the split end: values that dequantise to zero, by masking
                // (the load is always issued: the wait counts below rely on it)
                const uint32_t keep = (kt0 + t < kt_end) ? 0xFFFFFFFFu : 0u;
                const uint32_t z = (FMT == RRA_Q4) ? (0x88888888u & ~keep) : 0u;
                q[t][r] = uint4{(v.x & keep) | z, (v.y & keep) | z, (v.z & keep) | z,
                                (v.w & keep) | z};
            }
    };

    floatx4 acc[RPW][CT];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[r][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Branch-free: row tiles past N repeat the last tile's values (never stored).
    auto compute = [&](const uint4 (&q)[KTW][RPW], int buf) {
#pragma unroll
        for (int t = 0; t < KTW; ++t) {
            const uint8_t *bp = xs[buf][t];
            // scales of this wave's row tiles for K tile t: rows 4g+i, blocks b
            _Float16 sh[RPW][4 * NB];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const uint8_t *sp = sl[buf] + (((wave * RPW + r) * KTW) + t) * SB;
                if (FMT == RRA_Q4) {
                    const half8_t h0 = *reinterpret_cast<const half8_t *>(sp + 32 * g);
                    const half8_t h1 = *reinterpret_cast<const half8_t *>(sp + 32 * g + 16);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sh[r][e] = h0[e];
                        sh[r][8 + e] = h1[e];
                    }
                } else {
                    const half8_t h0 = *reinterpret_cast<const half8_t *>(sp + 16 * g);
#pragma unroll
                    for (int e = 0; e < 8; ++e) sh[r][e] = h0[e];
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                half8_t Bh[CT], Bl[CT];
                const int slot = frag_slot<FMT>(lane >> 4, lane & 15, b);
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    Bh[c] = *reinterpret_cast<const half8_t *>(bp + ((b * CT + c) * 2 + 0) * 1024 + slot * 16);
                    Bl[c] = *reinterpret_cast<const half8_t *>(bp + ((b * CT + c) * 2 + 1) * 1024 + slot * 16);
                }
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    const uint4 qv = q[t][r];
                    const half8_t a = (FMT == RRA_Q4)
                                          ? dequant_q4(u32_at(qv, b))
                                          : dequant_q8(u32_at(qv, 2 * b), u32_at(qv, 2 * b + 1));
#pragma unroll
                    for (int c = 0; c < CT; ++c) {
                        floatx4 tt = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            a, Bh[c], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        tt = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, Bl[c], tt, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[r][c][i] = fmaf((float)sh[r][i * NB + b], tt[i], acc[r][c][i]);
                    }
                }
            }
        }
    };

    // The LDS written by DMA must be complete before the barrier: wait for
    // the DMA but not for the weight loads issued after it (KTW*RPW each).
    uint4 q0[KTW][RPW], q1[KTW][RPW], q2[KTW][RPW];
    stage(0, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep every DMA ahead of the weight loads
    issue(q0, 0);
    if (nch > 1) {
        issue(q1, 1);
        wait_vm<2 * KTW * RPW>();
    } else {
        wait_vm<KTW * RPW>();
    }
    __syncthreads();
    // qc: chunk c (landed); chunk c+1 in flight; qf: chunk c+2 (issued here)
    auto iter = [&](const uint4 (&qc)[KTW][RPW], uint4 (&qf)[KTW][RPW], int c) {
        if (c + 1 < nch) stage(c + 1, (c + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 2 < nch) issue(qf, c + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(qc, c & 1);
        if (c + 2 < nch)
            wait_vm<KTW * RPW>();
        else
            wait_vm<0>();
        __syncthreads();
    };
    for (int c = 0; c < nch; c += 3) {
        iter(q0, q2, c);
        if (c + 1 < nch) iter(q1, q0, c + 1);
        if (c + 2 < nch) iter(q2, q1, c + 2);
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
            const float iv = inv_s[m];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = rt * 16 + 4 * g + i;
                if (row < N) o[(size_t)m * N + row] = acc[r][c][i] * iv;
            }
        }
    }
}

// Writes x (fp32 [M][K], canonical) as the B-operand image of a GEMV with
// `ct` column tiles; groups in [K, kpad) are zeros.  One thread per group.
template <int FMT>
__global__ void x_to_image_kernel(const float *__restrict__ x, uint8_t *__restrict__ img, int M,
                                  int K, int kpad, int ct) {
    const int groups = kpad / 8;
    const int gi = blockIdx.x * blockDim.x + threadIdx.x;
    const int m = blockIdx.y;
    if (gi >= groups) return;
    const int k0 = gi * 8;
    float v[8];
    if (k0 < K) {
        const float4 a0 = *reinterpret_cast<const float4 *>(x + (size_t)m * K + k0);
        const float4 a1 = *reinterpret_cast<const float4 *>(x + (size_t)m * K + k0 + 4);
        v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
        v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    write_frag8<FMT>(img, ct, m, k0, v);
}

// fp32 weights: one wave per output row, lanes stride K, all M inputs.
__global__ __launch_bounds__(256) void gemv_f32_kernel(const float *__restrict__ w,
                                                       const float *__restrict__ x,
                                                       float *__restrict__ out, int M, int N,
                                                       int K, NormIn nrm) {
    __shared__ float inv_s[RRA_M_MAX];
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < RRA_M_MAX) {
        float inv = 1.f;
        if (nrm.ss && (int)threadIdx.x < M) {
            float sq = 0.f;
            for (int p = 0; p < nrm.nparts; ++p) sq += nrm.ss[threadIdx.x * nrm.nparts + p];
            inv = 1.0f / sqrtf(sq / (float)K + nrm.eps);
        }
        inv_s[threadIdx.x] = inv;
    }
    __syncthreads();
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
            if (lane == 0) out[(size_t)m * N + row] = v * inv_s[m];
        }
    }
}

// y = sum over the split planes, 4 independent loads in flight per step.
__device__ __forceinline__ float sum_splits(const float *__restrict__ p, int split,
                                           long long stride) {
    float a = 0.f, b = 0.f, c = 0.f, d = 0.f;
    int s = 0;
    for (; s + 4 <= split; s += 4) {
        a += p[(size_t)s * stride];
        b += p[(size_t)(s + 1) * stride];
        c += p[(size_t)(s + 2) * stride];
        d += p[(size_t)(s + 3) * stride];
    }
    for (; s < split; ++s) a += p[(size_t)s * stride];
    return (a + b) + (c + d);
}

__global__ void reduce_splits_kernel(const float *__restrict__ part, int split,
                                     long long split_stride, float *__restrict__ y,
                                     long long total) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    y[i] = sum_splits(part + i, split, split_stride);
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

// K tiles per chunk: 16 KiB of activation image per chunk and LDS buffer.
constexpr int ktw_of(int fmt, int ct) {
    return fmt == RRA_Q4 ? (ct == 2 ? 1 : 2) : (ct == 2 ? 2 : 4);
}

template <int FMT, int CT, int RPW>
rra_status launch_q(const rra_weight &w, const GemvPlan &p, const uint8_t *img, int m, float *out,
                    size_t stride, const NormIn &nrm, hipStream_t s) {
    const int n_rt = (int)cdiv(w.n, 16);
    const int nkt = (int)cdiv(w.k, TileFmt<FMT>::KT);
    dim3 grid((unsigned)cdiv(n_rt, 4 * RPW), (unsigned)p.split);
    constexpr int KTW = ktw_of(FMT, CT);
    hipLaunchKernelGGL((gemv_q_kernel<FMT, CT, RPW, KTW>), grid, dim3(256), 0, s,
                       static_cast<const uint8_t *>(w.data), img, out, m, (int)w.n, (int)w.k, nkt,
                       p.kt_per_split, (long long)stride, nrm);
    return check_launch("gemv_q_kernel");
}

template <int FMT>
rra_status launch_fmt(const rra_weight &w, const GemvPlan &p, const uint8_t *img, int m,
                      float *out, size_t stride, const NormIn &nrm, hipStream_t s) {
    if (m <= 16) {
        if (p.rpw >= 2) return launch_q<FMT, 1, 2>(w, p, img, m, out, stride, nrm, s);
        return launch_q<FMT, 1, 1>(w, p, img, m, out, stride, nrm, s);
    }
    if (p.rpw >= 2) return launch_q<FMT, 2, 2>(w, p, img, m, out, stride, nrm, s);
    return launch_q<FMT, 2, 1>(w, p, img, m, out, stride, nrm, s);
}

}  // namespace

GemvPlan gemv_plan(const rra_weight &w, int m) {
    GemvPlan p;
    if (w.fmt == RRA_F32) return p;
    const int n_rt = (int)cdiv(w.n, 16);
    const int nkt = (int)cdiv(w.k, tile_k(w.fmt));
    const int ktw = ktw_of(w.fmt, frag_ct(m));
    // Row tiles per wave: 2, or 1 when that leaves too few row blocks.
    p.rpw = 2;
    if (cdiv(n_rt, 4 * p.rpw) < 128) p.rpw = 1;
    const int n_rb = (int)cdiv(n_rt, 4 * p.rpw);
    // K splits: aim for ~1024 workgroups (4 per compute unit), each split at
    // least one chunk of K tiles.
    const int target = 1024;
    int split = (int)std::max<int64_t>(1, cdiv(target, n_rb));
    split = std::min<int>(split, (int)cdiv(nkt, ktw));
    p.kt_per_split = (int)cdiv(nkt, split);
    p.split = (int)cdiv(nkt, p.kt_per_split);
    return p;
}

rra_status launch_gemv(const rra_weight &w, const GemvPlan &p, const void *x, int m, float *out,
                       size_t stride, hipStream_t s, const NormIn *nrm) {
    const NormIn none{nullptr, 0, 0.f};
    const NormIn &n = nrm ? *nrm : none;
    if (w.fmt == RRA_F32) {
        dim3 grid((unsigned)cdiv(w.n, 4));
        hipLaunchKernelGGL(gemv_f32_kernel, grid, dim3(256), 0, s,
                           static_cast<const float *>(w.data), static_cast<const float *>(x), out,
                           m, (int)w.n, (int)w.k, n);
        return check_launch("gemv_f32_kernel");
    }
    const auto *img = static_cast<const uint8_t *>(x);
    if (w.fmt == RRA_Q4) return launch_fmt<RRA_Q4>(w, p, img, m, out, stride, n, s);
    return launch_fmt<RRA_Q8>(w, p, img, m, out, stride, n, s);
}

rra_status launch_x_to_image(const float *x, uint8_t *img, int fmt, int m, int k, hipStream_t s) {
    const int kpad = (int)(cdiv(k, tile_k(fmt)) * tile_k(fmt));
    const int ct = frag_ct(m);
    dim3 grid((unsigned)cdiv(kpad / 8, 256), (unsigned)m);
    if (fmt == RRA_Q4)
        hipLaunchKernelGGL(x_to_image_kernel<RRA_Q4>, grid, dim3(256), 0, s, x, img, m, k, kpad, ct);
    else
        hipLaunchKernelGGL(x_to_image_kernel<RRA_Q8>, grid, dim3(256), 0, s, x, img, m, k, kpad, ct);
    return check_launch("x_to_image_kernel");
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

// Workspace of the public GEMV: the activation image (Q8/Q4), then the
// split-K partial sums when K is split.
static size_t gemv_ws_layout(const rra_weight &w, int m, size_t *part_off) {
    const GemvPlan p = gemv_plan(w, m);
    size_t img = 0;
    if (w.fmt != RRA_F32) img = align_up(frag_image_bytes(w.fmt, frag_ct(m), w.k), 256);
    *part_off = img;
    const size_t part = p.split > 1 ? (size_t)p.split * (size_t)m * (size_t)w.n * sizeof(float) : 0;
    return img + part;
}

extern "C" size_t rra_batched_gemv_workspace_bytes(const rra_weight *w, int32_t m) {
    if (!w || m < 1 || m > RRA_M_MAX || w->n <= 0 || w->k <= 0) return 0;
    size_t off;
    return gemv_ws_layout(*w, m, &off);
}

extern "C" rra_status rra_batched_gemv(const rra_weight *w, const float *x, float *y, int32_t m,
                                       void *ws, size_t ws_bytes, hipStream_t s) {
    clear_error();
    if (!w || !x || !y) return fail(RRA_EINVAL, "rra_batched_gemv: null argument");
    if (m < 1 || m > RRA_M_MAX) return fail(RRA_EINVAL, "rra_batched_gemv: m=%d not in 1..32", m);
    RRA_TRY(validate_weight(w, "rra_batched_gemv", true));
    size_t part_off;
    const size_t need = gemv_ws_layout(*w, m, &part_off);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(RRA_ENOTINIT, "rra_batched_gemv: workspace has %zu bytes, needs %zu",
                    ws ? ws_bytes : (size_t)0, need);
    const GemvPlan p = gemv_plan(*w, m);
    const void *in = x;
    if (w->fmt != RRA_F32) {
        auto *img = static_cast<uint8_t *>(ws);
        RRA_TRY(launch_x_to_image(x, img, w->fmt, m, (int)w->k, s));
        in = img;
    }
    if (p.split == 1) return launch_gemv(*w, p, in, m, y, 0, s);
    float *part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + part_off);
    const size_t stride = (size_t)m * (size_t)w->n;
    RRA_TRY(launch_gemv(*w, p, in, m, part, stride, s));
    return launch_reduce_splits(part, p.split, stride, y, m, (int)w->n, s);
}
