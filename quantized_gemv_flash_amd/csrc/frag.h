// frag.h -- the activation "B-operand image" shared by the GEMV (consumer) and
// the kernels that produce GEMV inputs.
//
// The quantised GEMV multiplies on the matrix cores with the fp32 activation x
// split as x = hi + lo (hi = fp16(x), lo = fp16(x - hi)).  Instead of every
// GEMV workgroup converting x again, the producer of a GEMV input writes it
// once in the exact layout the GEMV copies into LDS:
//
//   per K tile kt (KT = 128 for Q4 and Q6K, 64 for Q8 and FP8; NB = KT / 32
//   blocks), for
//   block b, column tile c (16 sequences), part h (0 = hi, 1 = lo): a 1 KiB
//   fragment of 64 slots x 16 bytes at
//       ((((kt * NB + b) * CT + c) * 2 + h) * 1024 + slot * 16;
//   slot frag_slot(j, r, b) holds the 8 fp16 values of sequence 16c + r,
//   elements kt*KT + 32b + 8j + [0..8) in the order the weight operand uses
//   (Q4 and Q6K: 0,4,1,5,2,6,3,7; Q8 and FP8: 0..7).
//
// CT = 1 for M <= 16 rows, 2 for M <= 32 (decode steps), 4 for M <= 64 and
// 8 for M <= 128 (prompt chunks).  Elements k >= K up to the K tile end must
// be written as zeros; columns past M hold anything (their outputs are never
// stored, and a column's products never mix with another column's).
#pragma once

#include "rra_internal.h"

namespace rra {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

inline int frag_ct(int m) { return m <= 16 ? 1 : m <= 32 ? 2 : m <= 64 ? 4 : 8; }
inline size_t frag_image_bytes(int fmt, int ct, int64_t k) {
    return (size_t)cdiv(k, tile_k(fmt)) * (size_t)tile_blocks(fmt) * (size_t)ct * 2 * 1024;
}

// LDS/image slot of B-operand lane (j, r) (lane = 16j + r) in the fragment of
// block b: the lane's own slot, so a wave's fragment read is one contiguous
// 1 KiB.  On gfx950 (64 LDS banks) that reads at the full 256 B per clock;
// an XOR swizzle that depends on j (spreading the writes of one row over the
// banks) halves the read rate, and the reads are the frequent side: every
// wave of a GEMV workgroup reads every fragment, while only the small-batch
// prologues write fragments into LDS at all (DMA copies whole fragments).
template <int FMT>
__device__ __forceinline__ int frag_slot(int j, int r, int b) {
    (void)b;
    return j * 16 + r;
}

// The producer's value as the fp32 number it is: an empty asm the compiler
// cannot see through, so that the fp16 conversions below start from the
// rounded fp32 value.  Without it the compiler may fold the producer's
// multiply (gamma x, silu(g) u, ...) into the conversion used for x - hi
// (v_fma_mixlo_f16 of the exact product, one rounding) while the stored high
// part converts the fp32-rounded product (two roundings): for a value on an
// fp16 midpoint the two disagree, hi + lo is then off by one fp16 unit, and
// kernels that inline the split differently write different bits.
__device__ __forceinline__ float as_fp32(float x) {
    asm("" : "+v"(x));
    return x;
}

// Splits 8 consecutive fp32 activations (k order) into hi/lo fp16 operands:
// hi = fp16(x), lo = fp16(x - hi) (x - hi is exact in fp32).  Returns false
// if a value has |x| >= 65504 (its fp16 high part may not be finite) or is
// NaN.
template <int FMT>
__device__ __forceinline__ bool split8(const float (&v)[8], half8_t &hi, half8_t &lo) {
#pragma clang fp contract(off)
    bool ok = true;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int src = (FMT == RRA_Q4) ? (e >> 1) + 4 * (e & 1) : e;
        const float x = as_fp32(v[src]);
        const _Float16 h = (_Float16)x;
        hi[e] = h;
        lo[e] = (_Float16)(x - (float)h);
        ok = ok && __builtin_fabsf(x) < 65504.0f;
    }
    return ok;
}

// Writes the group x[m][kk .. kk+8) of one K tile (kk = column within the
// tile, a multiple of 8) into that tile's image at `tile` (global memory or
// LDS: one tile is NB * ct * 2 KiB), with `ct` column tiles.
// x = hi + lo for 8 values in their own order (hi = fp16(x), lo = fp16(x - hi)).
__device__ __forceinline__ void split_exact(const float (&v)[8], half8_t &hi, half8_t &lo) {
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = as_fp32(v[e]);
        const _Float16 h = (_Float16)x;
        hi[e] = h;
        lo[e] = (_Float16)(x - (float)h);
    }
}

// Returns split8's range check.
template <int FMT>
__device__ __forceinline__ bool write_frag8_tile(uint8_t *tile, int ct, int m, int kk,
                                                 const float (&v)[8]) {
    const int b = kk >> 5, j = (kk & 31) >> 3;
    half8_t hi, lo;
    const bool ok = split8<FMT>(v, hi, lo);
    const int base = ((b * ct + (m >> 4)) * 2) * 1024 + frag_slot<FMT>(j, m & 15, b) * 16;
    *reinterpret_cast<half8_t *>(tile + base) = hi;
    *reinterpret_cast<half8_t *>(tile + base + 1024) = lo;
    return ok;
}

// Writes the group x[m][k0 .. k0+8) (k0 % 8 == 0) into an image with `ct`
// column tiles.
template <int FMT>
__device__ __forceinline__ bool write_frag8(uint8_t *img, int ct, int m, int k0,
                                            const float (&v)[8]) {
    constexpr int KT = (FMT == RRA_Q4) ? 128 : 64, NB = KT / 32;
    const int kt = k0 / KT;
    return write_frag8_tile<FMT>(img + (size_t)kt * NB * ct * 2 * 1024, ct, m, k0 - kt * KT, v);
}

__device__ __forceinline__ bool write_frag8_fmt(int fmt, uint8_t *img, int ct, int m, int k0,
                                                const float (&v)[8]) {
    if (fmt == RRA_Q4 || fmt == RRA_Q6K) return write_frag8<RRA_Q4>(img, ct, m, k0, v);
    return write_frag8<RRA_Q8>(img, ct, m, k0, v);
}

// A producer's image write of 8 values of row m, reporting kErrRange.
__device__ __forceinline__ void frag_out8(const FragOut &fo, int m, int k0, const float (&v)[8]) {
    if (!write_frag8_fmt(fo.fmt, fo.img, fo.ct, m, k0, v)) report_error(fo.err, kErrRange);
}

}  // namespace rra
