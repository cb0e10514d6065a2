// gemv.hip -- weights-once dequantising batched GEMV (y = W x for M inputs).
//
// [batched_forward] forward_batched_to_token_ids: every weight block is read
// and dequantised once for all M inputs.
//
// Quantised path (Q8, Q4, FP8, Q6K; gfx950 matrix cores).  One
// v_mfma_f32_16x16x32_f16 takes a 16-row x 32-column slab of W -- exactly one
// quantisation block per row -- and a 32 x 16 slab of X^T (16 sequences).  The
// dequantised operands are exact in fp16 (Q8 and Q4 values are small integers,
// E4M3 values are a subset of fp16, a Q6K value is split into two exact
// parts); the fp16 block scale (Q6K: the super-block scale) is applied in fp32
// after the products, so W is never rounded.  X is fp32 and enters as
// x = hi + lo with hi = fp16(x), lo = fp16(x - hi): two MFMAs per slab give
// ~22 significant bits, i.e. fp32-like dot products (products are exact in the
// fp32 accumulator: 11-bit x 11-bit mantissas).  A workgroup of NW waves owns
// NW * RPW row tiles and one K split; all its waves share each staged
// activation tile.
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
#include <mutex>

#include "epilogue.h"
#include "frag.h"
#include "rra_internal.h"

namespace rra {
namespace {

// Weight loads are marked nontemporal: every weight byte is read once per
// step, so it should not displace the activation image and scales the other
// workgroups re-read (MI355X: the Q8 128256 x 4096 GEMV at M=1 goes from
// about 5.4 to 6.1 TB/s).
typedef uint32_t rra_u4v __attribute__((ext_vector_type(4)));
typedef uint32_t rra_u2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ldnt16(const uint8_t *p) {
    const rra_u4v v = __builtin_nontemporal_load(reinterpret_cast<const rra_u4v *>(p));
    return uint4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ uint2 ldnt8(const uint8_t *p) {
    const rra_u2v v = __builtin_nontemporal_load(reinterpret_cast<const rra_u2v *>(p));
    return uint2{v.x, v.y};
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int FMT>
struct TileFmt;
// KT columns, NB blocks of 32, TB bytes per tile, scales at byte SO of a tile,
// IMG = the activation image layout the format reads (frag.h).
template <>
struct TileFmt<RRA_Q4> {
    static constexpr int KT = 128, NB = 4, TB = 1024 + 128, SO = 1024, IMG = RRA_Q4;
};
template <>
struct TileFmt<RRA_Q8> {
    static constexpr int KT = 64, NB = 2, TB = 1024 + 64, SO = 1024, IMG = RRA_Q8;
};
template <>
struct TileFmt<RRA_FP8> : TileFmt<RRA_Q8> {};  // one byte per value, same tiles
// Q6K: 1 KiB of low 4 bits, 512 B of high 2 bits, then 128 B of int8
// sub-scales ([lane half j/2][row][block]) and the 16 rows' fp16 d.  A K tile
// is half a 256-value super-block, so d repeats in the two tiles of one.
template <>
struct TileFmt<RRA_Q6K> {
    static constexpr int KT = 128, NB = 4, TB = 1024 + 512 + 128 + 32, SO = 1536, IMG = RRA_Q4;
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

// Q4: one dword = 8 nibbles of a group (byte u holds element 2u low, 2u+1
// high) -> fp16 (q - 8) in element order [0, 4, 1, 5, 2, 6, 3, 7].  Each pair
// comes from one v_and_or_b32 that drops two nibbles into the mantissas of
// the fp16 pair 1024 + n (low nibbles) or 1024 + 16 n (high nibbles), and one
// packed fp16 op that maps it to n - 8 (exact: small integers).
//
// The compiler splits (w & mask) | bits into v_and_b32 + v_or_b32 because a
// VOP3 instruction takes no literal operand on this target; the inline form
// keeps one instruction by taking the mask from an SGPR and the fp16 exponent
// bits from a VGPR (one scalar operand per VALU instruction).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(bits));
    return r;
}

__device__ __forceinline__ half8_t dequant_q4(uint32_t w) {
    const uint32_t w8 = w >> 8, e = 0x64006400u;
    const half2_t lo_a = __builtin_bit_cast(half2_t, and_or(w, 0x000F000Fu, e));
    const half2_t hi_a = __builtin_bit_cast(half2_t, and_or(w, 0x00F000F0u, e));
    const half2_t lo_b = __builtin_bit_cast(half2_t, and_or(w8, 0x000F000Fu, e));
    const half2_t hi_b = __builtin_bit_cast(half2_t, and_or(w8, 0x00F000F0u, e));
    const half2_t k1032 = {(_Float16)1032.f, (_Float16)1032.f};
    const half2_t r16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2_t k72 = {(_Float16)-72.f, (_Float16)-72.f};
    const half2_t e04 = lo_a - k1032;
    const half2_t e15 = __builtin_elementwise_fma(hi_a, r16, k72);
    const half2_t e26 = lo_b - k1032;
    const half2_t e37 = __builtin_elementwise_fma(hi_b, r16, k72);
    return half8_t{e04[0], e04[1], e15[0], e15[1], e26[0], e26[1], e37[0], e37[1]};
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

// FP8 (OCP E4M3): two dwords = codes of elements 0..7 -> fp16, exactly (E4M3
// values are a subset of fp16), in element order.  v_cvt_scalef32_pk_f16_fp8
// converts two codes (bytes 0,1 or 2,3 of a dword) at a time; scale 1.
__device__ __forceinline__ half8_t dequant_fp8(uint32_t d0, uint32_t d1) {
    const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
    const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
    const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
    const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
    return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Q6K: elements 0..7 of a group (low 4 bits n in one dword, as Q4; high 2
// bits t at bits 2e of h16) with sub-scale sc -> two fp16 operands whose sum
// is sc * (q - 32), q = 16 t + n, in Q4's order [0, 4, 1, 5, 2, 6, 3, 7]:
//   a2 = sc * n            (|.| <= 128 * 15 < 2048: exact in fp16)
//   a1 = 16 sc (t - 2)     (|.| <= 4096, a multiple of 16: exact)
// Nibbles land in fp16 mantissas as 1024 + n (low) or 1024 + 16 n (high).
// Low: (x - 1024) * sc.  High: one fused multiply-add (1024 + 16 n) sc/16 -
// 64 sc, a single rounding of an exactly representable value (the same form
// for the low nibbles would need the constant 1024 sc, past fp16's range for
// |sc| > 63).  For a1 the 2-bit fields of elements e and e + 4 are brought 16
// bits apart (h16 | h16 << 8), dropped into the mantissas of 1024 + t, then
// (x - 1026) * 16 sc.
__device__ __forceinline__ void dequant_q6k(uint32_t nib, uint32_t h16, _Float16 sc, half8_t &a1,
                                            half8_t &a2) {
    const half2_t s2 = {sc, sc};
    const half2_t k1024 = {(_Float16)1024.f, (_Float16)1024.f};
    const half2_t s_16 = s2 * half2_t{(_Float16)0.0625f, (_Float16)0.0625f};
    const half2_t s_64 = s2 * half2_t{(_Float16)-64.f, (_Float16)-64.f};
    const half2_t s_t = s2 * half2_t{(_Float16)16.f, (_Float16)16.f};
    const uint32_t e = 0x64006400u, w8 = nib >> 8;
    const half2_t p04 = (__builtin_bit_cast(half2_t, and_or(nib, 0x000F000Fu, e)) - k1024) * s2;
    const half2_t p15 = __builtin_elementwise_fma(
        __builtin_bit_cast(half2_t, and_or(nib, 0x00F000F0u, e)), s_16, s_64);
    const half2_t p26 = (__builtin_bit_cast(half2_t, and_or(w8, 0x000F000Fu, e)) - k1024) * s2;
    const half2_t p37 = __builtin_elementwise_fma(
        __builtin_bit_cast(half2_t, and_or(w8, 0x00F000F0u, e)), s_16, s_64);
    a2 = half8_t{p04[0], p04[1], p15[0], p15[1], p26[0], p26[1], p37[0], p37[1]};
    const uint32_t y = h16 | (h16 << 8);
    const half2_t k1026 = {(_Float16)1026.f, (_Float16)1026.f};
    const half2_t t0 = (__builtin_bit_cast(half2_t, and_or(y, 0x00030003u, e)) - k1026) * s_t;
    const half2_t t1 = (__builtin_bit_cast(half2_t, and_or(y >> 2, 0x00030003u, e)) - k1026) * s_t;
    const half2_t t2 = (__builtin_bit_cast(half2_t, and_or(y >> 4, 0x00030003u, e)) - k1026) * s_t;
    const half2_t t3 = (__builtin_bit_cast(half2_t, and_or(y >> 6, 0x00030003u, e)) - k1026) * s_t;
    a1 = half8_t{t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
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

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes of global memory -> LDS at byte address `lds` + 16 * lane
// (LDS-DMA).  `lds` must be the same for the whole wave.  Issued as inline
// assembly on purpose: the compiler cannot tell which LDS buffer a DMA fills
// and would otherwise wait for every DMA in flight (vmcnt(0)) before any LDS
// read, serialising the pipeline.  The caller waits for its DMA explicitly
// (wait_vm) before the barrier that publishes the buffer.  M0 holds the LDS
// address; s_nop covers the M0 -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds), "v"(src)
        : "memory", "m0");
}
__device__ __forceinline__ void dma16(const void *src, void *lds) {
    dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(lds)));
}

// Waits until at most N vector-memory instructions of this wave are in
// flight (s_waitcnt vmcnt(N); expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS barrier without a memory fence.  A fence would wait for every vector
// memory operation in flight (vmcnt(0)), including the weight loads issued
// for later chunks; instead the caller waits for exactly the LDS-DMA it needs
// (wait_vm) and this waits for the wave's own LDS reads (lgkmcnt(0)).  The
// asm "memory" clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

template <int FMT, int CT, int RPW, int NW>
struct QGemv {
    using F = TileFmt<FMT>;
    static constexpr int NB = F::NB, TB = F::TB;
    static constexpr int FRAG = NB * CT * 2;        // 1 KiB image fragments per K tile
    static constexpr int SB = TB - F::SO;           // scale bytes per tile
    static constexpr bool Q6 = FMT == RRA_Q6K;      // high-bit plane, sub-scales
    static constexpr int WL = Q6 ? 2 : 1;           // weight loads per row tile
    static constexpr int SCH = NW * RPW * SB / 16;  // 16-byte scale pieces per K tile
    static constexpr int XB = FRAG * 1024;          // image bytes per K tile
    static constexpr int XDW = (FRAG + NW - 1) / NW;  // image DMAs per wave per K tile
    static constexpr int SCW = (SCH + 63) / 64;     // waves that DMA one scale piece each
    static constexpr int SCB = SCW * 1024;          // scale bytes per LDS buffer
    static_assert(SCW <= NW, "scale DMA split over the waves");
    // fragment wave + NW * j exists (every wave has XDW when NW divides FRAG)
    __device__ __forceinline__ bool has_frag(int j) const {
        return FRAG % NW == 0 || wave + NW * j < FRAG;
    }
    struct Ring {
        uint4 q[RPW];  // this lane's 16 B of each row tile (Q6K: the low 4 bits)
        uint2 h[RPW];  // Q6K: this lane's 8 B of the high 2-bit plane
    };
    typedef floatx4 Acc[RPW][CT];

    const uint8_t *wt, *ximg;
    int lane, g, wave, n_rt, rt_wg, rt0, nkt, kt_begin, kt_end;

    // LDS-DMA of K tile kt_begin + c: XDW image fragments per wave, and the
    // workgroup's scales (waves < SCW, 64 pieces each).  A tile past the split end (the look-ahead
    // of the last step, never computed) is clamped to the last valid one.
    __device__ __forceinline__ void stage(int c, uint8_t *xd, uint8_t *sd) const {
        const int kt = min(kt_begin + c, kt_end - 1);
#pragma unroll
        for (int j = 0; j < XDW; ++j) {
            const int f = wave + NW * j;
            if (has_frag(j)) dma16(ximg + ((size_t)kt * FRAG + f) * 1024 + lane * 16, xd + f * 1024);
        }
        stage_scales(c, sd);
    }
    // The scales part of stage() alone.
    __device__ __forceinline__ void stage_scales(int c, uint8_t *sd) const {
        const int kt = min(kt_begin + c, kt_end - 1);
        if (wave < SCW) {  // piece e -> (row tile, piece)
            const int e = min(wave * 64 + lane, SCH - 1);
            const int piece = e % (SB / 16), rr = e / (SB / 16);
            const int rt = min(rt_wg + rr, n_rt - 1);
            dma16(wt + ((size_t)rt * nkt + kt) * TB + F::SO + piece * 16, sd + wave * 1024);
        }
    }

    // Addresses of one K tile for this lane; the next tile's are a constant
    // stride away, so the main loop only adds (no clamping: it never looks
    // past the split's last tile).
    struct Cursor {
        const uint8_t *x;       // image fragment `wave` of the tile, this lane's 16 B
        const uint8_t *s;       // scale piece of this lane (waves < SCW)
        const uint8_t *w[RPW];  // this lane's 16 B of each of the wave's row tiles
    };
    __device__ __forceinline__ Cursor cursor(int c) const {
        Cursor k;
        const int kt = kt_begin + c;
        k.x = ximg + ((size_t)kt * FRAG + wave) * 1024 + lane * 16;
        const int e = min(wave * 64 + lane, SCH - 1);
        const int rts = min(rt_wg + e / (SB / 16), n_rt - 1);
        k.s = wt + ((size_t)rts * nkt + kt) * TB + F::SO + (e % (SB / 16)) * 16;
#pragma unroll
        for (int r = 0; r < RPW; ++r)
            k.w[r] = wt + ((size_t)min(rt0 + r, n_rt - 1) * nkt + kt) * TB + lane * 16;
        return k;
    }
    __device__ __forceinline__ void advance(Cursor &k) const {
        k.x += FRAG * 1024;
        k.s += TB;
#pragma unroll
        for (int r = 0; r < RPW; ++r) k.w[r] += TB;
    }
    // stage()/issue() at a cursor; xd, sd are LDS byte addresses of the buffers.
    __device__ __forceinline__ void stage_at(const Cursor &k, uint32_t xd, uint32_t sd) const {
#pragma unroll
        for (int j = 0; j < XDW; ++j)
            if (has_frag(j)) dma16(k.x + (size_t)NW * j * 1024, xd + (uint32_t)(wave + NW * j) * 1024);
        if (wave < SCW) dma16(k.s, sd + (uint32_t)wave * 1024);
    }
    __device__ __forceinline__ void issue_at(const Cursor &k, Ring &q) const {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            q.q[r] = ldnt16(k.w[r]);
            if (Q6) q.h[r] = ldnt8(k.w[r] + 1024 - 8 * lane);
        }
    }

    // Quantised values of K tile kt_begin + c for this wave's row tiles,
    // straight into registers (no arithmetic on them here: that would make
    // the wave wait for the load at once).
    __device__ __forceinline__ void issue(Ring &q, int c) const {
        const int kt = min(kt_begin + c, kt_end - 1);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int rt = min(rt0 + r, n_rt - 1);
            const uint8_t *t = wt + ((size_t)rt * nkt + kt) * TB;
            q.q[r] = ldnt16(t + lane * 16);
            if (Q6) q.h[r] = ldnt8(t + 1024 + lane * 8);
        }
    }

    // Dequantise + MFMA + block scale of one K tile (always one inside the
    // split).  Branch-free: row tiles past N repeat the last tile's values
    // (never stored).
    __device__ __forceinline__ void compute(const Ring &q, const uint8_t *xs, const uint8_t *ss,
                                            Acc &acc) const {
        if constexpr (Q6)
            compute_q6k(q, xs, ss, acc);
        else
            compute_blocks(q, xs, ss, acc);
        // The tile's accumulator updates stay here: left free, the compiler
        // sinks them past the step's barrier, keeping every MFMA result of the
        // tile live (registers) and leaving the matrix unit idle meanwhile.
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int cc = 0; cc < CT; ++cc) asm volatile("" : "+v"(acc[r][cc]));
    }

    // B fragments (hi, lo per column tile) of block b of the staged tile.
    __device__ __forceinline__ void load_b(const uint8_t *xs, int b, half8_t (&Bh)[CT],
                                           half8_t (&Bl)[CT]) const {
        const int slot = frag_slot<F::IMG>(lane >> 4, lane & 15, b);
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) {
            Bh[cc] = *reinterpret_cast<const half8_t *>(xs + ((b * CT + cc) * 2 + 0) * 1024 + slot * 16);
            Bl[cc] = *reinterpret_cast<const half8_t *>(xs + ((b * CT + cc) * 2 + 1) * 1024 + slot * 16);
        }
    }

    // Q8 / Q4 / FP8: one fp16 scale per (row, block of 32), applied to each
    // block's MFMA result in fp32.
    __device__ __forceinline__ void compute_blocks(const Ring &q, const uint8_t *xs,
                                                   const uint8_t *ss, Acc &acc) const {
        // scales of this wave's row tiles: rows 4g+i, blocks b at (g, i, b)
        _Float16 sh[RPW][4 * NB];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const uint8_t *sp = ss + (wave * RPW + r) * SB;
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
        if constexpr (CT > 2) {
            // prompt chunks (4 or 8 column tiles): the dequantised block stays
            // in registers while the column tiles' B fragments are read one
            // tile at a time (all of them at once would take 16 CT registers)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                asm volatile("" ::: "memory");
                half8_t a[RPW];
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    const uint4 qv = q.q[r];
                    a[r] = (FMT == RRA_Q4)    ? dequant_q4(u32_at(qv, b))
                           : (FMT == RRA_FP8) ? dequant_fp8(u32_at(qv, 2 * b), u32_at(qv, 2 * b + 1))
                                              : dequant_q8(u32_at(qv, 2 * b), u32_at(qv, 2 * b + 1));
                }
                const int slot = frag_slot<F::IMG>(lane >> 4, lane & 15, b);
#pragma unroll
                for (int cc = 0; cc < CT; ++cc) {
                    const half8_t bh = *reinterpret_cast<const half8_t *>(
                        xs + ((b * CT + cc) * 2 + 0) * 1024 + slot * 16);
                    const half8_t bl = *reinterpret_cast<const half8_t *>(
                        xs + ((b * CT + cc) * 2 + 1) * 1024 + slot * 16);
#pragma unroll
                    for (int r = 0; r < RPW; ++r) {
                        floatx4 tt = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            a[r], bh, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        tt = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[r], bl, tt, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[r][cc][i] = fmaf((float)sh[r][i * NB + b], tt[i], acc[r][cc][i]);
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            // one block's B fragments at a time (a compiler memory barrier keeps
            // all four from being loaded up front, which costs registers)
            asm volatile("" ::: "memory");
            half8_t Bh[CT], Bl[CT];
            load_b(xs, b, Bh, Bl);
            half8_t a[RPW];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const uint4 qv = q.q[r];
                a[r] = (FMT == RRA_Q4)    ? dequant_q4(u32_at(qv, b))
                       : (FMT == RRA_FP8) ? dequant_fp8(u32_at(qv, 2 * b), u32_at(qv, 2 * b + 1))
                                          : dequant_q8(u32_at(qv, 2 * b), u32_at(qv, 2 * b + 1));
            }
            floatx4 tt[RPW][CT];
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int cc = 0; cc < CT; ++cc)
                    tt[r][cc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        a[r], Bh[cc], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int cc = 0; cc < CT; ++cc)
                    tt[r][cc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[r], Bl[cc], tt[r][cc], 0, 0, 0);
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int cc = 0; cc < CT; ++cc)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[r][cc][i] = fmaf((float)sh[r][i * NB + b], tt[r][cc][i], acc[r][cc][i]);
        }
    }

    // Q6K: the int8 sub-scale is folded exactly into the fp16 operands
    // (dequant_q6k), so the MFMAs accumulate the whole tile and d is applied
    // once per tile.  Lane (j, r) needs the sub-scale of row r, sub-block
    // 2b + j/2 of its half super-block: one dword per row tile holds blocks
    // 0..3; the MFMA result rows 4g + i take d of those rows.
    __device__ __forceinline__ void compute_q6k(const Ring &q, const uint8_t *xs,
                                                const uint8_t *ss, Acc &acc) const {
        uint32_t scw[RPW];
        _Float16 dv[RPW][4];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const uint8_t *sp = ss + (wave * RPW + r) * SB;
            scw[r] = *reinterpret_cast<const uint32_t *>(sp + (((lane >> 5) * 16 + (lane & 15)) * 4));
            const uint2 d2 = *reinterpret_cast<const uint2 *>(sp + 128 + 8 * g);
            const half2_t d01 = __builtin_bit_cast(half2_t, d2.x), d23 = __builtin_bit_cast(half2_t, d2.y);
            dv[r][0] = d01[0];
            dv[r][1] = d01[1];
            dv[r][2] = d23[0];
            dv[r][3] = d23[1];
        }
        floatx4 tt[RPW][CT];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int cc = 0; cc < CT; ++cc) tt[r][cc] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            asm volatile("" ::: "memory");
            half8_t Bh[CT], Bl[CT];
            load_b(xs, b, Bh, Bl);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const uint32_t hw = (b < 2) ? q.h[r].x : q.h[r].y;
                const uint32_t h16 = (b & 1) ? (hw >> 16) : (hw & 0xFFFFu);
                const _Float16 sc = (_Float16)(int)(int8_t)(scw[r] >> (8 * b));
                half8_t a1, a2;
                dequant_q6k(u32_at(q.q[r], b), h16, sc, a1, a2);
#pragma unroll
                for (int cc = 0; cc < CT; ++cc) {
                    floatx4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, Bh[cc], tt[r][cc], 0, 0, 0);
                    t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, Bl[cc], t, 0, 0, 0);
                    t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bh[cc], t, 0, 0, 0);
                    tt[r][cc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bl[cc], t, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int cc = 0; cc < CT; ++cc)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[r][cc][i] = fmaf((float)dv[r][i], tt[r][cc][i], acc[r][cc][i]);
    }

    // One pipeline iteration: DMA of the next tile (cursor kn) into xw/sw and
    // its weight loads into qf, compute of the current tile from qc and xr/sr,
    // then a wait for everything in flight (the next tile's data) and a
    // barrier.  The DMA is invisible to the compiler (inline asm); the full
    // wait keeps its own count of the register loads exact.
    __device__ __forceinline__ void step(const Ring &qc, Ring &qf, const Cursor &kn, uint32_t xw,
                                         uint32_t sw, const uint8_t *xr, const uint8_t *sr,
                                         Acc &acc) const {
        stage_at(kn, xw, sw);
        __builtin_amdgcn_sched_barrier(0);
        issue_at(kn, qf);
        __builtin_amdgcn_sched_barrier(0);
        compute(qc, xr, sr, acc);
        wait_vm<0>();
        lds_barrier();
    }

    // RMSNorm inputs: the first SSP partial sums of squares of this lane's
    // columns, loaded early (clamped, fixed count) and summed after a wait.
    static constexpr int SSP = 8;
    __device__ __forceinline__ void load_ss(const NormIn &nrm, int M, float (&sv)[CT][SSP]) const {
        if (!nrm.ss) return;
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) {
            const int m = min(16 * cc + (lane & 15), M - 1);
#pragma unroll
            for (int q = 0; q < SSP; ++q)
                sv[cc][q] = nrm.ss[(size_t)m * nrm.nparts + min(q, nrm.nparts - 1)];
        }
    }
    __device__ __forceinline__ void sum_ss(const NormIn &nrm, const float (&sv)[CT][SSP],
                                           float (&sq)[CT]) const {
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) {
            sq[cc] = 0.f;
            if (nrm.ss) {
#pragma unroll
                for (int q = 0; q < SSP; ++q) sq[cc] += (q < nrm.nparts) ? sv[cc][q] : 0.f;
            }
        }
    }

    // Result layout of a 16x16 MFMA: lane holds rows 4g..4g+3 of column
    // lane%16.  Multiplies by inv[m] (RMSNorm, when nrm.ss is set).
    // RMSNorm factor of column tile cc's row m (1 without a norm)
    __device__ __forceinline__ float col_inv(int cc, int m, const float (&sq)[CT],
                                             const NormIn &nrm, int K) const {
        float iv = 1.f;
        if (nrm.ss) {
            float t = sq[cc];
            for (int q = SSP; q < nrm.nparts; ++q) t += nrm.ss[(size_t)m * nrm.nparts + q];
            iv = 1.0f / sqrtf(t / (float)K + nrm.eps);
        }
        return iv;
    }
    // Greedy-argmax partial of the outputs store() writes (the same products,
    // acc * iv): per row m, the largest value with the lowest index among this
    // workgroup's output rows, to ao.val/idx[m * ao.stride + blockIdx.x].
    // Lanes 16 apart hold the same row's columns; the waves meet in LDS.
    // Every thread of the workgroup calls it (it synchronises the block).
    __device__ __forceinline__ void store_argmax(const Acc &acc, const float (&sq)[CT],
                                                 const NormIn &nrm, int M, int N, int K,
                                                 const ArgOut &ao, float (*av)[16 * CT],
                                                 uint32_t (*ai)[16 * CT]) const {
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) {
            const int m = 16 * cc + (lane & 15);
            float best = -INFINITY;
            uint32_t bidx = 0xFFFFFFFFu;
            if (m < M) {
                const float iv = col_inv(cc, m, sq, nrm, K);
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    const int rt = rt0 + r;
                    if (rt >= n_rt) continue;
                    const int row0 = rt * 16 + 4 * g;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (row0 + i < N)
                            arg_combine(best, bidx, acc[r][cc][i] * iv, (uint32_t)(row0 + i));
                }
            }
            arg_combine(best, bidx, __shfl_xor(best, 16, 64), __shfl_xor(bidx, 16, 64));
            arg_combine(best, bidx, __shfl_xor(best, 32, 64), __shfl_xor(bidx, 32, 64));
            if (g == 0) {
                av[wave][16 * cc + lane] = best;
                ai[wave][16 * cc + lane] = bidx;
            }
        }
        __syncthreads();
        if (wave == 0 && lane < 16 * CT && lane < M) {
            float best = av[0][lane];
            uint32_t bidx = ai[0][lane];
            for (int w = 1; w < NW; ++w) arg_combine(best, bidx, av[w][lane], ai[w][lane]);
            ao.val[(size_t)lane * ao.stride + blockIdx.x] = best;
            ao.idx[(size_t)lane * ao.stride + blockIdx.x] = bidx;
        }
    }
    __device__ __forceinline__ void store(const Acc &acc, const float (&sq)[CT], const NormIn &nrm,
                                          float *o, int M, int N, int K) const {
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) {
            const int m = 16 * cc + (lane & 15);
            if (m >= M) continue;
            const float iv = col_inv(cc, m, sq, nrm, K);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int rt = rt0 + r;
                if (rt >= n_rt) continue;
                // rows 4g .. 4g + 3: one 16-byte store when whole and aligned
                const int row0 = rt * 16 + 4 * g;
                float *dst = o + (size_t)m * N + row0;
                if (((N & 3) | (reinterpret_cast<uintptr_t>(o) & 15)) == 0 && row0 + 4 <= N) {
                    *reinterpret_cast<float4 *>(dst) =
                        make_float4(acc[r][cc][0] * iv, acc[r][cc][1] * iv, acc[r][cc][2] * iv,
                                    acc[r][cc][3] * iv);
                    continue;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (row0 + i < N) dst[i] = acc[r][cc][i] * iv;
            }
        }
    }

    __device__ __forceinline__ void init(const uint8_t *wt_, const uint8_t *ximg_, int N, int nkt_,
                                         int kt_per_split) {
        wt = wt_;
        ximg = ximg_;
        lane = threadIdx.x & 63;
        g = lane >> 4;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        n_rt = (N + 15) >> 4;
        rt_wg = blockIdx.x * NW * RPW;
        rt0 = rt_wg + wave * RPW;
        nkt = nkt_;
        kt_begin = blockIdx.y * kt_per_split;
        kt_end = min(nkt, kt_begin + kt_per_split);
    }
};

// Grid (row blocks of 16*NW*RPW rows, K splits); NW waves; wave w owns row
// tiles [(blockIdx.x*NW + w)*RPW, +RPW).  All NW waves share each staged
// activation tile, so more waves per workgroup move fewer image bytes per
// weight byte.  The split's K tiles are
// processed in a two-stage software pipeline (QGemv::step): while tile c is
// computed from registers and one LDS buffer, tile c+1's weights load into
// the other register set and its activation image and scales into the other
// LDS buffer by LDS-DMA.  Outputs are multiplied by inv[m] (RMSNorm, when
// nrm.ss is set) and written to out[split][m][n] (split_stride floats apart).
template <int FMT, int CT, int RPW, int NW>
__global__ __launch_bounds__(64 * NW) void gemv_q_kernel(const uint8_t *__restrict__ wt,
                                                         const uint8_t *__restrict__ ximg,
                                                         float *__restrict__ out, int M, int N,
                                                         int K, int nkt, int kt_per_split,
                                                         long long split_stride, NormIn nrm,
                                                         ArgOut ao) {
    using G = QGemv<FMT, CT, RPW, NW>;
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][G::XB];
    __shared__ __attribute__((aligned(16))) uint8_t sl[2][G::SCB];
    // argmax partials (decode batches only: CT <= 2)
    __shared__ float av[CT <= 2 ? NW : 1][16 * CT];
    __shared__ uint32_t ai[CT <= 2 ? NW : 1][16 * CT];

    G p;
    p.init(wt, ximg, N, nkt, kt_per_split);
    const int nch = p.kt_end - p.kt_begin;

    float sv[CT][G::SSP];
    p.load_ss(nrm, M, sv);

    typename G::Acc acc;
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) acc[r][cc] = floatx4{0.f, 0.f, 0.f, 0.f};

    typename G::Ring q0, q1;
    p.stage(0, xs[0], sl[0]);
    __builtin_amdgcn_sched_barrier(0);
    p.issue(q0, 0);
    wait_vm<0>();
    lds_barrier();
    float sq[CT];
    p.sum_ss(nrm, sv, sq);
    // Tile c lives in buffer c & 1 and register set c & 1.  Every step
    // prefetches a tile inside the split; the last tile is computed alone.
    const uint32_t x0 = lds_addr(xs[0]), x1 = lds_addr(xs[1]);
    const uint32_t s0 = lds_addr(sl[0]), s1 = lds_addr(sl[1]);
    typename G::Cursor kn = p.cursor(nch > 1 ? 1 : 0);
    int c = 0;
    for (; c + 2 < nch; c += 2) {
        p.step(q0, q1, kn, x1, s1, xs[0], sl[0], acc);
        p.advance(kn);
        p.step(q1, q0, kn, x0, s0, xs[1], sl[1], acc);
        p.advance(kn);
    }
    if (c + 1 < nch) {
        p.step(q0, q1, kn, x1, s1, xs[0], sl[0], acc);
        p.compute(q1, xs[1], sl[1], acc);
    } else if (c < nch) {
        p.compute(q0, xs[0], sl[0], acc);
    }
    p.store(acc, sq, nrm, out + (size_t)blockIdx.y * split_stride, M, N, K);
    if constexpr (CT <= 2)
        if (ao.val) p.store_argmax(acc, sq, nrm, M, N, K, ao, av, ai);  // uniform: one K split
}

// Short splits (at most NT K tiles): every K tile's image, scales and
// weights are requested up front -- all LDS-DMA first, then the weight
// loads -- so the workgroup pays one memory round trip instead of one per
// tile.  Tiles past the split end are clamped copies, never computed.
// Because no DMA follows a weight load, the compiler's own count of the
// loads in flight matches the hardware's and it adds no waits.
// Prologues (GemvPrologue): the image of K tiles kt_begin + t (t < nch) of
// this workgroup's split, built in LDS (xs[t]) for rows m < M, one column
// tile (M <= 16), four waves.  PRO: kProSwiglu, or kProAttn + HD.
template <int IMG, int KT, int XB>
__device__ __forceinline__ void prologue_swiglu(const GemvPrologue &pro, int M, int kt_begin,
                                                int nch, uint8_t (*xs)[XB], float *red) {
    // groups of 8 columns: gidx = (m * nch + t) * (KT / 8) + kk
    constexpr int GPT = KT / 8;
    const int total = M * nch * GPT, inter = pro.n;
    for (int g0 = 0; g0 < total; g0 += 64) {
        const int gidx = g0 + (threadIdx.x & 63);
        const bool valid = gidx < total;
        const int gc = valid ? gidx : 0;
        const int kk = gc % GPT, t = (gc / GPT) % nch, m = gc / (GPT * nch);
        const int k0 = (kt_begin + t) * KT + 8 * kk;
        const size_t gi = (size_t)m * 2 * inter + k0;
        float acc[2][8];
        const float *const pp[2] = {pro.part + gi, pro.part + gi + inter};
        group_split_sum<2>(pp, valid && k0 < inter, pro.split, pro.stride, acc, red);
        if (threadIdx.x < 64 && valid) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = k0 < inter ? swiglu1(acc[0][e], acc[1][e]) : 0.f;
            if (!write_frag8_tile<IMG>(xs[t], 1, m, 8 * kk, v)) report_error(pro.err, kErrRange);
        }
        __syncthreads();  // `red` is reused by the next pass
    }
}

template <int IMG, int KT, int XB, int HD>
__device__ __forceinline__ void prologue_attn(const GemvPrologue &pro, int M, int kt_begin,
                                              int nch, uint8_t (*xs)[XB], float *so) {
    // heads overlapping columns [kt_begin KT, (kt_begin + nch) KT), one wave
    // per (sequence, head) pair; so = 4 waves x HD floats.
    constexpr int PER = HD / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int k_lo = kt_begin * KT, k_hi = (kt_begin + nch) * KT, nqhd = pro.n * HD;
    const int h_lo = k_lo / HD, h_hi = min(pro.n, (k_hi + HD - 1) / HD);
    const int pairs = M * max(0, h_hi - h_lo);
    float *sw = so + wave * HD;
    for (int pidx = wave; pidx < pairs; pidx += 4) {
        const int m = pidx / (h_hi - h_lo), h = h_lo + pidx % (h_hi - h_lo);
        const int L = (int)min(pro.seq_len[m], (uint32_t)pro.max_len);
        float acc[PER];
        fd_combine<HD>(pro.part, pro.lse, m, h, pro.n, pro.nc_max, L, lane, acc);
#pragma unroll
        for (int j = 0; j < PER; ++j) sw[lane + 64 * j] = acc[j];
        __builtin_amdgcn_wave_barrier();
        if (lane < HD / 8) {
            const int k0 = h * HD + lane * 8;
            if (k0 >= k_lo && k0 < k_hi) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = sw[lane * 8 + e];
                if (!write_frag8_tile<IMG>(xs[k0 / KT - kt_begin], 1, m, k0 % KT, v))
                    report_error(pro.err, kErrRange);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    // zeros for the groups in [nq hd, kpad)
    for (int gidx = threadIdx.x; gidx < M * nch * (KT / 8); gidx += blockDim.x) {
        const int kk = gidx % (KT / 8), t = (gidx / (KT / 8)) % nch, m = gidx / (nch * (KT / 8));
        if ((kt_begin + t) * KT + 8 * kk >= nqhd) {
            const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            write_frag8_tile<IMG>(xs[t], 1, m, 8 * kk, z);
        }
    }
}

// The residual step for rows m < M (residual_ss_kernel's work, with its
// thread mapping and order of operations): for each (row, 512-column chunk)
// pair, lane g of the four waves holds columns chunk*512 + 8g .. + 7, the
// waves share the split sum (group_split_sum), and wave 0 forms
// x_out = x_in + sum, the chunk's sum of squares (a wave sum, as the block sum
// of the separate kernel: the other waves add zeros) and x_out * gamma, whose
// columns in this split's K tiles go to the image.  tsum[m] = the sum over
// the row's chunks, in chunk order.  parts: M * ceil(n/512) floats.
template <int IMG, int KT, int XB>
__device__ __forceinline__ void prologue_resid(const GemvPrologue &pro, int M, int kt_begin,
                                               int nch, uint8_t (*xs)[XB], float *red,
                                               float *parts, float *tsum) {
    const int H = pro.n, np = ss_parts(H), pairs = M * np;
    const int lane = threadIdx.x & 63;
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
    const int k_lo = kt_begin * KT, k_hi = (kt_begin + nch) * KT;
    for (int p0 = 0; p0 < pairs; p0 += 2) {
        int k0[2];
        size_t base[2];
        const float *pp[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int pidx = min(p0 + v, pairs - 1), m = pidx / np, ch = pidx % np;
            k0[v] = ch * 512 + lane * 8;
            base[v] = (size_t)m * H + (k0[v] < H ? k0[v] : 0);  // clamped: never used
            pp[v] = pro.part + base[v];
        }
        float xv[2][8], gm[2][8];
        if (threadIdx.x < 64) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                load8(pro.x_in + base[v], xv[v]);
                load8(pro.gamma + (k0[v] < H ? k0[v] : 0), gm[v]);
            }
        }
        float acc[2][8];
        group_split_sum<2>(pp, true, pro.split, pro.stride, acc, red);
        if (threadIdx.x < 64) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int pidx = p0 + v;
                if (pidx >= pairs) break;
                const int m = pidx / np;
                float sq = 0.f;
                if (k0[v] < H) {
                    float gv[8];
                    resid8(xv[v], acc[v], true, gm[v], gv, sq);
                    if (writer) store8(pro.x_out + base[v], xv[v]);
                    if (k0[v] >= k_lo && k0[v] < k_hi)
                        if (!write_frag8_tile<IMG>(xs[k0[v] / KT - kt_begin], 1, m, k0[v] % KT, gv))
                            report_error(pro.err, kErrRange);
                }
                sq = wave_sum(sq);
                if (lane == 0) parts[pidx] = 0.f + sq;
            }
        }
        __syncthreads();  // `red` is reused by the next pass; parts complete
    }
    if ((int)threadIdx.x < M) {
        float t = 0.f;
        for (int c = 0; c < np; ++c) t += parts[threadIdx.x * np + c];
        tsum[threadIdx.x] = t;
    }
    // zeros for the groups in [H, kpad)
    for (int gidx = threadIdx.x; gidx < M * nch * (KT / 8); gidx += blockDim.x) {
        const int kk = gidx % (KT / 8), t = (gidx / (KT / 8)) % nch, m = gidx / (nch * (KT / 8));
        if ((kt_begin + t) * KT + 8 * kk >= H) {
            const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            write_frag8_tile<IMG>(xs[t], 1, m, 8 * kk, z);
        }
    }
}

// Prompt-chunk GEMM (up to 128 rows of x, 8 column tiles): the decode
// GEMV's operand flow with the work split two ways.  8 waves = 4 row groups
// x 2 column groups; wave (rg, cg) owns row tiles 4 rg .. 4 rg + 3 of the
// workgroup's 16 (256 output rows) and column tiles 4 cg .. 4 cg + 3.  Each B
// fragment read from LDS then feeds 4 row tiles and each dequantised weight
// block 4 column tiles, so a matrix-core op costs a quarter of an LDS read
// (one row tile per wave would cost a whole one).  The two column groups
// load the same weights (the second read is an L2 hit) and each dequantise
// them.  K tiles are double-buffered as in gemv_q_kernel: the next tile's
// image and scales go to LDS by LDS-DMA and its weights to registers while
// the current one is computed.  Outputs are multiplied by inv[m] (RMSNorm,
// when nrm.ss is set) and written to out[split][m][n].
template <int FMT>
struct QGemm {
    using F = TileFmt<FMT>;
    static constexpr int NB = F::NB, TB = F::TB, SB = TB - F::SO;
    static constexpr int CT = 8, NW = 8, RG = 4, RPW = 4, CW = 4;  // CW column tiles per wave
    static constexpr int FRAG = NB * CT * 2;      // 1 KiB image fragments per K tile
    static constexpr int XB = FRAG * 1024;
    static constexpr int XDW = FRAG / NW;         // image DMAs per wave per K tile
    static constexpr int SCH = RG * RPW * SB / 16;  // 16-byte scale pieces per K tile
    static constexpr int SCW = (SCH + 63) / 64;     // waves that DMA scale pieces
    static_assert(FRAG % NW == 0 && SCW <= NW, "DMA split");
    typedef floatx4 Acc[RPW][CW];

    const uint8_t *wt, *ximg;
    int lane, g, wave, rg, cg, n_rt, rt_wg, rt0, nkt, kt_begin, kt_end;

    __device__ __forceinline__ void init(const uint8_t *wt_, const uint8_t *ximg_, int N, int nkt_,
                                         int kt_per_split) {
        wt = wt_;
        ximg = ximg_;
        lane = threadIdx.x & 63;
        g = lane >> 4;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rg = wave & (RG - 1);
        cg = wave / RG;
        n_rt = (N + 15) >> 4;
        rt_wg = blockIdx.x * RG * RPW;
        rt0 = rt_wg + rg * RPW;
        nkt = nkt_;
        kt_begin = blockIdx.y * kt_per_split;
        kt_end = min(nkt, kt_begin + kt_per_split);
    }
    // LDS-DMA of K tile kt_begin + c's image and the workgroup's scales
    // (clamped to the split's last tile: the look-ahead past it is never used)
    __device__ __forceinline__ void stage(int c, uint8_t *xd, uint8_t *sd) const {
        const int kt = min(kt_begin + c, kt_end - 1);
#pragma unroll
        for (int j = 0; j < XDW; ++j) {
            const int f = wave + NW * j;
            dma16(ximg + ((size_t)kt * FRAG + f) * 1024 + lane * 16, xd + f * 1024);
        }
        if (wave < SCW) {
            const int e = min(wave * 64 + lane, SCH - 1);
            const int piece = e % (SB / 16), rr = e / (SB / 16);
            const int rt = min(rt_wg + rr, n_rt - 1);
            dma16(wt + ((size_t)rt * nkt + kt) * TB + F::SO + piece * 16, sd + wave * 1024);
        }
    }
    __device__ __forceinline__ void issue(uint4 (&q)[RPW], int c) const {
        const int kt = min(kt_begin + c, kt_end - 1);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int rt = min(rt0 + r, n_rt - 1);
            q[r] = ldnt16(wt + ((size_t)rt * nkt + kt) * TB + lane * 16);
        }
    }
    __device__ __forceinline__ void compute(const uint4 (&q)[RPW], const uint8_t *xs,
                                            const uint8_t *ss, Acc &acc) const {
        // scales of this wave's row tiles: rows 4g + i, blocks b at (g, i, b)
        _Float16 sh[RPW][4 * NB];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const uint8_t *sp = ss + (rg * RPW + r) * SB;
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
            asm volatile("" ::: "memory");
            half8_t a[RPW];
#pragma unroll
            for (int r = 0; r < RPW; ++r)
                a[r] = (FMT == RRA_Q4)    ? dequant_q4(u32_at(q[r], b))
                       : (FMT == RRA_FP8) ? dequant_fp8(u32_at(q[r], 2 * b), u32_at(q[r], 2 * b + 1))
                                          : dequant_q8(u32_at(q[r], 2 * b), u32_at(q[r], 2 * b + 1));
            const int slot = frag_slot<F::IMG>(lane >> 4, lane & 15, b);
#pragma unroll
            for (int cw = 0; cw < CW; ++cw) {
                const int cc = cg * CW + cw;
                const half8_t bh = *reinterpret_cast<const half8_t *>(
                    xs + ((b * CT + cc) * 2 + 0) * 1024 + slot * 16);
                const half8_t bl = *reinterpret_cast<const half8_t *>(
                    xs + ((b * CT + cc) * 2 + 1) * 1024 + slot * 16);
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    floatx4 tt = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        a[r], bh, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    tt = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[r], bl, tt, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[r][cw][i] = fmaf((float)sh[r][i * NB + b], tt[i], acc[r][cw][i]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int cw = 0; cw < CW; ++cw) asm volatile("" : "+v"(acc[r][cw]));
    }
    __device__ __forceinline__ void step(const uint4 (&qc)[RPW], uint4 (&qn)[RPW], int c,
                                         uint8_t *xw, uint8_t *sw, const uint8_t *xr,
                                         const uint8_t *sr, Acc &acc) const {
        stage(c + 1, xw, sw);
        __builtin_amdgcn_sched_barrier(0);
        issue(qn, c + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(qc, xr, sr, acc);
        wait_vm<0>();
        lds_barrier();
    }
};

template <int FMT>
__global__ __launch_bounds__(512) void gemm_q_kernel(const uint8_t *__restrict__ wt,
                                                     const uint8_t *__restrict__ ximg,
                                                     float *__restrict__ out, int M, int N, int K,
                                                     int nkt, int kt_per_split,
                                                     long long split_stride, NormIn nrm) {
    using G = QGemm<FMT>;
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][G::XB];
    __shared__ __attribute__((aligned(16))) uint8_t sl[2][G::SCW * 1024];
    G p;
    p.init(wt, ximg, N, nkt, kt_per_split);
    const int nch = p.kt_end - p.kt_begin;
    typename G::Acc acc;
#pragma unroll
    for (int r = 0; r < G::RPW; ++r)
#pragma unroll
        for (int cw = 0; cw < G::CW; ++cw) acc[r][cw] = floatx4{0.f, 0.f, 0.f, 0.f};
    uint4 q0[G::RPW], q1[G::RPW];
    p.stage(0, xs[0], sl[0]);
    __builtin_amdgcn_sched_barrier(0);
    p.issue(q0, 0);
    wait_vm<0>();
    lds_barrier();
    int c = 0;
    for (; c + 2 < nch; c += 2) {
        p.step(q0, q1, c, xs[1], sl[1], xs[0], sl[0], acc);
        p.step(q1, q0, c + 1, xs[0], sl[0], xs[1], sl[1], acc);
    }
    if (c + 1 < nch) {
        p.step(q0, q1, c, xs[1], sl[1], xs[0], sl[0], acc);
        p.compute(q1, xs[1], sl[1], acc);
    } else if (c < nch) {
        p.compute(q0, xs[0], sl[0], acc);
    }
    // RMSNorm: inv of this lane's columns, then the 16 x 16 result tiles
    // (lane holds rows 4g .. 4g + 3 of column lane % 16: one 16-byte store
    // when the rows are whole and aligned, so the four lanes of a column
    // write its 64 contiguous bytes together)
    float *o = out + (size_t)blockIdx.y * split_stride;
    const bool vec = ((N & 3) | (reinterpret_cast<uintptr_t>(o) & 15)) == 0;
#pragma unroll
    for (int cw = 0; cw < G::CW; ++cw) {
        const int m = 16 * (p.cg * G::CW + cw) + (p.lane & 15);
        if (m >= M) continue;
        float iv = 1.f;
        if (nrm.ss) {
            float t = 0.f;
            for (int qq = 0; qq < nrm.nparts; ++qq) t += nrm.ss[(size_t)m * nrm.nparts + qq];
            iv = 1.0f / sqrtf(t / (float)K + nrm.eps);
        }
#pragma unroll
        for (int r = 0; r < G::RPW; ++r) {
            const int rt = p.rt0 + r;
            if (rt >= p.n_rt) continue;
            const int row0 = rt * 16 + 4 * p.g;
            float *dst = o + (size_t)m * N + row0;
            if (vec && row0 + 4 <= N) {
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(acc[r][cw][0] * iv, acc[r][cw][1] * iv, acc[r][cw][2] * iv,
                                acc[r][cw][3] * iv);
                continue;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (row0 + i < N) dst[i] = acc[r][cw][i] * iv;
        }
    }
}

template <int FMT, int CT, int RPW, int NW, int NT, int PRO = 0>
__global__ __launch_bounds__(64 * NW) void gemv_q_short_kernel(const uint8_t *__restrict__ wt,
                                                               const uint8_t *__restrict__ ximg,
                                                               float *__restrict__ out, int M,
                                                               int N, int K, int nkt,
                                                               int kt_per_split,
                                                               long long split_stride, NormIn nrm,
                                                               GemvPrologue pro) {
    using G = QGemv<FMT, CT, RPW, NW>;
    static_assert(PRO == 0 || (CT == 1 && NW == 4), "prologues build one column tile, 4 waves");
    __shared__ __attribute__((aligned(16))) uint8_t xs[NT][G::XB];
    __shared__ __attribute__((aligned(16))) uint8_t sl[NT][G::SCB];
    constexpr int RED = PRO == kProSwiglu ? 3 * 64 * 16
                        : PRO == kProResid ? 3 * 64 * 16 + 4 * 8 + 4
                        : PRO >= kProAttn  ? 4 * 128
                                           : 1;
    __shared__ float red[RED];

    G p;
    p.init(wt, ximg, N, nkt, kt_per_split);
    const int nch = p.kt_end - p.kt_begin;

    float sv[CT][G::SSP];
    p.load_ss(nrm, M, sv);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (PRO == 0)
            p.stage(t, xs[t], sl[t]);
        else
            p.stage_scales(t, sl[t]);
    }
    __builtin_amdgcn_sched_barrier(0);
    typename G::Ring q[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) p.issue(q[t], t);
    __builtin_amdgcn_sched_barrier(0);

    typename G::Acc acc;
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) acc[r][cc] = floatx4{0.f, 0.f, 0.f, 0.f};

    if constexpr (PRO == kProSwiglu)
        prologue_swiglu<TileFmt<FMT>::IMG, TileFmt<FMT>::KT, G::XB>(pro, M, p.kt_begin, nch, xs, red);
    else if constexpr (PRO == kProAttn)
        prologue_attn<TileFmt<FMT>::IMG, TileFmt<FMT>::KT, G::XB, 64>(pro, M, p.kt_begin, nch, xs, red);
    else if constexpr (PRO == kProAttn + 1)
        prologue_attn<TileFmt<FMT>::IMG, TileFmt<FMT>::KT, G::XB, 128>(pro, M, p.kt_begin, nch, xs, red);
    else if constexpr (PRO == kProResid)
        prologue_resid<TileFmt<FMT>::IMG, TileFmt<FMT>::KT, G::XB>(pro, M, p.kt_begin, nch, xs, red,
                                                                   red + 3 * 64 * 16,
                                                                   red + 3 * 64 * 16 + 4 * 8);
    wait_vm<NT * RPW * G::WL>();  // every DMA landed; weight loads may be in flight
    lds_barrier();
    float sq[CT];
    p.sum_ss(nrm, sv, sq);
    if constexpr (PRO == kProResid) {
        // the norm from the prologue's sums (one total per row, no more parts)
        const float *tsum = red + 3 * 64 * 16 + 4 * 8;
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) sq[cc] = tsum[min(16 * cc + (p.lane & 15), M - 1)];
        nrm = NormIn{tsum, 1, pro.eps};
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < nch) p.compute(q[t], xs[t], sl[t], acc);
    }
    wait_vm<0>();  // nothing in flight when the workgroup ends
    p.store(acc, sq, nrm, out + (size_t)blockIdx.y * split_stride, M, N, K);
}

// The same product on the vector ALUs, for comparison with the matrix-core
// path at small M (rra_batched_gemv_valu): one wave per 16-row tile of the
// tiled layout, lane (j, r) holding row r's bytes of sub-range j of each of
// the tile's blocks; the block's values are converted to fp32 (q or q - 8,
// exact) and multiplied with fp32 x from LDS (the split's K range of all
// rows, staged once per workgroup) in plain fp32 FMAs, the fp16 block scale
// applied per block; the four lanes of a row are summed with cross-lane adds.
// Q4's -8 offset is folded as sum (q - 8) x = sum q x - 8 sum x, with the sum
// of each 8-element group of x staged beside x.
template <int FMT, int MR>
__global__ __launch_bounds__(256) void gemv_valu_kernel(const uint8_t *__restrict__ wt,
                                                        const float *__restrict__ x,
                                                        float *__restrict__ out, int M, int N,
                                                        int K, int nkt, int kt_per_split,
                                                        long long split_stride) {
    using F = TileFmt<FMT>;
    constexpr int KT = F::KT, NB = F::NB, TB = F::TB;
    extern __shared__ __attribute__((aligned(16))) float xs[];  // [MR][kspan], then [MR][kspan / 8]
    const int kt_begin = blockIdx.y * kt_per_split, kt_end = min(nkt, kt_begin + kt_per_split);
    const int k_lo = kt_begin * KT, kspan = kt_per_split * KT;
    float *gs = xs + MR * kspan;
    for (int i = threadIdx.x; i < MR * kspan / 8; i += blockDim.x) {
        const int m = i / (kspan / 8), g8 = i % (kspan / 8), k = k_lo + 8 * g8;
        float v[8];
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[e] = (m < M && k + e < K) ? x[(size_t)m * K + k + e] : 0.f;
            sum += v[e];
        }
        store8(xs + m * kspan + 8 * g8, v);
        gs[m * (kspan / 8) + g8] = sum;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, j = lane >> 4, r = lane & 15;
    const int n_rt = (N + 15) >> 4;
    const int rt = blockIdx.x * 4 + (threadIdx.x >> 6);
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;
    if (rt < n_rt) {
        for (int kt = kt_begin; kt < kt_end; ++kt) {
            const uint8_t *tile = wt + ((size_t)rt * nkt + kt) * TB;
            const uint4 wv = ldnt16(tile + lane * 16);
            const uint16_t *sc = reinterpret_cast<const uint16_t *>(tile + F::SO) + r * NB;
            const int kl = (kt - kt_begin) * KT;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float w[8];
                if (FMT == RRA_Q4) {
                    const uint32_t d = u32_at(wv, b);
                    const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {  // byte u: element 2u (low), 2u + 1 (high)
                        w[2 * u] = (float)((lo >> (8 * u)) & 0xFFu);
                        w[2 * u + 1] = (float)((hi >> (8 * u)) & 0xFFu);
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t d = u32_at(wv, 2 * b + h);
#pragma unroll
                        for (int u = 0; u < 4; ++u) w[4 * h + u] = (float)(int8_t)(d >> (8 * u));
                    }
                }
                const float s = (float)__builtin_bit_cast(_Float16, sc[b]);
                const int k0 = kl + 32 * b + 8 * j;
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    float xv[8];
                    load8(xs + m * kspan + k0, xv);
                    float t = FMT == RRA_Q4 ? -8.f * gs[m * (kspan / 8) + k0 / 8] : 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) t = fmaf(w[e], xv[e], t);
                    acc[m] = fmaf(s, t, acc[m]);
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        float v = acc[m];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        const int row = rt * 16 + r;
        if (j == 0 && m < M && rt < n_rt && row < N)
            out[(size_t)blockIdx.y * split_stride + (size_t)m * N + row] = v;
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

// y = sum over the split planes in plane order, up to 8 loads in flight.
__device__ __forceinline__ float sum_splits(const float *__restrict__ p, int split,
                                           long long stride) {
    float acc = 0.f;
    for (int s0 = 0; s0 < split; s0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = p[(size_t)min(s0 + j, split - 1) * stride];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += (s0 + j < split) ? v[j] : 0.f;
    }
    return acc;
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

// Q6K tile (rt, kt) = half (kt & 1) of super-block kt / 2.  Lane (r, j):
// 16 B of low 4 bits (dword b = the 8 nibbles of elements 32b + 8j + [0, 8) of
// the half, as the planar bytes hold them) at 16 lane; 8 B of high 2-bit fields
// (16 bits per block, blocks 0,1 in the first dword, 2,3 in the second) at
// 1024 + 8 lane.  Sub-scales at 1536: byte ((h * 16 + r) * 4 + b) = sub-block
// 8 (kt & 1) + 2b + h of row r; d of row r at 1664 + 2r.  Rows >= N are zero.
__global__ void repack_q6k_kernel(const uint8_t *__restrict__ codes,
                                  const uint8_t *__restrict__ recs, uint8_t *__restrict__ tiled,
                                  int N, int K, int nkt) {
    const long long tile = blockIdx.x;
    const int lane = threadIdx.x;
    const int rt = (int)(tile / nkt), kt = (int)(tile % nkt);
    uint8_t *dst = tiled + tile * TileFmt<RRA_Q6K>::TB;
    const int nsb = K / 256, sb = kt >> 1, half = kt & 1;
    const int r = lane & 15, j = lane >> 4;
    const int row = rt * 16 + r;
    const bool ok = row < N;
    const uint8_t *cb = codes + ((size_t)(ok ? row : 0) * nsb + sb) * 192;
    uint32_t d[4], h[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int e0 = half * 128 + 32 * b + 8 * j;
        d[b] = ok ? *reinterpret_cast<const uint32_t *>(cb + e0 / 2) : 0u;
        h[b] = ok ? *reinterpret_cast<const uint16_t *>(cb + 128 + e0 / 4) : 0u;
    }
    *reinterpret_cast<uint4 *>(dst + lane * 16) = uint4{d[0], d[1], d[2], d[3]};
    *reinterpret_cast<uint2 *>(dst + 1024 + lane * 8) = uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int idx = 2 * lane + t;  // (hh * 16 + rr) * 4 + bb
        const int hh = idx >> 6, rr = (idx >> 2) & 15, bb = idx & 3;
        const int srow = rt * 16 + rr;
        dst[1536 + idx] = srow < N ? recs[((size_t)srow * nsb + sb) * 18 + half * 8 + 2 * bb + hh] : 0;
    }
    if (lane < 16) {
        const int srow = rt * 16 + lane;
        const uint8_t *rec = recs + ((size_t)(srow < N ? srow : 0) * nsb + sb) * 18;
        reinterpret_cast<uint16_t *>(dst + 1664)[lane] =
            srow < N ? (uint16_t)(rec[16] | (rec[17] << 8)) : (uint16_t)0;
    }
}

__global__ void unpack_q6k_kernel(const uint8_t *__restrict__ tiled, uint8_t *__restrict__ codes,
                                  uint8_t *__restrict__ recs, int N, int K, int nkt) {
    const long long tile = blockIdx.x;
    const int lane = threadIdx.x;
    const int rt = (int)(tile / nkt), kt = (int)(tile % nkt);
    const uint8_t *src = tiled + tile * TileFmt<RRA_Q6K>::TB;
    const int nsb = K / 256, sb = kt >> 1, half = kt & 1;
    const int r = lane & 15, j = lane >> 4;
    const int row = rt * 16 + r;
    if (row < N) {
        uint8_t *cb = codes + ((size_t)row * nsb + sb) * 192;
        const uint4 v = *reinterpret_cast<const uint4 *>(src + lane * 16);
        const uint2 hv = *reinterpret_cast<const uint2 *>(src + 1024 + lane * 8);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        const uint32_t h[4] = {hv.x & 0xFFFFu, hv.x >> 16, hv.y & 0xFFFFu, hv.y >> 16};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int e0 = half * 128 + 32 * b + 8 * j;
            *reinterpret_cast<uint32_t *>(cb + e0 / 2) = d[b];
            *reinterpret_cast<uint16_t *>(cb + 128 + e0 / 4) = (uint16_t)h[b];
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int idx = 2 * lane + t;
        const int hh = idx >> 6, rr = (idx >> 2) & 15, bb = idx & 3;
        const int srow = rt * 16 + rr;
        if (srow < N) recs[((size_t)srow * nsb + sb) * 18 + half * 8 + 2 * bb + hh] = src[1536 + idx];
    }
    if (lane < 16 && half == 0) {
        const int srow = rt * 16 + lane;
        if (srow < N) {
            const uint16_t dd = reinterpret_cast<const uint16_t *>(src + 1664)[lane];
            uint8_t *rec = recs + ((size_t)srow * nsb + sb) * 18;
            rec[16] = (uint8_t)(dd & 0xFF);
            rec[17] = (uint8_t)(dd >> 8);
        }
    }
}

template <int FMT, int CT, int RPW, int NW, int NT>
rra_status launch_short(const rra_weight &w, const GemvPlan &p, const uint8_t *img, int m,
                        float *out, size_t stride, const NormIn &nrm, const GemvPrologue &pro,
                        dim3 grid, int nkt, hipStream_t s) {
    const auto *wd = static_cast<const uint8_t *>(w.data);
#define RRA_SHORT(PRO)                                                                         \
    hipLaunchKernelGGL((gemv_q_short_kernel<FMT, CT, RPW, NW, NT, PRO>), grid, dim3(64 * NW), 0, \
                       s, wd, img, out, m, (int)w.n, (int)w.k, nkt, p.kt_per_split,           \
                       (long long)stride, nrm, pro)
    if constexpr (CT == 1 && NW == 4) {
        const int hd = pro.kind == kProAttn ? (int)(w.k / pro.n) : 0;
        if (pro.kind == kProSwiglu)
            RRA_SHORT(kProSwiglu);
        else if (pro.kind == kProAttn && hd == 64)
            RRA_SHORT(kProAttn);
        else if (pro.kind == kProAttn && hd == 128)
            RRA_SHORT(kProAttn + 1);
        else if (pro.kind == kProResid)
            RRA_SHORT(kProResid);
        else if (pro.kind != kProNone)
            return fail(RRA_EINVAL, "gemv prologue: unsupported kind %d (hd %d)", pro.kind, hd);
        else
            RRA_SHORT(kProNone);
    } else {
        if (pro.kind != kProNone) return fail(RRA_EINVAL, "gemv prologue: m > 16");
        RRA_SHORT(kProNone);
    }
#undef RRA_SHORT
    return check_launch("gemv_q_short_kernel");
}

template <int FMT, int CT, int RPW, int NW>
rra_status launch_q(const rra_weight &w, const GemvPlan &p, const uint8_t *img, int m, float *out,
                    size_t stride, const NormIn &nrm, const GemvPrologue &pro, hipStream_t s,
                    ArgOut *ao) {
    const int n_rt = (int)cdiv(w.n, 16);
    const int nkt = (int)cdiv(w.k, TileFmt<FMT>::KT);
    dim3 grid((unsigned)cdiv(n_rt, NW * RPW), (unsigned)p.split), block(64 * NW);
    const auto *wd = static_cast<const uint8_t *>(w.data);
    if constexpr (CT <= 2) {  // prompt chunks hold too large an image for NT K tiles in LDS
        if (p.kt_per_split <= 2)
            return launch_short<FMT, CT, RPW, NW, 2>(w, p, img, m, out, stride, nrm, pro, grid,
                                                     nkt, s);
        if (p.kt_per_split <= 4)
            return launch_short<FMT, CT, RPW, NW, 4>(w, p, img, m, out, stride, nrm, pro, grid,
                                                     nkt, s);
    }
    if (pro.kind != kProNone) return fail(RRA_EINVAL, "gemv prologue: split longer than 4 tiles");
    // argmax partials: one K split only, within the buffers' partials per row
    ArgOut a;
    if (CT <= 2 && ao && p.split == 1 && (int)grid.x <= ao->stride) {
        a = *ao;
        ao->blocks = (int)grid.x;
    }
    hipLaunchKernelGGL((gemv_q_kernel<FMT, CT, RPW, NW>), grid, block, 0, s, wd, img, out, m,
                       (int)w.n, (int)w.k, nkt, p.kt_per_split, (long long)stride, nrm, a);
    return check_launch("gemv_q_kernel");
}

template <int FMT>
rra_status launch_fmt(const rra_weight &w, const GemvPlan &p, const uint8_t *img, int m,
                      float *out, size_t stride, const NormIn &nrm, const GemvPrologue &pro,
                      hipStream_t s, ArgOut *ao) {
    if (m <= 16) {
        if (p.rpw >= 2) return launch_q<FMT, 1, 2, 4>(w, p, img, m, out, stride, nrm, pro, s, ao);
        return launch_q<FMT, 1, 1, 4>(w, p, img, m, out, stride, nrm, pro, s, ao);
    }
    if (m > 32) {  // prompt chunks
        if (pro.kind != kProNone) return fail(RRA_EINVAL, "gemv prologue: m > 16");
        if (m <= 64) return launch_q<FMT, 4, 1, 8>(w, p, img, m, out, stride, nrm, pro, s, ao);
        if constexpr (FMT != RRA_Q6K) {
            const int n_rt = (int)cdiv(w.n, 16);
            const int nkt = (int)cdiv(w.k, TileFmt<FMT>::KT);
            const dim3 grid((unsigned)cdiv(n_rt, 16), (unsigned)p.split);
            hipLaunchKernelGGL(gemm_q_kernel<FMT>, grid, dim3(512), 0, s,
                               static_cast<const uint8_t *>(w.data), img, out, m, (int)w.n,
                               (int)w.k, nkt, p.kt_per_split, (long long)stride, nrm);
            return check_launch("gemm_q_kernel");
        }
        return launch_q<FMT, 8, 1, 8>(w, p, img, m, out, stride, nrm, pro, s, ao);
    }
    if (p.nw == 8) {
        if (p.rpw >= 2) return launch_q<FMT, 2, 2, 8>(w, p, img, m, out, stride, nrm, pro, s, ao);
        return launch_q<FMT, 2, 1, 8>(w, p, img, m, out, stride, nrm, pro, s, ao);
    }
    // At m > 16, two row tiles per wave whatever the plan says (the row
    // tiling never changes a row's arithmetic).  Short splits: half the
    // workgroups, each with 4 K tiles of two-column-tile image in LDS, fit one
    // round on the chip (MI355X, 8B-shaped step at M=32: 7.51 -> 7.43 ms).
    // Long splits: each LDS fragment read feeds two row tiles (the 8B down
    // GEMV: 512 -> 256 workgroups, step 6.95 -> 6.91 ms; four row tiles in
    // the gate/up GEMV, 448 -> 224 workgroups, lost 0.2 %).  Three row tiles
    // where that turns more than one workgroup per compute unit into at most
    // one (the 8B QKV GEMV: 384 -> 256 workgroups, 16.0 -> 15.4 us, step
    // +0.35 %): with 1.5 workgroups per unit, half the units run two and set
    // the kernel's time.
    if (p.kt_per_split <= 4 && p.rpw < 2) {
        const int n_rt = (int)cdiv(w.n, 16);
        if (cdiv(n_rt, 12) * p.split <= 256 && cdiv(n_rt, 8) * p.split > 256)
            return launch_q<FMT, 2, 3, 4>(w, p, img, m, out, stride, nrm, pro, s, ao);
    }
    return launch_q<FMT, 2, 2, 4>(w, p, img, m, out, stride, nrm, pro, s, ao);
}

}  // namespace

GemvPlan gemv_plan(const rra_weight &w, int m) {
    GemvPlan p;
    if (w.fmt == RRA_F32) return p;
    const int n_rt = (int)cdiv(w.n, 16);
    const int nkt = (int)cdiv(w.k, tile_k(w.fmt));
    // Row tiles per wave: 2 (fewer activation bytes per weight byte), or 1
    // when that leaves fewer than 128 row blocks.
    p.rpw = cdiv(n_rt, 8) >= 128 ? 2 : 1;
    // 8 waves per workgroup (one activation tile shared by twice the rows:
    // half the image bytes per weight byte) where that still leaves at least
    // 256 workgroups, i.e. LM-head-sized N; used at m > 16, where the image
    // has two column tiles.  Each output is computed the same way either way.
    p.nw = cdiv(n_rt, 8 * p.rpw) >= 256 ? 8 : 4;
    const int n_rb = (int)cdiv(n_rt, p.nw * p.rpw);
    // K splits: a power of two giving about 768 workgroups (3 per compute
    // unit).  The plan depends on the weight shape only, never on m, so a
    // sequence's result is bit-identical whatever batch it is computed in.
    (void)m;
    int split = 1;
    while (split * 2 * n_rb <= 768 && split * 2 <= nkt) split *= 2;
    p.kt_per_split = (int)cdiv(nkt, split);
    p.split = (int)cdiv(nkt, p.kt_per_split);
    return p;
}

GemvPlan gemm_plan(const rra_weight &w) {
    GemvPlan p;
    if (w.fmt == RRA_F32) return p;
    const int n_rt = (int)cdiv(w.n, 16);
    const int nkt = (int)cdiv(w.k, tile_k(w.fmt));
    // Prompt chunks (33..128 rows): compute-bound, one 8-wave workgroup of
    // 256 output rows (gemm_q_kernel; 128 rows for chunks of up to 64 rows)
    // per compute unit at a time, its double-buffered image taking most of
    // the LDS; K splits until the grid has about 192 workgroups (each split
    // at least two K tiles long), fewer splits than a full chip's worth since
    // every split adds a plane of partial sums.
    p.rpw = 1;
    p.nw = 8;
    const int n_rb = (int)cdiv(n_rt, 16);
    int split = 1;
    while (split * n_rb < 192 && split * 4 <= nkt) split *= 2;
    p.kt_per_split = (int)cdiv(nkt, split);
    p.split = (int)cdiv(nkt, p.kt_per_split);
    return p;
}

bool gemv_takes_prologue(const rra_weight &w, const GemvPlan &p, int m) {
    return is_quantised(w.fmt) && m <= 4 && p.kt_per_split <= 4;
}

bool gemv_takes_resid_prologue(const rra_weight &w, const GemvPlan &p, int m, int planes) {
    // every workgroup reads planes x m x K floats: at most 64 (row, chunk,
    // plane) triples of 512 columns, about two memory round trips
    return gemv_takes_prologue(w, p, m) && m * ss_parts((int)w.k) <= 32 &&
           (int64_t)planes * m * ss_parts((int)w.k) <= 64;
}

rra_status launch_gemv(const rra_weight &w, const GemvPlan &p, const void *x, int m, float *out,
                       size_t stride, hipStream_t s, const NormIn *nrm, const GemvPrologue *pro,
                       ArgOut *ao) {
    if (ao) ao->blocks = 0;
    const NormIn none{nullptr, 0, 0.f};
    const NormIn &n = nrm ? *nrm : none;
    const GemvPrologue no_pro{kProNone, nullptr, nullptr, nullptr, 0, 0, 0, 0, 0};
    const GemvPrologue &pr = pro ? *pro : no_pro;
    if (pr.kind != kProNone && !gemv_takes_prologue(w, p, m))
        return fail(RRA_EINVAL, "gemv prologue: needs a quantised weight, m <= 4 and short splits");
    if (w.fmt == RRA_F32) {
        // up to 32 rows per launch (one accumulator per row in registers)
        dim3 grid((unsigned)cdiv(w.n, 4));
        for (int m0 = 0; m0 < m; m0 += RRA_M_MAX) {
            NormIn ns = n;
            if (ns.ss) ns.ss += (size_t)m0 * ns.nparts;
            hipLaunchKernelGGL(gemv_f32_kernel, grid, dim3(256), 0, s,
                               static_cast<const float *>(w.data),
                               static_cast<const float *>(x) + (size_t)m0 * w.k,
                               out + (size_t)m0 * w.n, std::min(RRA_M_MAX, m - m0), (int)w.n,
                               (int)w.k, ns);
            RRA_TRY(check_launch("gemv_f32_kernel"));
        }
        return RRA_OK;
    }
    const auto *img = static_cast<const uint8_t *>(x);
    if (w.fmt == RRA_Q4) return launch_fmt<RRA_Q4>(w, p, img, m, out, stride, n, pr, s, ao);
    if (w.fmt == RRA_Q6K) return launch_fmt<RRA_Q6K>(w, p, img, m, out, stride, n, pr, s, ao);
    if (w.fmt == RRA_FP8) return launch_fmt<RRA_FP8>(w, p, img, m, out, stride, n, pr, s, ao);
    return launch_fmt<RRA_Q8>(w, p, img, m, out, stride, n, pr, s, ao);
}

rra_status launch_x_to_image(const float *x, uint8_t *img, int fmt, int m, int k, hipStream_t s) {
    const int kpad = (int)(cdiv(k, tile_k(fmt)) * tile_k(fmt));
    const int ct = frag_ct(m);
    dim3 grid((unsigned)cdiv(kpad / 8, 256), (unsigned)m);
    if (k128_tiles(fmt))
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
    if (!is_quantised(fmt) || n <= 0 || k <= 0 || k % (fmt == RRA_Q6K ? 256 : 32)) return 0;
    return (size_t)cdiv(n, 16) * (size_t)cdiv(k, tile_k(fmt)) * (size_t)tile_bytes(fmt);
}

extern "C" rra_status rra_repack_weight(const rra_weight *planar, void *tiled, size_t tiled_bytes,
                                        rra_weight *out, hipStream_t s) {
    clear_error();
    if (!planar || !tiled || !out) return fail(RRA_EINVAL, "rra_repack_weight: null argument");
    if (!is_quantised(planar->fmt))
        return fail(RRA_EINVAL, "rra_repack_weight: only Q8/Q4/FP8/Q6K weights are tiled");
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
    if (planar->fmt == RRA_Q6K)
        hipLaunchKernelGGL(repack_q6k_kernel, dim3((unsigned)tiles), dim3(64), 0, s, q,
                           reinterpret_cast<const uint8_t *>(planar->scale), dst, (int)planar->n,
                           (int)planar->k, nkt);
    else if (planar->fmt == RRA_Q4)
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
    if (!is_quantised(tiled->fmt) || tiled->layout != RRA_TILED)
        return fail(RRA_EINVAL, "rra_unpack_weight: input must be a tiled Q8/Q4/FP8/Q6K weight");
    RRA_TRY(validate_weight(tiled, "rra_unpack_weight", true));
    const int nkt = (int)cdiv(tiled->k, tile_k(tiled->fmt));
    const long long tiles = cdiv(tiled->n, 16) * (long long)nkt;
    auto src = static_cast<const uint8_t *>(tiled->data);
    auto q = static_cast<uint8_t *>(data);
    if (tiled->fmt == RRA_Q6K)
        hipLaunchKernelGGL(unpack_q6k_kernel, dim3((unsigned)tiles), dim3(64), 0, s, src, q,
                           reinterpret_cast<uint8_t *>(scale), (int)tiled->n, (int)tiled->k, nkt);
    else if (tiled->fmt == RRA_Q4)
        hipLaunchKernelGGL(unpack_kernel<RRA_Q4>, dim3((unsigned)tiles), dim3(64), 0, s, src, q,
                           scale, (int)tiled->n, (int)tiled->k, nkt);
    else
        hipLaunchKernelGGL(unpack_kernel<RRA_Q8>, dim3((unsigned)tiles), dim3(64), 0, s, src, q,
                           scale, (int)tiled->n, (int)tiled->k, nkt);
    return check_launch("unpack_kernel");
}

// Workspace of the public GEMV: the activation image (quantised weights), then the
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

// ------------------------------------------------------------ no-allocation GEMV
// rra_batched_gemv_noalloc: the same kernels as rra_batched_gemv, with the
// workspace (activation image + split-K partials) in a file-scope device
// array instead of caller memory.  Each GPU the library runs on holds its own
// copy of the array until the process ends; its device address is looked up
// once per device (hipGetSymbolAddress with that device current) and only
// that address is handed to kernels -- the array's name in host code is a
// host-side stand-in, not a device pointer.  Every workspace byte a call reads
// is written earlier in the same call (the image by x_to_image_kernel, each
// split plane by its GEMV workgroups), so nothing needs clearing between calls.
namespace {
constexpr size_t kStaticScratchBytes = (size_t)RRA_GEMV_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of stream s (the null stream:
// the current device).
rra_status static_scratch(hipStream_t s, uint8_t **out) {
    int dev = -1;
    if (s)
        RRA_TRY_HIP(hipStreamGetDevice(s, &dev));
    else
        RRA_TRY_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(RRA_EINVAL, "rra_batched_gemv_noalloc: device %d not in 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        RRA_TRY_HIP(hipGetDevice(&cur));
        if (cur != dev) RRA_TRY_HIP(hipSetDevice(dev));
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return fail(RRA_EHIP, "rra_batched_gemv_noalloc: hipGetSymbolAddress(scratch) on "
                        "device %d failed: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<uint8_t *>(g_scratch_ptr[dev]);
    return RRA_OK;
}
}  // namespace

extern "C" rra_status rra_batched_gemv_noalloc(const rra_weight *w, const float *x, float *y,
                                               int32_t m, hipStream_t s) {
    clear_error();
    if (!w || !x || !y) return fail(RRA_EINVAL, "rra_batched_gemv_noalloc: null argument");
    if (m < 1 || m > RRA_M_MAX)
        return fail(RRA_EINVAL, "rra_batched_gemv_noalloc: m=%d not in 1..32", m);
    RRA_TRY(validate_weight(w, "rra_batched_gemv_noalloc", true));
    size_t part_off;
    const size_t need = gemv_ws_layout(*w, m, &part_off);
    if (need > kStaticScratchBytes)
        return fail(RRA_EINVAL, "rra_batched_gemv_noalloc: this call needs %zu workspace bytes; "
                    "the static scratch holds %zu (use rra_batched_gemv)", need,
                    kStaticScratchBytes);
    const GemvPlan p = gemv_plan(*w, m);
    if (need == 0) return launch_gemv(*w, p, x, m, y, 0, s);  // fp32, one split: no scratch
    uint8_t *ws = nullptr;
    RRA_TRY(static_scratch(s, &ws));
    const void *in = x;
    if (w->fmt != RRA_F32) {
        RRA_TRY(launch_x_to_image(x, ws, w->fmt, m, (int)w->k, s));
        in = ws;
    }
    if (p.split == 1) return launch_gemv(*w, p, in, m, y, 0, s);
    float *part = reinterpret_cast<float *>(ws + part_off);
    const size_t stride = (size_t)m * (size_t)w->n;
    RRA_TRY(launch_gemv(*w, p, in, m, part, stride, s));
    return launch_reduce_splits(part, p.split, stride, y, m, (int)w->n, s);
}

// ------------------------------------------------------------ VALU GEMV (comparison)
extern "C" rra_status rra_batched_gemv_valu(const rra_weight *w, const float *x, float *y,
                                            int32_t m, void *ws, size_t ws_bytes, hipStream_t s) {
    clear_error();
    if (!w || !x || !y) return fail(RRA_EINVAL, "rra_batched_gemv_valu: null argument");
    if (m < 1 || m > 8) return fail(RRA_EINVAL, "rra_batched_gemv_valu: m=%d not in 1..8", m);
    RRA_TRY(validate_weight(w, "rra_batched_gemv_valu", true));
    if (w->fmt != RRA_Q4 && w->fmt != RRA_Q8)
        return fail(RRA_EINVAL, "rra_batched_gemv_valu: Q4 and Q8 weights only");
    const GemvPlan p = gemv_plan(*w, m);
    const int kt = tile_k(w->fmt), nkt = (int)cdiv(w->k, kt);
    const int mr = m == 1 ? 1 : m <= 4 ? 4 : 8;
    const size_t shm = sizeof(float) * (size_t)mr * p.kt_per_split * kt * 9 / 8;
    if (shm > 65536)
        return fail(RRA_EINVAL, "rra_batched_gemv_valu: a split of %d K values needs %zu bytes of LDS",
                    p.kt_per_split * kt, shm);
    const size_t need = p.split > 1 ? (size_t)p.split * m * w->n * sizeof(float) : 0;
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(RRA_ENOTINIT, "rra_batched_gemv_valu: workspace has %zu bytes, needs %zu",
                    ws ? ws_bytes : (size_t)0, need);
    float *dst = p.split > 1 ? static_cast<float *>(ws) : y;
    const size_t stride = (size_t)m * w->n;
    const dim3 grid((unsigned)cdiv(cdiv(w->n, 16), 4), (unsigned)p.split);
    const auto *wd = static_cast<const uint8_t *>(w->data);
#define RRA_VG(F, MRV)                                                                         \
    hipLaunchKernelGGL((gemv_valu_kernel<F, MRV>), grid, dim3(256), shm, s, wd, x, dst, m,      \
                       (int)w->n, (int)w->k, nkt, p.kt_per_split, (long long)stride)
    if (w->fmt == RRA_Q4) {
        if (mr == 1) RRA_VG(RRA_Q4, 1); else if (mr == 4) RRA_VG(RRA_Q4, 4); else RRA_VG(RRA_Q4, 8);
    } else {
        if (mr == 1) RRA_VG(RRA_Q8, 1); else if (mr == 4) RRA_VG(RRA_Q8, 4); else RRA_VG(RRA_Q8, 8);
    }
#undef RRA_VG
    RRA_TRY(check_launch("gemv_valu_kernel"));
    if (p.split == 1) return RRA_OK;
    return launch_reduce_splits(dst, p.split, stride, y, m, (int)w->n, s);
}
