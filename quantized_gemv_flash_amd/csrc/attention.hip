// attention.hip -- KV-cache scatter and split-K flash-decoding attention.
//
// [head_dim] flash_decoding_attention_into: the new K/V row is written into
// the cache at the sequence's position; the cached rows are split into chunks
// processed in parallel, each giving a partial softmax result, and a second
// pass combines the partials with softmax (log-sum-exp) rescaling.  Q has nq
// heads; K/V have nkv heads, query head h reading KV head h / (nq / nkv).
//
// MI355X design.  One 256-thread workgroup per (split, KV head, sequence)
// serves all G = nq/nkv query heads of its KV head, so every cached K/V byte
// is read from HBM exactly once per step (the pages' kernel runs one 32-lane
// group per *query* head).  Scores: 8 lanes per cached row, each lane a 128-bit
// load per 32 columns, dot products for the G heads, 3-step butterfly.  The G
// score rows of the chunk live in LDS; one wave per head forms max / exp /
// sum; values: hd/4 lanes per row with 128-bit loads, G accumulators per lane,
// then a cross-wave sum in LDS.  The grid has nc = ceil(max_len / chunk)
// splits per (sequence, KV head), and split c takes rows c, c + nc, c + 2nc,
// ... (at most `chunk` of them) rather than one contiguous chunk: the softmax
// partials and their log-sum-exp combination hold for any partition of the
// rows, and with the rows dealt round-robin the nc workgroups of a sequence
// sweep its cache region together, so the reads in flight stay within a
// narrow window of HBM (measured on MI355X: 6.0-6.2 TB/s for the bare reads
// with 8 splits, against 5.4 for contiguous chunks).  A split with no rows
// (c >= seq_len) returns at once, so a captured graph stays valid as
// positions advance.
#include "epilogue.h"
#include "frag.h"
#include "rra_internal.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>
#include <vector>

namespace rra {
namespace {

// 128-bit load marked nontemporal (the cached K/V rows are read once per
// step, so they should not displace reused lines).  On MI355X this lifts the
// chunk kernel's K/V stream from about 5.5 to 6.05 TB/s.
typedef float rra_f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ldnt(const float *p) {
    const rra_f4v v = __builtin_nontemporal_load(reinterpret_cast<const rra_f4v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__global__ __launch_bounds__(256) void kv_scatter_kernel(const float *__restrict__ k_rows,
                                                         const float *__restrict__ v_rows,
                                                         float *__restrict__ kc,
                                                         float *__restrict__ vc,
                                                         const uint32_t *__restrict__ pos, int nkv,
                                                         int hd, int max_len) {
    const int m = blockIdx.x;
    const uint32_t p = pos[m];
    if (p >= (uint32_t)max_len) return;
    const int row = nkv * hd;
    for (int idx = threadIdx.x; idx < row; idx += blockDim.x) {
        const int g = idx / hd, d = idx - g * hd;
        const size_t dst = (((size_t)m * nkv + g) * max_len + p) * hd + d;
        kc[dst] = k_rows[(size_t)m * row + idx];
        vc[dst] = v_rows[(size_t)m * row + idx];
    }
}

// Partial result of split c (rows t = c + i nc_max) for query head h of
// sequence m:
//   part_o[((m*nq + h)*nc_max + c)*HD + d] = sum_t p_t v_t[d] / l,
//   part_lse[(m*nq + h)*nc_max + c]      = max_t s_t + ln l,
// with s_t = <q_h, k_t>/sqrt(HD), p_t = e^(s_t - max), l = sum_t p_t.
//
// A workgroup serves G query heads of KV head g = blockIdx.y / hs: the KV
// head's nq/nkv = G hs query heads are dealt to hs workgroups.  hs = 1 reads
// every KV byte once (bandwidth-bound grids); hs > 1 shortens each
// workgroup's work where the grid is small and latency-bound (the other
// workgroups' K/V reads are cache hits).  A head's arithmetic is the same
// whatever G and hs are.
//
// QF: the QKV GEMV's split planes stand in for q and seq_len (QkvIn).  The
// workgroup owning row pos (c = pos mod nc_max) forms the new K/V row in LDS,
// takes it in place of the cache row (which its loads still read: the values
// it writes there are the same), and the first of the hs workgroups of its
// KV head writes it to the cache.  The arithmetic is qkv_post_kernel's
// (sum_splits2, rope_pair), so the results equal the unfused path bitwise.
//
// EARLY (fused input, grids of at most one workgroup per compute unit): the
// first round's K rows and V rows depend neither on the query nor on the
// position, so they are requested before either is read, clamped to the
// split's rows in the allocated cache rather than to those below the position
// (rows past the sequence are loaded and never used): the position, the QKV
// partials and the first K/V rows then share one memory round trip.  With
// more workgroups per compute unit that loses (a wave's loads return in
// order, so rows requested ahead delay the partials, and the rows past the
// sequence add traffic).
template <int HD, int G, bool QF, bool EARLY = false, bool LF = false, bool PRE = false>
__global__ __launch_bounds__(256) void fd_chunk_kernel(
    const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vc,
    const uint32_t *__restrict__ seq_len, const uint32_t *__restrict__ slot_seq,
    float *__restrict__ part_o, float *__restrict__ part_lse, int nq, int nkv, int max_len,
    int chunk, int nc_max, int hs, QkvIn qi) {
    constexpr int GP = (G + 3) & ~3;  // probabilities stored key-major, G padded to 4
    const int c = blockIdx.x, g = blockIdx.y / hs;
    const int hq0 = blockIdx.y * G;  // first query head: g G hs + (blockIdx.y mod hs) G
    static_assert(QF || !EARLY, "early K/V rows need the fused QKV input");
    static_assert(!(LF && QF), "longest first: the unfused instance only");
    static_assert(!(PRE && (EARLY || LF)), "PRE: the index-order instances without EARLY");
    // The sequence served: blockIdx.z, or in the LF instance the
    // blockIdx.z-th longest (ties: lower index first).  Workgroups are
    // dispatched in blockIdx order, so the first ones then take the longest
    // splits and those that wait for a free compute unit the shortest.  Every
    // lane loads one sequence's length in the round trip that would load this
    // sequence's alone; the ranking is a serial loop over the batch (about
    // 1 us), paid back only where lengths differ widely.  The ranking takes
    // one sequence per lane; a grid of more than 64 (the entry points allow
    // 32) would keep blockIdx.z.
    const uint32_t *src = QF ? qi.pos : seq_len;  // position (QF) or length
    int m = blockIdx.z;
    uint32_t mv = 0;  // src[m]
    if (LF && gridDim.z <= 64) {
        const int ln = threadIdx.x & 63, nseq = gridDim.z;
        const uint32_t v = ln < nseq ? src[ln] : 0u;
        const uint32_t len = QF ? (v < (uint32_t)max_len ? v + 1 : 0u) : min(v, (uint32_t)max_len);
        int rank = 0;  // sequences ahead of this lane's
        for (int k = 0; k < nseq; ++k) {  // k is wave-uniform: a scalar broadcast
            const uint32_t lk = (uint32_t)__builtin_amdgcn_readlane((int)len, k);
            rank += (lk > len || (lk == len && k < ln)) ? 1 : 0;
        }
        const unsigned long long hit = __ballot(ln < nseq && rank == (int)blockIdx.z);
        // the ranks are a permutation of 0 .. nseq - 1: exactly one lane hits
        m = hit ? __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1) : (int)blockIdx.z;
        mv = (uint32_t)__builtin_amdgcn_readlane((int)v, m);
    }
    float4 ek[2][HD / 32], ev[8];  // EARLY: the first K rows and V rows
    if constexpr (EARLY) {
        // the index maps of the score loop (8 lanes per K row, 2 rows per lane)
        // and of the value loop (hd/4 lanes per V row, 8 rows per lane); the
        // fused input has no slot map, sequence m's cache is slot m
        const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
        const int ln = threadIdx.x & 63, e0 = ln & 7, ks0 = ln >> 3;
        constexpr int LPK = HD / 4, KPW = 64 / LPK;
        const int ncap = (max_len - c + nc_max - 1) / nc_max;  // >= 1: c < nc_max <= max_len
        const size_t at0 = (((size_t)m * nkv + g) * max_len + c) * HD;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (u * 32 + wv * 8 >= ncap) break;  // wave-uniform: no rows left
            const int tc = min(u * 32 + wv * 8 + ks0, ncap - 1);
#pragma unroll
            for (int i = 0; i < HD / 32; ++i)
                ek[u][i] = ldnt(kc + at0 + (size_t)tc * nc_max * HD + 4 * (e0 + 8 * i));
        }
        const int d4 = ln % LPK, r0 = wv * KPW + ln / LPK;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tr = min(r0 + u * 4 * KPW, ncap - 1);
            ev[u] = ldnt(vc + at0 + (size_t)tr * nc_max * HD + 4 * d4);
        }
    }
    // Index order (fused or not): the first round's K rows do not depend on
    // the length or the query either, so they too are requested before the
    // length or position is read (clamped to the split's rows in the allocated
    // cache; rows past the length are loaded and never used): the length, the
    // first rows and (fused) the QKV partials' round trips overlap.  K only:
    // with the V rows as well (EARLY) the G = 4 kernel needs 153 VGPRs, 3 waves
    // per SIMD instead of 4.  The PRE instance, on grids of few splits per
    // sequence (the splits past a short sequence's length load rows for
    // nothing).
    constexpr bool KPRE = PRE;
    if constexpr (KPRE) {
        const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
        const int ln = threadIdx.x & 63, e0 = ln & 7, ks0 = ln >> 3;
        const int ncap = (max_len - c + nc_max - 1) / nc_max;  // >= 1: c < nc_max <= max_len
        const size_t cs0 = slot_seq ? slot_seq[m] : (uint32_t)m;
        const float *K0 = kc + ((cs0 * nkv + g) * max_len + c) * HD;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (u * 32 + wv * 8 >= ncap) break;  // wave-uniform: no rows left
            const int tc = min(u * 32 + wv * 8 + ks0, ncap - 1);
#pragma unroll
            for (int i = 0; i < HD / 32; ++i)
                ek[u][i] = ldnt(K0 + (size_t)tc * nc_max * HD + 4 * (e0 + 8 * i));
        }
    }
    if (!LF || gridDim.z > 64) mv = src[m];
    uint32_t p = 0;
    bool ok = false;
    int L;
    if constexpr (QF) {
        p = mv;
        ok = p < (uint32_t)max_len;  // false for an empty slot (RRA_POS_NONE) too
        // an empty slot attends to nothing; any other bad position is an error
        const uint32_t lr = ok ? p + 1 : (p == RRA_POS_NONE ? 0u : (uint32_t)max_len);
        if (c == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
            qi.seq_len[m] = lr;
            if (!ok && p != RRA_POS_NONE) report_error(qi.err, kErrPos);
        }
        L = (int)min(lr, (uint32_t)max_len);
    } else {
        L = (int)min(mv, (uint32_t)max_len);
    }
    if (c >= L) return;
    // Rows c, c + nc_max, c + 2 nc_max, ... < L (local row i is cache row
    // c + i nc_max): the nc_max workgroups of one (sequence, KV head) sweep its
    // cache region together, front to back.
    const int n = (L - c + nc_max - 1) / nc_max;  // <= chunk

    // LDS regions, each starting on a 16-byte boundary (they are read with
    // 128-bit loads): GP and HD are multiples of 4 floats, and the statistics
    // region is padded to 2 GP floats.
    static_assert(GP % 4 == 0 && HD % 4 == 0, "16-byte aligned LDS regions");
    extern __shared__ __attribute__((aligned(16))) float smem[];
    float *sc = smem;                 // [chunk][GP] scores, then probabilities
    float *red = smem + GP * chunk;   // [4 waves][G][HD]
    float *stat = red + 4 * G * HD;   // [G] max, [G] sum (2 GP floats)
    float *qs = stat + 2 * GP;        // QF: [G][HD] queries, then [HD] new K, [HD] new V
    float *kn = qs + G * HD, *vn = kn + HD;
    // QF: the new row's local index in this split, or -1
    const int tp = (QF && ok && (int)(p % (uint32_t)nc_max) == c) ? (int)(p / (uint32_t)nc_max) : -1;
    // The first round's K rows (see the score loop): requested before the
    // length was known (EARLY, KPRE), or (the other fused instances) now,
    // before the QKV partials are summed; the unfused ones without KPRE load
    // them in the loop.
    constexpr int F4 = HD / 32;  // 128-bit loads per lane per row
    constexpr int UK = 2;        // rows per lane per score round (see below)
    float4 kv0[UK][F4];
    static_assert(UK == 2, "the early loads take two K rows per lane");
    if constexpr (EARLY || KPRE) {
#pragma unroll
        for (int u = 0; u < UK; ++u)
#pragma unroll
            for (int i = 0; i < F4; ++i) kv0[u][i] = ek[u][i];
    } else if constexpr (QF) {
        const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
        const int ln = threadIdx.x & 63, e0 = ln & 7, ks0 = ln >> 3;
        const size_t cs0 = slot_seq ? slot_seq[m] : (uint32_t)m;
        const float *K0 = kc + ((cs0 * nkv + g) * max_len + c) * HD;
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            if (u * 32 + wv * 8 >= n) break;  // wave-uniform: no rows left
            const int tc = min(u * 32 + wv * 8 + ks0, n - 1);
#pragma unroll
            for (int i = 0; i < F4; ++i)
                kv0[u][i] = ldnt(K0 + (size_t)tc * nc_max * HD + 4 * (e0 + 8 * i));
        }
    }
    if constexpr (QF) {
        constexpr int HALF = HD / 2;
        const int nrow = (nq + 2 * nkv) * HD;
        const int npairs = (G + (tp >= 0 ? 2 : 0)) * HALF;
        for (int idx = threadIdx.x; idx < npairs; idx += blockDim.x) {
            const int hh = idx / HALF, j = idx % HALF;
            const int head = hh < G ? hq0 + hh : hh == G ? nq + g : nq + nkv + g;
            const size_t b = (size_t)m * nrow + (size_t)head * HD;
            float a, cc;
            sum_splits2(qi.part + b + j, qi.part + b + j + HALF, qi.split, qi.stride, a, cc);
            if (hh <= G && ok)
                rope_pair(a, cc, qi.table[((size_t)p * HALF + j) * 2],
                          qi.table[((size_t)p * HALF + j) * 2 + 1]);
            float *dst = qs + hh * HD;  // qs rows, then kn, vn
            dst[j] = a;
            dst[j + HALF] = cc;
        }
        __syncthreads();
        if (tp >= 0 && blockIdx.y % hs == 0 && qi.k_cache) {
            const size_t at = (((size_t)m * nkv + g) * max_len + p) * HD;
            for (int d = threadIdx.x; d < HD; d += blockDim.x) {
                qi.k_cache[at + d] = kn[d];
                qi.v_cache[at + d] = vn[d];
            }
        }
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t cs = slot_seq ? slot_seq[m] : (uint32_t)m;  // cache slot of query row m
    const size_t row0 = (cs * nkv + g) * max_len + c;
    const size_t rs = (size_t)nc_max * HD;  // floats between consecutive local rows
    const float *K = kc + row0 * HD;
    const float *V = vc + row0 * HD;

    // ---- scores: 8 lanes per cached row, UK rows per lane per round.  UK = 2
    // keeps the kernel at 117 VGPRs (4 waves per SIMD; UK = 4 needs 152, 3
    // waves): on MI355X 1-2 % faster at 512-row splits, 16 % at 32-row ones.
    const int e = lane & 7, ks = lane >> 3;
    const float qscale = 1.0f / sqrtf((float)HD);
    float4 qr[G][F4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float *qh = QF ? qs + h * HD : q + ((size_t)m * nq + hq0 + h) * HD;
#pragma unroll
        for (int i = 0; i < F4; ++i) {
            float4 v = *reinterpret_cast<const float4 *>(qh + 4 * (e + 8 * i));
            qr[h][i] = make_float4(v.x * qscale, v.y * qscale, v.z * qscale, v.w * qscale);
        }
    }
    for (int base = 0; base < n; base += 32 * UK) {
        float4 kv[UK][F4];
        int tt[UK];
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            tt[u] = base + u * 32 + wave * 8 + ks;
            if (base + u * 32 + wave * 8 >= n) break;  // wave-uniform: no rows left
            const int tc = min(tt[u], n - 1);  // clamped: unconditional 128-bit loads
            if ((QF || KPRE) && base == 0) {
#pragma unroll
                for (int i = 0; i < F4; ++i) kv[u][i] = kv0[u][i];
            } else {
#pragma unroll
                for (int i = 0; i < F4; ++i)
                    kv[u][i] = ldnt(K + (size_t)tc * rs + 4 * (e + 8 * i));
            }
            if (QF && tt[u] == tp) {
#pragma unroll
                for (int i = 0; i < F4; ++i)
                    kv[u][i] = *reinterpret_cast<const float4 *>(kn + 4 * (e + 8 * i));
            }
        }
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            if (base + u * 32 + wave * 8 >= n) break;
            float s[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < F4; ++i) {
                    a = fmaf(qr[h][i].x, kv[u][i].x, a);
                    a = fmaf(qr[h][i].y, kv[u][i].y, a);
                    a = fmaf(qr[h][i].z, kv[u][i].z, a);
                    a = fmaf(qr[h][i].w, kv[u][i].w, a);
                }
                a += __shfl_xor(a, 1, 64);
                a += __shfl_xor(a, 2, 64);
                a += __shfl_xor(a, 4, 64);
                s[h] = a;
            }
            if (tt[u] < n) {
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if (e == (h & 7)) sc[tt[u] * GP + h] = s[h];
            }
        }
    }
    // ---- values, first round: requested now, in flight during the softmax.
    // hd/4 lanes per row, rows r0 + 4 KPW u of each round of RS rows; rows
    // past n are clamped loads, never used.
    constexpr int LPK = HD / 4, KPW = 64 / LPK, UV = 8, RS = 4 * KPW * UV;
    static_assert(UV == 8, "EARLY loads eight V rows per lane");
    const int d4 = lane % LPK, r0 = wave * KPW + lane / LPK;
    float4 vb[UV];
    auto vload = [&](int base) {
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int t = min(base + r0 + u * 4 * KPW, n - 1);
            vb[u] = ldnt(V + (size_t)t * rs + 4 * d4);
            if (QF && base + r0 + u * 4 * KPW == tp)
                vb[u] = *reinterpret_cast<const float4 *>(vn + 4 * d4);
        }
    };
    if constexpr (EARLY) {
#pragma unroll
        for (int u = 0; u < UV; ++u)
            vb[u] = r0 + u * 4 * KPW == tp ? *reinterpret_cast<const float4 *>(vn + 4 * d4) : ev[u];
    } else {
        vload(0);
    }
    __syncthreads();

    // ---- per-head max, exponentials, sum
    for (int h = wave; h < G; h += 4) {
        float mx = -INFINITY;
        for (int t = lane; t < n; t += 64) mx = fmaxf(mx, sc[t * GP + h]);
        mx = wave_max(mx);
        float l = 0.f;
        for (int t = lane; t < n; t += 64) {
            const float p = expf(sc[t * GP + h] - mx);
            sc[t * GP + h] = p;
            l += p;
        }
        l = wave_sum(l);
        if (lane == 0) {
            stat[h] = mx;
            stat[G + h] = l;
        }
    }
    __syncthreads();

    // ---- probability-weighted values: each round's rows are loaded one round
    // ahead (the first before the softmax), so a round's loads overlap the
    // previous round's arithmetic.
    const int kslot = lane / LPK;
    float4 o[G];
#pragma unroll
    for (int h = 0; h < G; ++h) o[h] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int base = 0; base < n; base += RS) {
        float4 v[UV];
#pragma unroll
        for (int u = 0; u < UV; ++u) v[u] = vb[u];
        if (base + RS < n) vload(base + RS);  // uniform over the workgroup
        const int tb = base + r0;
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int t = tb + u * 4 * KPW;
            if (t < n) {
                float p[GP];
#pragma unroll
                for (int h4 = 0; h4 < GP; h4 += 4) {
                    const float4 pv = *reinterpret_cast<const float4 *>(sc + t * GP + h4);
                    p[h4] = pv.x;
                    p[h4 + 1] = pv.y;
                    p[h4 + 2] = pv.z;
                    p[h4 + 3] = pv.w;
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    o[h].x = fmaf(p[h], v[u].x, o[h].x);
                    o[h].y = fmaf(p[h], v[u].y, o[h].y);
                    o[h].z = fmaf(p[h], v[u].z, o[h].z);
                    o[h].w = fmaf(p[h], v[u].w, o[h].w);
                }
            }
        }
    }
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            o[h].x += __shfl_xor(o[h].x, off, 64);
            o[h].y += __shfl_xor(o[h].y, off, 64);
            o[h].z += __shfl_xor(o[h].z, off, 64);
            o[h].w += __shfl_xor(o[h].w, off, 64);
        }
    }
    if (kslot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
            *reinterpret_cast<float4 *>(red + (wave * G + h) * HD + 4 * d4) = o[h];
    }
    __syncthreads();

    for (int idx = tid; idx < G * HD; idx += blockDim.x) {
        const int h = idx / HD, d = idx - h * HD;
        const float v = red[(0 * G + h) * HD + d] + red[(1 * G + h) * HD + d] +
                        red[(2 * G + h) * HD + d] + red[(3 * G + h) * HD + d];
        part_o[(((size_t)m * nq + hq0 + h) * nc_max + c) * HD + d] = v / stat[G + h];
    }
    if (tid < G)
        part_lse[((size_t)m * nq + hq0 + tid) * nc_max + c] = stat[tid] + logf(stat[G + tid]);
}

// Causal attention of a prompt chunk on the matrix cores ([head_dim]
// tensor_core_attention: the prompt's tokens attend to themselves and the
// tokens before them, on the tensor cores).  Rows t < n of q sit at
// positions start + t of one cache slot; row t attends to the slot's cache
// rows [0, start + t] (the chunk's own K/V rows are already in the cache).
//
// One workgroup per (16-row query tile, KV head), one wave per query head of
// the KV head's group, so the K/V rows are staged once for the G heads.  Keys
// go in blocks of 32, staged in LDS as fp16 high and low parts laid out as
// matrix-core B operands.  S = Q K^T and O += P V use
// v_mfma_f32_16x16x32_f16 with the fp32 operands split x = hi + lo
// (hi = fp16(x), lo = fp16(x - hi)): each product is taken as hi*hi + hi*lo
// + lo*hi, which drops only the lo*lo term (relative size 2^-22), so the
// scores and outputs carry fp32-level error.  The softmax is the online
// (running max and sum) form: per block, m' = max(m, max s), l' = l e^(m-m')
// + sum e^(s-m'), O' = O e^(m-m') + P V with P = e^(s-m'); at the end O / l.
// Keys past a row's position get probability 0; cache rows past the chunk's
// last position are staged as zeros (never read as data).
//
// With ks_n > 1 the key blocks are dealt to ks_n workgroups (blockIdx.z = ks
// takes blocks ks, ks + ks_n, ...), so short grids fill the chip; each
// writes its normalised partial output and log-sum-exp in flash decode's
// partials layout (split = ks; an empty split writes 0 and -inf), and
// fd_reduce_kernel combines them.
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int HD, int G>
__global__ __launch_bounds__(64 * G) void prefill_attn_kernel(
    const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vc,
    float *__restrict__ out, int n, int nq, int nkv, int max_len, uint32_t start, FragOut fo,
    int ks_n, float *__restrict__ part_o, float *__restrict__ part_lse) {
    constexpr int DS = HD / 32;  // 32-wide d steps of S = Q K^T
    constexpr int DT = HD / 16;  // 16-wide d tiles of O
    constexpr int OS = HD + 4;   // row stride of the output staging (floats)
    __shared__ __attribute__((aligned(16))) uint8_t kf[2 * DS * 2 * 1024];  // [key tile][d step][part]
    __shared__ __attribute__((aligned(16))) uint8_t vf[DT * 2 * 1024];      // [d tile][part]
    __shared__ __attribute__((aligned(16))) _Float16 pf[G][2][16 * 32];     // [wave][part][row][key]
    __shared__ __attribute__((aligned(16))) float of[G][16 * OS];           // [wave][row][d]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int g = blockIdx.y, h = g * G + wave, t0 = blockIdx.x * 16;
    const int j = lane >> 4, r = lane & 15;
    const int last = n - 1;
    const float *K = kc + (size_t)g * max_len * HD;
    const float *V = vc + (size_t)g * max_len * HD;

    // Q as A operands: lane (j, r) holds row t0 + r, d = 32 s + 8 j + [0, 8)
    half8_t qh[DS], ql[DS];
    {
        const float *qr = q + ((size_t)min(t0 + r, last) * nq + h) * HD;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            float v[8];
            load8(qr + 32 * s + 8 * j, v);
            split_exact(v, qh[s], ql[s]);
        }
    }
    const float scale = 1.0f / sqrtf((float)HD);
    float mrow[4], lrow[4];
    floatx4 o[DT];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        mrow[i] = -INFINITY;
        lrow[i] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    // this lane's rows of S and O: 4 j + i; their positions
    int prow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) prow[i] = (int)start + min(t0 + 4 * j + i, last);
    const int kvalid = (int)start + last;            // last cache row holding data
    const int kmax = (int)start + min(t0 + 15, last);  // last key any row of the tile reads
    const int ks = blockIdx.z;
    for (int k0 = 32 * ks; k0 <= kmax; k0 += 32 * ks_n) {
        // ---- stage keys k0 .. k0 + 31: K as B[32 d][16 keys] per (key tile, d step),
        // V as B[32 keys][16 d] per d tile; hi and lo parts
        for (int it = threadIdx.x; it < 32 * (HD / 8); it += 64 * G) {
            const int key = it / (HD / 8), dg = it % (HD / 8);  // (key, group of 8 d)
            float v[8];
            if (k0 + key <= kvalid) {
                load8(K + (size_t)(k0 + key) * HD + 8 * dg, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
            }
            half8_t hi, lo;
            split_exact(v, hi, lo);
            const int nt = key >> 4, s = dg >> 2, jj = dg & 3, slot = 16 * jj + (key & 15);
            uint8_t *f = kf + ((nt * DS + s) * 2) * 1024 + slot * 16;
            *reinterpret_cast<half8_t *>(f) = hi;
            *reinterpret_cast<half8_t *>(f + 1024) = lo;
        }
        for (int it = threadIdx.x; it < HD * 4; it += 64 * G) {
            const int d = it % HD, kg = it / HD;  // (d, group of 8 keys)
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = k0 + 8 * kg + e;
                v[e] = key <= kvalid ? V[(size_t)key * HD + d] : 0.f;
            }
            half8_t hi, lo;
            split_exact(v, hi, lo);
            const int t = d >> 4, slot = 16 * kg + (d & 15);
            uint8_t *f = vf + (t * 2) * 1024 + slot * 16;
            *reinterpret_cast<half8_t *>(f) = hi;
            *reinterpret_cast<half8_t *>(f + 1024) = lo;
        }
        __syncthreads();
        // ---- S = Q K^T for the two key tiles
        floatx4 sc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            floatx4 a = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const uint8_t *f = kf + ((nt * DS + s) * 2) * 1024 + lane * 16;
                const half8_t kh = *reinterpret_cast<const half8_t *>(f);
                const half8_t kl = *reinterpret_cast<const half8_t *>(f + 1024);
                a = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[s], kh, a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[s], kl, a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[s], kh, a, 0, 0, 0);
            }
            sc[nt] = a;
        }
        // ---- online softmax over this block (rows 4 j + i, keys k0 + 16 nt + r)
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s0 = sc[0][i] * scale, s1 = sc[1][i] * scale;
            if (k0 + r > prow[i]) s0 = -INFINITY;
            if (k0 + 16 + r > prow[i]) s1 = -INFINITY;
            float mx = fmaxf(s0, s1);
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            // -inf only while this workgroup has seen no key of the row (a
            // later key split's first blocks): nothing to add, nothing to scale
            const float mn = fmaxf(mrow[i], mx);
            const bool none = mn == -INFINITY;
            alpha[i] = none ? 1.f : expf(mrow[i] - mn);
            const float p0 = none ? 0.f : expf(s0 - mn), p1 = none ? 0.f : expf(s1 - mn);
            float ps = p0 + p1;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off, 64);
            lrow[i] = lrow[i] * alpha[i] + ps;
            mrow[i] = mn;
            // P into [row][key] fp16 hi / lo (the A operand layout is read back below)
            const int row = 4 * j + i;
            const float x0 = as_fp32(p0), x1 = as_fp32(p1);
            const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
            pf[wave][0][row * 32 + r] = h0;
            pf[wave][1][row * 32 + r] = (_Float16)(x0 - (float)h0);
            pf[wave][0][row * 32 + 16 + r] = h1;
            pf[wave][1][row * 32 + 16 + r] = (_Float16)(x1 - (float)h1);
        }
        __builtin_amdgcn_wave_barrier();
        // ---- O = O alpha + P V: A = P[16 rows][32 keys] (lane (j, r): row r, keys 8 j ..)
        const half8_t ph = *reinterpret_cast<const half8_t *>(&pf[wave][0][r * 32 + 8 * j]);
        const half8_t pl = *reinterpret_cast<const half8_t *>(&pf[wave][1][r * 32 + 8 * j]);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            floatx4 a = o[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] *= alpha[i];
            const uint8_t *f = vf + (t * 2) * 1024 + lane * 16;
            const half8_t vh = *reinterpret_cast<const half8_t *>(f);
            const half8_t vl = *reinterpret_cast<const half8_t *>(f + 1024);
            a = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, vh, a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, vl, a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, vh, a, 0, 0, 0);
            o[t] = a;
        }
        __syncthreads();  // kf, vf and pf are refilled next block
    }
    // ---- O / l, through LDS, to the output rows and the O GEMV's image
    // (or, split over keys, to this split's partials)
    float *os = of[wave];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            os[(4 * j + i) * OS + 16 * t + r] = lrow[i] > 0.f ? o[t][i] / lrow[i] : 0.f;
    __builtin_amdgcn_wave_barrier();
    if (ks_n > 1) {
        if (r == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 4 * j + i;
                if (t <= last)
                    part_lse[((size_t)t * nq + h) * ks_n + ks] =
                        lrow[i] > 0.f ? mrow[i] + logf(lrow[i]) : -INFINITY;
            }
        }
        for (int it = lane; it < 16 * (HD / 8); it += 64) {
            const int row = it / (HD / 8), dg = it % (HD / 8), t = t0 + row;
            if (t > last) continue;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = os[row * OS + 8 * dg + e];
            store8(part_o + (((size_t)t * nq + h) * ks_n + ks) * HD + 8 * dg, v);
        }
        return;
    }
    for (int it = lane; it < 16 * (HD / 8); it += 64) {
        const int row = it / (HD / 8), dg = it % (HD / 8), t = t0 + row;
        if (t > last) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = os[row * OS + 8 * dg + e];
        store8(out + ((size_t)t * nq + h) * HD + 8 * dg, v);
        if (fo.img) frag_out8(fo, t, h * HD + 8 * dg, v);
    }
    if (fo.img && h == nq - 1) {  // zeros for the groups in [nq hd, kpad) of the tile's rows
        const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int it = lane; it < 16 * 64; it += 64) {
            const int row = it / 64, k = nq * HD + 8 * (it % 64), t = t0 + row;
            if (t <= last && k < fo.kpad) frag_out8(fo, t, k, z);
        }
    }
}

// out[m][h] = sum_c w_c o~_c / sum_c w_c, w_c = e^(lse_c - max lse), over the
// chunks that hold rows of the sequence.  One wave per (head, sequence).  With
// fo.img set, the head's slice is also written as the output projection's
// activation image (the last head also zeros the groups in [nq hd, kpad)).
template <int HD>
__global__ __launch_bounds__(64) void fd_reduce_kernel(const float *__restrict__ part_o,
                                                       const float *__restrict__ part_lse,
                                                       const uint32_t *__restrict__ seq_len,
                                                       float *__restrict__ out, int nq, int max_len,
                                                       int chunk, int nc_max, FragOut fo) {
    __shared__ float so[HD];
    const int h = blockIdx.x, m = blockIdx.y, lane = threadIdx.x;
    constexpr int PER = HD / 64;
    float acc[PER];
    fd_combine<HD, true>(part_o, part_lse, m, h, nq, nc_max, (int)seq_len[m], lane, acc, max_len);
    const int L = (int)min(seq_len[m], (uint32_t)max_len);
    if (L > 0) {
        float *o = out + ((size_t)m * nq + h) * HD;
#pragma unroll
        for (int j = 0; j < PER; ++j) o[lane + 64 * j] = acc[j];
    }
    if (!fo.img) return;
#pragma unroll
    for (int j = 0; j < PER; ++j) so[lane + 64 * j] = acc[j];
    __syncthreads();
    if (lane < HD / 8) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = so[lane * 8 + e];
        frag_out8(fo, m, h * HD + lane * 8, v);
    }
    if (h == nq - 1) {
        const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k0 = nq * HD + lane * 8; k0 < fo.kpad; k0 += 64 * 8)
            write_frag8_fmt(fo.fmt, fo.img, fo.ct, m, k0, z);
    }
}

template <int HD, int G>
rra_status launch_chunk(const float *q, const float *kc, const float *vc, const uint32_t *lens,
                        const uint32_t *slot_seq, float *po, float *pl, int m, int nq, int nkv,
                        int max_len, int chunk, int nc_max, int hs, bool longest_first,
                        const QkvIn *qi, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    constexpr int GP = (G + 3) & ~3;
    const size_t shm = sizeof(float) * ((size_t)GP * chunk + 4 * G * HD + 2 * GP +
                                        (qi ? (size_t)(G + 2) * HD : 0));
    const dim3 grid(nc_max, nkv * hs, m);
    const QkvIn qa = qi ? *qi : QkvIn{};
    // Longest first only on grids of a few rounds of resident workgroups
    // (four 4-wave workgroups per compute unit): over more rounds the
    // dispatcher already evens the tail out and the ranking is pure cost
    // (standalone attention, lengths U[1, 8192]: 2048 workgroups 180 -> 170 us,
    // 8192 workgroups 188 -> 192 us).
    longest_first = longest_first && (int64_t)nc_max * nkv * hs * m <= 4096;
    // First K rows before the length (index order, no EARLY) only on grids of
    // at most 20 splits per sequence, where the rows loaded for nothing are
    // confined to sequences under 20 x 64 rows (the decode steps' plans take
    // 5 to 18).  Lengths U[1, 8192] over 128 splits: 262 -> 331 us with it.
    const bool pre = nc_max <= 20;
    // Early K/V rows (fused input) only while every workgroup has a compute
    // unit to itself (the 1.5B-shaped decoder at M = 4, 864 workgroups, was
    // 1-2 % slower with them; M = 1 grids gain about 1 %), and while the
    // batch's whole cache is at most 4 MiB of K and V, the most that the rows
    // past short sequences can add (the 0.5B and 1.5B-shaped M = 1 caches
    // are 0.8 and 2.4 MB).
    const bool early = qi && (int64_t)nc_max * nkv * hs * m <= 256 &&
                       (int64_t)m * nkv * max_len * HD * 8 <= (int64_t)4 << 20;
    // Timed launches (ev0/ev1 set) go through hipExtLaunchKernel, whose event
    // pair is stamped at the kernel's own start and end.
    if (ev0 || ev1) {
        if (early)
            hipExtLaunchKernelGGL((fd_chunk_kernel<HD, G, true, true>), grid, dim3(256),
                                  (uint32_t)shm, s, ev0, ev1, 0u, q, kc, vc, lens, slot_seq, po,
                                  pl, nq, nkv, max_len, chunk, nc_max, hs, qa);
        else if (qi && pre)
            hipExtLaunchKernelGGL((fd_chunk_kernel<HD, G, true, false, false, true>), grid,
                                  dim3(256), (uint32_t)shm, s, ev0, ev1, 0u, q, kc, vc, lens,
                                  slot_seq, po, pl, nq, nkv, max_len, chunk, nc_max, hs, qa);
        else if (qi)
            hipExtLaunchKernelGGL((fd_chunk_kernel<HD, G, true>), grid, dim3(256), (uint32_t)shm, s,
                                  ev0, ev1, 0u, q, kc, vc, lens, slot_seq, po, pl, nq, nkv,
                                  max_len, chunk, nc_max, hs, qa);
        else if (longest_first)
            hipExtLaunchKernelGGL((fd_chunk_kernel<HD, G, false, false, true>), grid, dim3(256),
                                  (uint32_t)shm, s, ev0, ev1, 0u, q, kc, vc, lens, slot_seq, po,
                                  pl, nq, nkv, max_len, chunk, nc_max, hs, qa);
        else if (pre)
            hipExtLaunchKernelGGL((fd_chunk_kernel<HD, G, false, false, false, true>), grid,
                                  dim3(256), (uint32_t)shm, s, ev0, ev1, 0u, q, kc, vc, lens,
                                  slot_seq, po, pl, nq, nkv, max_len, chunk, nc_max, hs, qa);
        else
            hipExtLaunchKernelGGL((fd_chunk_kernel<HD, G, false>), grid, dim3(256), (uint32_t)shm,
                                  s, ev0, ev1, 0u, q, kc, vc, lens, slot_seq, po, pl, nq, nkv,
                                  max_len, chunk, nc_max, hs, qa);
    } else if (early) {
        hipLaunchKernelGGL((fd_chunk_kernel<HD, G, true, true>), grid, dim3(256), shm, s, q, kc, vc,
                           lens, slot_seq, po, pl, nq, nkv, max_len, chunk, nc_max, hs, qa);
    } else if (qi && pre) {
        hipLaunchKernelGGL((fd_chunk_kernel<HD, G, true, false, false, true>), grid, dim3(256), shm,
                           s, q, kc, vc, lens, slot_seq, po, pl, nq, nkv, max_len, chunk, nc_max,
                           hs, qa);
    } else if (qi) {
        hipLaunchKernelGGL((fd_chunk_kernel<HD, G, true>), grid, dim3(256), shm, s, q, kc, vc, lens,
                           slot_seq, po, pl, nq, nkv, max_len, chunk, nc_max, hs, qa);
    } else if (longest_first) {
        hipLaunchKernelGGL((fd_chunk_kernel<HD, G, false, false, true>), grid, dim3(256), shm, s,
                           q, kc, vc, lens, slot_seq, po, pl, nq, nkv, max_len, chunk, nc_max, hs,
                           qa);
    } else if (pre) {
        hipLaunchKernelGGL((fd_chunk_kernel<HD, G, false, false, false, true>), grid, dim3(256),
                           shm, s, q, kc, vc, lens, slot_seq, po, pl, nq, nkv, max_len, chunk,
                           nc_max, hs, qa);
    } else {
        hipLaunchKernelGGL((fd_chunk_kernel<HD, G, false>), grid, dim3(256), shm, s, q, kc, vc,
                           lens, slot_seq, po, pl, nq, nkv, max_len, chunk, nc_max, hs, qa);
    }
    return check_launch("fd_chunk_kernel");
}

// Workgroups per KV head's query-head group: 1 while the grid has at least
// 256 workgroups (one per compute unit); below that (short caches at small
// batch, latency-bound) the largest divisor of the group size that keeps the
// grid within 1024 workgroups.
int fd_head_split(int group, int m, int nkv, int nc_max) {
    const int64_t base = (int64_t)nc_max * nkv * m;
    if (base >= 256) return 1;
    int hs = 1;
    for (int d = 2; d <= group; ++d)
        if (group % d == 0 && base * d <= 1024) hs = d;
    return hs;
}

template <int HD>
rra_status launch_chunk_hd(int group, const float *q, const float *kc, const float *vc,
                           const uint32_t *lens, const uint32_t *slot_seq, float *po, float *pl,
                           int m, int nq, int nkv, int max_len, int chunk, int nc_max, int hs_want,
                           bool longest_first, const QkvIn *qi, hipStream_t s, hipEvent_t ev0,
                           hipEvent_t ev1) {
    if (group < 1 || group > 8) return fail(RRA_EINVAL, "flash decode: nq/nkv=%d not in 1..8", group);
    if (hs_want < 0 || (hs_want > 0 && group % hs_want))
        return fail(RRA_EINVAL, "flash decode: head split %d does not divide the group size %d",
                    hs_want, group);
    const int hs = hs_want > 0 ? hs_want : fd_head_split(group, m, nkv, nc_max);
    switch (group / hs) {
#define RRA_G(gv) \
    case gv:                                                                                    \
        return launch_chunk<HD, gv>(q, kc, vc, lens, slot_seq, po, pl, m, nq, nkv, max_len, chunk, \
                                    nc_max, hs, longest_first, qi, s, ev0, ev1);
        RRA_G(1) RRA_G(2) RRA_G(3) RRA_G(4) RRA_G(5) RRA_G(6) RRA_G(7) RRA_G(8)
#undef RRA_G
    }
    return fail(RRA_EINVAL, "flash decode: nq/nkv=%d not in 1..8", group);
}

}  // namespace

int fd_choose_chunk(int m, int nkv, int max_len, int chunk) {
    if (chunk > 0) return chunk;
    // About one workgroup per 512 cached rows, but at least 256 (one per
    // compute unit) and at most 4096; the splits per (sequence, KV head) then
    // give the rows per split, rounded up to a multiple of 32 in 64..1024.
    // Fewer, longer splits save per-workgroup cost (query load, softmax,
    // partial write) and reduce work; more keep short caches spread over the
    // chip.  Measured on MI355X over M = 1..32 at 0.5B, 1.5B and 8B-sized KV
    // heads: within 5 % of the best fixed split size everywhere.  Once the
    // grid has 1024 workgroups (four resident per compute unit) a sequence
    // gets at most 5 splits: more only add per-workgroup cost.  8B-shaped
    // layer at M = 32 (lengths 2112..4160, 8 KV heads): 5 splits 134-136 us,
    // 8 splits 140-141 us; an 8192-row cache (lengths U[1, 8192], 8 KV heads):
    // 8 and 16 splits within 1 % (183-187 us).
    const int64_t pairs = (int64_t)m * nkv;
    const int64_t wgs = std::min<int64_t>(4096, std::max<int64_t>(256, pairs * max_len / 512));
    const int64_t nc = std::max<int64_t>(
        1, std::min<int64_t>(wgs / pairs, std::max<int64_t>(5, (1024 + pairs - 1) / pairs)));
    const int64_t rows = (max_len + nc - 1) / nc;
    return (int)std::min<int64_t>(1024, std::max<int64_t>(64, (rows + 31) / 32 * 32));
}

int fd_candidates(int m, int nkv, int group, int max_len, int *chunks, int *head_splits, int cap) {
    // Splits per (sequence, KV head) to try; each gives the rows per split
    // (rounded up to a multiple of 32, in 32..1024), duplicates dropped.  A
    // head split hs > 1 (the group's query heads dealt to hs workgroups) is
    // tried only on grids of fewer than 1024 workgroups, where the kernel is
    // latency-bound; no candidate has more than 8192 workgroups.
    static const int kSplits[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16, 20, 24, 28, 32,
                                  40, 48, 56, 64, 80, 96, 112, 128, 160, 192, 224, 256};
    int n = 0, last_chunk = 0;
    for (int nc : kSplits) {
        const int64_t rows = (max_len + nc - 1) / nc;
        const int chunk = (int)((rows + 31) / 32 * 32);
        if (chunk > 1024) continue;
        if (chunk < 32 || chunk == last_chunk) continue;
        last_chunk = chunk;
        const int64_t base = cdiv(max_len, chunk) * (int64_t)nkv * m;
        if (base > 8192) break;  // the splits only grow from here
        for (int hs = 1; hs <= group; ++hs) {
            if (group % hs) continue;
            if (hs > 1 && (base >= 1024 || base * hs > 4096)) break;
            if (n < cap && chunks) chunks[n] = chunk;
            if (n < cap && head_splits) head_splits[n] = hs;
            ++n;
        }
    }
    return n;
}

size_t fd_tuned_floats(int m, int nq, int nkv, int hd, int max_len) {
    int chunks[256];
    const int n = std::min(256, fd_candidates(m, nkv, std::max(1, nq / std::max(1, nkv)), max_len,
                                              chunks, nullptr, 256));
    size_t best = fd_partials_floats(m, nq, hd, max_len, fd_choose_chunk(m, nkv, max_len, 0));
    for (int i = 0; i < n; ++i) best = std::max(best, fd_partials_floats(m, nq, hd, max_len, chunks[i]));
    return best;
}

rra_status fd_time_candidates(const float *q, const float *const *k_caches,
                              const float *const *v_caches, int n_caches,
                              const uint32_t *seq_len, float *out, int m, int nq, int nkv, int hd,
                              int max_len, float *part, hipStream_t s, int *chunk_out,
                              int *hs_out, float *us_out, const QkvIn *qi, bool longest_first) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    RRA_TRY_HIP(hipStreamIsCapturing(s, &cs));
    if (cs != hipStreamCaptureStatusNone)
        return fail(RRA_EINVAL, "flash-decode tuning: the stream is capturing a graph");
    int chunks[256], hss[256];
    const int n = std::min(256, fd_candidates(m, nkv, nq / nkv, max_len, chunks, hss, 256));
    if (n == 0) return fail(RRA_EINVAL, "flash-decode tuning: no candidate for this shape");
    hipEvent_t e0, e1;
    RRA_TRY_HIP(hipEventCreate(&e0));
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return fail(RRA_EHIP, "flash-decode tuning: hipEventCreate failed");
    }
    std::vector<float> best(n, 1e30f);
    rra_status st = RRA_OK;
    // Two rounds over every candidate (the fastest time of each kept), so a
    // slow moment of the machine does not decide alone; each time is the
    // mean of `reps` back-to-back launches (chunk kernel + combine).  The
    // launches walk through the n_caches caches (a model's layers), one
    // after another, so that at small batches, where one layer's cache fits
    // in the caches of the chip, a launch does not find its rows there from
    // the launch before, just as in a decode step.
    constexpr int reps = 4;
    int next = 0;
    auto launch = [&](int i) {
        const int l = next;
        next = (next + 1) % n_caches;
        return launch_flash_decode(q, k_caches[l], v_caches[l], seq_len, out, m, nq, nkv, hd,
                                   max_len, chunks[i], part, s, nullptr, nullptr, true, qi,
                                   nullptr, nullptr, hss[i], longest_first);
    };
    for (int round = 0; round < 2 && st == RRA_OK; ++round) {
        for (int i = 0; i < n && st == RRA_OK; ++i) {
            st = launch(i);
            if (st != RRA_OK) break;
            if (hipEventRecord(e0, s) != hipSuccess) { st = fail(RRA_EHIP, "hipEventRecord"); break; }
            for (int r = 0; r < reps && st == RRA_OK; ++r) st = launch(i);
            if (st != RRA_OK) break;
            float ms = 0.f;
            if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
                st = fail(RRA_EHIP, "flash-decode tuning: event timing failed");
                break;
            }
            best[i] = std::min(best[i], 1e3f * ms / reps);
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    RRA_TRY(st);
    // On bandwidth-bound grids (at least 1024 workgroups), among the
    // candidates within 3 % of the fastest, the one with the fewest
    // workgroups: timed alone, neighbouring split counts differ by less than
    // the run-to-run noise, and between the decode step's GEMVs the grid with
    // less per-workgroup work (query loads, softmax, partial writes) and fewer
    // partials holds up better (MI355X, 8B-shaped layer at M=32: 5 splits
    // 129 us in the step against 136 us for 7, within 1 % of each other alone).
    // Smaller grids are latency-bound and take the fastest: there the step
    // favoured the grid with more workgroups (1.5B-shaped decoder at M = 4
    // and 8: 160-row splits with head split 6 and 3, 1-2 % faster in the step
    // than the 96- and 160-row ones with head split 2 the rule picked).
    int fastest = 0;
    for (int i = 1; i < n; ++i)
        if (best[i] < best[fastest]) fastest = i;
    auto wgs = [&](int i) { return cdiv(max_len, chunks[i]) * (int64_t)hss[i]; };
    int bi = fastest;
    if (wgs(fastest) * nkv * m >= 1024)
        for (int i = 0; i < n; ++i)
            if (best[i] <= 1.03f * best[fastest] && wgs(i) < wgs(bi)) bi = i;
    *chunk_out = chunks[bi];
    *hs_out = hss[bi];
    if (us_out) *us_out = best[bi];
    return RRA_OK;
}

size_t fd_partials_floats(int m, int nq, int hd, int max_len, int chunk) {
    const int nc_max = (int)cdiv(max_len, chunk);
    return (size_t)m * nq * nc_max * (size_t)(hd + 1);
}

int prefill_key_splits(int n, int nkv, uint32_t start) {
    // about 256 workgroups, each split with at least one 32-key block
    const int base = (int)cdiv(n, 16) * nkv;
    const int blocks = (int)cdiv((int64_t)start + n, 32);
    return std::max(1, std::min({kPrefillKeySplits, 256 / std::max(1, base), blocks}));
}

rra_status launch_prefill_attention(const float *q, const float *k_slot, const float *v_slot,
                                    float *out, int n, int nq, int nkv, int hd, int max_len,
                                    uint32_t start, const FragOut *fo, float *part,
                                    const uint32_t *lens, hipStream_t s) {
    const FragOut img = fo ? *fo : FragOut{nullptr, 0, 1, 0};
    const int group = nq / nkv;
    const int ks_n = part ? prefill_key_splits(n, nkv, start) : 1;
    float *po = part, *pl = part ? const_cast<float *>(fd_part_lse(part, n, nq, hd, ks_n)) : nullptr;
    const dim3 grid((unsigned)cdiv(n, 16), (unsigned)nkv, (unsigned)ks_n);
#define RRA_PA(HDV, GV)                                                                       \
    if (hd == HDV && group == GV) {                                                          \
        hipLaunchKernelGGL((prefill_attn_kernel<HDV, GV>), grid, dim3(64 * GV), 0, s, q, k_slot, \
                           v_slot, out, n, nq, nkv, max_len, start, img, ks_n, po, pl);     \
        RRA_TRY(check_launch("prefill_attn_kernel"));                                        \
        if (ks_n == 1) return RRA_OK;                                                        \
        hipLaunchKernelGGL(fd_reduce_kernel<HDV>, dim3(nq, n), dim3(64), 0, s, po, pl, lens, out, \
                           nq, max_len, 0, ks_n, img);                                       \
        return check_launch("fd_reduce_kernel");                                             \
    }
    RRA_PA(64, 1) RRA_PA(64, 2) RRA_PA(64, 3) RRA_PA(64, 4) RRA_PA(64, 5) RRA_PA(64, 6)
    RRA_PA(64, 7) RRA_PA(64, 8) RRA_PA(128, 1) RRA_PA(128, 2) RRA_PA(128, 3) RRA_PA(128, 4)
    RRA_PA(128, 5) RRA_PA(128, 6) RRA_PA(128, 7) RRA_PA(128, 8)
#undef RRA_PA
    return fail(RRA_EINVAL, "prefill attention: hd=%d, group %d", hd, group);
}

rra_status launch_kv_scatter(const float *k_rows, const float *v_rows, float *k_cache,
                             float *v_cache, const uint32_t *pos, int m, int nkv, int hd,
                             int max_len, hipStream_t s) {
    hipLaunchKernelGGL(kv_scatter_kernel, dim3(m), dim3(256), 0, s, k_rows, v_rows, k_cache,
                       v_cache, pos, nkv, hd, max_len);
    return check_launch("kv_scatter_kernel");
}

rra_status launch_flash_decode(const float *q, const float *k_cache, const float *v_cache,
                               const uint32_t *seq_len, float *out, int m, int nq, int nkv,
                               int hd, int max_len, int chunk, float *part, hipStream_t s,
                               const FragOut *fo, const uint32_t *slot_seq, bool reduce,
                               const QkvIn *qi, hipEvent_t chunk_start, hipEvent_t chunk_stop,
                               int head_split, bool longest_first) {
    if (qi && slot_seq) return fail(RRA_EINVAL, "flash decode: fused QKV input needs no slot map");
    const FragOut img = fo ? *fo : FragOut{nullptr, 0, 1, 0};
    const int G = nq / nkv;
    const int nc_max = (int)cdiv(max_len, chunk);
    float *po = part;
    float *pl = const_cast<float *>(fd_part_lse(part, m, nq, hd, nc_max));
    if (hd == 128)
        RRA_TRY(launch_chunk_hd<128>(G, q, k_cache, v_cache, seq_len, slot_seq, po, pl, m, nq, nkv,
                                     max_len, chunk, nc_max, head_split, longest_first, qi, s,
                                     chunk_start, chunk_stop));
    else
        RRA_TRY(launch_chunk_hd<64>(G, q, k_cache, v_cache, seq_len, slot_seq, po, pl, m, nq, nkv,
                                    max_len, chunk, nc_max, head_split, longest_first, qi, s,
                                    chunk_start, chunk_stop));
    if (!reduce) return RRA_OK;
    if (hd == 128)
        hipLaunchKernelGGL(fd_reduce_kernel<128>, dim3(nq, m), dim3(64), 0, s, po, pl, seq_len,
                           out, nq, max_len, chunk, nc_max, img);
    else
        hipLaunchKernelGGL(fd_reduce_kernel<64>, dim3(nq, m), dim3(64), 0, s, po, pl, seq_len, out,
                           nq, max_len, chunk, nc_max, img);
    return check_launch("fd_reduce_kernel");
}

}  // namespace rra

using namespace rra;

extern "C" rra_status rra_kv_scatter(const float *k_rows, const float *v_rows, float *k_cache,
                                     float *v_cache, const uint32_t *pos, int32_t m, int32_t nkv,
                                     int32_t hd, int32_t max_len, hipStream_t s) {
    clear_error();
    if (!k_rows || !v_rows || !k_cache || !v_cache || !pos)
        return fail(RRA_EINVAL, "rra_kv_scatter: null argument");
    if (m < 1 || m > RRA_M_MAX) return fail(RRA_EINVAL, "rra_kv_scatter: m=%d not in 1..32", m);
    if (nkv < 1 || hd < 1 || max_len < 1)
        return fail(RRA_EINVAL, "rra_kv_scatter: nkv=%d hd=%d max_len=%d", nkv, hd, max_len);
    return launch_kv_scatter(k_rows, v_rows, k_cache, v_cache, pos, m, nkv, hd, max_len, s);
}

static rra_status fd_validate(int32_t m, int32_t nq, int32_t nkv, int32_t hd, int32_t max_len,
                              int32_t chunk) {
    if (m < 1 || m > RRA_M_MAX) return fail(RRA_EINVAL, "flash decode: m=%d not in 1..32", m);
    if (hd != 64 && hd != 128) return fail(RRA_EINVAL, "flash decode: hd=%d not 64 or 128", hd);
    if (nkv < 1 || nq < 1 || nq % nkv || nq / nkv > 8)
        return fail(RRA_EINVAL, "flash decode: nq=%d nkv=%d (need nq %% nkv == 0, nq/nkv <= 8)",
                    nq, nkv);
    if (max_len < 1) return fail(RRA_EINVAL, "flash decode: max_len=%d", max_len);
    if (chunk != 0 && (chunk < 32 || chunk > 1024 || chunk % 32))
        return fail(RRA_EINVAL, "flash decode: chunk=%d (0, or a multiple of 32 in 32..1024)",
                    chunk);
    return RRA_OK;
}

// Tuned choices of the standalone flash decode (rra_flash_decode_tune), by
// shape; a chunk = 0 call of that shape uses it.
namespace {
struct FdTuned {
    int m, nq, nkv, hd, max_len, chunk, hs;
};
std::mutex g_fd_mu;
std::vector<FdTuned> g_fd_tuned;

bool fd_lookup(int m, int nq, int nkv, int hd, int max_len, int *chunk, int *hs) {
    std::lock_guard<std::mutex> lock(g_fd_mu);
    for (const FdTuned &t : g_fd_tuned)
        if (t.m == m && t.nq == nq && t.nkv == nkv && t.hd == hd && t.max_len == max_len) {
            *chunk = t.chunk;
            *hs = t.hs;
            return true;
        }
    return false;
}
}  // namespace

extern "C" int32_t rra_flash_decode_candidates(int32_t m, int32_t nq, int32_t nkv, int32_t max_len,
                                               int32_t *chunks, int32_t *head_splits, int32_t cap) {
    if (m < 1 || m > RRA_M_MAX || nkv < 1 || nq < 1 || nq % nkv || nq / nkv > 8 || max_len < 1 ||
        cap < 0)
        return 0;
    return fd_candidates(m, nkv, nq / nkv, max_len, chunks, head_splits, cap);
}

extern "C" int32_t rra_flash_decode_chunk(int32_t m, int32_t nkv, int32_t max_len, int32_t chunk) {
    return fd_choose_chunk(m, nkv, max_len, chunk);
}

extern "C" size_t rra_flash_decode_workspace_bytes(int32_t m, int32_t nq, int32_t nkv, int32_t hd,
                                                   int32_t max_len, int32_t chunk) {
    if (fd_validate(m, nq, nkv, hd, max_len, chunk) != RRA_OK) {
        clear_error();
        return 0;
    }
    // chunk = 0: enough for the default rule and for every candidate the
    // tuner may pick, so tuning never outgrows a workspace sized before it
    if (chunk == 0) return sizeof(float) * fd_tuned_floats(m, nq, nkv, hd, max_len);
    return sizeof(float) * fd_partials_floats(m, nq, hd, max_len, chunk);
}

extern "C" rra_status rra_flash_decode(const float *q, const float *k_cache, const float *v_cache,
                                       const uint32_t *seq_len, float *out, int32_t m, int32_t nq,
                                       int32_t nkv, int32_t hd, int32_t max_len, int32_t chunk,
                                       void *ws, size_t ws_bytes, hipStream_t s) {
    clear_error();
    if (!q || !k_cache || !v_cache || !seq_len || !out || !ws)
        return fail(RRA_EINVAL, "rra_flash_decode: null argument");
    RRA_TRY(fd_validate(m, nq, nkv, hd, max_len, chunk));
    const size_t need = rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, chunk);
    if (ws_bytes < need)
        return fail(RRA_ENOTINIT, "rra_flash_decode: workspace has %zu bytes, needs %zu", ws_bytes,
                    need);
    int c = fd_choose_chunk(m, nkv, max_len, chunk), hs = 0;
    if (chunk == 0) {
        int tc, th;
        if (fd_lookup(m, nq, nkv, hd, max_len, &tc, &th)) {
            c = tc;
            hs = th;
        }
    }
    return launch_flash_decode(q, k_cache, v_cache, seq_len, out, m, nq, nkv, hd, max_len, c,
                               static_cast<float *>(ws), s, nullptr, nullptr, true, nullptr,
                               nullptr, nullptr, hs, true);
}

extern "C" rra_status rra_flash_decode_ex(const float *q, const float *k_cache,
                                          const float *v_cache, const uint32_t *seq_len,
                                          float *out, int32_t m, int32_t nq, int32_t nkv,
                                          int32_t hd, int32_t max_len, int32_t chunk,
                                          int32_t head_split, void *ws, size_t ws_bytes,
                                          hipStream_t s) {
    clear_error();
    if (!q || !k_cache || !v_cache || !seq_len || !out || !ws)
        return fail(RRA_EINVAL, "rra_flash_decode_ex: null argument");
    RRA_TRY(fd_validate(m, nq, nkv, hd, max_len, chunk));
    if (chunk == 0) return fail(RRA_EINVAL, "rra_flash_decode_ex: chunk must be given (32..1024)");
    if (head_split < 1 || (nq / nkv) % head_split)
        return fail(RRA_EINVAL, "rra_flash_decode_ex: head_split=%d does not divide nq/nkv=%d",
                    head_split, nq / nkv);
    const size_t need = sizeof(float) * fd_partials_floats(m, nq, hd, max_len, chunk);
    if (ws_bytes < need)
        return fail(RRA_ENOTINIT, "rra_flash_decode_ex: workspace has %zu bytes, needs %zu",
                    ws_bytes, need);
    return launch_flash_decode(q, k_cache, v_cache, seq_len, out, m, nq, nkv, hd, max_len, chunk,
                               static_cast<float *>(ws), s, nullptr, nullptr, true, nullptr,
                               nullptr, nullptr, head_split, true);
}

extern "C" rra_status rra_flash_decode_tune(const float *q, const float *k_cache,
                                            const float *v_cache, const uint32_t *seq_len,
                                            float *out, int32_t m, int32_t nq, int32_t nkv,
                                            int32_t hd, int32_t max_len, void *ws,
                                            size_t ws_bytes, hipStream_t s, int32_t *chunk_out,
                                            int32_t *head_split_out) {
    clear_error();
    if (!q || !k_cache || !v_cache || !seq_len || !out || !ws)
        return fail(RRA_EINVAL, "rra_flash_decode_tune: null argument");
    RRA_TRY(fd_validate(m, nq, nkv, hd, max_len, 0));
    const size_t need = rra_flash_decode_workspace_bytes(m, nq, nkv, hd, max_len, 0);
    if (ws_bytes < need)
        return fail(RRA_ENOTINIT, "rra_flash_decode_tune: workspace has %zu bytes, needs %zu",
                    ws_bytes, need);
    int c = 0, hs = 0;
    RRA_TRY(fd_time_candidates(q, &k_cache, &v_cache, 1, seq_len, out, m, nq, nkv, hd, max_len,
                               static_cast<float *>(ws), s, &c, &hs, nullptr, nullptr, true));
    {
        std::lock_guard<std::mutex> lock(g_fd_mu);
        bool found = false;
        for (FdTuned &t : g_fd_tuned)
            if (t.m == m && t.nq == nq && t.nkv == nkv && t.hd == hd && t.max_len == max_len) {
                t.chunk = c;
                t.hs = hs;
                found = true;
            }
        if (!found) g_fd_tuned.push_back(FdTuned{m, nq, nkv, hd, max_len, c, hs});
    }
    if (chunk_out) *chunk_out = c;
    if (head_split_out) *head_split_out = hs;
    return RRA_OK;
}
