// elementwise.hip -- RMSNorm, RoPE, SwiGLU, greedy argmax, embedding gather,
// and the fused epilogues the decode step runs after each GEMV (split-K sum +
// residual + RMSNorm; split-K sum + RoPE + KV scatter; split-K sum + SwiGLU).
//
// Readings of the steps the pages name without defining (a Llama-style block):
//   RMSNorm  x / sqrt(mean(x^2) + eps) * gamma
//   RoPE     pairs (j, j + hd/2) rotated by pos * theta^(-2j/hd); the cos/sin
//            table is built in fp64 on the host and rounded once to fp32
//   SwiGLU   silu(gate) * up, silu(z) = z / (1 + e^-z)
//   argmax   lowest index among the maximal logits ([reduces] gpu_argmax:
//            block-level (max, index) pairs, then a final reduce)
#include "epilogue.h"
#include "frag.h"
#include "rra_internal.h"

#include <cmath>

namespace rra {
namespace {

// Sums over the `split` K-split planes of a GEMV result (stride floats
// apart), in plane order, of two columns at once (p and q).  Up to 8 planes
// are loaded at once (clamped addresses, unconditional loads), so the latency
// is paid once per 8 planes, not once per plane.
// Sum over a 256-thread block; every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum(v);
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float t = 0.f;
    const int nw = blockDim.x >> 6;
    for (int i = 0; i < nw; ++i) t += sh[i];
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *x,
                                                      const float *__restrict__ gamma,
                                                      float *out, int h, float eps) {
    __shared__ float sh[4];
    const float *xr = x + (size_t)blockIdx.x * h;
    float ss = 0.f;
    for (int i = threadIdx.x; i < h; i += blockDim.x) ss = fmaf(xr[i], xr[i], ss);
    ss = block_sum(ss, sh);
    const float inv = 1.0f / sqrtf(ss / (float)h + eps);
    float *o = out + (size_t)blockIdx.x * h;
    for (int i = threadIdx.x; i < h; i += blockDim.x) o[i] = xr[i] * inv * gamma[i];
}

// Grid (ceil(h / 512), m), 256 threads: 64 groups of 8 columns per block,
// the four waves sharing each group's split sum (group_split_sum), wave 0
// finishing it: x[m][c] += sum_s part[s][m][c] (split may be 0: x unchanged);
// the block's sum of squares of the updated row -> ss[m * nblocks + block];
// xg = x * gamma (fp32) and, when fo.img is set, its GEMV activation image
// (zeros for the groups in [h, kpad)).  The next GEMV forms RMSNorm from ss
// (NormIn).  With gi.embed set (no planes) the input row is gathered from
// the embedding table instead of read from x_in (GatherIn's rules) and
// written to x, in place of a separate gather launch: the same values.
__global__ __launch_bounds__(256) void residual_ss_kernel(const float *__restrict__ part, int split,
                                                          long long split_stride,
                                                          const float *x_in, float *x,
                                                          float *__restrict__ ss,
                                                          const float *__restrict__ gamma,
                                                          float *__restrict__ xg, int h,
                                                          FragOut fo, GatherIn gi) {
    __shared__ float red[3 * 64 * 8];
    __shared__ float sh[4];
    const int ch = blockIdx.x, m = blockIdx.y, nch = gridDim.x;
    const int k0 = (ch * 64 + (threadIdx.x & 63)) * 8;
    const size_t base = (size_t)m * h + k0;
    float acc[1][8];
    const float *const pp[1] = {split > 0 ? part + base : nullptr};
    group_split_sum<1>(pp, split > 0 && k0 < h, split, split_stride, acc, red);
    float sq = 0.f;
    if (threadIdx.x < 64) {
        if (k0 < h) {
            float v[8], gm[8], gv[8];
            bool gathered = false;
            if (gi.embed && gi.pos[m] != RRA_POS_NONE) {
                const uint32_t t = gi.tok[m];
                gathered = true;
                if (t < (uint32_t)gi.vocab) {
                    load8(gi.embed + (size_t)t * h + k0, v);
                } else {  // no read outside the table; reported once per row
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = 0.f;
                    if (ch == 0 && threadIdx.x == 0) report_error(gi.err, kErrToken);
                }
            } else {
                load8(x_in + base, v);
            }
            load8(gamma + k0, gm);
            resid8(v, acc[0], split > 0, gm, gv, sq);
            if (split > 0 || x_in != x || gathered) store8(x + base, v);
            store8(xg + base, gv);
            if (fo.img) frag_out8(fo, m, k0, gv);
        } else if (fo.img && k0 < fo.kpad) {
            const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            write_frag8_fmt(fo.fmt, fo.img, fo.ct, m, k0, z);
        }
    }
    sq = block_sum(sq, sh);
    if (threadIdx.x == 0) ss[(size_t)m * nch + ch] = sq;
}

// Grid (m, nq + 2 nkv heads), hd/2 threads: thread j handles pair (j, j + hd/2).
__global__ void qkv_post_kernel(const float *__restrict__ part, int split, long long split_stride,
                                const uint32_t *__restrict__ pos, const float *__restrict__ table,
                                float *__restrict__ q_out, float *__restrict__ kc,
                                float *__restrict__ vc, uint32_t *__restrict__ seq_len,
                                uint32_t *__restrict__ err, const uint32_t *__restrict__ slot_seq,
                                int nq, int nkv, int hd, int max_len) {
    const int m = blockIdx.x, head = blockIdx.y, j = threadIdx.x, half = hd >> 1;
    const size_t cs_row = slot_seq ? slot_seq[m] : (uint32_t)m;  // cache slot of row m
    const int nrow = (nq + 2 * nkv) * hd;
    const uint32_t p = pos[m];
    const bool ok = p < (uint32_t)max_len;  // also false for an empty slot (RRA_POS_NONE)
    const size_t b = (size_t)m * nrow + (size_t)head * hd;
    float a, c;
    sum_splits2(part + b + j, part + b + j + half, split, split_stride, a, c);
    if (head < nq + nkv && ok)
        rope_pair(a, c, table[((size_t)p * half + j) * 2], table[((size_t)p * half + j) * 2 + 1]);
    if (head < nq) {
        float *qo = q_out + ((size_t)m * nq + head) * hd;
        qo[j] = a;
        qo[j + half] = c;
    } else if (ok) {
        const bool is_k = head < nq + nkv;
        const int g = is_k ? head - nq : head - nq - nkv;
        float *dst = (is_k ? kc : vc) + ((cs_row * nkv + g) * max_len + p) * hd;
        dst[j] = a;
        dst[j + half] = c;
    }
    if (head == 0 && j == 0) {
        // an empty slot attends to nothing; any other bad position is an error
        seq_len[m] = ok ? p + 1 : (p == RRA_POS_NONE ? 0u : (uint32_t)max_len);
        if (!ok && p != RRA_POS_NONE) report_error(err, kErrPos);
    }
}

__global__ void rope_kernel(float *__restrict__ z, const uint32_t *__restrict__ pos,
                            const float *__restrict__ table, int n_heads, int hd, int max_len) {
    const int m = blockIdx.x, head = blockIdx.y, j = threadIdx.x, half = hd >> 1;
    const uint32_t p = pos[m];
    if (p >= (uint32_t)max_len) return;
    float *zr = z + ((size_t)m * n_heads + head) * hd;
    const float cs = table[((size_t)p * half + j) * 2], sn = table[((size_t)p * half + j) * 2 + 1];
    float a = zr[j], c = zr[j + half];
    rope_pair(a, c, cs, sn);
    zr[j] = a;
    zr[j + half] = c;
}

__global__ void swiglu_kernel(const float *gate, const float *up, float *out, int n,
                              long long gate_stride, long long up_stride, long long total) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const long long m = i / n, j = i - m * n;
    out[i] = silu(gate[m * gate_stride + j]) * up[m * up_stride + j];
}

// act[m][j] = silu(sum_s part[s][m][j]) * sum_s part[s][m][inter + j], and
// its activation image for the down GEMV.  Grid (ceil(max(inter, kpad) / 512),
// m), 256 threads: 64 groups of 8 columns per block, the four waves sharing
// each group's gate and up split sums (group_split_sum), wave 0 finishing.
__global__ __launch_bounds__(256) void swiglu_reduce_kernel(const float *__restrict__ part,
                                                            int split, long long split_stride,
                                                            float *__restrict__ act, int inter,
                                                            FragOut fo) {
    __shared__ float red[3 * 64 * 16];
    const int m = blockIdx.y;
    const int k0 = (blockIdx.x * 64 + (threadIdx.x & 63)) * 8;
    const size_t gi = (size_t)m * 2 * inter + k0, ui = gi + inter;
    float acc[2][8];
    const float *const pp[2] = {part + gi, part + ui};
    group_split_sum<2>(pp, k0 < inter, split, split_stride, acc, red);
    if (threadIdx.x >= 64) return;
    if (k0 < inter) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = swiglu1(acc[0][e], acc[1][e]);
        store8(act + (size_t)m * inter + k0, v);
        if (fo.img) frag_out8(fo, m, k0, v);
    } else if (fo.img && k0 < fo.kpad) {
        const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        write_frag8_fmt(fo.fmt, fo.img, fo.ct, m, k0, z);
    }
}

__global__ void embed_gather_kernel(const float *__restrict__ embed, const uint32_t *__restrict__ tok,
                                    const uint32_t *__restrict__ pos, float *__restrict__ x, int h,
                                    int vocab, uint32_t *__restrict__ err) {
    const int m = blockIdx.x;
    if (pos[m] == RRA_POS_NONE) return;  // empty slot: x row left as it is
    const uint32_t t = tok[m];
    float *xr = x + (size_t)m * h;
    if (t >= (uint32_t)vocab) {  // no read outside the table; reported
        for (int i = threadIdx.x; i < h; i += blockDim.x) xr[i] = 0.f;
        if (threadIdx.x == 0) report_error(err, kErrToken);
        return;
    }
    const float *er = embed + (size_t)t * h;
    if ((h & 3) == 0) {
        // 16-byte copies, four per thread in flight before any store (one
        // memory round trip for a 4096-wide row instead of sixteen)
        const float4 *e4 = reinterpret_cast<const float4 *>(er);
        float4 *x4 = reinterpret_cast<float4 *>(xr);
        const int h4 = h >> 2;
        for (int i0 = threadIdx.x; i0 < h4; i0 += 4 * blockDim.x) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = e4[min(i0 + u * (int)blockDim.x, h4 - 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i0 + u * (int)blockDim.x < h4) x4[i0 + u * blockDim.x] = v[u];
        }
        return;
    }
    for (int i = threadIdx.x; i < h; i += blockDim.x) xr[i] = er[i];
}

constexpr int kArgmaxPerBlock = 4096;  // 256 threads x 16 logits

__global__ __launch_bounds__(256) void argmax_pass1_kernel(const float *__restrict__ logits,
                                                           float *__restrict__ bv,
                                                           uint32_t *__restrict__ bi, int v,
                                                           int nb) {
    __shared__ float sv[4];
    __shared__ uint32_t si[4];
    const int blk = blockIdx.x, m = blockIdx.y;
    const float *l = logits + (size_t)m * v;
    float best = -INFINITY;
    uint32_t bidx = 0xFFFFFFFFu;
    // every load first (clamped index), then the combines: one memory round
    // trip; arg_combine's order (value, then lowest index) makes the result
    // independent of the order the candidates are taken in
    constexpr int PER = kArgmaxPerBlock / 256;
    float x[PER];
    const int base = blk * kArgmaxPerBlock + (int)threadIdx.x;
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] = l[min(base + i * 256, v - 1)];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (base + i * 256 < v) arg_combine(best, bidx, x[i], (uint32_t)(base + i * 256));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        arg_combine(best, bidx, __shfl_xor(best, off, 64), __shfl_xor(bidx, off, 64));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wave] = best;
        si[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) arg_combine(best, bidx, sv[w], si[w]);
        bv[(size_t)m * nb + blk] = best;
        bi[(size_t)m * nb + blk] = bidx;
    }
}

__global__ __launch_bounds__(256) void argmax_pass2_kernel(const float *__restrict__ bv,
                                                           const uint32_t *__restrict__ bi,
                                                           uint32_t *__restrict__ tok,
                                                           uint32_t *__restrict__ pos,
                                                           int advance, int nb, int stride) {
    __shared__ float sv[4];
    __shared__ uint32_t si[4];
    const int m = blockIdx.x;
    if (pos && pos[m] == RRA_POS_NONE) return;  // empty slot: tok and pos unchanged
    float best = -INFINITY;
    uint32_t bidx = 0xFFFFFFFFu;
    for (int i = threadIdx.x; i < nb; i += blockDim.x)
        arg_combine(best, bidx, bv[(size_t)m * stride + i], bi[(size_t)m * stride + i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        arg_combine(best, bidx, __shfl_xor(best, off, 64), __shfl_xor(bidx, off, 64));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wave] = best;
        si[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) arg_combine(best, bidx, sv[w], si[w]);
        tok[m] = bidx == 0xFFFFFFFFu ? 0u : bidx;
        if (advance) pos[m] += 1u;
    }
}

// Plain streaming read of n4 16-byte words: grid-stride, eight independent
// 128-bit loads in flight per thread, marked nontemporal as the decode step's
// weight and K/V streams are; each block writes the fp32 sum of the values it
// read (so the reads cannot be dropped, and the result is checkable).
typedef float rra_f4v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void hbm_read_kernel(const float4 *__restrict__ p, size_t n4,
                                                       float *__restrict__ sums) {
    constexpr int U = 8;
    __shared__ float sh[4];
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    float acc = 0.f;
    for (; i + (U - 1) * stride < n4; i += U * stride) {
        float4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const rra_f4v v =
                __builtin_nontemporal_load(reinterpret_cast<const rra_f4v *>(p + i + u * stride));
            a[u] = make_float4(v.x, v.y, v.z, v.w);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc += (a[u].x + a[u].y) + (a[u].z + a[u].w);
    }
    for (; i < n4; i += stride) {
        const float4 a = p[i];
        acc += (a.x + a.y) + (a.z + a.w);
    }
    acc = block_sum(acc, sh);
    if (threadIdx.x == 0) sums[blockIdx.x] = acc;
}

}  // namespace

rra_status launch_rmsnorm(const float *x, const float *gamma, float *out, int m, int h, float eps,
                          hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(m), dim3(256), 0, s, x, gamma, out, h, eps);
    return check_launch("rmsnorm_kernel");
}

rra_status launch_residual_ss(const float *part, int split, size_t split_stride, const float *x_in,
                              float *x, float *ss, const float *gamma, float *xg, int m, int h,
                              const FragOut &fo, hipStream_t s) {
    hipLaunchKernelGGL(residual_ss_kernel, dim3((unsigned)ss_parts(h), m), dim3(256), 0, s, part,
                       split, (long long)split_stride, x_in ? x_in : x, x, ss, gamma, xg, h, fo,
                       GatherIn{});
    return check_launch("residual_ss_kernel");
}

rra_status launch_gather_residual_ss(const GatherIn &g, float *x, float *ss, const float *gamma,
                                     float *xg, int m, int h, const FragOut &fo, hipStream_t s) {
    hipLaunchKernelGGL(residual_ss_kernel, dim3((unsigned)ss_parts(h), m), dim3(256), 0, s,
                       nullptr, 0, 0LL, x, x, ss, gamma, xg, h, fo, g);
    return check_launch("residual_ss_kernel");
}

rra_status launch_qkv_post(const float *part, int split, size_t split_stride, const uint32_t *pos,
                           const float *table, float *q_out, float *k_cache, float *v_cache,
                           uint32_t *seq_len, uint32_t *err, int m, int nq, int nkv, int hd,
                           int max_len, const uint32_t *slot_seq, hipStream_t s) {
    hipLaunchKernelGGL(qkv_post_kernel, dim3(m, nq + 2 * nkv), dim3(hd / 2), 0, s, part, split,
                       (long long)split_stride, pos, table, q_out, k_cache, v_cache, seq_len, err,
                       slot_seq, nq, nkv, hd, max_len);
    return check_launch("qkv_post_kernel");
}

rra_status launch_rope(float *z, const uint32_t *pos, const float *table, int m, int n_heads,
                       int hd, int max_len, hipStream_t s) {
    hipLaunchKernelGGL(rope_kernel, dim3(m, n_heads), dim3(hd / 2), 0, s, z, pos, table, n_heads,
                       hd, max_len);
    return check_launch("rope_kernel");
}

rra_status launch_swiglu(const float *gate, const float *up, float *out, int m, int n,
                         size_t gate_stride, size_t up_stride, hipStream_t s) {
    const long long total = (long long)m * n;
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s, gate, up,
                       out, n, (long long)gate_stride, (long long)up_stride, total);
    return check_launch("swiglu_kernel");
}

rra_status launch_swiglu_reduce(const float *part, int split, size_t split_stride, float *act,
                                int m, int inter, const FragOut &fo, hipStream_t s) {
    const int groups = (int)cdiv(std::max(inter, fo.img ? fo.kpad : inter), 8);
    hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)cdiv(groups, 64), m), dim3(256), 0, s,
                       part, split, (long long)split_stride, act, inter, fo);
    return check_launch("swiglu_reduce_kernel");
}

__global__ void prefill_rows_kernel(uint32_t *pos, uint32_t *slot_seq, uint32_t base,
                                    uint32_t seq, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        pos[i] = base + (uint32_t)i;
        slot_seq[i] = seq;
    }
}

rra_status launch_prefill_rows(uint32_t *pos, uint32_t *slot_seq, uint32_t base, uint32_t seq,
                               int n, hipStream_t s) {
    hipLaunchKernelGGL(prefill_rows_kernel, dim3((unsigned)cdiv(n, 64)), dim3(64), 0, s, pos,
                       slot_seq, base, seq, n);
    return check_launch("prefill_rows_kernel");
}

rra_status launch_embed_gather(const float *embed, const uint32_t *tok, const uint32_t *pos,
                               float *x, int m, int h, int vocab, uint32_t *err, hipStream_t s) {
    hipLaunchKernelGGL(embed_gather_kernel, dim3(m), dim3(256), 0, s, embed, tok, pos, x, h, vocab,
                       err);
    return check_launch("embed_gather_kernel");
}

size_t argmax_ws_bytes(int m, int v) {
    const size_t nb = (size_t)cdiv(v, kArgmaxPerBlock);
    return align_up((size_t)m * nb * sizeof(float), 256) + (size_t)m * nb * sizeof(uint32_t);
}

rra_status launch_argmax(const float *logits, uint32_t *tok, int m, int v, void *ws,
                         uint32_t *pos, bool advance, hipStream_t s) {
    const int nb = (int)cdiv(v, kArgmaxPerBlock);
    float *bv = static_cast<float *>(ws);
    uint32_t *bi = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) +
                                                align_up((size_t)m * nb * sizeof(float), 256));
    hipLaunchKernelGGL(argmax_pass1_kernel, dim3(nb, m), dim3(256), 0, s, logits, bv, bi, v, nb);
    RRA_TRY(check_launch("argmax_pass1_kernel"));
    hipLaunchKernelGGL(argmax_pass2_kernel, dim3(m), dim3(256), 0, s, bv, bi, tok, pos,
                       (pos && advance) ? 1 : 0, nb, nb);
    return check_launch("argmax_pass2_kernel");
}

rra_status launch_argmax_partials(const ArgOut &ao, uint32_t *tok, int m, uint32_t *pos,
                                  bool advance, hipStream_t s) {
    hipLaunchKernelGGL(argmax_pass2_kernel, dim3(m), dim3(256), 0, s, ao.val, ao.idx, tok, pos,
                       (pos && advance) ? 1 : 0, ao.blocks, ao.stride);
    return check_launch("argmax_pass2_kernel");
}

size_t gemv_argmax_ws_bytes(int m, int n) {
    const size_t cap = (size_t)gemv_argmax_blocks_max(n);
    return align_up((size_t)m * cap * sizeof(float), 256) + (size_t)m * cap * sizeof(uint32_t);
}

ArgOut gemv_argmax_out(void *ws, int m, int n) {
    const int cap = gemv_argmax_blocks_max(n);
    ArgOut ao;
    ao.val = static_cast<float *>(ws);
    ao.idx = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) +
                                          align_up((size_t)m * cap * sizeof(float), 256));
    ao.stride = cap;
    return ao;
}

void rope_table_host(float *table, int max_len, int hd, double theta) {
    const int half = hd / 2;
    for (int p = 0; p < max_len; ++p)
        for (int j = 0; j < half; ++j) {
            const double ang = (double)p * std::pow(theta, -2.0 * j / hd);
            table[((size_t)p * half + j) * 2] = (float)std::cos(ang);
            table[((size_t)p * half + j) * 2 + 1] = (float)std::sin(ang);
        }
}

rra_status launch_hbm_read(const void *buf, size_t bytes, float *sums, int blocks, hipStream_t s) {
    hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const float4 *>(buf), bytes / 16, sums);
    return check_launch("hbm_read_kernel");
}

}  // namespace rra
