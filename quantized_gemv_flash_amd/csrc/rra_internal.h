// Internal declarations shared by librra's sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "rra.h"

namespace rra {

// Records a thread-local message and returns `st`.
rra_status fail(rra_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
bool verbose();
bool capture_failure_requested();

#define RRA_TRY_HIP(call)                                                               \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess)                                                           \
            return ::rra::fail(RRA_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

#define RRA_TRY(expr)                       \
    do {                                    \
        rra_status st_ = (expr);            \
        if (st_ != RRA_OK) return st_;      \
    } while (0)

// Checks the launch status of the kernel just enqueued.
rra_status check_launch(const char *what);

// Bits of the model's device error word (read and cleared by rra_model_check).
constexpr uint32_t kErrPos = 1;    // a position >= max_len (nothing written for it)
constexpr uint32_t kErrToken = 2;  // a gathered token id >= vocab (a zero row was used)
constexpr uint32_t kErrRange = 4;  // a GEMV input element with |x| >= 65504 or not a number
// Sets `bit` in *err (no-op for a null err).  A vector-memory atomic: rare path.
__device__ __forceinline__ void report_error(uint32_t *err, uint32_t bit) {
    if (err) __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ tiles
// A tile covers 16 rows and KT columns: 1 KiB of quantised values (Q6K: the
// low 4 bits, then 512 B of high 2 bits), then the scales of its 16 rows.
constexpr int kRowTile = 16;
// Q8 and FP8 share one tile geometry (one byte per value); Q4 and Q6K share
// theirs (128 columns, 4 blocks of 32).
inline bool is_quantised(int fmt) {
    return fmt == RRA_Q8 || fmt == RRA_Q4 || fmt == RRA_FP8 || fmt == RRA_Q6K;
}
inline bool k128_tiles(int fmt) { return fmt == RRA_Q4 || fmt == RRA_Q6K; }
inline int tile_k(int fmt) { return k128_tiles(fmt) ? 128 : 64; }
inline int tile_blocks(int fmt) { return k128_tiles(fmt) ? 4 : 2; }
inline int tile_bytes(int fmt) {
    return fmt == RRA_Q6K ? 1024 + 512 + 128 + 32 : fmt == RRA_Q4 ? 1024 + 128 : 1024 + 64;
}

rra_status validate_weight(const rra_weight *w, const char *what, bool need_tiled_q);

// ------------------------------------------------------------------ GEMV
// How one GEMV is spread over the chip: `split` K-splits, each writing
// partial sums [split][m][n]; workgroups of `nw` waves, each wave owning
// `rpw` row tiles.
struct GemvPlan {
    int split = 1;
    int rpw = 1;  // row tiles (16 rows) per wave
    int nw = 4;   // waves per workgroup sharing one activation tile
    int kt_per_split = 1;
};
GemvPlan gemv_plan(const rra_weight &w, int m);
// The plan of a prompt chunk of 33..128 rows (decode steps use gemv_plan).
GemvPlan gemm_plan(const rra_weight &w);
// Rows of one prompt chunk at most (rra_prefill).
constexpr int kPrefillMax = 128;
// RMSNorm folded into a GEMV.  The GEMV input holds x[m][k] * gamma[k] (the
// producer applies gamma) and every output of row m is multiplied by
// inv[m] = 1 / sqrt(ss[m] / K + eps), ss[m] = sum of the `nparts` partial sums
// of squares of the un-scaled row x[m], ss[m*nparts + p]: since inv[m] is one
// scalar per row, W (x gamma inv) = inv (W (x gamma)).
struct NormIn {
    const float *ss;  // [M][nparts], or nullptr: no norm
    int nparts;
    float eps;
};
// A quantised GEMV's input formed inside the GEMV (small batches, short
// splits): instead of copying a finished activation image, each workgroup
// builds the image of its own K range from the producing step's partial
// results, with the same arithmetic as the kernel that would otherwise write
// the image (epilogue.h), so the result is bit-identical either way.
// kProResid: the residual step before an RMSNorm-fused GEMV (residual_ss):
// x_out = x_in + sum of the previous GEMV's split planes, the sums of squares
// of x_out (the norm is then applied from them, not from NormIn), and the
// image of x_out * gamma; x_out is written by one workgroup and must not
// alias x_in.
enum GemvPrologueKind { kProNone = 0, kProSwiglu = 1, kProAttn = 2, kProResid = 4 };
struct GemvPrologue {
    int kind;                 // GemvPrologueKind
    const float *part;        // SwiGLU: gate/up split partials [split][m][2 n]; attention: part_o;
                              // residual: the previous GEMV's partials [split][m][n]
    const float *lse;         // attention: part_lse
    const uint32_t *seq_len;  // attention: per-sequence lengths (clamped to max_len)
    long long stride;         // SwiGLU, residual: floats between split planes
    int split;                // SwiGLU, residual: split planes
    int n;                    // SwiGLU: intermediate size; attention: query heads; residual: hidden
    int nc_max, max_len;      // attention
    const float *x_in = nullptr;   // residual
    float *x_out = nullptr;        // residual
    const float *gamma = nullptr;  // residual
    float eps = 0.f;               // residual
    uint32_t *err = nullptr;       // error word: kErrRange when an image input leaves fp16's range
};
// Whether a GEMV of this plan can take a prologue (short splits, m <= 4).
bool gemv_takes_prologue(const rra_weight &w, const GemvPlan &p, int m);
// Whether it can take the residual prologue: besides the above, few enough
// split planes to read (each workgroup reads every plane of the whole rows).
bool gemv_takes_resid_prologue(const rra_weight &w, const GemvPlan &p, int m, int planes);

// Enqueues the GEMV; the result (or its K-split partial sums) goes to
// out[split][m][n] with out_split_stride floats between splits.  For quantised
// weights `x` is the activation image (frag.h) with frag_ct(m) column tiles;
// for F32 weights it is fp32 [m][k].
// Greedy-argmax partials of a GEMV's outputs (the LM head): when the GEMV
// runs as one K split of gemv_q_kernel, its workgroup b also writes, for each
// row m, the (largest stored value, lowest index) among the outputs it stores
// to val[m * stride + b] / idx[m * stride + b] and sets blocks to the number
// of workgroups; otherwise blocks stays 0 and the caller runs launch_argmax
// on the stored outputs.  Either way the ids are the same.
struct ArgOut {
    float *val = nullptr;
    uint32_t *idx = nullptr;
    int stride = 0;  // partials per row the buffers hold
    int blocks = 0;  // set by launch_gemv
};
// Partials per row that any launch shape of an n-row GEMV can produce.
inline int gemv_argmax_blocks_max(int64_t n) { return (int)((n + 63) / 64); }
size_t gemv_argmax_ws_bytes(int m, int n);
ArgOut gemv_argmax_out(void *ws, int m, int n);
rra_status launch_gemv(const rra_weight &w, const GemvPlan &p, const void *x, int m, float *out,
                       size_t out_split_stride, hipStream_t s, const NormIn *nrm = nullptr,
                       const GemvPrologue *pro = nullptr, ArgOut *ao = nullptr);
// The greedy ids from a GEMV's argmax partials (ao.blocks of them per row).
rra_status launch_argmax_partials(const ArgOut &ao, uint32_t *tok, int m, uint32_t *pos,
                                  bool advance, hipStream_t s);
// Converts fp32 x [m][k] into the activation image of a quantised GEMV.
rra_status launch_x_to_image(const float *x, uint8_t *img, int fmt, int m, int k, hipStream_t s);
// y[i][r] = sum over `split` partial planes (+ y[i][r] if accumulate).
rra_status launch_reduce_splits(const float *part, int split, size_t split_stride, float *y,
                                int m, int n, hipStream_t s);

// Where a producer writes the next GEMV's activation image (frag.h).
struct FragOut {
    uint8_t *img;  // nullptr: no image (fp32 weights)
    int fmt;       // the consumer's format: RRA_Q4 / RRA_Q6K, or RRA_Q8 / RRA_FP8
                   // (each pair reads the same image)
    int ct;        // column tiles (1 for m <= 16, 2 otherwise)
    int kpad;      // K rounded up to the K tile; groups in [K, kpad) are zeros
    uint32_t *err = nullptr;  // error word: kErrRange when an input leaves fp16's range
};

// ------------------------------------------------------------------ attention
int fd_choose_chunk(int m, int nkv, int max_len, int chunk);
size_t fd_partials_floats(int m, int nq, int hd, int max_len, int chunk);
// The (rows per split, head split) pairs the flash-decode tuner tries for m
// sequences, nkv KV heads of `group` query heads each and max_len cache rows;
// writes up to cap of them and returns their count.
int fd_candidates(int m, int nkv, int group, int max_len, int *chunks, int *head_splits, int cap);
// Partial floats enough for the default rule and every candidate.
size_t fd_tuned_floats(int m, int nq, int nkv, int hd, int max_len);
struct QkvIn;
// Times every candidate (chunk kernel + combine, synchronously on s) on the
// given inputs, its launches taking the n_caches K/V caches in turn, and
// returns the fastest (and its time in us if us_out).  With qi the chunk
// kernel is the QKV-fused one (qi.k_cache null: no cache write);
// longest_first as in launch_flash_decode.
rra_status fd_time_candidates(const float *q, const float *const *k_caches,
                              const float *const *v_caches, int n_caches,
                              const uint32_t *seq_len, float *out, int m, int nq, int nkv, int hd,
                              int max_len, float *part, hipStream_t s, int *chunk_out,
                              int *hs_out, float *us_out, const QkvIn *qi,
                              bool longest_first = false);
rra_status launch_kv_scatter(const float *k_rows, const float *v_rows, float *k_cache,
                             float *v_cache, const uint32_t *pos, int m, int nkv, int hd,
                             int max_len, hipStream_t s);
// The QKV GEMV's output taken by flash decode itself (qkv_post's work, at
// small batch in the decode step): the split kernel sums the split planes of
// its query heads and applies RoPE at pos; the workgroup that holds row pos
// of a sequence forms the new K/V row (summed, K roped), uses it in place of
// the cache row and writes it to the cache; one workgroup per sequence
// writes seq_len (and err), with qkv_post's rules.
struct QkvIn {
    const float *part = nullptr;  // [split][m][(nq + 2 nkv) hd]
    int split = 0;
    long long stride = 0;         // floats between split planes
    const uint32_t *pos = nullptr;
    const float *table = nullptr;  // RoPE table [max_len][hd/2][2]
    // the new K/V row is written at row pos; null: formed and attended to
    // but not written (the attention tuner times the fused kernel this way)
    float *k_cache = nullptr, *v_cache = nullptr;
    uint32_t *seq_len = nullptr, *err = nullptr;
};
// Row i of q attends to cache slot slot_seq[i] (slot i when slot_seq is null).
// head_split: workgroups per KV head's query-head group (a divisor of
// nq / nkv), or 0 for the default rule (fd_head_split).
// reduce = false launches the split kernel only (the O GEMV then combines the
// partials in its prologue).  longest_first: the chunk kernel's workgroups
// take the sequences longest first (grids of at most 4096 workgroups), so
// that the grid's tail holds short work; it costs each workgroup about 1 us
// and pays where the lengths differ widely (the standalone entry points), not
// in the decode step, whose nearly equal lengths it slowed by 1-2 %.  With qi, q and seq_len are ignored (the split
// kernel forms them; slot_seq must be null).
rra_status launch_flash_decode(const float *q, const float *k_cache, const float *v_cache,
                               const uint32_t *seq_len, float *out, int m, int nq, int nkv,
                               int hd, int max_len, int chunk, float *part, hipStream_t s,
                               const FragOut *fo = nullptr, const uint32_t *slot_seq = nullptr,
                               bool reduce = true, const QkvIn *qi = nullptr,
                               hipEvent_t chunk_start = nullptr, hipEvent_t chunk_stop = nullptr,
                               int head_split = 0, bool longest_first = false);
// Causal attention of a prompt chunk (matrix cores): q [n][nq][hd] at
// positions start .. start + n - 1 of one cache slot (k_slot, v_slot: that
// slot's [nkv][max_len][hd]), row t over the slot's rows [0, start + t];
// out [n][nq][hd] and, with fo, the O GEMV's activation image.  With `part`
// (n * nq * ks * (hd + 1) floats for ks = prefill_key_splits(n, nkv, start))
// the keys are split over workgroups and combined by fd_reduce_kernel, which
// reads lens[t] = start + t + 1.
constexpr int kPrefillKeySplits = 8;
int prefill_key_splits(int n, int nkv, uint32_t start);
rra_status launch_prefill_attention(const float *q, const float *k_slot, const float *v_slot,
                                    float *out, int n, int nq, int nkv, int hd, int max_len,
                                    uint32_t start, const FragOut *fo, float *part,
                                    const uint32_t *lens, hipStream_t s);
// Where rra_flash_decode's partials live in `part` (m sequences, nq heads).
inline const float *fd_part_lse(const float *part, int m, int nq, int hd, int nc_max) {
    return part + (size_t)m * nq * nc_max * hd;
}

// ------------------------------------------------------------------ elementwise
rra_status launch_rmsnorm(const float *x, const float *gamma, float *out, int m, int h,
                          float eps, hipStream_t s);
rra_status launch_rope(float *z, const uint32_t *pos, const float *table, int m, int n_heads,
                       int hd, int max_len, hipStream_t s);
rra_status launch_swiglu(const float *gate, const float *up, float *out, int m, int n,
                         size_t gate_stride, size_t up_stride, hipStream_t s);
size_t argmax_ws_bytes(int m, int v);
// tok[i] = argmax of logits row i (lowest index among equal maxima).  With
// pos: rows whose pos is RRA_POS_NONE are skipped (tok, pos unchanged), and
// pos[i] += 1 for the others when advance is set.
rra_status launch_argmax(const float *logits, uint32_t *tok, int m, int v, void *ws,
                         uint32_t *pos, bool advance, hipStream_t s);
void rope_table_host(float *table, int max_len, int hd, double theta);

// Fused epilogues used by the decode step.
// x[i] = x_in[i] + sum_s part[s][i] (x_in null: x itself; split may be 0);
// per 512-column chunk c the sum
// of squares of the updated row, ss[i * ss_parts(h) + c]; and xg = x * gamma,
// the input of the next RMSNorm-fused GEMV (fp32, and its image if fo.img).
// h % 8 == 0.
rra_status launch_residual_ss(const float *part, int split, size_t split_stride, const float *x_in,
                              float *x, float *ss, const float *gamma, float *xg, int m, int h,
                              const FragOut &fo, hipStream_t s);
// The step input gathered on the device (embed_gather_kernel's rules: row m
// of x becomes embedding row tok[m]; an empty slot, pos[m] == RRA_POS_NONE,
// keeps its row; a token id >= vocab gives a zero row and kErrToken).
struct GatherIn {
    const float *embed = nullptr;  // [vocab][h]
    const uint32_t *tok = nullptr, *pos = nullptr;
    int vocab = 0;
    uint32_t *err = nullptr;
};
// launch_residual_ss with no planes on the gathered rows: the gather and the
// first sums of squares and activation image in one launch.
rra_status launch_gather_residual_ss(const GatherIn &g, float *x, float *ss, const float *gamma,
                                     float *xg, int m, int h, const FragOut &fo, hipStream_t s);
__host__ __device__ inline int ss_parts(int h) { return (h + 511) / 512; }
// qkv = sum_s part[s]; rope(q, k) at pos; q -> q_out [m][nq][hd]; k, v rows
// scattered into the caches at pos, in cache slot slot_seq[i] (slot i when
// slot_seq is null); seq_len[i] = min(pos[i] + 1, max_len); pos >= max_len
// sets *err.
rra_status launch_qkv_post(const float *part, int split, size_t split_stride, const uint32_t *pos,
                           const float *table, float *q_out, float *k_cache, float *v_cache,
                           uint32_t *seq_len, uint32_t *err, int m, int nq, int nkv, int hd,
                           int max_len, const uint32_t *slot_seq, hipStream_t s);
// act[i][j] = silu(sum_s part[s][i][j]) * sum_s part[s][i][inter + j], and
// its activation image for the down GEMV.
rra_status launch_swiglu_reduce(const float *part, int split, size_t split_stride, float *act,
                                int m, int inter, const FragOut &fo, hipStream_t s);
// pos[i] = base + i, slot_seq[i] = seq for i < n (one prefill chunk).
rra_status launch_prefill_rows(uint32_t *pos, uint32_t *slot_seq, uint32_t base, uint32_t seq,
                               int n, hipStream_t s);
// Streaming read of `bytes` (a multiple of 16) with `blocks` workgroups;
// sums[b] = the fp32 sum of the values block b read.
rra_status launch_hbm_read(const void *buf, size_t bytes, float *sums, int blocks, hipStream_t s);
// x[i] = embed[tok[i]] for every slot whose pos is not RRA_POS_NONE; a token
// id >= vocab gives a zero row and sets kErrToken in *err (err may be null).
rra_status launch_embed_gather(const float *embed, const uint32_t *tok, const uint32_t *pos,
                               float *x, int m, int h, int vocab, uint32_t *err, hipStream_t s);

}  // namespace rra
