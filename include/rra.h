/*
 * rra.h -- C ABI of librra, the MI355X (gfx950) batched single-token decode
 * step: a weights-once dequantising batched GEMV, split-K flash-decoding
 * attention over an fp32 KV cache with grouped KV heads, and the RMSNorm /
 * RoPE / SwiGLU / residual / greedy-argmax steps around them, replayable as
 * one HIP graph.
 *
 * Sources (docs.rs source pages), cited per entry point below:
 *   [reduces]          realizar 0.8.5, src/cuda/executor/layers/reduces.rs
 *   [batched_forward]  realizar 0.8.5, src/cuda/executor/layers/batched_forward.rs
 *   [head_dim]         realizar 0.8.5, src/cuda/executor/head_dim.rs
 *   [graph]            aprender-serve 0.70.2, src/gguf/cuda/forward_qwen35_cuda_graph.rs
 *
 * Conventions for every call:
 *   - Pointers named as "device" are device (HBM) addresses owned by the
 *     caller; the library never allocates or frees device memory.  Scratch
 *     space is a caller-provided workspace whose size a *_workspace_bytes()
 *     call returns.  Host pointers are named as such.
 *   - Every call enqueues work only on the stream `s` it is given and returns
 *     without waiting for it, unless stated otherwise ([reduces]: host-to-device
 *     copies go on the launch stream so the legacy stream cannot reorder them).
 *     `s` may be 0 (the null stream) except where stated.
 *   - All activations are fp32, row-major, sequence-major: [M][...].
 *   - On a non-RRA_OK return nothing was enqueued unless stated, no partial
 *     outputs are promised, and rra_last_error() returns a message for the
 *     calling thread.
 *   - M (the number of sequences) is 1..32 ([batched_forward]
 *     forward_batched_to_token_ids rejects batch sizes outside 1..32).
 */
#ifndef RRA_H
#define RRA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RRA_VERSION 1
#define RRA_M_MAX 32

typedef enum rra_status {
    RRA_OK = 0,
    RRA_EINVAL = 1,   /* an argument is out of range, null, or inconsistent */
    RRA_ENOTINIT = 2, /* workspace too small, or model not created */
    RRA_EHIP = 3,     /* a HIP runtime call failed; message has its text */
    RRA_ECAPTURE = 4  /* graph capture failed and the eager fallback failed too */
} rra_status;

/* Weight formats.  Blocks are 32 consecutive elements along K of one row
 * (Q6K: super-blocks of 256).
 *   RRA_F32: fp32 weights.
 *   RRA_Q8 : 32 int8 values q and one fp16 scale per block; w = scale * q.
 *   RRA_Q4 : 32 unsigned 4-bit values q and one fp16 scale per block;
 *            w = scale * (q - 8).
 *   RRA_FP8: 32 OCP FP8 E4M3 codes q (sign, 4-bit exponent with bias 7,
 *            3-bit fraction; no infinity; S.1111.111 is NaN) and one fp16
 *            scale per block; w = scale * e4m3(q).  The pages run the LM head
 *            in FP8 ([batched_forward] batched_output_norm_lm_head_argmax);
 *            here it is one more block format of the same weights-once GEMV,
 *            usable for any matrix.
 *   RRA_Q6K: the 6-bit K-quant the pages name for LM heads (its block
 *            layout is not on the pages; read as the K-quant family's 6-bit
 *            format): super-blocks of 256 values along K, each of 16
 *            sub-blocks of 16 with a signed int8 scale sc, and one fp16 scale d
 *            per super-block; 6-bit codes q in 0..63; w = d * sc * (q - 32).
 *            k must be a multiple of 256. */
typedef enum rra_wfmt {
    RRA_F32 = 0,
    RRA_Q8 = 1,
    RRA_Q4 = 2,
    RRA_FP8 = 3,
    RRA_Q6K = 4
} rra_wfmt;

/* Storage layouts.
 *   RRA_PLANAR: F32 float[n][k]; Q8 data int8[n][k]; FP8 data uint8 codes
 *     [n][k]; Q4 data uint8[n][k/2] where byte j of a row holds element 2j in
 *     its low nibble and element 2j+1 in its high nibble; scales fp16 bit
 *     patterns [n][k/32].  Q6K data uint8[n][k/256][192]: per super-block 128
 *     bytes of the codes' low 4 bits (byte j: element 2j low nibble, 2j+1 high
 *     nibble), then 64 bytes of their high 2 bits (byte j: element 4j + e at
 *     bits 2e, 2e+1); Q6K `scale` points to uint8[n][k/256][18] records: the
 *     16 sub-scales, then d (fp16, low byte first).
 *   RRA_TILED (Q8/Q4/FP8/Q6K): the layout the GEMV streams.  Rows are grouped
 *     in tiles of 16 and K in tiles of 128 (Q4, Q6K) or 64 (Q8, FP8), one tile
 *     = 1 KiB of quantised values (Q6K: their low 4 bits, then 512 B of their
 *     high 2 bits) followed by its scales (128 B for Q4, 64 B for Q8/FP8; Q6K:
 *     128 B of sub-scales and the 16 rows' d); the scales live inside `data`
 *     and `scale` is NULL.  Rows are padded to a multiple of 16 and K to a
 *     multiple of the K tile with zero-valued blocks.  Produced by
 *     rra_repack_weight; rra_tiled_bytes gives its size. */
typedef enum rra_wlayout { RRA_PLANAR = 0, RRA_TILED = 1 } rra_wlayout;

/* A weight matrix W [n][k] (n outputs, k inputs); y = W x. */
typedef struct rra_weight {
    int32_t fmt;           /* rra_wfmt */
    int32_t layout;        /* rra_wlayout; RRA_F32 must be RRA_PLANAR */
    int64_t n, k;          /* k % 32 == 0 for Q8/Q4/FP8, k % 256 == 0 for Q6K */
    const void *data;      /* device, see the layouts above */
    const uint16_t *scale; /* device: planar Q8/Q4/FP8 fp16 bits [n][k/32], planar
                              Q6K byte records (above); tiled and F32: NULL */
} rra_weight;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *rra_last_error(void);
/* Static name of a status code. */
const char *rra_status_name(rra_status st);
int32_t rra_version(void);

/* ------------------------------------------------------------------ layout */

/* Bytes of the RRA_TILED form of an [n][k] weight of format fmt (Q8/Q4/FP8/Q6K);
 * 0 for an invalid shape or format. */
size_t rra_tiled_bytes(int32_t fmt, int64_t n, int64_t k);

/* Converts a planar Q8/Q4/FP8/Q6K weight into the tiled layout at `tiled`
 * (device, tiled_bytes >= rra_tiled_bytes) and fills *out (host) with its
 * descriptor.  Bit-exact: no value is changed, only moved.  EINVAL on F32, on
 * a non-planar input, on k % 32 != 0 (Q6K: k % 256) or on a short buffer. */
rra_status rra_repack_weight(const rra_weight *planar, void *tiled, size_t tiled_bytes,
                             rra_weight *out, hipStream_t s);

/* Inverse of rra_repack_weight: writes the planar data and scales (device,
 * the RRA_PLANAR layout of the weight's format; for Q6K `scale` receives the
 * byte records). */
rra_status rra_unpack_weight(const rra_weight *tiled, void *data, uint16_t *scale,
                             hipStream_t s);

/* -------------------------------------------------------- batched GEMV (a3)
 * [batched_forward] forward_batched_to_token_ids: batched GEMV kernels read
 * and dequantise every weight block once for all M inputs.
 *   y[i][r] = sum_c W[r][c] * x[i][c]   for i < m, r < n.
 * w   : F32 planar, or a tiled quantised weight (planar -> EINVAL, repack first:
 *       the kernel streams only the tiled layout, whose 16-row x K-tile records
 *       put each lane's bytes in matrix-core operand order; converting on every
 *       call would move the weights twice).
 * x   : device fp32 [m][k]; |x| must stay below 65504 for quantised weights (the
 *       activations enter the matrix cores as an fp16 high part plus an fp16
 *       low part).
 * y   : device fp32 [m][n]; must not overlap x.
 * ws  : device scratch, ws_bytes >= rra_batched_gemv_workspace_bytes(w, m),
 *       owned by the caller and reused freely after the call completes on s.
 *       It holds the activations converted once into the matrix-core operand
 *       image (quantised weights) and the split-K partial sums (when K is
 *       split).  May be NULL only when that size is 0; otherwise a missing or
 *       short ws gives RRA_ENOTINIT and nothing is launched.
 * Results do not depend on the stream, the call or the run (no atomics). */
size_t rra_batched_gemv_workspace_bytes(const rra_weight *w, int32_t m);
rra_status rra_batched_gemv(const rra_weight *w, const float *x, float *y, int32_t m,
                            void *ws, size_t ws_bytes, hipStream_t s);

/* The same GEMV on the vector ALUs (Q4 and Q8 tiled weights, m in 1..8),
 * kept to measure the matrix-core path against: one wave per 16-row tile,
 * each lane converting its bytes of every block to fp32 and accumulating fp32
 * FMAs with fp32 x staged in LDS, the four lanes of a row summed by cross-lane
 * adds.  Same y up to fp32 rounding order; ws as for rra_batched_gemv (only
 * its split-K partials are used); RRA_EINVAL when a K split would need more
 * than 64 KiB of LDS. */
rra_status rra_batched_gemv_valu(const rra_weight *w, const float *x, float *y, int32_t m,
                                 void *ws, size_t ws_bytes, hipStream_t s);

/* rra_batched_gemv for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation with the same kernels, bitwise the same y, with no
 * workspace argument.  Its scratch is a library-owned static device array of
 * RRA_GEMV_STATIC_SCRATCH_BYTES (16 MiB) per GPU, held until the process
 * ends; the call allocates nothing.  A call whose workspace would exceed that
 * size (rra_batched_gemv_workspace_bytes(w, m) > RRA_GEMV_STATIC_SCRATCH_BYTES)
 * returns RRA_EINVAL without launching.  All calls on one GPU share the one
 * array: calls that may overlap on that GPU (different streams without an
 * ordering between them, or different threads) race on it and must be
 * serialised by the caller.  Nothing in the array needs to start at zero.
 * s: the kernels run on s's device, whose copy of the array is used. */
#define RRA_GEMV_STATIC_SCRATCH_BYTES (16u << 20)
rra_status rra_batched_gemv_noalloc(const rra_weight *w, const float *x, float *y, int32_t m,
                                    hipStream_t s);

/* ---------------------------------------------------------- KV scatter (a5)
 * [head_dim] flash_decoding_attention_into, step 1: this token's K and V rows
 * are written into the caches at the sequence's position.
 *   k_cache[i][g][pos[i]][d] = k_rows[i][g*hd + d], same for V,
 *   for i < m, g < nkv, d < hd.
 * k_rows, v_rows : device fp32 [m][nkv*hd].
 * k_cache, v_cache : device fp32 [>= m][nkv][max_len][hd].
 * pos : device uint32 [m] (read on the device, so the call is graph-safe).
 * A sequence with pos[i] >= max_len is not written (no out-of-bounds store).
 * Pure copy: bit-exact. */
rra_status rra_kv_scatter(const float *k_rows, const float *v_rows, float *k_cache,
                          float *v_cache, const uint32_t *pos, int32_t m, int32_t nkv,
                          int32_t hd, int32_t max_len, hipStream_t s);

/* ------------------------------------------------ flash decoding (a6, a7)
 * [head_dim] flash_decoding_attention_into: the cache is split into chunks
 * processed in parallel, then the partial results are combined with softmax
 * rescaling; Q has num_heads heads, K/V num_kv_heads.
 *   out[i][h] = sum_{t < seq_len[i]} softmax_t(<q[i][h], K[i][g][t]> / sqrt(hd))
 *               * V[i][g][t],   g = h / (nq / nkv).
 * q   : device fp32 [m][nq][hd];  out : device fp32 [m][nq][hd].
 * k_cache, v_cache : device fp32 [>= m][nkv][max_len][hd].
 * seq_len : device uint32 [m]; values are clamped to max_len; a sequence with
 *       seq_len 0 leaves its out rows untouched.
 * hd in {64, 128}; nq % nkv == 0; nq / nkv <= 8.
 * chunk : at most this many rows per split, a multiple of 32 in [32, 1024],
 *       or 0 for the autotuned choice: the one rra_flash_decode_tune cached for
 *       this (m, nq, nkv, hd, max_len), else a default rule of (m, nkv,
 *       max_len) (rra_flash_decode_chunk).  The rows of a sequence are dealt
 *       round-robin to nc = ceil(max_len / chunk) splits (split c takes rows
 *       c, c + nc, ...); the result is the same softmax.  On grids of at most
 *       4096 workgroups (nc * nkv * m, times the head split) the workgroups
 *       launched first take the longest sequences, so that short work fills
 *       the grid's tail; a sequence's result does not depend on which
 *       workgroup computes it.
 * ws  : device scratch, ws_bytes >= rra_flash_decode_workspace_bytes(...) with
 *       the same chunk argument (for chunk 0: enough for every candidate the
 *       tuner may pick). */
size_t rra_flash_decode_workspace_bytes(int32_t m, int32_t nq, int32_t nkv, int32_t hd,
                                        int32_t max_len, int32_t chunk);
/* The default rule's rows per split (chunk 0), or chunk itself. */
int32_t rra_flash_decode_chunk(int32_t m, int32_t nkv, int32_t max_len, int32_t chunk);
rra_status rra_flash_decode(const float *q, const float *k_cache, const float *v_cache,
                            const uint32_t *seq_len, float *out, int32_t m, int32_t nq,
                            int32_t nkv, int32_t hd, int32_t max_len, int32_t chunk,
                            void *ws, size_t ws_bytes, hipStream_t s);

/* Split-size autotuning ([head_dim] flash_decoding_attention_into takes its
 * chunk size from a fixed constant; here it is chosen by timing on the GPU).
 * A candidate is (chunk, head_split): rows per split as above, and the number
 * of workgroups that share a KV head's nq/nkv query heads (a divisor of
 * nq/nkv; head_split 1 reads every K/V byte once, more shorten each
 * workgroup's work on small, latency-bound grids at the cost of cache-hit
 * re-reads).  The result is the same softmax for every candidate.
 *
 * rra_flash_decode_candidates: writes up to cap candidates for this shape
 * into chunks[] and head_splits[] (host; either may be NULL) and returns how
 * many there are (0 for an invalid shape).  The list depends only on the
 * arguments. */
int32_t rra_flash_decode_candidates(int32_t m, int32_t nq, int32_t nkv, int32_t max_len,
                                    int32_t *chunks, int32_t *head_splits, int32_t cap);
/* rra_flash_decode with an explicit candidate (chunk 32..1024, a multiple of
 * 32; head_split dividing nq/nkv); ws as for that chunk. */
rra_status rra_flash_decode_ex(const float *q, const float *k_cache, const float *v_cache,
                               const uint32_t *seq_len, float *out, int32_t m, int32_t nq,
                               int32_t nkv, int32_t hd, int32_t max_len, int32_t chunk,
                               int32_t head_split, void *ws, size_t ws_bytes, hipStream_t s);
/* Times every candidate on the caller's inputs (synchronous on s; s must not
 * be capturing a graph; `out` and ws are overwritten), writes the fastest to
 * *chunk_out / *head_split_out (host, nullable) and caches it process-wide
 * for this (m, nq, nkv, hd, max_len): later chunk = 0 calls of that shape use
 * it, so the choice stays fixed (and graph-safe) once made.  ws_bytes >=
 * rra_flash_decode_workspace_bytes(..., chunk = 0). */
rra_status rra_flash_decode_tune(const float *q, const float *k_cache, const float *v_cache,
                                 const uint32_t *seq_len, float *out, int32_t m, int32_t nq,
                                 int32_t nkv, int32_t hd, int32_t max_len, void *ws,
                                 size_t ws_bytes, hipStream_t s, int32_t *chunk_out,
                                 int32_t *head_split_out);

/* ------------------------------------------------------- step kernels
 * Exposed for per-step parity checks; rra_decode_step uses fused forms. */

/* RMSNorm (a2, a9, a12; [batched_forward] batched_output_norm_lm_head_argmax:
 * one launch for all M rows): out[i] = x[i] / sqrt(mean(x[i]^2) + eps) * gamma.
 * x, out: device fp32 [m][h] (may alias); gamma: device fp32 [h]. */
rra_status rra_rmsnorm(const float *x, const float *gamma, float *out, int32_t m, int32_t h,
                       float eps, hipStream_t s);

/* RoPE table for rra_rope: device fp32 [max_len][hd/2][2] holding (cos, sin)
 * of pos * theta^(-2i/hd), computed in fp64 on the host and rounded once.
 * Synchronous: returns after the copy has completed. */
rra_status rra_rope_table(float *table, int32_t max_len, int32_t hd, double theta,
                          hipStream_t s);

/* RoPE (a4; [graph] module doc: the position is read from device memory):
 * rotates every head of z in place by pos[i]: for each pair (j, j + hd/2),
 * (a, b) -> (a cos - b sin, a sin + b cos).  z: device fp32 [m][n_heads][hd];
 * pos: device uint32 [m]; a sequence with pos >= max_len is left unchanged. */
rra_status rra_rope(float *z, const uint32_t *pos, const float *table, int32_t m,
                    int32_t n_heads, int32_t hd, int32_t max_len, hipStream_t s);

/* SwiGLU (a10; [graph] module doc names the fused SwiGLU):
 * out[i][j] = silu(gate[i][j]) * up[i][j], silu(z) = z / (1 + e^-z).
 * All device fp32 [m][n]; out may alias gate or up. */
rra_status rra_swiglu(const float *gate, const float *up, float *out, int32_t m, int32_t n,
                      hipStream_t s);

/* Measurement aid, not a step of the decode path: a plain streaming read of
 * `bytes` bytes at `buf` (device memory, 16-byte aligned, bytes a non-zero
 * multiple of 16) by `blocks` 256-thread workgroups (1 .. 2^20) with 128-bit
 * loads, the practical HBM ceiling that the kernels' rates are compared
 * with.  sums: device fp32 [blocks], written with the sum of the fp32 values
 * each workgroup read (the buffer is read as floats).  Asynchronous on s;
 * argument errors return RRA_EINVAL without launching. */
rra_status rra_hbm_read(const void *buf, size_t bytes, float *sums, int32_t blocks, hipStream_t s);

/* Greedy argmax (a14; [reduces] gpu_argmax / batched_gpu_argmax: block-level
 * (max, index) pairs, then a final reduce, for all M rows with no host sync):
 * tok[i] = the lowest index among the maximal logits[i][*].  NaN logits are
 * never selected.  logits: device fp32 [m][v]; tok: device uint32 [m]. */
size_t rra_argmax_workspace_bytes(int32_t m, int32_t v);
rra_status rra_argmax(const float *logits, uint32_t *tok, int32_t m, int32_t v, void *ws,
                      size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------- decode step (a1-a15)
 * [batched_forward] forward_batched_to_token_ids: M embeddings and M positions
 * in, every layer, then output norm -> LM head -> argmax, M token ids out.
 * Layer body (a Llama pre-norm block):
 *   u = rmsnorm(x, attn_gamma); [q k v] = Wqkv u; rope(q, k); scatter k, v
 *   at pos; a = attention(q, cache, pos + 1); x += Wo a;
 *   u = rmsnorm(x, ffn_gamma); x += Wd (silu(Wg u) * Wu u).
 * Tail: logits = W_lm rmsnorm(x, out_gamma); tok = argmax(logits). */
typedef struct rra_layer_desc {
    rra_weight wqkv;          /* [(nq + 2 nkv) hd][hidden]: q rows, k rows, v rows */
    rra_weight wo;            /* [hidden][nq hd] */
    rra_weight wgu;           /* [2 inter][hidden]: gate rows, then up rows */
    rra_weight wd;            /* [hidden][inter] */
    const float *attn_gamma;  /* device [hidden] */
    const float *ffn_gamma;   /* device [hidden] */
    float *k_cache;           /* device [m_max][nkv][max_len][hd] */
    float *v_cache;           /* device [m_max][nkv][max_len][hd] */
} rra_layer_desc;

typedef struct rra_model_desc {
    int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab;
    float rms_eps;
    double rope_theta;
    int32_t max_len;               /* cache rows per sequence */
    int32_t m_max;                 /* cache slots; every step has m <= m_max <= 32 */
    const rra_layer_desc *layers;  /* host array [n_layers], copied at create */
    const float *out_gamma;        /* device [hidden] */
    rra_weight lm_head;            /* [vocab][hidden] */
    const float *embed;            /* device [vocab][hidden] fp32, or NULL (needed for RRA_STEP_GATHER) */
    int32_t attn_chunk;            /* flash-decode rows per split; 0 = chosen by the library
                                      for each step from its m, nkv and max_len */
    int32_t prefill_rows;          /* prompt tokens per rra_prefill chunk, 0..128 (0 = 128);
                                      the workspace holds max(m_max, prefill_rows) rows */
} rra_model_desc;

typedef struct rra_model rra_model;

/* Step flags. */
#define RRA_GRAPH 1        /* run as a captured HIP graph (captured on the first
                              call for a given (m, flags, pointers) key, replayed
                              after; [graph] module doc, [batched_forward]
                              forward_batched_to_token_ids_graphed).  If the
                              capture fails it is discarded, the stream leaves
                              capture mode and the step runs eagerly ([reduces]
                              try_graph_capture); the environment variable
                              RRA_FAIL_CAPTURE=1 makes every capture fail, to
                              test that path.  RRA_VERBOSE=1 logs captures and
                              fallbacks to stderr. */
#define RRA_STEP_GATHER 2  /* x[i] = embed[tok[i]] first (tok read as input) */
#define RRA_STEP_ADVANCE 4 /* pos[i] += 1 after the step */

/* A slot whose position is RRA_POS_NONE is empty ([head_dim]
 * flash_decoding_attention_into: a sequence with nothing to attend to is
 * skipped, the done-mask early exit).  Continuous batching: a slot leaves by
 * setting its position to RRA_POS_NONE and joins by setting a real position,
 * on the device, between steps, with no recapture of the step graph.  The
 * step leaves an empty slot's cache rows, tok and pos unchanged and does not
 * gather its x row; its x and logits rows after the step are unspecified.
 * The other slots' results do not depend on empty slots in any way. */
#define RRA_POS_NONE 0xFFFFFFFFu

size_t rra_model_workspace_bytes(const rra_model_desc *d);
/* The same size under the name the decode-step contract uses: the workspace
 * rra_model_create needs for descriptor d (0 if d is invalid). */
size_t rra_decode_workspace_bytes(const rra_model_desc *d);

/* Validates d, lays the workspace out (device, ws_bytes >=
 * rra_model_workspace_bytes(d)), fills its RoPE table on stream s (and waits
 * for it), and returns a host handle in *out.  Weights, caches and gammas are
 * referenced, not copied: they must outlive the model. */
rra_status rra_model_create(const rra_model_desc *d, void *ws, size_t ws_bytes, hipStream_t s,
                            rra_model **out);

/* One decode step for sequences 0..m-1.
 * x      : device fp32 [m][hidden], in/out: the step input (embedding rows)
 *          and, on return, the final residual stream (before the output norm).
 * pos    : device uint32 [m], this token's position per sequence; the K/V rows
 *          are written there and attention covers rows [0, pos]; RRA_POS_NONE
 *          marks an empty slot (see above); any other position >= max_len
 *          writes nothing, and is reported by rra_model_check.
 * tok    : device uint32 [m], out (and in under RRA_STEP_GATHER, where an id
 *          >= vocab gathers a zero row and is reported by rra_model_check).
 * tok_host : host uint32 [m] or NULL.  When non-NULL the call waits for the
 *          stream and copies the ids there (the one sync of the step).
 * logits : device fp32 [m][vocab] or NULL (then an internal buffer is used).
 * flags  : RRA_GRAPH | RRA_STEP_GATHER | RRA_STEP_ADVANCE.  RRA_GRAPH needs a
 *          non-null stream.  If capture fails the step runs eagerly.
 * Writes k_cache/v_cache[l][i][*][pos[i]] for every layer. */
rra_status rra_decode_step(rra_model *mdl, float *x, uint32_t *pos, uint32_t *tok,
                           uint32_t *tok_host, float *logits, int32_t m, int32_t flags,
                           hipStream_t s);

/* The decode step with a non-blocking hand-off of its ids ([reduces]
 * forward_graphed_replay: a completion event recorded after each replay, to
 * be queried for pipelining): rra_decode_step (tok_host = NULL), then an
 * asynchronous copy of the m ids into tok_pinned and a record of `done`, all
 * on s; returns without waiting.  Once `done` has completed
 * (hipEventQuery / hipEventSynchronize), tok_pinned holds this step's ids.
 * tok_pinned: page-locked host memory (hipHostMalloc) [m], else RRA_EINVAL;
 * done: an event created by the caller.  With RRA_STEP_GATHER |
 * RRA_STEP_ADVANCE the device feeds the ids back itself, so a caller can
 * enqueue step t+1 before reading step t's ids: with two tok_pinned buffers
 * and two events used alternately, the host reads one step's ids while the
 * next step runs.  A buffer must not be reused until its event has completed
 * and the host has read it. */
rra_status rra_decode_step_async(rra_model *mdl, float *x, uint32_t *pos, uint32_t *tok,
                                 uint32_t *tok_pinned, hipEvent_t done, float *logits, int32_t m,
                                 int32_t flags, hipStream_t s);

/* Prefill (context ingestion; [head_dim] tensor_core_attention: causal
 * attention of every prompt token to itself and the tokens before it).
 * Runs the n_tokens prompt tokens of cache slot `seq` through the model at
 * positions start .. start + n_tokens - 1: every layer's K/V rows for those
 * positions are written into the slot's cache, each token attending to cache
 * rows [0, its position] -- the rows already there (a context ingested
 * earlier) and the prompt tokens before it -- the same result as the tokens
 * fed one at a time through rra_decode_step (up to rounding).  The tokens go
 * through in chunks of prefill_rows: per chunk and layer, each weight matrix
 * is streamed once for all of the chunk's rows (a matrix-core GEMM with the
 * decode GEMV's exact-integer weights and fp16 high + low activation parts),
 * RoPE is applied and the chunk's K/V rows are written into the slot, and a
 * matrix-core causal attention (scores and outputs from fp16 high + low
 * operand parts, fp32 accumulation, online softmax) takes each row over the
 * slot's rows up to its position.  Only the last token reaches the output
 * norm, LM head and argmax.
 * tokens   : device uint32 [n_tokens], ids < vocab.
 * seq      : cache slot in [0, m_max).  Other slots are not touched.
 * start    : position of tokens[0]; start + n_tokens <= max_len (else
 *            RRA_EINVAL, nothing enqueued).
 * next_tok : device uint32 [1] or NULL: the greedy id after the last token
 *            (the first token a decode step for this slot then consumes at
 *            position start + n_tokens).
 * logits   : device fp32 [vocab] or NULL: the last token's logits.
 * Needs the model's embedding table.  Enqueued on s without a sync and
 * without graph capture; it uses the model's workspace, so calls on one model
 * (prefill or decode) must be ordered on one stream. */
rra_status rra_prefill(rra_model *mdl, const uint32_t *tokens, int32_t n_tokens, int32_t seq,
                       uint32_t start, uint32_t *next_tok, float *logits, hipStream_t s);

/* The model's flash-decode plan for steps of m sequences (m in 1..
 * max(m_max, prefill_rows)): rows per split and head split (0: the default
 * rule, which may split heads on small grids).  Initially the default rule
 * of (m, n_kv_heads, max_len), or attn_chunk when the descriptor sets one. */
rra_status rra_model_attention_plan(const rra_model *mdl, int32_t m, int32_t *chunk,
                                    int32_t *head_split);
/* Sets that plan (chunk: a multiple of 32 in 32..1024 whose partials fit the
 * workspace, which holds every tuner candidate; head_split: 0 or a divisor of
 * n_heads / n_kv_heads).  A change drops the model's captured graphs (they
 * hold the old grid); the next RRA_GRAPH step captures again. */
rra_status rra_model_set_attention_plan(rra_model *mdl, int32_t m, int32_t chunk,
                                        int32_t head_split);
/* Autotunes the plan for each batch size in ms[0..n_ms) (host; NULL or n_ms
 * <= 0: every m in 1..m_max): times every rra_flash_decode_candidates pair on
 * layer 0's caches with sequence lengths lengths[i] (host [m_max], clamped to
 * max_len; NULL: max_len) and keeps the fastest, as rra_model_set_attention_plan
 * would.  Synchronous on s, which must not be capturing; it overwrites the
 * model's workspace (not the caches), so it must not overlap steps of the
 * model.  The cache contents do not matter for the timing. */
rra_status rra_model_tune_attention(rra_model *mdl, const int32_t *ms, int32_t n_ms,
                                    const uint32_t *lengths, hipStream_t s);

/* Waits for stream s and reports (and clears) the device-side error word:
 * RRA_EINVAL, with a message naming each condition, if a step or prefill
 * since the last check saw
 *   - a position >= max_len (other than RRA_POS_NONE): nothing was written
 *     for that sequence;
 *   - a gathered token id >= vocab (RRA_STEP_GATHER, rra_prefill): a zero row
 *     was used as its embedding;
 *   - an activation entering a quantised GEMV with |x| >= 65504 or NaN: its
 *     fp16 operand parts are not exact there, so that step's results are not
 *     to be trusted.
 * These are detected inside the kernels (no fault, no extra sync per step). */
rra_status rra_model_check(rra_model *mdl, hipStream_t s);

/* Graph counters ([graph] decode_graph_replays: the evidence that decode ran
 * through the graph): captures made, replays launched, and kernel nodes in the
 * most recent graph.  Any pointer may be NULL. */
rra_status rra_graph_stats(const rra_model *mdl, uint64_t *captures, uint64_t *replays,
                           uint32_t *kernels);

/* Attention timing, for measurement ([reduces] forward_graphed_replay_to_token_id
 * splits a decode step's time into sub-phases on request; this times the
 * step's dominant kernel on the device).  events: n = 2 x n_layers
 * hipEvent_t handles created by the caller with timing enabled, or NULL / n = 0
 * to stop.  Every eager decode step (flags without RRA_GRAPH) enqueued
 * afterwards launches layer l's split-K flash-decode chunk kernel with
 * hipExtLaunchKernel's event pair (events[2l], events[2l + 1]): the runtime
 * stamps them at that kernel's own start and end, so after the step
 * hipEventElapsedTime(events[2l], events[2l + 1]) is that layer's chunk-kernel
 * time inside the step.  Graph steps record nothing.  Prefill records
 * nothing.  The events stay the caller's and must outlive the steps that
 * record them.  Errors: RRA_ENOTINIT for a null model, RRA_EINVAL for a wrong
 * n or a null event. */
rra_status rra_model_set_attention_events(rra_model *mdl, void *const *events, int32_t n);

/* Sub-phase timing of the decode step, for measurement ([reduces]
 * forward_graphed_replay_to_token_id splits a decode step's time into
 * sub-phases on request).  events: n = 4 x n_layers + 3 hipEvent_t handles
 * created by the caller with timing enabled, or NULL / n = 0 to stop.  Every
 * eager decode step (flags without RRA_GRAPH) enqueued afterwards records them
 * on its stream between its kernel groups:
 *   events[0]            step start (before the gather and the first norm inputs)
 *   events[1 + 4l]       layer l start (QKV GEMV)
 *   events[2 + 4l]       layer l attention (flash decode and its combine)
 *   events[3 + 4l]       layer l O GEMV
 *   events[4 + 4l]       layer l feed-forward (norm, gate/up, SwiGLU, down, residual)
 *   events[1 + 4 n_layers]  output norm, LM head, argmax
 *   events[2 + 4 n_layers]  step end
 * so hipEventElapsedTime(events[i], events[i + 1]) is the group's time,
 * launch gaps included.  Where the small-batch path fuses work across groups
 * (a GEMV prologue doing the residual step or the attention combine, flash
 * decode taking the QKV partials), a group holds the kernels launched
 * between its records.  Results are unchanged; graph steps and prefill record
 * nothing.  The events stay the caller's.  Errors: RRA_ENOTINIT for a null
 * model, RRA_EINVAL for a wrong n or a null event. */
rra_status rra_model_set_phase_events(rra_model *mdl, void *const *events, int32_t n);

/* Releases the host handle and its graphs (not the caller's memory). */
void rra_model_destroy(rra_model *mdl);

#ifdef __cplusplus
}
#endif
#endif /* RRA_H */
