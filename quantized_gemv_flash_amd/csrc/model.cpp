// model.cpp -- host side of librra: error reporting, argument validation, the
// standalone step entry points, and the decode step with its HIP graph cache.
//
// [batched_forward] forward_batched_to_token_ids / ..._graphed and
// [graph] (module doc, graph_step, graph_capture): the whole step -- every
// layer, the output norm, the LM head and the argmax -- is one graph whose
// per-token inputs (positions, token ids, the step input) sit at fixed device
// addresses; a graph is keyed by those addresses and by M, captured on first
// use and replayed after; a failed capture leaves the stream out of capture
// mode and the step runs eagerly instead.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "frag.h"
#include "rra_internal.h"

namespace rra {

static thread_local std::string g_error;

rra_status fail(rra_status st, const char *fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    if (verbose()) fprintf(stderr, "[rra] %s: %s\n", rra_status_name(st), buf);
    return st;
}

void clear_error() { g_error.clear(); }

bool verbose() {
    static const bool v = [] {
        const char *e = getenv("RRA_VERBOSE");
        return e && *e && strcmp(e, "0") != 0;
    }();
    return v;
}

// RRA_FAIL_CAPTURE set (and not "0"): every graph capture reports its body as
// failed, so tests can drive the discard-and-run-eagerly path from the host.
// Read at each capture (captures are rare), so a test can set and clear it.
bool capture_failure_requested() {
    const char *e = getenv("RRA_FAIL_CAPTURE");
    return e && *e && strcmp(e, "0") != 0;
}

rra_status check_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(RRA_EHIP, "launch of %s failed: %s", what, hipGetErrorString(e));
    return RRA_OK;
}

rra_status validate_weight(const rra_weight *w, const char *what, bool need_tiled_q) {
    if (!w) return fail(RRA_EINVAL, "%s: null weight", what);
    if (w->fmt != RRA_F32 && !is_quantised(w->fmt))
        return fail(RRA_EINVAL, "%s: unknown weight format %d", what, w->fmt);
    if (w->n <= 0 || w->k <= 0 || w->n > (1LL << 30) || w->k > (1LL << 24))
        return fail(RRA_EINVAL, "%s: bad shape %lld x %lld", what, (long long)w->n,
                    (long long)w->k);
    if (!w->data) return fail(RRA_EINVAL, "%s: null weight data", what);
    if (w->fmt == RRA_F32) {
        if (w->layout != RRA_PLANAR) return fail(RRA_EINVAL, "%s: F32 weights are planar", what);
        return RRA_OK;
    }
    if (w->k % 32) return fail(RRA_EINVAL, "%s: k=%lld is not a multiple of 32", what, (long long)w->k);
    if (w->fmt == RRA_Q6K && w->k % 256)
        return fail(RRA_EINVAL, "%s: Q6K needs k (%lld) to be a multiple of 256", what,
                    (long long)w->k);
    if (w->layout == RRA_PLANAR) {
        if (need_tiled_q)
            return fail(RRA_EINVAL, "%s: planar quantised weight; convert it with rra_repack_weight",
                        what);
        if (!w->scale) return fail(RRA_EINVAL, "%s: planar quantised weight without scales", what);
        return RRA_OK;
    }
    if (w->layout != RRA_TILED) return fail(RRA_EINVAL, "%s: unknown layout %d", what, w->layout);
    return RRA_OK;
}

}  // namespace rra

using namespace rra;

// ---------------------------------------------------------------- basics
extern "C" const char *rra_last_error(void) { return g_error.c_str(); }

extern "C" const char *rra_status_name(rra_status st) {
    switch (st) {
        case RRA_OK: return "RRA_OK";
        case RRA_EINVAL: return "RRA_EINVAL";
        case RRA_ENOTINIT: return "RRA_ENOTINIT";
        case RRA_EHIP: return "RRA_EHIP";
        case RRA_ECAPTURE: return "RRA_ECAPTURE";
    }
    return "RRA_UNKNOWN";
}

extern "C" int32_t rra_version(void) { return RRA_VERSION; }

// ---------------------------------------------------------------- step kernels
extern "C" rra_status rra_rmsnorm(const float *x, const float *gamma, float *out, int32_t m,
                                  int32_t h, float eps, hipStream_t s) {
    clear_error();
    if (!x || !gamma || !out) return fail(RRA_EINVAL, "rra_rmsnorm: null argument");
    if (m < 1 || m > RRA_M_MAX || h < 1) return fail(RRA_EINVAL, "rra_rmsnorm: m=%d h=%d", m, h);
    if (!(eps >= 0.f)) return fail(RRA_EINVAL, "rra_rmsnorm: eps must be >= 0");
    return launch_rmsnorm(x, gamma, out, m, h, eps, s);
}

extern "C" rra_status rra_rope_table(float *table, int32_t max_len, int32_t hd, double theta,
                                     hipStream_t s) {
    clear_error();
    if (!table) return fail(RRA_EINVAL, "rra_rope_table: null table");
    if (max_len < 1 || hd < 2 || hd % 2 || !(theta > 0.0))
        return fail(RRA_EINVAL, "rra_rope_table: max_len=%d hd=%d theta=%g", max_len, hd, theta);
    std::vector<float> host((size_t)max_len * hd);
    rope_table_host(host.data(), max_len, hd, theta);
    RRA_TRY_HIP(hipMemcpyAsync(table, host.data(), host.size() * sizeof(float),
                               hipMemcpyHostToDevice, s));
    RRA_TRY_HIP(hipStreamSynchronize(s));
    return RRA_OK;
}

extern "C" rra_status rra_rope(float *z, const uint32_t *pos, const float *table, int32_t m,
                               int32_t n_heads, int32_t hd, int32_t max_len, hipStream_t s) {
    clear_error();
    if (!z || !pos || !table) return fail(RRA_EINVAL, "rra_rope: null argument");
    if (m < 1 || m > RRA_M_MAX || n_heads < 1 || hd < 2 || hd % 2 || hd > 2048 || max_len < 1)
        return fail(RRA_EINVAL, "rra_rope: m=%d heads=%d hd=%d max_len=%d", m, n_heads, hd, max_len);
    return launch_rope(z, pos, table, m, n_heads, hd, max_len, s);
}

extern "C" rra_status rra_swiglu(const float *gate, const float *up, float *out, int32_t m,
                                 int32_t n, hipStream_t s) {
    clear_error();
    if (!gate || !up || !out) return fail(RRA_EINVAL, "rra_swiglu: null argument");
    if (m < 1 || m > RRA_M_MAX || n < 1) return fail(RRA_EINVAL, "rra_swiglu: m=%d n=%d", m, n);
    return launch_swiglu(gate, up, out, m, n, (size_t)n, (size_t)n, s);
}

extern "C" size_t rra_argmax_workspace_bytes(int32_t m, int32_t v) {
    if (m < 1 || m > RRA_M_MAX || v < 1) return 0;
    return argmax_ws_bytes(m, v);
}

extern "C" rra_status rra_argmax(const float *logits, uint32_t *tok, int32_t m, int32_t v,
                                 void *ws, size_t ws_bytes, hipStream_t s) {
    clear_error();
    if (!logits || !tok || !ws) return fail(RRA_EINVAL, "rra_argmax: null argument");
    if (m < 1 || m > RRA_M_MAX || v < 1) return fail(RRA_EINVAL, "rra_argmax: m=%d v=%d", m, v);
    const size_t need = argmax_ws_bytes(m, v);
    if (ws_bytes < need)
        return fail(RRA_ENOTINIT, "rra_argmax: workspace has %zu bytes, needs %zu", ws_bytes, need);
    return launch_argmax(logits, tok, m, v, ws, nullptr, false, s);
}

extern "C" rra_status rra_hbm_read(const void *buf, size_t bytes, float *sums, int32_t blocks,
                                   hipStream_t s) {
    clear_error();
    if (!buf || !sums) return fail(RRA_EINVAL, "rra_hbm_read: null argument");
    if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
        return fail(RRA_EINVAL, "rra_hbm_read: %zu bytes at %p: need a non-zero multiple of 16, "
                    "16-byte aligned", bytes, buf);
    if (blocks < 1 || blocks > (1 << 20))
        return fail(RRA_EINVAL, "rra_hbm_read: blocks=%d not in 1..2^20", blocks);
    return launch_hbm_read(buf, bytes, sums, blocks, s);
}

// ---------------------------------------------------------------- model
struct GraphKey {
    int32_t m, flags;
    const void *x, *pos, *tok, *logits;
    bool operator==(const GraphKey &o) const {
        return m == o.m && flags == o.flags && x == o.x && pos == o.pos && tok == o.tok &&
               logits == o.logits;
    }
};

struct GraphEntry {
    GraphKey key;
    hipGraphExec_t exec;
    uint32_t kernels;
};

struct rra_model {
    rra_model_desc d{};
    std::vector<rra_layer_desc> layers;
    int chunk[RRA_M_MAX + 1] = {};  // flash-decode rows per split, per batch size
    int hsplit[RRA_M_MAX + 1] = {}; // flash-decode head split per batch size (0: default rule)
    // workspace carve-up
    float *ss = nullptr, *xg = nullptr, *part = nullptr, *q = nullptr, *attn = nullptr, *act = nullptr;
    float *part_d = nullptr;  // the O and down GEMVs' partials (the next GEMV's prologue may read
                              // them while writing `part`)
    float *xalt = nullptr;    // the residual stream's second buffer (residual prologues)
    float *fd = nullptr, *logits = nullptr, *rope = nullptr;
    uint32_t *lens = nullptr, *err = nullptr;
    void *argmax_ws = nullptr;
    uint8_t *img = nullptr;  // activation image of the next quantised GEMV
    int rows = 0;            // batch rows the workspace holds: max(m_max, prefill rows)
    int prefill_rows = 0;    // prompt tokens per prefill chunk
    // prefill chunk state: x rows, positions, cache slot per row, token ids
    float *px = nullptr;
    uint32_t *ppos = nullptr, *pseq = nullptr, *ptok = nullptr;
    // per-M plans (index m), and the plans of prompt chunks of more than 32 rows
    GemvPlan plan_qkv[RRA_M_MAX + 1], plan_o[RRA_M_MAX + 1], plan_gu[RRA_M_MAX + 1],
        plan_d[RRA_M_MAX + 1], plan_lm[RRA_M_MAX + 1];
    GemvPlan pf_qkv, pf_o, pf_gu, pf_d;
    std::vector<GraphEntry> graphs;
    // attention timing: a pair of caller-owned events per layer, stamped at the
    // start and end of that layer's flash-decode chunk kernel in eager steps
    // (empty: none)
    std::vector<hipEvent_t> attn_events;
    std::vector<hipEvent_t> phase_events;  // 4 x n_layers + 3 boundaries (eager steps)
    uint64_t captures = 0, replays = 0;
    uint32_t last_kernels = 0;
};

namespace {

struct Layout {
    size_t ss, xg, img, part, part_d, q, lens, attn, act, fd, logits, argmax, rope, err, px, pidx,
        xalt, total;
};

// Rows of one prefill chunk, and the batch rows the workspace is laid out for.
int prefill_rows_of(const rra_model_desc &d) { return d.prefill_rows ? d.prefill_rows : kPrefillMax; }
int rows_of(const rra_model_desc &d) { return std::max(d.m_max, prefill_rows_of(d)); }

// Largest activation image any GEMV of the model reads (0 if all are fp32).
size_t image_bytes(const rra_model_desc &d) {
    const int ct = frag_ct(rows_of(d));
    size_t best = 0;
    auto need = [&](const rra_weight &w) {
        if (w.fmt != RRA_F32) best = std::max(best, frag_image_bytes(w.fmt, ct, w.k));
    };
    const rra_layer_desc &l = d.layers[0];
    need(l.wqkv);
    need(l.wo);
    need(l.wgu);
    need(l.wd);
    need(d.lm_head);
    return best;
}

// The GEMV plan of a step or prompt chunk of m rows.
GemvPlan plan_for(const rra_weight &w, int m) {
    return m > RRA_M_MAX ? gemm_plan(w) : gemv_plan(w, m);
}

size_t part_floats(const rra_model_desc &d, const rra_layer_desc &l) {
    size_t best = 0;
    for (int m = 1; m <= rows_of(d); ++m) {
        const rra_weight *ws[4] = {&l.wqkv, &l.wo, &l.wgu, &l.wd};
        for (const rra_weight *w : ws) {
            const GemvPlan p = plan_for(*w, m);
            best = std::max(best, (size_t)p.split * (size_t)m * (size_t)w->n);
        }
    }
    return best;
}

// Flash-decode chunk used for a step of m sequences.
int chunk_for(const rra_model_desc &d, int m) {
    return fd_choose_chunk(m, d.n_kv_heads, d.max_len, d.attn_chunk);
}

// Flash-decode partials: enough for the plan of every batch size, whether
// the default rule's, a fixed attn_chunk's or any candidate the tuner may pick.
size_t fd_floats(const rra_model_desc &d) {
    size_t best = 0;
    for (int m = 1; m <= d.m_max; ++m) {
        best = std::max(best, fd_partials_floats(m, d.n_heads, d.head_dim, d.max_len, chunk_for(d, m)));
        best = std::max(best, fd_tuned_floats(m, d.n_heads, d.n_kv_heads, d.head_dim, d.max_len));
    }
    // a prompt chunk's attention split over keys (at most kPrefillKeySplits)
    const size_t pr = (size_t)prefill_rows_of(d);
    return std::max(best, pr * d.n_heads * kPrefillKeySplits * (size_t)(d.head_dim + 1));
}

Layout layout_of(const rra_model_desc &d) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t M = (size_t)rows_of(d);
    size_t partf = 0;
    for (int i = 0; i < d.n_layers; ++i) partf = std::max(partf, part_floats(d, d.layers[i]));
    L.ss = take(4 * M * ss_parts(d.hidden));
    L.xg = take(4 * M * d.hidden);
    L.img = take(image_bytes(d));
    L.part = take(4 * partf);
    L.part_d = take(4 * partf);
    L.q = take(4 * M * d.n_heads * d.head_dim);
    L.lens = take(4 * M);
    L.attn = take(4 * M * d.n_heads * d.head_dim);
    L.act = take(4 * M * d.intermediate);
    L.fd = take(4 * fd_floats(d));
    L.logits = take(4 * (size_t)d.m_max * (size_t)d.vocab);  // prompts: the last row only
    // the argmax pass over the logits, or the LM head's own partials
    L.argmax = take(std::max(argmax_ws_bytes(d.m_max, d.vocab),
                             gemv_argmax_ws_bytes(d.m_max, d.vocab)));
    L.rope = take(4 * (size_t)d.max_len * d.head_dim);
    L.err = take(256);
    L.px = take(4 * M * d.hidden);
    L.pidx = take(3 * 4 * M);
    L.xalt = take(4 * M * d.hidden);
    L.total = off;
    return L;
}

rra_status check_shape(const rra_weight &w, int64_t n, int64_t k, const char *what) {
    RRA_TRY(validate_weight(&w, what, true));
    if (w.n != n || w.k != k)
        return fail(RRA_EINVAL, "%s: shape %lld x %lld, expected %lld x %lld", what,
                    (long long)w.n, (long long)w.k, (long long)n, (long long)k);
    return RRA_OK;
}

rra_status validate_desc(const rra_model_desc *d) {
    if (!d) return fail(RRA_EINVAL, "model: null descriptor");
    if (d->n_layers < 1 || d->hidden < 1 || d->n_heads < 1 || d->n_kv_heads < 1 ||
        d->intermediate < 1 || d->vocab < 1)
        return fail(RRA_EINVAL, "model: non-positive dimension");
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(RRA_EINVAL, "model: head_dim=%d not 64 or 128", d->head_dim);
    if (d->n_heads % d->n_kv_heads || d->n_heads / d->n_kv_heads > 8)
        return fail(RRA_EINVAL, "model: n_heads=%d n_kv_heads=%d (need a group size 1..8)",
                    d->n_heads, d->n_kv_heads);
    if (d->hidden % 8 || d->intermediate % 8)
        return fail(RRA_EINVAL, "model: hidden and intermediate must be multiples of 8");
    if (d->m_max < 1 || d->m_max > RRA_M_MAX)
        return fail(RRA_EINVAL, "model: m_max=%d not in 1..32", d->m_max);
    if (d->prefill_rows < 0 || d->prefill_rows > kPrefillMax)
        return fail(RRA_EINVAL, "model: prefill_rows=%d not in 0..%d", d->prefill_rows,
                    kPrefillMax);
    if (d->max_len < 1) return fail(RRA_EINVAL, "model: max_len=%d", d->max_len);
    if (!(d->rms_eps >= 0.f) || !(d->rope_theta > 0.0))
        return fail(RRA_EINVAL, "model: bad rms_eps or rope_theta");
    if (d->attn_chunk != 0 && (d->attn_chunk < 32 || d->attn_chunk > 1024 || d->attn_chunk % 32))
        return fail(RRA_EINVAL, "model: attn_chunk=%d", d->attn_chunk);
    if (!d->layers || !d->out_gamma) return fail(RRA_EINVAL, "model: null layers or out_gamma");
    const int64_t H = d->hidden, hd = d->head_dim, nq = d->n_heads, nkv = d->n_kv_heads,
                  I = d->intermediate;
    for (int i = 0; i < d->n_layers; ++i) {
        const rra_layer_desc &l = d->layers[i];
        RRA_TRY(check_shape(l.wqkv, (nq + 2 * nkv) * hd, H, "layer wqkv"));
        RRA_TRY(check_shape(l.wo, H, nq * hd, "layer wo"));
        RRA_TRY(check_shape(l.wgu, 2 * I, H, "layer wgu"));
        RRA_TRY(check_shape(l.wd, H, I, "layer wd"));
        if (!l.attn_gamma || !l.ffn_gamma || !l.k_cache || !l.v_cache)
            return fail(RRA_EINVAL, "layer %d: null gamma or cache", i);
        const rra_layer_desc &l0 = d->layers[0];
        if (l.wqkv.fmt != l0.wqkv.fmt || l.wo.fmt != l0.wo.fmt || l.wgu.fmt != l0.wgu.fmt ||
            l.wd.fmt != l0.wd.fmt)
            return fail(RRA_EINVAL, "layer %d: weight formats differ from layer 0's", i);
    }
    RRA_TRY(check_shape(d->lm_head, d->vocab, H, "lm_head"));
    return RRA_OK;
}

// Where the producer of a GEMV's input writes its activation image: nowhere
// for fp32 weights (the GEMV reads the fp32 rows).
FragOut image_for(const rra_model *M, const rra_weight &w, int m) {
    if (w.fmt == RRA_F32) return FragOut{nullptr, 0, 1, 0};
    const int kt = tile_k(w.fmt);
    return FragOut{M->img, w.fmt, frag_ct(m), (int)(cdiv(w.k, kt) * kt), M->err};
}
const void *gemv_input(const rra_model *M, const rra_weight &w, const float *rows) {
    return w.fmt == RRA_F32 ? static_cast<const void *>(rows) : M->img;
}

// Internal step flag: stop after the last layer (no LM head, no argmax).
constexpr int kStepNoHead = 1 << 16;

// At small m flash decode takes the QKV partials itself (QkvIn: sum, RoPE,
// the new K/V row, seq_len); otherwise qkv_post does that work.  Every split
// of a query head sums that head's planes again, so the fused form wins only
// while that is cheaper than a launch: on MI355X the 1.5B-shaped decoder
// gained 2.9 % at M = 8 and lost 0.9 % at M = 16, the 8B-shaped one lost
// 1.9 % at M = 32.
bool step_fuses_qkv(int m) { return m <= 8; }

// The launches of one decode step, in stream order, as phases: begin() (the
// step input), then per layer pre(l) (the QKV GEMV and its epilogue),
// attn(l) (flash decode) and post(l) (the O GEMV, the feed-forward block and
// the residual steps), then head() (LM head and argmax); enqueue_step runs
// them in that order.  Row i reads token tok_in[i] (under
// RRA_STEP_GATHER), sits at position pos[i] and uses cache slot i; the
// greedy ids go to tok_out.
struct Stepper {
    rra_model *M;
    float *x;
    uint32_t *pos;
    const uint32_t *tok_in;
    uint32_t *tok_out;
    float *logits;
    int m, flags;
    hipStream_t s;
    int H = 0, nq = 0, nkv = 0, hd = 0, I = 0, nqkv = 0;
    NormIn nrm{nullptr, 0, 0.f};
    bool phased = false;  // sub-phase boundaries (eager steps only)
    // The residual stream lives in x or in M->xalt.  At small m an
    // RMSNorm-fused GEMV can do the residual step itself (kProResid): it reads
    // the stream and the previous GEMV's partials and one of its workgroups
    // writes the new stream to the other buffer.  The last residual step
    // always writes x.
    float *xc = nullptr;
    GemvPrologue pr_qkv{kProNone, nullptr, nullptr, nullptr, 0, 0, 0, 0, 0};

    Stepper(rra_model *M_, float *x_, uint32_t *pos_, const uint32_t *tok_in_,
            uint32_t *tok_out_, float *logits_, int m_, int flags_, hipStream_t s_)
        : M(M_), x(x_), pos(pos_), tok_in(tok_in_), tok_out(tok_out_), logits(logits_), m(m_),
          flags(flags_), s(s_) {
        const rra_model_desc &d = M->d;
        H = d.hidden;
        nq = d.n_heads;
        nkv = d.n_kv_heads;
        hd = d.head_dim;
        I = d.intermediate;
        nqkv = (nq + 2 * nkv) * hd;
        nrm = NormIn{M->ss, ss_parts(H), d.rms_eps};
        phased = !M->phase_events.empty() && !(flags & RRA_GRAPH);
        xc = x;
    }
    // a record on the step's stream between kernel groups, so each pair of
    // records spans that group
    rra_status mark(int i) {
        if (phased) RRA_TRY_HIP(hipEventRecord(M->phase_events[i], s));
        return RRA_OK;
    }
    float *other(const float *p) const { return p == x ? M->xalt : x; }
    GemvPrologue resid_pro(const float *planes, int split, const float *gamma) {
        GemvPrologue r{kProResid, planes, nullptr, nullptr, (long long)m * H, split, H, 0, 0};
        r.x_in = xc;
        r.x_out = other(xc);
        r.gamma = gamma;
        r.eps = M->d.rms_eps;
        r.err = M->err;
        xc = r.x_out;
        return r;
    }
    bool fuse_qkv() const { return step_fuses_qkv(m); }

    rra_status begin() {
        const rra_model_desc &d = M->d;
        RRA_TRY(mark(0));
        // RMSNorm is formed inside each consuming GEMV from per-chunk sums of
        // squares of x; the first ones come from the step input (gathered
        // from the embedding table by the same launch under
        // RRA_STEP_GATHER).  Each producer also writes the next GEMV's
        // activation image.
        const rra_layer_desc &L0 = M->layers[0];
        if (flags & RRA_STEP_GATHER)
            return launch_gather_residual_ss(GatherIn{d.embed, tok_in, pos, d.vocab, M->err}, x,
                                             M->ss, L0.attn_gamma, M->xg, m, H,
                                             image_for(M, L0.wqkv, m), s);
        return launch_residual_ss(nullptr, 0, 0, x, x, M->ss, L0.attn_gamma, M->xg, m, H,
                                  image_for(M, L0.wqkv, m), s);
    }

    rra_status pre(int l) {
        const rra_model_desc &d = M->d;
        const rra_layer_desc &L = M->layers[l];
        RRA_TRY(mark(1 + 4 * l));
        const GemvPlan &pq = M->plan_qkv[m];
        const bool rq = pr_qkv.kind == kProResid;
        RRA_TRY(launch_gemv(L.wqkv, pq, gemv_input(M, L.wqkv, M->xg), m, M->part, (size_t)m * nqkv,
                            s, rq ? nullptr : &nrm, rq ? &pr_qkv : nullptr));
        if (!fuse_qkv())
            RRA_TRY(launch_qkv_post(M->part, pq.split, (size_t)m * nqkv, pos, M->rope, M->q,
                                    L.k_cache, L.v_cache, M->lens, M->err, m, nq, nkv, hd,
                                    d.max_len, nullptr, s));
        return RRA_OK;
    }

    rra_status attn(int l) {
        const rra_model_desc &d = M->d;
        const rra_layer_desc &L = M->layers[l];
        const GemvPlan &pq = M->plan_qkv[m];
        const QkvIn qi{M->part, pq.split, (long long)m * nqkv, pos, M->rope,
                       L.k_cache, L.v_cache, M->lens, M->err};
        // At small m the O GEMV combines the attention partials itself and
        // the down GEMV forms SwiGLU itself (GemvPrologue): two launches
        // fewer per layer, with the same arithmetic as the kernels they
        // stand in for.
        const bool pro_o = gemv_takes_prologue(L.wo, M->plan_o[m], m);
        const FragOut fo_o = image_for(M, L.wo, m);
        RRA_TRY(mark(2 + 4 * l));
        // (eager steps only: the timed launch is not one a graph captures)
        const bool timed = !M->attn_events.empty() && !(flags & RRA_GRAPH);
        return launch_flash_decode(M->q, L.k_cache, L.v_cache, M->lens, M->attn, m, nq, nkv, hd,
                                   d.max_len, M->chunk[m], M->fd, s, &fo_o, nullptr, !pro_o,
                                   fuse_qkv() ? &qi : nullptr,
                                   timed ? M->attn_events[2 * l] : nullptr,
                                   timed ? M->attn_events[2 * l + 1] : nullptr, M->hsplit[m]);
    }

    rra_status post(int l) {
        const rra_model_desc &d = M->d;
        const rra_layer_desc &L = M->layers[l];
        const GemvPlan &pq = M->plan_qkv[m];
        const GemvPlan &po = M->plan_o[m];
        const bool pro_o = gemv_takes_prologue(L.wo, po, m);
        const int nc_max = (int)cdiv(d.max_len, M->chunk[m]);
        GemvPrologue pa{kProAttn, M->fd, fd_part_lse(M->fd, m, nq, hd, nc_max), M->lens,
                        0, 0, nq, nc_max, d.max_len};
        pa.err = M->err;
        RRA_TRY(mark(3 + 4 * l));
        RRA_TRY(launch_gemv(L.wo, po, gemv_input(M, L.wo, M->attn), m, M->part_d, (size_t)m * H, s,
                            nullptr, pro_o ? &pa : nullptr));
        RRA_TRY(mark(4 + 4 * l));
        // feed-forward block
        const GemvPlan &pg = M->plan_gu[m];
        if (gemv_takes_resid_prologue(L.wgu, pg, m, po.split)) {
            const GemvPrologue rg = resid_pro(M->part_d, po.split, L.ffn_gamma);
            RRA_TRY(launch_gemv(L.wgu, pg, gemv_input(M, L.wgu, M->xg), m, M->part,
                                (size_t)m * 2 * I, s, nullptr, &rg));
        } else {
            RRA_TRY(launch_residual_ss(M->part_d, po.split, (size_t)m * H, xc, xc, M->ss,
                                       L.ffn_gamma, M->xg, m, H, image_for(M, L.wgu, m), s));
            RRA_TRY(launch_gemv(L.wgu, pg, gemv_input(M, L.wgu, M->xg), m, M->part,
                                (size_t)m * 2 * I, s, &nrm));
        }
        const GemvPlan &pd = M->plan_d[m];
        const bool pro_d = gemv_takes_prologue(L.wd, pd, m);
        if (!pro_d)
            RRA_TRY(launch_swiglu_reduce(M->part, pg.split, (size_t)m * 2 * I, M->act, m, I,
                                         image_for(M, L.wd, m), s));
        GemvPrologue ps{kProSwiglu, M->part, nullptr, nullptr, (long long)m * 2 * I, pg.split,
                        I, 0, 0};
        ps.err = M->err;
        RRA_TRY(launch_gemv(L.wd, pd, gemv_input(M, L.wd, M->act), m, M->part_d, (size_t)m * H, s,
                            nullptr, pro_d ? &ps : nullptr));
        const bool last = l + 1 == d.n_layers;
        pr_qkv.kind = kProNone;
        if (!last && gemv_takes_resid_prologue(M->layers[l + 1].wqkv, pq, m, pd.split)) {
            pr_qkv = resid_pro(M->part_d, pd.split, M->layers[l + 1].attn_gamma);
        } else {
            const float *next_gamma = last ? d.out_gamma : M->layers[l + 1].attn_gamma;
            const rra_weight &next_w = last ? d.lm_head : M->layers[l + 1].wqkv;
            float *x_out = last ? x : xc;
            RRA_TRY(launch_residual_ss(M->part_d, pd.split, (size_t)m * H, xc, x_out, M->ss,
                                       next_gamma, M->xg, m, H, image_for(M, next_w, m), s));
            xc = x_out;
        }
        return RRA_OK;
    }

    rra_status head() {
        const rra_model_desc &d = M->d;
        RRA_TRY(mark(1 + 4 * d.n_layers));
        if (flags & kStepNoHead) return mark(2 + 4 * d.n_layers);
        // The LM head leaves per-workgroup argmax partials when it runs as one
        // K split, and the ids come from those; otherwise from the logits.
        ArgOut ao = gemv_argmax_out(M->argmax_ws, m, d.vocab);
        RRA_TRY(launch_gemv(d.lm_head, M->plan_lm[m], gemv_input(M, d.lm_head, M->xg), m, logits,
                            0, s, &nrm, nullptr, &ao));
        const bool adv = (flags & RRA_STEP_ADVANCE) != 0;
        if (ao.blocks)
            RRA_TRY(launch_argmax_partials(ao, tok_out, m, pos, adv, s));
        else
            RRA_TRY(launch_argmax(logits, tok_out, m, d.vocab, M->argmax_ws, pos, adv, s));
        return mark(2 + 4 * d.n_layers);
    }
};

rra_status enqueue_step(rra_model *M, float *x, uint32_t *pos, const uint32_t *tok_in,
                        uint32_t *tok_out, float *logits, int m, int flags, hipStream_t s) {
    Stepper st(M, x, pos, tok_in, tok_out, logits, m, flags, s);
    RRA_TRY(st.begin());
    for (int l = 0; l < M->d.n_layers; ++l) {
        RRA_TRY(st.pre(l));
        RRA_TRY(st.attn(l));
        RRA_TRY(st.post(l));
    }
    return st.head();
}

// One prompt chunk: tokens[0..n) of cache slot `seq` at positions start ..
// start + n - 1 ([head_dim] tensor_core_attention: the prompt's causal
// attention on the tensor cores).  Every layer: the QKV GEMM for all n rows
// (weights read once), RoPE and the K/V rows written to the slot's cache, the
// matrix-core causal attention, the O GEMM, the residual step, the gate/up
// GEMM, SwiGLU, the down GEMM.  With `last`, the last row alone then goes
// through the output norm, the LM head and the argmax (ids to M->ptok[0],
// logits to M->logits row 0).
rra_status enqueue_prompt_chunk(rra_model *M, const uint32_t *tokens, int n, int seq,
                                uint32_t start, bool last, hipStream_t s) {
    const rra_model_desc &d = M->d;
    const int H = d.hidden, nq = d.n_heads, nkv = d.n_kv_heads, hd = d.head_dim,
              I = d.intermediate;
    const int nqkv = (nq + 2 * nkv) * hd;
    auto plan = [&](const GemvPlan &pf, const GemvPlan *pm) { return n > RRA_M_MAX ? pf : pm[n]; };
    float *x = M->px;
    RRA_TRY(launch_prefill_rows(M->ppos, M->pseq, start, (uint32_t)seq, n, s));
    RRA_TRY(launch_embed_gather(d.embed, tokens, M->ppos, x, n, H, d.vocab, M->err, s));
    const NormIn nrm{M->ss, ss_parts(H), d.rms_eps};
    const size_t slot = (size_t)seq * nkv * d.max_len * hd;
    RRA_TRY(launch_residual_ss(nullptr, 0, 0, x, x, M->ss, M->layers[0].attn_gamma, M->xg, n, H,
                               image_for(M, M->layers[0].wqkv, n), s));
    for (int l = 0; l < d.n_layers; ++l) {
        const rra_layer_desc &L = M->layers[l];
        const GemvPlan pq = plan(M->pf_qkv, M->plan_qkv), po = plan(M->pf_o, M->plan_o),
                       pg = plan(M->pf_gu, M->plan_gu), pd = plan(M->pf_d, M->plan_d);
        RRA_TRY(launch_gemv(L.wqkv, pq, gemv_input(M, L.wqkv, M->xg), n, M->part, (size_t)n * nqkv,
                            s, &nrm));
        RRA_TRY(launch_qkv_post(M->part, pq.split, (size_t)n * nqkv, M->ppos, M->rope, M->q,
                                L.k_cache, L.v_cache, M->lens, M->err, n, nq, nkv, hd, d.max_len,
                                M->pseq, s));
        const FragOut fo_o = image_for(M, L.wo, n);
        RRA_TRY(launch_prefill_attention(M->q, L.k_cache + slot, L.v_cache + slot, M->attn, n, nq,
                                         nkv, hd, d.max_len, start, &fo_o, M->fd, M->lens, s));
        RRA_TRY(launch_gemv(L.wo, po, gemv_input(M, L.wo, M->attn), n, M->part_d, (size_t)n * H,
                            s));
        RRA_TRY(launch_residual_ss(M->part_d, po.split, (size_t)n * H, x, x, M->ss, L.ffn_gamma,
                                   M->xg, n, H, image_for(M, L.wgu, n), s));
        RRA_TRY(launch_gemv(L.wgu, pg, gemv_input(M, L.wgu, M->xg), n, M->part, (size_t)n * 2 * I,
                            s, &nrm));
        RRA_TRY(launch_swiglu_reduce(M->part, pg.split, (size_t)n * 2 * I, M->act, n, I,
                                     image_for(M, L.wd, n), s));
        RRA_TRY(launch_gemv(L.wd, pd, gemv_input(M, L.wd, M->act), n, M->part_d, (size_t)n * H, s));
        if (l + 1 < d.n_layers) {
            const rra_layer_desc &Ln = M->layers[l + 1];
            RRA_TRY(launch_residual_ss(M->part_d, pd.split, (size_t)n * H, x, x, M->ss,
                                       Ln.attn_gamma, M->xg, n, H, image_for(M, Ln.wqkv, n), s));
        } else if (last) {
            // the last row alone: its residual step and the output norm's inputs
            float *xl = x + (size_t)(n - 1) * H;
            RRA_TRY(launch_residual_ss(M->part_d + (size_t)(n - 1) * H, pd.split, (size_t)n * H,
                                       xl, xl, M->ss, d.out_gamma, M->xg, 1, H,
                                       image_for(M, d.lm_head, 1), s));
        }
    }
    if (!last) return RRA_OK;
    RRA_TRY(launch_gemv(d.lm_head, M->plan_lm[1], gemv_input(M, d.lm_head, M->xg), 1, M->logits,
                        0, s, &nrm));
    return launch_argmax(M->logits, M->ptok, 1, d.vocab, M->argmax_ws, nullptr, false, s);
}

}  // namespace

extern "C" size_t rra_model_workspace_bytes(const rra_model_desc *d) {
    if (validate_desc(d) != RRA_OK) return 0;
    return layout_of(*d).total;
}

extern "C" size_t rra_decode_workspace_bytes(const rra_model_desc *d) {
    return rra_model_workspace_bytes(d);
}

extern "C" rra_status rra_model_create(const rra_model_desc *d, void *ws, size_t ws_bytes,
                                       hipStream_t s, rra_model **out) {
    clear_error();
    if (!out) return fail(RRA_EINVAL, "rra_model_create: null out");
    *out = nullptr;
    RRA_TRY(validate_desc(d));
    if (!ws) return fail(RRA_EINVAL, "rra_model_create: null workspace");
    const Layout L = layout_of(*d);
    if (ws_bytes < L.total)
        return fail(RRA_ENOTINIT, "rra_model_create: workspace has %zu bytes, needs %zu", ws_bytes,
                    L.total);
    auto *M = new rra_model();
    M->d = *d;
    M->layers.assign(d->layers, d->layers + d->n_layers);
    M->d.layers = M->layers.data();
    char *b = static_cast<char *>(ws);
    M->ss = reinterpret_cast<float *>(b + L.ss);
    M->xg = reinterpret_cast<float *>(b + L.xg);
    M->img = reinterpret_cast<uint8_t *>(b + L.img);
    M->part = reinterpret_cast<float *>(b + L.part);
    M->part_d = reinterpret_cast<float *>(b + L.part_d);
    M->q = reinterpret_cast<float *>(b + L.q);
    M->lens = reinterpret_cast<uint32_t *>(b + L.lens);
    M->attn = reinterpret_cast<float *>(b + L.attn);
    M->act = reinterpret_cast<float *>(b + L.act);
    M->fd = reinterpret_cast<float *>(b + L.fd);
    M->logits = reinterpret_cast<float *>(b + L.logits);
    M->argmax_ws = b + L.argmax;
    M->rope = reinterpret_cast<float *>(b + L.rope);
    M->err = reinterpret_cast<uint32_t *>(b + L.err);
    M->px = reinterpret_cast<float *>(b + L.px);
    M->xalt = reinterpret_cast<float *>(b + L.xalt);
    M->rows = rows_of(*d);
    M->prefill_rows = prefill_rows_of(*d);
    M->ppos = reinterpret_cast<uint32_t *>(b + L.pidx);
    M->pseq = M->ppos + M->rows;
    M->ptok = M->pseq + M->rows;
    for (int m = 1; m <= std::min(M->rows, RRA_M_MAX); ++m) {
        M->chunk[m] = chunk_for(*d, m);
        const rra_layer_desc &l0 = d->layers[0];
        M->plan_qkv[m] = gemv_plan(l0.wqkv, m);
        M->plan_o[m] = gemv_plan(l0.wo, m);
        M->plan_gu[m] = gemv_plan(l0.wgu, m);
        M->plan_d[m] = gemv_plan(l0.wd, m);
        GemvPlan lm = gemv_plan(d->lm_head, m);
        lm.kt_per_split = d->lm_head.fmt == RRA_F32 ? 1 : (int)cdiv(d->lm_head.k, tile_k(d->lm_head.fmt));
        lm.split = 1;
        M->plan_lm[m] = lm;
    }
    {
        const rra_layer_desc &l0 = d->layers[0];
        M->pf_qkv = gemm_plan(l0.wqkv);
        M->pf_o = gemm_plan(l0.wo);
        M->pf_gu = gemm_plan(l0.wgu);
        M->pf_d = gemm_plan(l0.wd);
    }
    std::vector<float> table((size_t)d->max_len * d->head_dim);
    rope_table_host(table.data(), d->max_len, d->head_dim, d->rope_theta);
    const uint32_t zero[64] = {0};
    hipError_t e = hipMemcpyAsync(M->rope, table.data(), table.size() * sizeof(float),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(M->err, zero, sizeof zero, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete M;
        return fail(RRA_EHIP, "rra_model_create: %s", hipGetErrorString(e));
    }
    *out = M;
    return RRA_OK;
}

extern "C" void rra_model_destroy(rra_model *M) {
    if (!M) return;
    for (GraphEntry &g : M->graphs) (void)hipGraphExecDestroy(g.exec);
    delete M;
}

extern "C" rra_status rra_graph_stats(const rra_model *M, uint64_t *captures, uint64_t *replays,
                                      uint32_t *kernels) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_graph_stats: null model");
    if (captures) *captures = M->captures;
    if (replays) *replays = M->replays;
    if (kernels) *kernels = M->last_kernels;
    return RRA_OK;
}

extern "C" rra_status rra_model_check(rra_model *M, hipStream_t s) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_model_check: null model");
    uint32_t flag = 0;
    const uint32_t zero = 0;
    RRA_TRY_HIP(hipMemcpyAsync(&flag, M->err, sizeof flag, hipMemcpyDeviceToHost, s));
    RRA_TRY_HIP(hipStreamSynchronize(s));
    if (flag) {
        RRA_TRY_HIP(hipMemcpyAsync(M->err, &zero, sizeof zero, hipMemcpyHostToDevice, s));
        RRA_TRY_HIP(hipStreamSynchronize(s));
        std::string what;
        auto add = [&](const std::string &t) { what += (what.empty() ? "" : "; ") + t; };
        if (flag & kErrPos) add("a position >= max_len (" + std::to_string(M->d.max_len) + ")");
        if (flag & kErrToken) add("a token id >= vocab (" + std::to_string(M->d.vocab) + ")");
        if (flag & kErrRange)
            add("a GEMV input element with |x| >= 65504 or NaN (outside the fp16 operand range)");
        return fail(RRA_EINVAL, "a step saw %s", what.c_str());
    }
    return RRA_OK;
}

static rra_status capture_and_launch(rra_model *M, const GraphKey &key, float *x, uint32_t *pos,
                                     uint32_t *tok, float *logits, int m, int flags,
                                     hipStream_t s) {
    // Stream capture in thread-local mode ([reduces] try_graph_capture): a
    // failed capture cannot poison other threads' work.  End the capture
    // whatever happened, so the stream always leaves capture mode.
    RRA_TRY_HIP(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    rra_status body = enqueue_step(M, x, pos, tok, tok, logits, m, flags, s);
    if (body == RRA_OK && capture_failure_requested())
        body = fail(RRA_ECAPTURE, "capture failure requested by RRA_FAIL_CAPTURE");
    hipGraph_t graph = nullptr;
    const hipError_t end = hipStreamEndCapture(s, &graph);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    (void)hipStreamIsCapturing(s, &cs);
    if (cs != hipStreamCaptureStatusNone) (void)hipStreamSynchronize(s);
    if (body != RRA_OK || end != hipSuccess || !graph) {
        if (graph) (void)hipGraphDestroy(graph);
        (void)hipGetLastError();
        if (verbose())
            fprintf(stderr, "[rra] graph capture failed for M=%d (%s); running eagerly\n", m,
                    end != hipSuccess ? hipGetErrorString(end) : rra_last_error());
        return RRA_ECAPTURE;
    }
    size_t nodes = 0;
    (void)hipGraphGetNodes(graph, nullptr, &nodes);
    hipGraphExec_t exec = nullptr;
    const hipError_t inst = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (inst != hipSuccess) {
        (void)hipGetLastError();
        return RRA_ECAPTURE;
    }
    if (M->graphs.size() >= 16) {  // small cache: drop the oldest graph
        (void)hipGraphExecDestroy(M->graphs.front().exec);
        M->graphs.erase(M->graphs.begin());
    }
    M->graphs.push_back(GraphEntry{key, exec, (uint32_t)nodes});
    M->captures++;
    M->last_kernels = (uint32_t)nodes;
    if (verbose())
        fprintf(stderr, "[rra] captured decode graph: M=%d, %zu kernels\n", m, nodes);
    // Capture records without running: launch it now so this call's outputs
    // are real ([batched_forward] forward_batched_to_token_ids_graphed).
    RRA_TRY_HIP(hipGraphLaunch(exec, s));
    return RRA_OK;
}

extern "C" rra_status rra_decode_step(rra_model *M, float *x, uint32_t *pos, uint32_t *tok,
                                      uint32_t *tok_host, float *logits, int32_t m, int32_t flags,
                                      hipStream_t s) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_decode_step: null model");
    if (!x || !pos || !tok) return fail(RRA_EINVAL, "rra_decode_step: null x, pos or tok");
    if (m < 1 || m > M->d.m_max)
        return fail(RRA_EINVAL, "rra_decode_step: m=%d not in 1..m_max=%d", m, M->d.m_max);
    if (flags & ~(RRA_GRAPH | RRA_STEP_GATHER | RRA_STEP_ADVANCE))
        return fail(RRA_EINVAL, "rra_decode_step: unknown flags 0x%x", flags);
    if ((flags & RRA_STEP_GATHER) && !M->d.embed)
        return fail(RRA_EINVAL, "rra_decode_step: RRA_STEP_GATHER needs an embedding table");
    if ((flags & RRA_GRAPH) && !s)
        return fail(RRA_EINVAL, "rra_decode_step: RRA_GRAPH needs a non-null stream");
    float *lg = logits ? logits : M->logits;
    if (flags & RRA_GRAPH) {
        const GraphKey key{m, flags & ~RRA_GRAPH, x, pos, tok, lg};
        GraphEntry *hit = nullptr;
        for (GraphEntry &g : M->graphs)
            if (g.key == key) hit = &g;
        if (hit) {
            RRA_TRY_HIP(hipGraphLaunch(hit->exec, s));
            M->replays++;
            M->last_kernels = hit->kernels;
        } else {
            const rra_status st = capture_and_launch(M, key, x, pos, tok, lg, m, flags, s);
            if (st != RRA_OK) {
                clear_error();
                const rra_status eager = enqueue_step(M, x, pos, tok, tok, lg, m, flags, s);
                if (eager != RRA_OK) return fail(RRA_ECAPTURE, "capture and eager step failed: %s",
                                                 rra_last_error());
            }
        }
    } else {
        RRA_TRY(enqueue_step(M, x, pos, tok, tok, lg, m, flags, s));
    }
    if (tok_host) {
        RRA_TRY_HIP(hipMemcpyAsync(tok_host, tok, sizeof(uint32_t) * m, hipMemcpyDeviceToHost, s));
        RRA_TRY_HIP(hipStreamSynchronize(s));
    }
    return RRA_OK;
}

extern "C" rra_status rra_decode_step_async(rra_model *M, float *x, uint32_t *pos, uint32_t *tok,
                                            uint32_t *tok_pinned, hipEvent_t done, float *logits,
                                            int32_t m, int32_t flags, hipStream_t s) {
    clear_error();
    if (!tok_pinned || !done)
        return fail(RRA_EINVAL, "rra_decode_step_async: null tok_pinned or done event");
    // The copy must not block the host: only page-locked host memory is taken.
    hipPointerAttribute_t attr{};
    const hipError_t pe = hipPointerGetAttributes(&attr, tok_pinned);
    if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(RRA_EINVAL, "rra_decode_step_async: tok_pinned is not page-locked host memory "
                    "(allocate it with hipHostMalloc)");
    }
    RRA_TRY(rra_decode_step(M, x, pos, tok, nullptr, logits, m, flags, s));
    RRA_TRY_HIP(hipMemcpyAsync(tok_pinned, tok, sizeof(uint32_t) * m, hipMemcpyDeviceToHost, s));
    RRA_TRY_HIP(hipEventRecord(done, s));
    return RRA_OK;
}

extern "C" rra_status rra_model_set_attention_events(rra_model *M, void *const *events,
                                                     int32_t n) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_model_set_attention_events: null model");
    if (!events || n == 0) {
        M->attn_events.clear();
        return RRA_OK;
    }
    if (n != 2 * M->d.n_layers)
        return fail(RRA_EINVAL, "rra_model_set_attention_events: n=%d, need 2 x %d layers", n,
                    M->d.n_layers);
    for (int32_t i = 0; i < n; ++i)
        if (!events[i]) return fail(RRA_EINVAL, "rra_model_set_attention_events: null event %d", i);
    M->attn_events.assign(reinterpret_cast<const hipEvent_t *>(events),
                          reinterpret_cast<const hipEvent_t *>(events) + n);
    return RRA_OK;
}

extern "C" rra_status rra_model_set_phase_events(rra_model *M, void *const *events, int32_t n) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_model_set_phase_events: null model");
    if (!events || n == 0) {
        M->phase_events.clear();
        return RRA_OK;
    }
    if (n != 4 * M->d.n_layers + 3)
        return fail(RRA_EINVAL, "rra_model_set_phase_events: n=%d, need 4 x %d layers + 3", n,
                    M->d.n_layers);
    for (int32_t i = 0; i < n; ++i)
        if (!events[i]) return fail(RRA_EINVAL, "rra_model_set_phase_events: null event %d", i);
    M->phase_events.assign(reinterpret_cast<const hipEvent_t *>(events),
                           reinterpret_cast<const hipEvent_t *>(events) + n);
    return RRA_OK;
}

extern "C" rra_status rra_prefill(rra_model *M, const uint32_t *tokens, int32_t n_tokens,
                                  int32_t seq, uint32_t start, uint32_t *next_tok, float *logits,
                                  hipStream_t s) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_prefill: null model");
    const rra_model_desc &d = M->d;
    if (!tokens || n_tokens < 1) return fail(RRA_EINVAL, "rra_prefill: no tokens");
    if (seq < 0 || seq >= d.m_max)
        return fail(RRA_EINVAL, "rra_prefill: seq=%d not in 0..m_max-1=%d", seq, d.m_max - 1);
    if (!d.embed) return fail(RRA_EINVAL, "rra_prefill: the model has no embedding table");
    if ((int64_t)start + n_tokens > d.max_len)
        return fail(RRA_EINVAL, "rra_prefill: positions %u..%lld exceed max_len=%d", start,
                    (long long)start + n_tokens - 1, d.max_len);
    // Chunks of up to prefill_rows tokens; each chunk's GEMMs stream the
    // weights once for all of its rows, and its attention is causal within
    // the chunk and over the slot's earlier rows.
    const int R = M->prefill_rows;
    for (int c0 = 0; c0 < n_tokens; c0 += R) {
        const int n = std::min(R, n_tokens - c0);
        RRA_TRY(enqueue_prompt_chunk(M, tokens + c0, n, seq, start + (uint32_t)c0,
                                     c0 + n == n_tokens, s));
    }
    if (next_tok)
        RRA_TRY_HIP(hipMemcpyAsync(next_tok, M->ptok, sizeof(uint32_t), hipMemcpyDeviceToDevice, s));
    if (logits)
        RRA_TRY_HIP(hipMemcpyAsync(logits, M->logits, sizeof(float) * d.vocab,
                                   hipMemcpyDeviceToDevice, s));
    return RRA_OK;
}

// ---------------------------------------------------------------- attention plan
static void drop_graphs(rra_model *M) {
    for (GraphEntry &g : M->graphs) (void)hipGraphExecDestroy(g.exec);
    M->graphs.clear();
}

extern "C" rra_status rra_model_attention_plan(const rra_model *M, int32_t m, int32_t *chunk,
                                               int32_t *head_split) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_model_attention_plan: null model");
    if (m < 1 || m > M->d.m_max)
        return fail(RRA_EINVAL, "rra_model_attention_plan: m=%d not in 1..%d", m, M->d.m_max);
    if (chunk) *chunk = M->chunk[m];
    if (head_split) *head_split = M->hsplit[m];
    return RRA_OK;
}

extern "C" rra_status rra_model_set_attention_plan(rra_model *M, int32_t m, int32_t chunk,
                                                   int32_t head_split) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_model_set_attention_plan: null model");
    const rra_model_desc &d = M->d;
    if (m < 1 || m > d.m_max)
        return fail(RRA_EINVAL, "rra_model_set_attention_plan: m=%d not in 1..%d", m, d.m_max);
    if (chunk < 32 || chunk > 1024 || chunk % 32)
        return fail(RRA_EINVAL, "rra_model_set_attention_plan: chunk=%d (a multiple of 32 in "
                    "32..1024)", chunk);
    const int group = d.n_heads / d.n_kv_heads;
    if (head_split < 0 || (head_split > 0 && group % head_split))
        return fail(RRA_EINVAL, "rra_model_set_attention_plan: head_split=%d does not divide %d",
                    head_split, group);
    if (fd_partials_floats(m, d.n_heads, d.head_dim, d.max_len, chunk) > fd_floats(d))
        return fail(RRA_EINVAL, "rra_model_set_attention_plan: chunk=%d needs more partials than "
                    "the workspace holds", chunk);
    if (M->chunk[m] != chunk || M->hsplit[m] != head_split) {
        M->chunk[m] = chunk;
        M->hsplit[m] = head_split;
        drop_graphs(M);  // captured steps baked the old grid in
    }
    return RRA_OK;
}

extern "C" rra_status rra_model_tune_attention(rra_model *M, const int32_t *ms, int32_t n_ms,
                                               const uint32_t *lengths, hipStream_t s) {
    clear_error();
    if (!M) return fail(RRA_ENOTINIT, "rra_model_tune_attention: null model");
    const rra_model_desc &d = M->d;
    std::vector<int> todo;
    if (!ms || n_ms <= 0) {
        for (int m = 1; m <= d.m_max; ++m) todo.push_back(m);
    } else {
        for (int i = 0; i < n_ms; ++i) {
            if (ms[i] < 1 || ms[i] > d.m_max)
                return fail(RRA_EINVAL, "rra_model_tune_attention: m=%d not in 1..%d", ms[i],
                            d.m_max);
            todo.push_back(ms[i]);
        }
    }
    // lengths the steps will see (clamped to max_len); default: full caches
    std::vector<uint32_t> lens(d.m_max, (uint32_t)d.max_len);
    if (lengths)
        for (int i = 0; i < d.m_max; ++i) lens[i] = std::min<uint32_t>(lengths[i], d.max_len);
    RRA_TRY_HIP(hipMemcpyAsync(M->lens, lens.data(), sizeof(uint32_t) * d.m_max,
                               hipMemcpyHostToDevice, s));
    const int nqkv = (d.n_heads + 2 * d.n_kv_heads) * d.head_dim;
    std::vector<const float *> kcs(d.n_layers), vcs(d.n_layers);
    for (int l = 0; l < d.n_layers; ++l) {
        kcs[l] = M->layers[l].k_cache;
        vcs[l] = M->layers[l].v_cache;
    }
    // Positions for the fused kernel: the row before each length, so that
    // the sequence lengths it forms are the given ones; an empty slot for 0.
    std::vector<uint32_t> pos(d.m_max);
    for (int i = 0; i < d.m_max; ++i) pos[i] = lens[i] ? lens[i] - 1 : RRA_POS_NONE;
    for (int m : todo) {
        // time the kernel the step runs: at m where the step fuses the QKV
        // epilogue, the fused one, from zero split planes, attending to its
        // new row without writing it to the cache (QkvIn with null caches);
        // the positions sit in the q buffer, which the fused kernel does not read
        RRA_TRY_HIP(hipMemsetAsync(M->q, 0, sizeof(float) * d.m_max * d.n_heads * d.head_dim, s));
        QkvIn qi;
        const bool fused = step_fuses_qkv(m);
        if (fused) {
            const GemvPlan &pq = M->plan_qkv[m];
            uint32_t *pos_dev = reinterpret_cast<uint32_t *>(M->q);
            RRA_TRY_HIP(hipMemcpyAsync(pos_dev, pos.data(), sizeof(uint32_t) * d.m_max,
                                       hipMemcpyHostToDevice, s));
            RRA_TRY_HIP(hipMemsetAsync(M->part, 0,
                                       sizeof(float) * (size_t)pq.split * m * nqkv, s));
            qi = QkvIn{M->part, pq.split, (long long)m * nqkv, pos_dev, M->rope,
                       nullptr, nullptr, M->lens, M->err};
        }
        int c = 0, hs = 0;
        RRA_TRY(fd_time_candidates(M->q, kcs.data(), vcs.data(), d.n_layers, M->lens, M->attn, m,
                                   d.n_heads, d.n_kv_heads, d.head_dim, d.max_len, M->fd, s, &c,
                                   &hs, nullptr, fused ? &qi : nullptr));
        RRA_TRY(rra_model_set_attention_plan(M, m, c, hs));
    }
    RRA_TRY_HIP(hipStreamSynchronize(s));
    return RRA_OK;
}
