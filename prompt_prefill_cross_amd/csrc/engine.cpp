// Prefill scheduler, KV store, KVCP snapshots and the extern "C" entry points.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <mutex>
#include <string>
#include <vector>

#include "ppx_internal.h"

namespace ppx {
bool log_enabled();
int model_load(const uint8_t *b, size_t n, hipStream_t stream, void *weights_dev, size_t weights_bytes,
               size_t *need_bytes, ppx_model **out);
int ensure_rope(ppx_model *m, int n_ctx);
void model_free(ppx_model *m);

namespace {

#define PPX_TRY(x)                     \
    do {                               \
        const int st_ = (x);           \
        if (st_ != PPX_OK) return st_; \
    } while (0)

inline size_t al(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout of one prefill (offsets from the workspace base).  The
// per-ubatch buffers (x .. gpart) repeat once per slot, slot_stride apart:
// a prefill keeps up to nslots ubatches in flight, each in its own slot.
struct WsLayout {
    size_t tok;
    size_t x, a16, a16lo, q16, o16, h16, p16, ap_part, gpart;  // slot 0
    size_t q32, o16lo, h16lo, p16lo;                           // exact precision only (one ubatch at a time)
    size_t gpart_floats;                                       // split-K partials of one GEMM
    size_t slot_stride;
    int nslots;
    size_t xr, qr, orow, hr, pr;
    size_t at_part;
    size_t total;
};

WsLayout ws_layout(const ppx_model *m, int ub, int n_ctx, int nslots) {
    const ppx_model_info &I = m->info;
    const int d = I.d_model, qd = I.n_head * I.head_dim, F = I.n_ff, E = I.ple_dim;
    WsLayout w{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t r = o;
        o += al(bytes);
        return r;
    };
    const size_t ub16 = (size_t)(ub + 15) / 16 * 16;  // fragment-tiled buffers hold whole 16-row tiles
    w.tok = take(sizeof(int32_t) * (size_t)std::max(n_ctx, 1));
    const size_t s0 = o;
    w.x = take(4ull * ub * d);
    w.a16 = take(2ull * ub16 * std::max(d, 1));
    w.a16lo = take(2ull * ub16 * std::max(d, 1));
    w.q16 = take(2ull * ub * qd);
    w.o16 = take(2ull * ub16 * qd);
    w.h16 = take(2ull * ub16 * F);
    w.p16 = take(2ull * ub16 * std::max(E, 1));
    w.ap_part = take(4 * attn_prefill_scratch_floats(ub, I.n_head, I.head_dim, std::max(n_ctx, 1)));
    {
        const int kvd = I.kv_dim;
        const int shapes[][2] = {{qd, d}, {2 * kvd, d}, {d, qd}, {2 * F, d}, {d, F}, {E, d}, {d, E}};
        size_t pf = 0;
        for (const auto &nk : shapes)
            if (nk[0] > 0 && nk[1] > 0) pf = std::max(pf, gemm_part_floats(ub, nk[0], nk[1]));
        w.gpart_floats = pf;
        w.gpart = take(4 * std::max<size_t>(pf, 1));
    }
    w.slot_stride = o - s0;
    w.nslots = std::max(1, nslots);
    o += w.slot_stride * (w.nslots - 1);
    // exact precision: fp32 queries and the low parts of the split operands
    w.q32 = take(4ull * ub * qd);
    w.o16lo = take(2ull * ub16 * qd);
    w.h16lo = take(2ull * ub16 * F);
    w.p16lo = take(2ull * ub16 * std::max(E, 1));
    w.xr = take(4ull * d);
    w.qr = take(4ull * qd);
    w.orow = take(4ull * qd);
    w.hr = take(4ull * F);
    w.pr = take(4ull * std::max(E, 1));
    w.at_part = take(4 * attn1_scratch_floats(I.n_head, I.head_dim, std::max(n_ctx, 1)));
    w.total = o;
    return w;
}

// Ubatches a prefill keeps in flight: as many as the prompt has, at most one
// per layer they run through and at most kMaxUnits.
int prefill_slots(const ppx_model *m, int ub, int n_ctx) {
    const long nub = ((long)std::max(n_ctx, 1) + ub - 1) / ub;
    return (int)std::max(1L, std::min<long>({nub, (long)m->info.n_layer, (long)kMaxUnits}));
}

int predicate(int L, int Ls, int emb, int nseq, const uint8_t *inp, int crop) {
    bool ok = crop && Ls > 0 && Ls < L && !emb && nseq == 1;
    for (int il = Ls; ok && il <= L; ++il) ok = !(inp && inp[il]);
    return ok ? 1 : 0;
}

struct Ctx {
    ppx_model *m;
    ppx_kv *kv;
    hipStream_t s;
    uint8_t *ws;
    WsLayout L;
    ppx_timing *tm = nullptr;  // per-phase timing requested
    int slot = 0;              // buffers of the ubatch being enqueued
    bool exact = false;        // PPX_PRECISION_EXACT: the row-batched layers at ~fp32 accuracy
    // A row batch spanning several sequences, each with its own cache (null:
    // the rows are one sequence's consecutive positions, in kv).
    struct Rows {
        const int32_t *tok = nullptr, *pos = nullptr, *seq = nullptr;  // device, per row
        const KVRef *kv = nullptr;  // device, [Ls][nseq]: sequence s's cache of owning layer l at l * nseq + s
        int nseq = 0;
        const AttnWg *wg = nullptr;  // device: the attention workgroups of the batch
        int nwg = 0;
        AttnSplit split;
        double vis = 0;  // causal (query, key) pairs of the batch (timing only)
        bool gathered = false;  // the sequences' output rows, one each
    };
    const Rows *rows = nullptr;
    struct Rec { int phase; hipEvent_t a, b; bool glu; };
    std::vector<Rec> recs;
    size_t next_ev = 0;
    template <typename T>
    T *at(size_t off) const { return reinterpret_cast<T *>(ws + off); }
    // a per-ubatch buffer of slot k (default: the current slot)
    template <typename T>
    T *sl(size_t off, int k = -1) const {
        return reinterpret_cast<T *>(ws + off + (size_t)(k < 0 ? slot : k) * L.slot_stride);
    }
    // a row-batched GEMM of slot k, with that slot's split-K partial space
    GemmArgs gemm(int k = -1, const Rows *r = nullptr) const {
        GemmArgs g;
        g.part = sl<float>(L.gpart, k);
        g.part_floats = L.gpart_floats;
        g.few_rows = r ? r->gathered : rows && rows->gathered;
        return g;
    }

    hipEvent_t event() {
        if (next_ev == m->events.size()) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return nullptr;
            m->events.push_back(e);
        }
        return m->events[next_ev++];
    }
    hipEvent_t begin() {
        if (!tm) return nullptr;
        hipEvent_t e = event();
        if (e) (void)hipEventRecord(e, s);
        return e;
    }
    void end(int phase, hipEvent_t a, bool glu = false) {
        if (!tm || !a) return;
        hipEvent_t b = event();
        if (!b) return;
        (void)hipEventRecord(b, s);
        recs.push_back({phase, a, b, glu});
    }
    int finish() {
        if (!tm) return PPX_OK;
        if (hipStreamSynchronize(s) != hipSuccess) return PPX_E_HIP;
        for (const Rec &r : recs) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return PPX_E_HIP;
            tm->ms[r.phase] += ms;
            tm->launches[r.phase] += 1;
            if (r.glu) {
                tm->glu_ms += ms;
                tm->glu_launches += 1;
            }
        }
        return PPX_OK;
    }
};

// Run one launch, timed under `phase` when timing was requested.
#define PPX_LAUNCH(c, phase, expr)              \
    do {                                        \
        hipEvent_t ev0_ = (c).begin();          \
        PPX_TRY(expr);                          \
        (c).end((phase), ev0_);                 \
    } while (0)

inline double q4_bytes(const Q4R &w) { return (double)w.N * w.K * 18.0 / 32.0; }

// Layer il for M rows at ~fp32 accuracy (PPX_PRECISION_EXACT): every GEMM on
// the exact-weight kernel with split activations (norms write high and low
// parts; the epilogues of Q, GLU and PLE keep fp32 or write both parts), and
// attention of each row in fp32.  Slot 0's buffers only (one ubatch at a time).
int layer_rows_exact(Ctx &c, int il, int M, int row0, int pos0) {
    const ppx_model *m = c.m;
    const ppx_model_info &I = m->info;
    const LayerW &w = m->layers[il];
    const int d = I.d_model, hd = I.head_dim, qd = I.n_head * hd, kvd = I.kv_dim;
    float *x = c.sl<float>(c.L.x);
    __half *a16 = c.sl<__half>(c.L.a16), *a16lo = c.sl<__half>(c.L.a16lo);
    __half *o16 = c.sl<__half>(c.L.o16), *o16lo = c.at<__half>(c.L.o16lo);
    __half *h16 = c.sl<__half>(c.L.h16), *h16lo = c.at<__half>(c.L.h16lo);
    float *q32 = c.at<float>(c.L.q32);
    const Ctx::Rows *R = c.rows;
    const size_t lstride = R ? 0 : (size_t)c.kv->n_ctx * kvd;
    const size_t vstride = R ? 0 : (size_t)c.kv->vld * kvd;
    auto gemm = [&](const __half *A, const __half *A2, const Q4R &W, int epi) {
        GemmArgs g;
        g.A = A;
        g.A2 = A2;
        g.M = M;
        g.W = W;
        g.epi = epi;
        return g;
    };

    PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_rmsnorm_split(x, w.attn_norm, m->eps, M, d, a16, a16lo, c.s));
    GemmArgs g = gemm(a16, a16lo, w.wq, EPI_QKV);
    g.q32 = q32;
    g.qd = qd;
    g.kvd = 0;
    g.hd = hd;
    g.pos0 = pos0;
    g.rope = m->rope;
    if (R) g.row_pos = R->pos;
    PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_exact(g, c.s));
    if (w.own) {
        GemmArgs gk = g;
        gk.W = w.wkv;
        gk.q32 = nullptr;
        gk.qd = 0;
        gk.kvd = kvd;
        if (R) {
            gk.row_seq = R->seq;
            gk.seq_kv = R->kv + (size_t)il * R->nseq;
        } else {
            gk.kc = c.kv->k + il * lstride;
            gk.vc = c.kv->vt + il * vstride;
            gk.vld = c.kv->vld;
        }
        PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_exact(gk, c.s));
    }
    AttnArgs at;
    at.q32 = q32;
    at.o = o16;
    at.o_lo = o16lo;
    if (R) {
        at.seq_kv = R->kv + (size_t)w.src * R->nseq;
        at.row_pos = R->pos;
        at.row_seq = R->seq;
    } else {
        at.k = c.kv->k + (size_t)w.src * lstride;
        at.vt = c.kv->vt + (size_t)w.src * vstride;
        at.vld = c.kv->vld;
    }
    at.M = M;
    at.H = I.n_head;
    at.KVH = I.n_kv_head;
    at.hd = hd;
    at.pos0 = pos0;
    PPX_LAUNCH(c, PPX_PHASE_ATTN, launch_attn_rows_exact(at, c.s));
    GemmArgs go = gemm(o16, o16lo, w.wo, EPI_ADD);
    go.out_f32 = x;
    PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_exact(go, c.s));

    PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_rmsnorm_split(x, w.ffn_norm, m->eps, M, d, a16, a16lo, c.s));
    GemmArgs gu = gemm(a16, a16lo, w.wgu, EPI_GLU);
    gu.out_f16 = h16;
    gu.out_lo = h16lo;
    gu.act = I.act;
    PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_exact(gu, c.s));
    GemmArgs gd = gemm(h16, h16lo, w.wdown, EPI_ADD);
    gd.out_f32 = x;
    PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_exact(gd, c.s));
    if (I.ple_dim) {
        const int E = I.ple_dim;
        __half *p16 = c.sl<__half>(c.L.p16), *p16lo = c.at<__half>(c.L.p16lo);
        PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_rmsnorm_split(x, w.ple_norm, m->eps, M, d, a16, a16lo, c.s));
        GemmArgs gp = gemm(a16, a16lo, w.wpg, EPI_PLE);
        gp.out_f16 = p16;
        gp.out_lo = p16lo;
        gp.ple_raw = m->ple_raw;
        gp.tok = R ? R->tok : c.at<int32_t>(c.L.tok) + row0;
        gp.ple_row_blocks = I.n_layer * E / 32;
        gp.ple_col0 = il * E;
        gp.ple_s = w.ple_s;
        PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_exact(gp, c.s));
        GemmArgs gq = gemm(p16, p16lo, w.wpu, EPI_ADD);
        gq.out_f32 = x;
        PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_exact(gq, c.s));
    }
    if (c.tm) {
        double nk = (double)w.wq.N * w.wq.K + (double)w.wo.N * w.wo.K + (double)w.wgu.N * w.wgu.K +
                    (double)w.wdown.N * w.wdown.K;
        if (w.own) nk += (double)w.wkv.N * w.wkv.K;
        if (I.ple_dim) nk += (double)w.wpg.N * w.wpg.K + (double)w.wpu.N * w.wpu.K;
        c.tm->gemm_flop += 2.0 * M * nk;
        const double vis = R ? R->vis : (double)M * pos0 + 0.5 * (double)M * (M + 1);
        c.tm->attn_flop += 4.0 * I.n_head * hd * vis;
    }
    return PPX_OK;
}

// One ubatch in flight: rows [row0, row0 + M) of the call (token ids from
// row0 on), positions pos0 .., running layer il with the buffers of slot.
// R: the per-row tables of a batch spanning several sequences (null: one
// sequence in c.kv).
struct Unit {
    int il, M, row0, pos0, slot;
    const Ctx::Rows *R = nullptr;
};

// One step of the row-batched layers: every unit runs its own layer, and each
// operation of the layer is one launch over all the units (the same shapes,
// each unit with its own weights, activations and cache).
int layer_rows_group(Ctx &c, const Unit *U, int n) {
    if (n < 1 || n > kMaxUnits) return PPX_E_INVAL;
    if (c.exact) {
        if (n != 1) return PPX_E_INVAL;  // one ubatch at a time
        const Ctx::Rows *r0 = c.rows;
        const int s0 = c.slot;
        c.rows = U[0].R;
        c.slot = U[0].slot;
        const int st = layer_rows_exact(c, U[0].il, U[0].M, U[0].row0, U[0].pos0);
        c.rows = r0;
        c.slot = s0;
        return st;
    }
    const ppx_model *m = c.m;
    const ppx_model_info &I = m->info;
    const int d = I.d_model, hd = I.head_dim, qd = I.n_head * hd, kvd = I.kv_dim;
    for (int i = 1; i < n; ++i)
        if (!U[i].R != !U[0].R) return PPX_E_INVAL;  // one kind of cache per launch
    const size_t lstride = U[0].R ? 0 : (size_t)c.kv->n_ctx * kvd;
    const size_t vstride = U[0].R ? 0 : (size_t)c.kv->vld * kvd;
    auto W = [&](int i) -> const LayerW & { return m->layers[U[i].il]; };
    auto X = [&](int i) { return c.sl<float>(c.L.x, U[i].slot); };
    auto H16 = [&](int i, size_t off) { return c.sl<__half>(off, U[i].slot); };

    // attention RMSNorm: owning layers also write the low part (the K|V operand)
    {
        NormUnit own[kMaxUnits], shr[kMaxUnits];
        int no = 0, ns = 0;
        for (int i = 0; i < n; ++i) {
            NormUnit u;
            u.x = X(i);
            u.g = W(i).attn_norm;
            u.hi = H16(i, c.L.a16);
            u.M = U[i].M;
            if (W(i).own) {
                u.lo = H16(i, c.L.a16lo);
                own[no++] = u;
            } else {
                shr[ns++] = u;
            }
        }
        if (no) PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_rmsnorm_group(own, no, m->eps, d, true, c.s));
        if (ns) PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_rmsnorm_group(shr, ns, m->eps, d, false, c.s));
    }
    GemmArgs g[kMaxUnits];
    for (int i = 0; i < n; ++i) {
        g[i] = c.gemm(U[i].slot, U[i].R);
        g[i].A = H16(i, c.L.a16);
        g[i].lda = d;
        g[i].M = U[i].M;
        g[i].W = W(i).wq;
        g[i].epi = EPI_QKV;
        g[i].out_f16 = H16(i, c.L.q16);
        g[i].qd = qd;
        g[i].kvd = 0;
        g[i].hd = hd;
        g[i].pos0 = U[i].pos0;
        g[i].rope = m->rope;
        if (U[i].R) g[i].row_pos = U[i].R->pos;
    }
    PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_group(g, n, c.s));
    {
        // K and V on the exact-weight path, straight into the owning layers' cache rows
        GemmArgs gk[kMaxUnits];
        int nk = 0;
        for (int i = 0; i < n; ++i) {
            if (!W(i).own) continue;
            GemmArgs &k = gk[nk++];
            k = g[i];
            k.A2 = H16(i, c.L.a16lo);
            k.W = W(i).wkv;
            k.qd = 0;
            k.kvd = kvd;
            k.out_f16 = nullptr;
            if (const Ctx::Rows *R = U[i].R) {
                k.row_seq = R->seq;
                k.seq_kv = R->kv + (size_t)U[i].il * R->nseq;
            } else {
                k.kc = c.kv->k + U[i].il * lstride;
                k.vc = c.kv->vt + U[i].il * vstride;
                k.vld = c.kv->vld;
            }
        }
        if (nk) PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_exact_group(gk, nk, c.s));
    }
    {
        // causal attention over the cache of each unit's KV source layer
        AttnArgs at[kMaxUnits];
        for (int i = 0; i < n; ++i) {
            AttnArgs &a = at[i];
            const int src = W(i).src;
            a.q = H16(i, c.L.q16);
            if (const Ctx::Rows *R = U[i].R) {
                a.wg = R->wg;
                a.nwg = R->nwg;
                a.seq_kv = R->kv + (size_t)src * R->nseq;
                a.row_pos = R->pos;
                a.kc = R->split.kc;
                a.nkc = R->split.nkc;
            } else {
                a.k = c.kv->k + (size_t)src * lstride;
                a.vt = c.kv->vt + (size_t)src * vstride;
                a.vld = c.kv->vld;
            }
            a.part = c.sl<float>(c.L.ap_part, U[i].slot);
            a.o = H16(i, c.L.o16);
            a.M = U[i].M;
            a.H = I.n_head;
            a.KVH = I.n_kv_head;
            a.hd = hd;
            a.pos0 = U[i].pos0;
        }
        PPX_LAUNCH(c, PPX_PHASE_ATTN, launch_attn_prefill_group(at, n, c.s));
    }
    for (int i = 0; i < n; ++i) {
        g[i] = c.gemm(U[i].slot, U[i].R);
        g[i].A = H16(i, c.L.o16);
        g[i].lda = qd;
        g[i].M = U[i].M;
        g[i].W = W(i).wo;
        g[i].epi = EPI_ADD;
        g[i].out_f32 = X(i);
    }
    PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_group(g, n, c.s));
    {
        NormUnit nu[kMaxUnits];
        for (int i = 0; i < n; ++i) {
            nu[i].x = X(i);
            nu[i].g = W(i).ffn_norm;
            nu[i].hi = H16(i, c.L.a16);
            nu[i].M = U[i].M;
        }
        PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_rmsnorm_group(nu, n, m->eps, d, false, c.s));
    }
    for (int i = 0; i < n; ++i) {
        g[i] = c.gemm(U[i].slot, U[i].R);
        g[i].A = H16(i, c.L.a16);
        g[i].lda = d;
        g[i].M = U[i].M;
        g[i].W = W(i).wgu;
        g[i].epi = EPI_GLU;
        g[i].out_f16 = H16(i, c.L.h16);
        g[i].act = I.act;
    }
    {
        hipEvent_t ev0 = c.begin();
        PPX_TRY(launch_gemm_group(g, n, c.s));
        c.end(PPX_PHASE_GEMM, ev0, true);
    }
    for (int i = 0; i < n; ++i) {
        g[i] = c.gemm(U[i].slot, U[i].R);
        g[i].A = H16(i, c.L.h16);
        g[i].lda = I.n_ff;
        g[i].M = U[i].M;
        g[i].W = W(i).wdown;
        g[i].epi = EPI_ADD;
        g[i].out_f32 = X(i);
        if (I.ple_dim) {
            // the per-layer-embedding block's RMSNorm of the updated rows rides on the down projection
            g[i].norm_g = W(i).ple_norm;
            g[i].norm_eps = m->eps;
            g[i].norm_out = H16(i, c.L.a16);
        }
    }
    PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_group(g, n, c.s));
    if (I.ple_dim && ple_fused_supported(I.ple_dim, d)) {
        // the whole block in one launch: p stays in LDS
        const int E = I.ple_dim;
        PleArgs pa[kMaxUnits];
        for (int i = 0; i < n; ++i) {
            pa[i].a = H16(i, c.L.a16);
            pa[i].x = X(i);
            pa[i].wg = W(i).wpg;
            pa[i].wu = W(i).wpu;
            pa[i].ple_raw = m->ple_raw;
            pa[i].tok = U[i].R ? U[i].R->tok : c.at<int32_t>(c.L.tok) + U[i].row0;
            pa[i].ple_row_blocks = I.n_layer * E / 32;
            pa[i].ple_col0 = U[i].il * E;
            pa[i].ple_s = W(i).ple_s;
            pa[i].M = U[i].M;
        }
        PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_ple_group(pa, n, c.s));
    } else if (I.ple_dim) {
        const int E = I.ple_dim;
        for (int i = 0; i < n; ++i) {
            g[i] = c.gemm(U[i].slot, U[i].R);
            g[i].A = H16(i, c.L.a16);
            g[i].lda = d;
            g[i].M = U[i].M;
            g[i].W = W(i).wpg;
            g[i].epi = EPI_PLE;
            g[i].out_f16 = H16(i, c.L.p16);
            g[i].ple_raw = m->ple_raw;
            g[i].tok = U[i].R ? U[i].R->tok : c.at<int32_t>(c.L.tok) + U[i].row0;
            g[i].ple_row_blocks = I.n_layer * E / 32;
            g[i].ple_col0 = U[i].il * E;
            g[i].ple_s = W(i).ple_s;
        }
        PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_group(g, n, c.s));
        for (int i = 0; i < n; ++i) {
            g[i] = c.gemm(U[i].slot, U[i].R);
            g[i].A = H16(i, c.L.p16);
            g[i].lda = E;
            g[i].M = U[i].M;
            g[i].W = W(i).wpu;
            g[i].epi = EPI_ADD;
            g[i].out_f32 = X(i);
        }
        PPX_LAUNCH(c, PPX_PHASE_GEMM, launch_gemm_group(g, n, c.s));
    }
    if (c.tm) {
        for (int i = 0; i < n; ++i) {
            const LayerW &w = W(i);
            const int M = U[i].M, pos0 = U[i].pos0;
            double nk = (double)w.wq.N * w.wq.K + (double)w.wo.N * w.wo.K + (double)w.wgu.N * w.wgu.K +
                        (double)w.wdown.N * w.wdown.K;
            if (w.own) nk += (double)w.wkv.N * w.wkv.K;
            if (I.ple_dim) nk += (double)w.wpg.N * w.wpg.K + (double)w.wpu.N * w.wpu.K;
            c.tm->gemm_flop += 2.0 * M * nk;
            c.tm->glu_flop += 2.0 * M * w.wgu.N * w.wgu.K;
            const double vis = U[i].R ? U[i].R->vis
                                      : (double)M * pos0 + 0.5 * (double)M * (M + 1);  // causal (query, key) pairs
            c.tm->attn_flop += 4.0 * I.n_head * hd * vis;
        }
    }
    return PPX_OK;
}

// One ubatch of M rows through layer il on the MFMA path (the current slot).
int layer_rows(Ctx &c, int il, int M, int row0, int pos0) {
    const Unit u{il, M, row0, pos0, c.slot, c.rows};
    return layer_rows_group(c, &u, 1);
}

GemvArgs gemv_base(Ctx &c, const float *x, const Q4R &W, int epi, float *out) {
    GemvArgs a;
    a.x = x;
    a.W = W;
    a.epi = epi;
    a.out = out;
    (void)c;
    return a;
}

// Layer il for one row at position pos, fp32 throughout: the pruned KV-shared
// layers of a prefill, and every layer of a decode step (where an owning layer
// first writes the row's K and V at pos).
int layer_row(Ctx &c, int il, int pos, const int32_t *tok, bool write_kv = false) {
    const ppx_model *m = c.m;
    const ppx_model_info &I = m->info;
    const LayerW &w = m->layers[il];
    const int hd = I.head_dim, kvd = I.kv_dim;
    float *xr = c.at<float>(c.L.xr);
    float *qr = c.at<float>(c.L.qr), *orow = c.at<float>(c.L.orow);
    float *hr = c.at<float>(c.L.hr), *pr = c.at<float>(c.L.pr);
    const size_t lstride = (size_t)c.kv->n_ctx * kvd;

    // each projection that follows an RMSNorm normalises the row itself
    GemvArgs gq = gemv_base(c, xr, w.wq, GV_QROPE, qr);
    gq.norm_g = w.attn_norm;
    gq.eps = m->eps;
    gq.hd = hd;
    gq.pos = pos;
    gq.rope = m->rope;
    if (write_kv && w.own) {
        // the K|V projection of the same normalised row, in the same launch:
        // the roped K row and the V^T column at pos
        gq.W2 = w.wkv;
        gq.epi2 = GV_KV;
        gq.kc = c.kv->k + (size_t)il * lstride;
        gq.vt = c.kv->vt + (size_t)il * c.kv->vld * kvd;
        gq.kvd = kvd;
        gq.vld = c.kv->vld;
        if (c.tm) c.tm->row_bytes += q4_bytes(w.wkv);
    }
    PPX_LAUNCH(c, PPX_PHASE_ROW, launch_gemv(gq, c.s));
    Attn1Args at;
    at.q = qr;
    at.k = c.kv->k + (size_t)w.src * lstride;
    at.vt = c.kv->vt + (size_t)w.src * c.kv->vld * kvd;
    at.vld = c.kv->vld;
    at.o = orow;
    at.H = I.n_head;
    at.KVH = I.n_kv_head;
    at.hd = hd;
    at.pos = pos;
    at.partial = c.at<float>(c.L.at_part);
    PPX_LAUNCH(c, PPX_PHASE_ROW, launch_attn_1row(at, c.s));
    PPX_LAUNCH(c, PPX_PHASE_ROW, launch_gemv(gemv_base(c, orow, w.wo, GV_ADD, xr), c.s));
    GemvArgs gg = gemv_base(c, xr, w.wgu, GV_GLU, hr);
    gg.norm_g = w.ffn_norm;
    gg.eps = m->eps;
    gg.act = I.act;
    PPX_LAUNCH(c, PPX_PHASE_ROW, launch_gemv(gg, c.s));
    PPX_LAUNCH(c, PPX_PHASE_ROW, launch_gemv(gemv_base(c, hr, w.wdown, GV_ADD, xr), c.s));
    if (c.tm) {
        c.tm->row_bytes += q4_bytes(w.wq) + q4_bytes(w.wo) + q4_bytes(w.wgu) + q4_bytes(w.wdown) +
                           4.0 * (pos + 1) * kvd;
        if (I.ple_dim) c.tm->row_bytes += q4_bytes(w.wpg) + q4_bytes(w.wpu);
    }
    if (I.ple_dim) {
        GemvArgs gp = gemv_base(c, xr, w.wpg, GV_PLE, pr);
        gp.norm_g = w.ple_norm;
        gp.eps = m->eps;
        gp.ple_raw = m->ple_raw;
        gp.tok = tok;
        gp.ple_row_blocks = I.n_layer * I.ple_dim / 32;
        gp.ple_col0 = il * I.ple_dim;
        gp.ple_s = w.ple_s;
        PPX_LAUNCH(c, PPX_PHASE_ROW, launch_gemv(gp, c.s));
        PPX_LAUNCH(c, PPX_PHASE_ROW, launch_gemv(gemv_base(c, pr, w.wpu, GV_ADD, xr), c.s));
    }
    return PPX_OK;
}

// logits = W_out rms(x, gain); gain defaults to the output norm's
int head_row(Ctx &c, const float *x_last, float *logits, const float *gain = nullptr) {
    const ppx_model *m = c.m;
    GemvArgs gh = gemv_base(c, x_last, m->out, GV_F32, logits);
    gh.norm_g = gain ? gain : m->out_norm;
    gh.eps = m->eps;
    PPX_LAUNCH(c, PPX_PHASE_ROW, launch_gemv(gh, c.s));
    if (c.tm) c.tm->row_bytes += q4_bytes(m->out);
    return PPX_OK;
}

// The launch sequence of one prefill call (all ubatches, the pruned tail and
// the head).  Token ids are read from tok_dev, so the sequence can be recorded
// once and replayed for any prompt of the same shape.
//
// Ubatches go through the row-batched layers together: up to L.nslots of them
// are in flight, each in its own slot of buffers, and every step runs each
// in-flight ubatch through its next layer, one launch per operation over all
// of them (layer_rows_group).  A ubatch is admitted when a slot is free, so
// ubatches admitted together advance in lockstep and a later one may trail.
// Within a step the K|V launch of every unit precedes the attention launch,
// and a ubatch is never ahead of an earlier one: when ubatch u attends at
// layer l, every earlier ubatch's K/V of layer l is written, so each ubatch
// sees exactly the cache of the serial order and its rows go through the same
// kernels with the same per-ubatch launch shapes (the results are bit for bit
// those of the serial order).  Debug outputs, extraction and exact precision
// run one ubatch at a time.
int enqueue_prefill(Ctx &c, const ppx_prefill_params *p, const int32_t *tok_dev, int n, int p0, int ub,
                    bool prune, float *logits) {
    ppx_model *m = c.m;
    const ppx_model_info &I = m->info;
    const int L = I.n_layer, Ls = I.n_layer_kv_from_start, d = I.d_model;
    const int nub = (n + ub - 1) / ub;
    const int full_layers = prune ? Ls : L;
    // extraction: the flagged layers' inputs, each in its own [n][d] slab
    std::vector<int> slab(L + 1, -1);
    int nslab = 0;
    if (p->embeddings_layer_inp)
        for (int il = 0; il <= L; ++il)
            if (p->embeddings_layer_inp[il]) slab[il] = nslab++;
    auto extract = [&](int il, const float *x, int M, int s0) -> int {
        if (slab[il] < 0) return PPX_OK;
        return launch_copy_f32(x, p->layer_inp_out + ((size_t)slab[il] * n + s0) * d, M * d, c.s);
    };
    const bool serial = c.exact || p->debug_rows || p->debug_hidden || nslab || p->embeddings;
    const int NU = serial ? 1 : std::max(1, std::min({nub, full_layers, c.L.nslots}));

    struct Flight {
        int u, il, slot;
    };
    std::vector<Flight> fl;
    std::vector<int> free_slots;
    for (int k = NU - 1; k >= 0; --k) free_slots.push_back(k);
    int next_u = 0;
    while (next_u < nub || !fl.empty()) {
        // admit ubatches into free slots: their first layer runs in this step
        while ((int)fl.size() < NU && next_u < nub) {
            const int slot = free_slots.back();
            free_slots.pop_back();
            const int s0 = next_u * ub, M = std::min(ub, n - s0);
            PPX_LAUNCH(c, PPX_PHASE_OTHER,
                       launch_embed(m->tok, tok_dev + s0, M, m->embd_scale, c.sl<float>(c.L.x, slot), c.s));
            fl.push_back({next_u, 0, slot});
            ++next_u;
        }
        Unit U[kMaxUnits];
        const int nu = (int)fl.size();
        for (int i = 0; i < nu; ++i) {
            const int s0 = fl[i].u * ub;
            U[i] = Unit{fl[i].il, std::min(ub, n - s0), s0, p0 + s0, fl[i].slot};
        }
        if (serial) {
            const float *x = c.sl<float>(c.L.x, U[0].slot);
            if (p->debug_rows)
                PPX_TRY(launch_copy_f32(x, p->debug_rows + ((size_t)U[0].il * n + U[0].row0) * d, U[0].M * d, c.s));
            PPX_TRY(extract(U[0].il, x, U[0].M, U[0].row0));
        }
        PPX_TRY(layer_rows_group(c, U, nu));
        // advance; a ubatch past its last row-batched layer leaves its slot
        for (int i = nu - 1; i >= 0; --i) {
            Flight &f = fl[i];
            const Unit &u = U[i];
            float *x = c.sl<float>(c.L.x, f.slot);
            const bool last = f.u == nub - 1;
            if (last && p->debug_hidden)
                PPX_TRY(launch_copy_f32(x + (size_t)(u.M - 1) * d, p->debug_hidden + (size_t)f.il * d, d, c.s));
            if (++f.il < full_layers) continue;
            if (full_layers == L) {
                // every row reached the end (the predicate keeps these off pruned runs)
                PPX_TRY(extract(L, x, u.M, u.row0));
                if (p->embeddings)
                    PPX_TRY(launch_rmsnorm_f32(x, m->out_norm, m->eps, u.M, d, p->embd_out + (size_t)u.row0 * d, c.s));
                if (p->nextn_logits && n - 2 >= u.row0 && n - 2 < u.row0 + u.M) {
                    // next-n head: the second-to-last row's final state plus the
                    // last token's embedding (xr is free: no pruned tail runs)
                    float *z = c.at<float>(c.L.xr);
                    PPX_LAUNCH(c, PPX_PHASE_OTHER,
                               launch_embed_add(m->tok, tok_dev + n - 1, m->embd_scale,
                                                x + (size_t)(n - 2 - u.row0) * d, z, c.s));
                    PPX_TRY(head_row(c, z, p->nextn_logits, m->nextn_norm));
                }
            }
            if (last) {
                const float *x_last = x + (size_t)(u.M - 1) * d;
                if (prune) {
                    float *xr = c.at<float>(c.L.xr);
                    PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_copy_f32(x_last, xr, d, c.s));  // the one row kept
                    const int pos = p0 + n - 1;
                    for (int il = Ls; il < L; ++il) {
                        if (p->debug_rows)
                            PPX_TRY(launch_copy_f32(xr, p->debug_rows + ((size_t)il * n + n - 1) * d, d, c.s));
                        PPX_TRY(layer_row(c, il, pos, tok_dev + n - 1));
                        if (p->debug_hidden) PPX_TRY(launch_copy_f32(xr, p->debug_hidden + (size_t)il * d, d, c.s));
                    }
                    x_last = xr;
                }
                PPX_TRY(head_row(c, x_last, logits));
            }
            free_slots.push_back(f.slot);
            fl.erase(fl.begin() + i);
        }
    }
    return PPX_OK;
}

bool graphs_enabled() {
    static const bool on = [] {
        const char *v = std::getenv("PPX_NO_GRAPH");
        return !(v && *v && *v != '0');
    }();
    return on;
}

// Replay the recorded launch sequence for this call's shape and buffers, or
// record it first (on a private stream: recording runs nothing).  At most
// kMaxGraphs sequences are kept per model, least recently used first out.
constexpr size_t kMaxGraphs = 8;
int run_graph(Ctx &c, const ppx_prefill_params *p, const int32_t *tok_dev, int n, int p0, int ub, bool prune,
              float *logits) {
    ppx_model *m = c.m;
    ppx_model::Graph key;
    key.kv_k = c.kv->k;
    key.kv_vt = c.kv->vt;
    key.ws = c.ws;
    key.logits = logits;
    key.nextn = p->nextn_logits;
    key.n_ctx = c.kv->n_ctx;
    key.n = n;
    key.p0 = p0;
    key.ub = ub;
    key.prune = prune;
    key.exact = c.exact;
    for (auto &g : m->graphs) {
        if (g.kv_k == key.kv_k && g.kv_vt == key.kv_vt && g.ws == key.ws && g.logits == key.logits &&
            g.nextn == key.nextn && g.n_ctx == key.n_ctx && g.n == key.n && g.p0 == key.p0 && g.ub == key.ub && g.prune == key.prune &&
            g.exact == key.exact) {
            g.last_use = ++m->graph_clock;
            return hipGraphLaunch(g.exec, c.s) == hipSuccess ? PPX_OK : PPX_E_HIP;
        }
    }
    if (!m->capture_stream && hipStreamCreateWithFlags(&m->capture_stream, hipStreamNonBlocking) != hipSuccess)
        return PPX_E_HIP;
    Ctx rc = c;
    rc.s = m->capture_stream;
    if (hipStreamBeginCapture(rc.s, hipStreamCaptureModeThreadLocal) != hipSuccess) return PPX_E_HIP;
    const int st = enqueue_prefill(rc, p, tok_dev, n, p0, ub, prune, logits);
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(rc.s, &graph);
    if (st != PPX_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
    }
    if (ec != hipSuccess || !graph) return PPX_E_HIP;
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return PPX_E_HIP;
    if (m->graphs.size() >= kMaxGraphs) {
        auto old = std::min_element(m->graphs.begin(), m->graphs.end(),
                                    [](const ppx_model::Graph &x, const ppx_model::Graph &y) {
                                        return x.last_use < y.last_use;
                                    });
        (void)hipGraphExecDestroy(old->exec);
        m->graphs.erase(old);
    }
    key.exec = exec;
    key.last_use = ++m->graph_clock;
    m->graphs.push_back(key);
    return hipGraphLaunch(exec, c.s) == hipSuccess ? PPX_OK : PPX_E_HIP;
}

// Replay the launch sequence recorded under `key` (everything the launches'
// arguments depend on), or record it first on the model's private stream.
// Up to kMaxGraphs such sequences are kept, least recently used first out.
template <class F>
int run_keyed_graph(Ctx &c, std::vector<long long> key, F &&enqueue) {
    ppx_model *m = c.m;
    for (auto &g : m->keyed_graphs)
        if (g.key == key) {
            g.last_use = ++m->graph_clock;
            return hipGraphLaunch(g.exec, c.s) == hipSuccess ? PPX_OK : PPX_E_HIP;
        }
    if (!m->capture_stream && hipStreamCreateWithFlags(&m->capture_stream, hipStreamNonBlocking) != hipSuccess)
        return PPX_E_HIP;
    Ctx rc = c;
    rc.s = m->capture_stream;
    if (hipStreamBeginCapture(rc.s, hipStreamCaptureModeThreadLocal) != hipSuccess) return PPX_E_HIP;
    const int st = enqueue(rc);
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(rc.s, &graph);
    if (st != PPX_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
    }
    if (ec != hipSuccess || !graph) return PPX_E_HIP;
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return PPX_E_HIP;
    if (m->keyed_graphs.size() >= kMaxGraphs) {
        auto old = std::min_element(m->keyed_graphs.begin(), m->keyed_graphs.end(),
                                    [](const ppx_model::KeyedGraph &x, const ppx_model::KeyedGraph &y) {
                                        return x.last_use < y.last_use;
                                    });
        (void)hipGraphExecDestroy(old->exec);
        m->keyed_graphs.erase(old);
    }
    m->keyed_graphs.push_back({std::move(key), exec, ++m->graph_clock});
    return hipGraphLaunch(exec, c.s) == hipSuccess ? PPX_OK : PPX_E_HIP;
}

int prefill(ppx_model *m, ppx_kv *kv, const int32_t *tokens, int n, const ppx_prefill_params *p, void *ws,
            size_t ws_bytes, float *logits, hipStream_t s) {
    if (!m || !kv || !p || !logits || !ws) return PPX_E_INVAL;
    if (kv->m != m) return PPX_E_INVAL;
    if (n <= 0) return PPX_E_EMPTY;
    if (!tokens) return PPX_E_INVAL;
    const ppx_model_info &I = m->info;
    if (p->n_seq_max != 1) return PPX_E_UNSUPPORTED;
    if (p->embeddings && !p->embd_out) return PPX_E_INVAL;
    if (p->embeddings_layer_inp && !p->layer_inp_out)
        for (int il = 0; il <= I.n_layer; ++il)
            if (p->embeddings_layer_inp[il]) return PPX_E_INVAL;
    if (p->n_ubatch < 1 || p->n_ubatch > PPX_MAX_UBATCH) return PPX_E_INVAL;
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= I.n_vocab) return PPX_E_TOKEN;
    const int p0 = kv->n_pos;
    if ((long)p0 + n > kv->n_ctx) return PPX_E_CTX;
    if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return PPX_E_INVAL;
    const int ub = p->n_ubatch;
    Ctx c{m, kv, s, static_cast<uint8_t *>(ws), ws_layout(m, ub, kv->n_ctx, prefill_slots(m, ub, kv->n_ctx))};
    if (p->timing) {
        std::memset(p->timing, 0, sizeof(*p->timing));
        c.tm = p->timing;
    }
    if (ws_bytes < c.L.total) return PPX_E_NOMEM;
    if (p->precision != PPX_PRECISION_FAST && p->precision != PPX_PRECISION_EXACT) return PPX_E_INVAL;
    c.exact = p->precision == PPX_PRECISION_EXACT;
    if (p->nextn_logits) {
        if (!I.has_nextn) return PPX_E_UNSUPPORTED;
        if (n < 2) return PPX_E_INVAL;
    }
    const int L = I.n_layer, Ls = I.n_layer_kv_from_start, d = I.d_model;
    // a next-n head reads a row other than the output row: the rows cannot be cropped before it
    const int can = predicate(L, Ls, p->embeddings, p->n_seq_max, p->embeddings_layer_inp, p->nextn_logits == nullptr);
    bool prune;
    if (p->prune == PPX_PRUNE_AUTO) prune = can;
    else if (p->prune == PPX_PRUNE_OFF) prune = false;
    else if (p->prune == PPX_PRUNE_ON) {
        if (!can) return PPX_E_UNSUPPORTED;
        prune = true;
    } else return PPX_E_INVAL;

    int32_t *tok_dev = c.at<int32_t>(c.L.tok);
    if (hipMemcpyAsync(tok_dev, tokens, sizeof(int32_t) * n, hipMemcpyHostToDevice, s) != hipSuccess)
        return PPX_E_HIP;
    if (log_enabled())
        std::fprintf(stderr, "[ppx] prefill %d tokens at position %d, ubatch %d, prune %s\n", n, p0, ub,
                     prune ? "on" : "off");

    bool extract = p->embeddings != 0;
    if (p->embeddings_layer_inp)
        for (int il = 0; il <= L; ++il) extract = extract || p->embeddings_layer_inp[il];
    const bool graphable = !c.tm && !p->debug_rows && !p->debug_hidden && !extract && graphs_enabled();
    if (!graphable) {
        // timing, debug and extraction outputs run the launches directly
        PPX_TRY(enqueue_prefill(c, p, tok_dev, n, p0, ub, prune, logits));
    } else {
        PPX_TRY(run_graph(c, p, tok_dev, n, p0, ub, prune, logits));
    }
    PPX_TRY(c.finish());
    kv->n_pos = p0 + n;
    return PPX_OK;
}

// One generated token: the row at position n_pos through every layer on the
// single-row path (owning layers append its K and V), then the head.  The
// same computation as a prefill of that one token.
int decode(ppx_model *m, ppx_kv *kv, int32_t token, void *ws, size_t ws_bytes, float *logits, hipStream_t s) {
    if (!m || !kv || !logits || !ws) return PPX_E_INVAL;
    if (kv->m != m) return PPX_E_INVAL;
    const ppx_model_info &I = m->info;
    if (token < 0 || token >= I.n_vocab) return PPX_E_TOKEN;
    const int pos = kv->n_pos;
    if (pos + 1 > kv->n_ctx) return PPX_E_CTX;
    if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return PPX_E_INVAL;
    Ctx c{m, kv, s, static_cast<uint8_t *>(ws), ws_layout(m, 1, kv->n_ctx, 1)};
    if (ws_bytes < c.L.total) return PPX_E_NOMEM;
    int32_t *tok_dev = c.at<int32_t>(c.L.tok);
    PPX_TRY(launch_fill_u32(reinterpret_cast<uint32_t *>(tok_dev), (uint32_t)token, 1, s));  // by value: no host buffer to outlive
    float *xr = c.at<float>(c.L.xr);
    PPX_TRY(launch_embed(m->tok, tok_dev, 1, m->embd_scale, xr, s));
    for (int il = 0; il < I.n_layer; ++il) PPX_TRY(layer_row(c, il, pos, tok_dev, true));
    PPX_TRY(head_row(c, xr, logits));
    PPX_TRY(c.finish());
    kv->n_pos = pos + 1;
    return PPX_OK;
}

// ------------------------------------------------------------------ several sequences

// Workspace of a multi-sequence prefill: the single-sequence buffers sized for
// max(n_ubatch, n_seq) rows (every ubatch and the gathered output rows use
// them in turn), the gathered rows, then the per-row tables, copied from the
// host in one transfer.
struct MultiLayout {
    WsLayout w;
    size_t xk;                  // fp32 [k][d]: each sequence's output row
    size_t blob;                // start of the tables (everything below is relative to it)
    size_t tok, pos, seq;       // int32 [T] over the rows laid end to end
    size_t ttok, tpos, tseq;    // int32 [k] of the gathered rows
    size_t kv;                  // KVRef [Ls][k]
    size_t wg;                  // AttnWg [max_wg]: every ubatch's workgroups, then the tail's
    size_t pairs;               // int2 [k]: (row in its ubatch, sequence) of each output row
    size_t pages;               // int32 [k][npg]: each sequence's page table (unified cache)
    size_t blob_bytes;
    size_t max_wg;
    size_t total;
};

MultiLayout multi_layout(const ppx_model *m, int ub, int k, long T, int n_ctx_max, int npg = 0) {
    const ppx_model_info &I = m->info;
    MultiLayout L{};
    // ubatch slots as in a single-sequence prefill of T rows
    const long nub_all = (T + ub - 1) / ub;
    const int nslots = (int)std::max(1L, std::min<long>({nub_all, (long)I.n_layer, (long)kMaxUnits}));
    L.w = ws_layout(m, std::max(ub, k), n_ctx_max, nslots);
    size_t o = L.w.total;
    L.xk = o;
    o += al(4ull * k * I.d_model);
    L.blob = o;
    size_t b = 0;
    auto take = [&](size_t bytes) {
        const size_t r = b;
        b += al(bytes);
        return r;
    };
    const int G = I.n_head / std::max(I.n_kv_head, 1);
    const int cb = attn_prefill_cols_per_wg(I.head_dim);
    const long nub = (T + ub - 1) / ub;
    // per ubatch: its rows' column blocks, plus one partial block per sequence boundary
    L.max_wg = (size_t)nub * ((ub * (size_t)G + cb - 1) / cb + 1) + 2 * (size_t)k;
    L.tok = take(4ull * T);
    L.pos = take(4ull * T);
    L.seq = take(4ull * T);
    L.ttok = take(4ull * k);
    L.tpos = take(4ull * k);
    L.tseq = take(4ull * k);
    L.kv = take(sizeof(KVRef) * (size_t)std::max(I.n_layer_kv_from_start, 1) * k);
    L.wg = take(sizeof(AttnWg) * L.max_wg);
    L.pairs = take(sizeof(int2) * (size_t)k);
    L.pages = take(4ull * k * npg);
    L.blob_bytes = b;
    L.total = L.blob + b;
    return L;
}

// The prune of a multi-sequence pass: one output row per sequence, so the
// single-sequence predicate holds per sequence.
int multi_prune(const ppx_model *m, const ppx_prefill_params *p, bool *prune) {
    const ppx_model_info &I = m->info;
    const int can = predicate(I.n_layer, I.n_layer_kv_from_start, p->embeddings, 1, nullptr, 1);
    if (p->prune == PPX_PRUNE_AUTO) *prune = can;
    else if (p->prune == PPX_PRUNE_OFF) *prune = false;
    else if (p->prune == PPX_PRUNE_ON) {
        if (!can) return PPX_E_UNSUPPORTED;
        *prune = true;
    } else return PPX_E_INVAL;
    return PPX_OK;
}

// Pinned staging for the tables: the previous copy out of it must be done
// before it is rewritten (the caller's stream may still be behind).
int stage_tables(ppx_model *m, size_t bytes, uint8_t **out) {
    if (m->stage_event && hipEventSynchronize(m->stage_event) != hipSuccess) return PPX_E_HIP;
    if (m->stage_bytes < bytes) {
        if (m->stage_host) (void)hipHostFree(m->stage_host);
        m->stage_host = nullptr;
        m->stage_bytes = 0;
        if (hipHostMalloc(&m->stage_host, bytes, hipHostMallocDefault) != hipSuccess) return PPX_E_NOMEM;
        m->stage_bytes = bytes;
    }
    if (!m->stage_event && hipEventCreateWithFlags(&m->stage_event, hipEventDisableTiming) != hipSuccess)
        return PPX_E_HIP;
    *out = static_cast<uint8_t *>(m->stage_host);
    return PPX_OK;
}

// One prompt of a multi-sequence pass: its tokens and first position, and
// where its cache lives -- split: its own ppx_kv; unified: its page table in
// the one buffer, covering every position the pass writes.
struct SeqRun {
    const int32_t *tok = nullptr;
    int n = 0, n_pos = 0;
    const ppx_kv *kv = nullptr;
    const std::vector<int32_t> *pages = nullptr;
};

// Several prompts in one pass (the arguments are already checked).  Their
// rows are laid end to end and cut into ubatches of n_ubatch rows; a ubatch
// row carries its own position and sequence, so the K|V projection writes
// each row into its own sequence's cache (or cells) and attention reads only
// that sequence's keys.  Pruning generalises the single-sequence rule to one
// output row per sequence: the ubatch that holds a prompt's last row gathers
// it after the owning layers, and the k gathered rows alone run the
// KV-shared layers (each against its own sequence's source-layer cache) and
// the head.  Without pruning they are gathered after the last layer.
// logits: fp32 [k][n_vocab].  u: the unified cache, or null (split caches).
int multi_pass(ppx_model *m, const SeqRun *sq, int k, const ppx_kvu *u, int nctx_max, bool prune,
               const ppx_prefill_params *p, void *ws, size_t ws_bytes, float *logits, hipStream_t s) {
    const ppx_model_info &I = m->info;
    const int L = I.n_layer, Ls = I.n_layer_kv_from_start, d = I.d_model, kvd = I.kv_dim;
    long T = 0;
    for (int q = 0; q < k; ++q) T += sq[q].n;
    const int npg = u ? u->n_cells / kKvPage : 0;
    const int ub = p->n_ubatch;
    const MultiLayout ML = multi_layout(m, ub, k, T, nctx_max, npg);
    if (ws_bytes < ML.total) return PPX_E_NOMEM;
    const int G = I.n_head / I.n_kv_head;
    const int cbw = attn_prefill_cols_per_wg(I.head_dim);
    if (G > cbw) return PPX_E_UNSUPPORTED;  // a one-row segment fits one column block

    // ---- the tables, built on the host
    uint8_t *hb = nullptr;
    PPX_TRY(stage_tables(m, ML.blob_bytes, &hb));
    auto H32 = [&](size_t off) { return reinterpret_cast<int32_t *>(hb + off); };
    int32_t *tok = H32(ML.tok), *pos = H32(ML.pos), *seq = H32(ML.seq);
    int32_t *ttok = H32(ML.ttok), *tpos = H32(ML.tpos), *tseq = H32(ML.tseq);
    std::vector<long> last(k);
    {
        long r = 0;
        for (int q = 0; q < k; ++q) {
            const SeqRun &sr = sq[q];
            for (int i = 0; i < sr.n; ++i, ++r) {
                tok[r] = sr.tok[i];
                pos[r] = sr.n_pos + i;
                seq[r] = q;
            }
            last[q] = r - 1;
            ttok[q] = sr.tok[sr.n - 1];
            tpos[q] = sr.n_pos + sr.n - 1;
            tseq[q] = q;
        }
    }
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    uint8_t *dblob = wsb + ML.blob;
    int32_t *pgt = H32(ML.pages);
    for (int q = 0; q < k && u; ++q) {
        const std::vector<int32_t> &pv = *sq[q].pages;
        std::copy(pv.begin(), pv.end(), pgt + (size_t)q * npg);
        std::fill(pgt + (size_t)q * npg + pv.size(), pgt + (size_t)(q + 1) * npg, 0);
    }
    KVRef *kvt = reinterpret_cast<KVRef *>(hb + ML.kv);
    for (int l = 0; l < Ls; ++l)
        for (int q = 0; q < k; ++q) {
            KVRef &ref = kvt[(size_t)l * k + q];
            if (u) {
                ref.k = u->k + (size_t)l * u->n_cells * kvd;
                ref.vt = u->vt + (size_t)l * kvd * u->n_cells;
                ref.vld = u->n_cells;
                ref.page = reinterpret_cast<const int32_t *>(dblob + ML.pages) + (size_t)q * npg;
            } else {
                const ppx_kv *kv = sq[q].kv;
                ref.k = kv->k + (size_t)l * kv->n_ctx * kvd;
                ref.vt = kv->vt + (size_t)l * kv->vld * kvd;
                ref.vld = kv->vld;
                ref.page = nullptr;
            }
            ref.pad = 0;
        }
    AttnWg *wgt = reinterpret_cast<AttnWg *>(hb + ML.wg);
    int2 *pairs = reinterpret_cast<int2 *>(hb + ML.pairs);
    struct Ub {
        long u0;
        int M;
        size_t wg0;
        int nwg;
        AttnSplit split;
        double vis;
        int pair0, npairs;
    };
    std::vector<Ub> ubs;
    size_t nw = 0;
    int np = 0;
    bool over = false;
    auto add_segment = [&](int row0, int Ms, int pos0, int q) {
        const int nb = (Ms * G + cbw - 1) / cbw;
        for (int b = 0; b < nb; ++b) {
            if (nw >= ML.max_wg) {
                over = true;
                return;
            }
            wgt[nw++] = AttnWg{row0, Ms, pos0, q, b, {0, 0, 0}};
        }
    };
    for (long u0 = 0; u0 < T; u0 += ub) {
        Ub U{};
        U.u0 = u0;
        U.M = (int)std::min<long>(ub, T - u0);
        U.wg0 = nw;
        U.pair0 = np;
        int P = 1;
        for (int r = 0; r < U.M;) {
            const int q = seq[u0 + r];
            int e = r + 1;
            while (e < U.M && seq[u0 + e] == q) ++e;
            const int Ms = e - r, p0 = pos[u0 + r];
            add_segment(r, Ms, p0, q);
            P = std::max(P, p0 + Ms);
            U.vis += (double)Ms * p0 + 0.5 * (double)Ms * (Ms + 1);
            if (last[q] < u0 + e) {
                if (np < k) pairs[np] = int2{(int)(last[q] - u0), q};
                ++np;
            }
            r = e;
        }
        U.nwg = (int)(nw - U.wg0);
        U.npairs = np - U.pair0;
        U.split = attn_split_cols(U.nwg, I.n_kv_head, P);
        ubs.push_back(U);
    }
    Ub tail{};
    tail.M = k;
    tail.wg0 = nw;
    {
        int P = 1;
        for (int q = 0; q < k; ++q) {
            add_segment(q, 1, tpos[q], q);
            P = std::max(P, tpos[q] + 1);
            tail.vis += tpos[q] + 1.0;
        }
        tail.nwg = (int)(nw - tail.wg0);
        tail.split = attn_split_cols(tail.nwg, I.n_kv_head, P);
    }
    if (over || np != k) return PPX_E_INVAL;  // cannot happen: the layout's bounds hold for any lengths

    if (hipMemcpyAsync(dblob, hb, ML.blob_bytes, hipMemcpyHostToDevice, s) != hipSuccess) return PPX_E_HIP;
    if (hipEventRecord(m->stage_event, s) != hipSuccess) return PPX_E_HIP;
    auto D32 = [&](size_t off) { return reinterpret_cast<const int32_t *>(dblob + off); };
    const KVRef *dkv = reinterpret_cast<const KVRef *>(dblob + ML.kv);
    const AttnWg *dwg = reinterpret_cast<const AttnWg *>(dblob + ML.wg);
    const int2 *dpairs = reinterpret_cast<const int2 *>(dblob + ML.pairs);
    float *xk = reinterpret_cast<float *>(wsb + ML.xk);

    Ctx c{m, nullptr, s, wsb, ML.w};
    c.exact = p->precision == PPX_PRECISION_EXACT;
    if (p->timing) {
        std::memset(p->timing, 0, sizeof(*p->timing));
        c.tm = p->timing;
    }
    if (log_enabled())
        std::fprintf(stderr, "[ppx] prefill of %d sequences, %ld rows, ubatch %d, prune %s, %s cache\n", k, T,
                     ub, prune ? "on" : "off", u ? "unified" : "split");
    // the launches (tables and tokens are already in device memory, so a
    // recorded sequence serves any prompts of the same shape)
    auto enqueue = [&](Ctx &c) -> int {
        const int full_layers = prune ? Ls : L;
        const int nub = (int)ubs.size();
        std::vector<Ctx::Rows> RU(nub);
        for (int j = 0; j < nub; ++j) {
            const Ub &U = ubs[j];
            Ctx::Rows &R = RU[j];
            R.tok = D32(ML.tok) + U.u0;
            R.pos = D32(ML.pos) + U.u0;
            R.seq = D32(ML.seq) + U.u0;
            R.kv = dkv;
            R.nseq = k;
            R.wg = dwg + U.wg0;
            R.nwg = U.nwg;
            R.split = U.split;
            R.vis = U.vis;
        }
        // the ubatches in lockstep, as in a single-sequence prefill: up to
        // nslots in flight, each step runs every one through its next layer
        // with one launch per operation; K|V of a step precede its attention,
        // and a ubatch never runs ahead of an earlier one, so every row sees
        // the keys of the serial order
        const int NU = c.exact ? 1 : std::max(1, std::min({nub, full_layers, c.L.nslots}));
        struct Flight {
            int u, il, slot;
        };
        std::vector<Flight> fl;
        std::vector<int> free_slots;
        for (int q = NU - 1; q >= 0; --q) free_slots.push_back(q);
        int next_u = 0;
        while (next_u < nub || !fl.empty()) {
            while ((int)fl.size() < NU && next_u < nub) {
                const int slot = free_slots.back();
                free_slots.pop_back();
                PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_embed(m->tok, RU[next_u].tok, ubs[next_u].M, m->embd_scale,
                                                            c.sl<float>(c.L.x, slot), c.s));
                fl.push_back({next_u, 0, slot});
                ++next_u;
            }
            Unit Us[kMaxUnits];
            const int nu = (int)fl.size();
            for (int i = 0; i < nu; ++i) Us[i] = Unit{fl[i].il, ubs[fl[i].u].M, 0, 0, fl[i].slot, &RU[fl[i].u]};
            PPX_TRY(layer_rows_group(c, Us, nu));
            for (int i = nu - 1; i >= 0; --i) {
                if (++fl[i].il < full_layers) continue;
                const Ub &U = ubs[fl[i].u];
                if (U.npairs)
                    PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_gather_rows(c.sl<float>(c.L.x, fl[i].slot), d,
                                                                      dpairs + U.pair0, U.npairs, xk, c.s));
                free_slots.push_back(fl[i].slot);
                fl.erase(fl.begin() + i);
            }
        }
        float *x = c.sl<float>(c.L.x, 0);
        PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_copy_f32(xk, x, k * d, c.s));
        Ctx::Rows R;
        R.tok = D32(ML.ttok);
        R.pos = D32(ML.tpos);
        R.seq = D32(ML.tseq);
        R.kv = dkv;
        R.nseq = k;
        R.wg = dwg + tail.wg0;
        R.nwg = tail.nwg;
        R.split = tail.split;
        R.vis = tail.vis;
        R.gathered = true;
        c.rows = &R;
        if (prune)
            for (int il = Ls; il < L; ++il) PPX_TRY(layer_rows(c, il, k, 0, 0));
        // the head of the k rows as one GEMM (the output matrix is read once)
        __half *a16 = c.sl<__half>(c.L.a16);
        PPX_LAUNCH(c, PPX_PHASE_OTHER, launch_rmsnorm_f16(x, m->out_norm, m->eps, k, d, a16, c.s));
        GemmArgs gh = c.gemm();
        gh.A = a16;
        gh.lda = d;
        gh.M = k;
        gh.W = m->out;
        gh.epi = EPI_F32;
        gh.out_f32 = logits;
        int st = PPX_OK;
        {
            hipEvent_t ev0 = c.begin();
            // exact precision keeps the head on the fp32-class single-row path
            st = c.exact ? PPX_E_UNSUPPORTED : launch_gemm(gh, c.s);
            if (st == PPX_E_UNSUPPORTED) {
                // an output width the MFMA tiles do not divide: one fp32 row at a time
                st = PPX_OK;
                for (int q = 0; q < k && st == PPX_OK; ++q) {
                    GemvArgs gv = gemv_base(c, x + (size_t)q * d, m->out, GV_F32, logits + (size_t)q * I.n_vocab);
                    gv.norm_g = m->out_norm;
                    gv.eps = m->eps;
                    st = launch_gemv(gv, c.s);
                }
            }
            PPX_TRY(st);
            c.end(PPX_PHASE_GEMM, ev0);
        }
        c.rows = nullptr;
        return PPX_OK;
    };
    if (!c.tm && graphs_enabled()) {
        std::vector<long long> key = {(long long)(uintptr_t)wsb, (long long)(uintptr_t)logits, T, ub, k, prune,
                                      nctx_max, (long long)ubs.size(), tail.nwg, tail.split.kc, tail.split.nkc,
                                      c.exact, npg};
        for (const Ub &U : ubs) {
            const long long v[] = {U.M, (long long)U.wg0, U.nwg, U.split.kc, U.split.nkc, U.pair0, U.npairs};
            key.insert(key.end(), v, v + 7);
        }
        PPX_TRY(run_keyed_graph(c, std::move(key), enqueue));
    } else {
        PPX_TRY(enqueue(c));
    }
    if (c.tm) c.tm->gemm_flop += 2.0 * k * (double)m->out.N * m->out.K;
    PPX_TRY(c.finish());
    return PPX_OK;
}

int prefill_multi(ppx_model *m, const ppx_seq *seqs, int k, const ppx_prefill_params *p, void *ws, size_t ws_bytes,
                  float *logits, hipStream_t s) {
    if (!m || !seqs || !p || !logits || !ws) return PPX_E_INVAL;
    if (k < 1 || k > PPX_MAX_SEQ) return PPX_E_INVAL;
    const ppx_model_info &I = m->info;
    if (p->embeddings != 0 || p->embeddings_layer_inp) return PPX_E_UNSUPPORTED;
    if (p->debug_rows || p->debug_hidden || p->nextn_logits) return PPX_E_UNSUPPORTED;
    if (p->n_seq_max < k) return PPX_E_INVAL;
    if (p->n_ubatch < 1 || p->n_ubatch > PPX_MAX_UBATCH) return PPX_E_INVAL;
    if (p->precision != PPX_PRECISION_FAST && p->precision != PPX_PRECISION_EXACT) return PPX_E_INVAL;
    int nctx_max = 1;
    for (int q = 0; q < k; ++q) {
        const ppx_seq &sq = seqs[q];
        if (!sq.kv || sq.kv->m != m) return PPX_E_INVAL;
        for (int r = 0; r < q; ++r)
            if (seqs[r].kv == sq.kv) return PPX_E_INVAL;  // each sequence needs its own cache
        if (sq.n_tokens <= 0) return PPX_E_EMPTY;
        if (!sq.tokens_host) return PPX_E_INVAL;
        for (int i = 0; i < sq.n_tokens; ++i)
            if (sq.tokens_host[i] < 0 || sq.tokens_host[i] >= I.n_vocab) return PPX_E_TOKEN;
        if ((long)sq.kv->n_pos + sq.n_tokens > sq.kv->n_ctx) return PPX_E_CTX;
        nctx_max = std::max(nctx_max, sq.kv->n_ctx);
    }
    if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return PPX_E_INVAL;
    if (k == 1) {
        // one sequence: exactly the single-sequence prefill
        ppx_prefill_params q1 = *p;
        q1.n_seq_max = 1;
        return prefill(m, seqs[0].kv, seqs[0].tokens_host, seqs[0].n_tokens, &q1, ws, ws_bytes, logits, s);
    }
    bool prune;
    PPX_TRY(multi_prune(m, p, &prune));
    std::vector<SeqRun> sr(k);
    for (int q = 0; q < k; ++q) sr[q] = SeqRun{seqs[q].tokens_host, seqs[q].n_tokens, seqs[q].kv->n_pos, seqs[q].kv};
    PPX_TRY(multi_pass(m, sr.data(), k, nullptr, nctx_max, prune, p, ws, ws_bytes, logits, s));
    for (int q = 0; q < k; ++q) seqs[q].kv->n_pos += seqs[q].n_tokens;
    return PPX_OK;
}

// Several prompts over one unified cache: each takes the pages its new
// positions need (lowest free first); they are committed to the sequence
// only once the pass has been queued.
int prefill_unified(ppx_model *m, ppx_kvu *u, const ppx_useq *seqs, int k, const ppx_prefill_params *p, void *ws,
                    size_t ws_bytes, float *logits, hipStream_t s) {
    if (!m || !u || !seqs || !p || !logits || !ws) return PPX_E_INVAL;
    if (u->m != m || k < 1 || k > PPX_MAX_SEQ) return PPX_E_INVAL;
    const ppx_model_info &I = m->info;
    if (p->embeddings != 0 || p->embeddings_layer_inp) return PPX_E_UNSUPPORTED;
    if (p->debug_rows || p->debug_hidden || p->nextn_logits) return PPX_E_UNSUPPORTED;
    if (p->n_seq_max < k) return PPX_E_INVAL;
    if (p->n_ubatch < 1 || p->n_ubatch > PPX_MAX_UBATCH) return PPX_E_INVAL;
    if (p->precision != PPX_PRECISION_FAST && p->precision != PPX_PRECISION_EXACT) return PPX_E_INVAL;
    long need = 0;
    for (int q = 0; q < k; ++q) {
        const ppx_useq &sq = seqs[q];
        if (sq.seq_id < 0 || sq.seq_id >= u->n_seq_max) return PPX_E_INVAL;
        for (int r = 0; r < q; ++r)
            if (seqs[r].seq_id == sq.seq_id) return PPX_E_INVAL;  // one prompt per sequence
        if (sq.n_tokens <= 0) return PPX_E_EMPTY;
        if (!sq.tokens_host) return PPX_E_INVAL;
        for (int i = 0; i < sq.n_tokens; ++i)
            if (sq.tokens_host[i] < 0 || sq.tokens_host[i] >= I.n_vocab) return PPX_E_TOKEN;
        const long end = (long)u->n_pos[sq.seq_id] + sq.n_tokens;
        if (end > u->n_cells) return PPX_E_CTX;
        need += (end + kKvPage - 1) / kKvPage - (long)u->pages[sq.seq_id].size();
    }
    if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return PPX_E_INVAL;
    std::vector<int32_t> freep;
    for (int pg = 0; pg < (int)u->page_seq.size() && (long)freep.size() < need; ++pg)
        if (u->page_seq[pg] < 0) freep.push_back(pg);
    if ((long)freep.size() < need) return PPX_E_CTX;
    bool prune;
    PPX_TRY(multi_prune(m, p, &prune));
    std::vector<std::vector<int32_t>> pv(k);
    std::vector<SeqRun> sr(k);
    size_t f = 0;
    for (int q = 0; q < k; ++q) {
        const ppx_useq &sq = seqs[q];
        pv[q] = u->pages[sq.seq_id];
        const int np = (u->n_pos[sq.seq_id] + sq.n_tokens + kKvPage - 1) / kKvPage;
        while ((int)pv[q].size() < np) pv[q].push_back(freep[f++]);
        sr[q] = SeqRun{sq.tokens_host, sq.n_tokens, u->n_pos[sq.seq_id], nullptr, &pv[q]};
    }
    PPX_TRY(multi_pass(m, sr.data(), k, u, u->n_cells, prune, p, ws, ws_bytes, logits, s));
    for (int q = 0; q < k; ++q) {
        const int sid = seqs[q].seq_id;
        for (size_t i = u->pages[sid].size(); i < pv[q].size(); ++i) u->page_seq[pv[q][i]] = sid;
        u->pages[sid] = std::move(pv[q]);
        u->n_pos[sid] += seqs[q].n_tokens;
    }
    return PPX_OK;
}

// ------------------------------------------------------------------ KVCP snapshots

// With tokens: the KVCP body is followed by a token section, "KVTK", int32
// count (= n_pos), then the count int32 token ids of the cached positions.
int kv_save(const ppx_kv *kv, const char *path, int n_pos, hipStream_t s, const int32_t *tokens = nullptr) {
    if (!kv || !path) return PPX_E_INVAL;
    if (n_pos < 0 || n_pos > kv->n_pos) return PPX_E_CTX;
    const ppx_model_info &I = kv->m->info;
    const int nl = I.n_layer_kv_from_start, kvd = I.kv_dim;
    const size_t row = (size_t)n_pos * kvd;
    std::vector<uint16_t> buf(2 * (size_t)nl * row);
    if (hipStreamSynchronize(s) != hipSuccess) return PPX_E_HIP;
    // V is held transposed on the device ([kvd][vld] per layer): back to
    // position-major rows in a temporary device buffer, then one copy
    uint16_t *vpos = nullptr;
    if (row && hipMalloc(&vpos, (size_t)nl * row * 2) != hipSuccess) return PPX_E_NOMEM;
    int st = PPX_OK;
    for (int il = 0; il < nl && row && st == PPX_OK; ++il) {
        const size_t src = (size_t)il * kv->n_ctx * kvd;
        if (hipMemcpy(buf.data() + il * row, kv->k + src, row * 2, hipMemcpyDeviceToHost) != hipSuccess)
            st = PPX_E_HIP;
        else
            st = launch_transpose_u16(reinterpret_cast<const uint16_t *>(kv->vt) + (size_t)il * kv->vld * kvd, kvd,
                                      n_pos, (size_t)kv->vld, vpos + (size_t)il * row, (size_t)kvd, s);
    }
    if (st == PPX_OK && row &&
        (hipStreamSynchronize(s) != hipSuccess ||
         hipMemcpy(buf.data() + (size_t)nl * row, vpos, (size_t)nl * row * 2, hipMemcpyDeviceToHost) != hipSuccess))
        st = PPX_E_HIP;
    if (vpos) (void)hipFree(vpos);
    if (st) return st;
    std::FILE *f = std::fopen(path, "wb");
    if (!f) return PPX_E_IO;
    const int32_t hdr[3] = {n_pos, nl, kvd};
    bool ok = std::fwrite("KVCP", 1, 4, f) == 4 && std::fwrite(hdr, 4, 3, f) == 3 &&
              std::fwrite(buf.data(), 2, buf.size(), f) == buf.size();
    if (ok && tokens) {
        const int32_t cnt = n_pos;
        ok = std::fwrite("KVTK", 1, 4, f) == 4 && std::fwrite(&cnt, 4, 1, f) == 1 &&
             std::fwrite(tokens, 4, (size_t)n_pos, f) == (size_t)n_pos;
    }
    ok = (std::fclose(f) == 0) && ok;
    return ok ? PPX_OK : PPX_E_IO;
}

// Validates a KVCP file; leaves *fpos = file positions when the header was read
// and *has_tokens = whether a token section follows the body.  The file is
// exactly the KVCP body, or the body and a token section of one id per
// cached position.
int kvfile_check(const char *path, int nl, int kvd, int n_pos, int n_ctx, int *fpos, bool *has_tokens = nullptr) {
    if (has_tokens) *has_tokens = false;
    std::FILE *f = std::fopen(path, "rb");
    if (!f) return PPX_E_IO;
    char mg[4];
    int32_t hdr[3];
    int st = PPX_OK;
    if (std::fread(mg, 1, 4, f) != 4 || std::memcmp(mg, "KVCP", 4) != 0 || std::fread(hdr, 4, 3, f) != 3) {
        st = PPX_E_FORMAT;
    } else {
        if (fpos) *fpos = hdr[0];
        // the body size in 64 bits without wrapping (the layer count and
        // width come from the model, the position count from the file)
        int64_t body = 0;
        const bool huge = nl <= 0 || kvd <= 0 || hdr[0] < 0 ||
                          __builtin_mul_overflow((int64_t)4 * nl, (int64_t)kvd, &body) ||
                          __builtin_mul_overflow(body, (int64_t)hdr[0], &body) || body > (int64_t)1 << 50;
        if (hdr[1] != nl || hdr[2] != kvd) {
            st = PPX_E_MISMATCH;
        } else if (huge) {
            st = PPX_E_FORMAT;
        } else {
            std::fseek(f, 0, SEEK_END);
            const int64_t sz = std::ftell(f);
            const int64_t want = 16 + body;
            bool tok = false;
            if (sz == want + 8 + 4ll * hdr[0]) {
                char tm[4];
                int32_t cnt = -1;
                std::fseek(f, want, SEEK_SET);
                tok = std::fread(tm, 1, 4, f) == 4 && std::memcmp(tm, "KVTK", 4) == 0 &&
                      std::fread(&cnt, 4, 1, f) == 1 && cnt == hdr[0];
            }
            if (has_tokens) *has_tokens = tok;
            if (sz != want && !tok) st = PPX_E_FORMAT;
            else if (n_pos < 0 || n_pos > hdr[0]) st = PPX_E_FORMAT;
            else if (n_pos > n_ctx) st = PPX_E_CTX;
        }
    }
    std::fclose(f);
    return st;
}

int kv_load(ppx_kv *kv, const char *path, int n_pos, hipStream_t s) {
    if (!kv || !path) return PPX_E_INVAL;
    kv->n_pos = 0;
    const ppx_model_info &I = kv->m->info;
    const int nl = I.n_layer_kv_from_start, kvd = I.kv_dim;
    int fpos = 0;
    int st = kvfile_check(path, nl, kvd, n_pos, kv->n_ctx, &fpos);
    if (st) {
        if (log_enabled()) std::fprintf(stderr, "[ppx] KV cache file %s rejected (%d)\n", path, st);
        return st;
    }
    std::FILE *f = std::fopen(path, "rb");
    if (!f) return PPX_E_IO;
    const size_t frow = (size_t)fpos * kvd, row = (size_t)n_pos * kvd;
    std::vector<uint16_t> buf(2 * (size_t)nl * row);
    for (int part = 0; part < 2 && row; ++part)
        for (int il = 0; il < nl; ++il) {
            std::fseek(f, 16 + (long)(((size_t)part * nl + il) * frow * 2), SEEK_SET);
            if (std::fread(buf.data() + ((size_t)part * nl + il) * row, 2, row, f) != row) st = PPX_E_IO;
        }
    std::fclose(f);
    if (st) return st;
    // V rows go up position-major into a temporary device buffer and are
    // transposed there into the cache's [kvd][vld] layout
    uint16_t *vpos = nullptr;
    if (row && hipMalloc(&vpos, (size_t)nl * row * 2) != hipSuccess) return PPX_E_NOMEM;
    if (row && hipMemcpyAsync(vpos, buf.data() + (size_t)nl * row, (size_t)nl * row * 2, hipMemcpyHostToDevice, s) !=
                   hipSuccess)
        st = PPX_E_HIP;
    for (int il = 0; il < nl && row && st == PPX_OK; ++il) {
        const size_t dst = (size_t)il * kv->n_ctx * kvd;
        if (hipMemcpyAsync(kv->k + dst, buf.data() + il * row, row * 2, hipMemcpyHostToDevice, s) != hipSuccess)
            st = PPX_E_HIP;
        else
            st = launch_transpose_u16(vpos + (size_t)il * row, n_pos, kvd, (size_t)kvd,
                                      reinterpret_cast<uint16_t *>(kv->vt) + (size_t)il * kv->vld * kvd,
                                      (size_t)kv->vld, s);
    }
    if (hipStreamSynchronize(s) != hipSuccess && st == PPX_OK) st = PPX_E_HIP;
    if (vpos) (void)hipFree(vpos);
    if (st) return st;
    kv->n_pos = n_pos;
    if (log_enabled())
        std::fprintf(stderr, "[ppx] snapshot %s: %d positions restored; the prefill resumes at position %d\n", path,
                     n_pos, n_pos);
    return PPX_OK;
}

// Token-verified prefix reuse: the longest common prefix of the snapshot's
// token ids and the new prompt, at most n_tokens - 1 positions (one token is
// left to prefill, which gives the logits), is loaded into the cache.
int kv_load_prefix(ppx_kv *kv, const char *path, const int32_t *tokens, int n_tokens, int *n_reused, hipStream_t s) {
    if (!kv || !path || !n_reused || (n_tokens > 0 && !tokens)) return PPX_E_INVAL;
    *n_reused = 0;
    kv->n_pos = 0;
    const ppx_model_info &I = kv->m->info;
    const int nl = I.n_layer_kv_from_start, kvd = I.kv_dim;
    int fpos = 0;
    bool has_tokens = false;
    const int st = kvfile_check(path, nl, kvd, 0, kv->n_ctx, &fpos, &has_tokens);
    if (st) return st;
    if (!has_tokens) return PPX_E_FORMAT;  // nothing to verify the prefix against
    std::vector<int32_t> ids((size_t)fpos);
    std::FILE *f = std::fopen(path, "rb");
    if (!f) return PPX_E_IO;
    std::fseek(f, 16 + 4l * nl * fpos * kvd + 8, SEEK_SET);
    const bool rd = std::fread(ids.data(), 4, (size_t)fpos, f) == (size_t)fpos;
    std::fclose(f);
    if (!rd) return PPX_E_IO;
    const int cap = std::min({fpos, n_tokens - 1, kv->n_ctx});
    int L = 0;
    while (L < cap && ids[(size_t)L] == tokens[L]) ++L;
    if (L == 0) return PPX_OK;
    PPX_TRY(kv_load(kv, path, L, s));
    *n_reused = L;
    return PPX_OK;
}

const Q4R *find_q4(const ppx_model *m, const char *name, int *kind) {
    if (!m || !name) return nullptr;
    auto it = m->q4.find(name);
    if (it == m->q4.end()) return nullptr;
    auto k = m->q4_kind.find(name);
    *kind = k == m->q4_kind.end() ? 0 : k->second;
    return &it->second;
}

}  // namespace
}  // namespace ppx

using namespace ppx;

// ====================================================================== C ABI

extern "C" {

int ppx_model_load(const void *container, size_t bytes, void *hip_stream, ppx_model **out) {
    if (!container || !out) return PPX_E_INVAL;
    *out = nullptr;
    return model_load(static_cast<const uint8_t *>(container), bytes, (hipStream_t)hip_stream, nullptr, 0, nullptr,
                      out);
}

size_t ppx_model_weight_bytes(const void *container, size_t bytes) {
    if (!container) return 0;
    size_t need = 0;
    if (model_load(static_cast<const uint8_t *>(container), bytes, nullptr, nullptr, 0, &need, nullptr) != PPX_OK)
        return 0;
    return need;
}

int ppx_model_load_into(const void *container, size_t bytes, void *weights_dev, size_t weights_bytes,
                        void *hip_stream, ppx_model **out) {
    if (!container || !out || !weights_dev) return PPX_E_INVAL;
    *out = nullptr;
    return model_load(static_cast<const uint8_t *>(container), bytes, (hipStream_t)hip_stream, weights_dev,
                      weights_bytes, nullptr, out);
}

int ppx_model_load_file(const char *path, void *hip_stream, ppx_model **out) {
    if (!path || !out) return PPX_E_INVAL;
    *out = nullptr;
    std::ifstream f(path, std::ios::binary | std::ios::ate);
    if (!f) return PPX_E_IO;
    const std::streamsize n = f.tellg();
    if (n <= 0) return PPX_E_IO;
    std::vector<uint8_t> buf((size_t)n);
    f.seekg(0);
    if (!f.read(reinterpret_cast<char *>(buf.data()), n)) return PPX_E_IO;
    return model_load(buf.data(), buf.size(), (hipStream_t)hip_stream, nullptr, 0, nullptr, out);
}

void ppx_model_free(ppx_model *m) { model_free(m); }

int ppx_model_get_info(const ppx_model *m, ppx_model_info *out) {
    if (!m || !out) return PPX_E_INVAL;
    *out = m->info;
    return PPX_OK;
}

size_t ppx_model_device_bytes(const ppx_model *m) { return m ? m->dev_bytes : 0; }

static int kv_vld(int n_ctx) { return (n_ctx + 63) / 64 * 64; }

size_t ppx_kv_bytes(const ppx_model *m, int n_ctx) {
    if (!m || n_ctx <= 0) return 0;
    const size_t ls = m->info.n_layer_kv_from_start, kvd = m->info.kv_dim;
    const size_t kbytes = (ls * (size_t)n_ctx * kvd * 2 + 255) / 256 * 256;
    return kbytes + ls * kvd * (size_t)kv_vld(n_ctx) * 2;
}

int ppx_kv_init(ppx_model *m, void *kv_dev, size_t bytes, int n_ctx, ppx_kv **out) {
    if (!m || !out || n_ctx <= 0) return PPX_E_INVAL;
    *out = nullptr;
    const size_t need = ppx_kv_bytes(m, n_ctx);
    if (need && !kv_dev) return PPX_E_INVAL;
    if (bytes < need) return PPX_E_NOMEM;
    if ((reinterpret_cast<uintptr_t>(kv_dev) & 255) != 0) return PPX_E_INVAL;
    PPX_TRY(ensure_rope(m, n_ctx));
    // a fresh cache holds zeros; the attention kernels never use a value
    // past the last written position (after kv_clear or a shorter kv_load the
    // old contents stay, and are masked or zeroed in the kernels)
    if (need && hipMemset(kv_dev, 0, need) != hipSuccess) return PPX_E_HIP;
    ppx_kv *kv = new ppx_kv();
    kv->m = m;
    const size_t kbytes = ((size_t)m->info.n_layer_kv_from_start * n_ctx * m->info.kv_dim * 2 + 255) / 256 * 256;
    kv->k = static_cast<__half *>(kv_dev);
    kv->vt = reinterpret_cast<__half *>(static_cast<uint8_t *>(kv_dev) + kbytes);
    kv->vld = kv_vld(n_ctx);
    kv->n_ctx = n_ctx;
    *out = kv;
    return PPX_OK;
}

void ppx_kv_free(ppx_kv *kv) { delete kv; }
int ppx_kv_n_pos(const ppx_kv *kv) { return kv ? kv->n_pos : PPX_E_INVAL; }
int ppx_kv_n_ctx(const ppx_kv *kv) { return kv ? kv->n_ctx : PPX_E_INVAL; }
int ppx_kv_clear(ppx_kv *kv) {
    if (!kv) return PPX_E_INVAL;
    kv->n_pos = 0;
    return PPX_OK;
}

int ppx_kv_save(const ppx_kv *kv, const char *path, int n_pos, void *hip_stream) {
    return kv_save(kv, path, n_pos, (hipStream_t)hip_stream);
}

int ppx_kv_load(ppx_kv *kv, const char *path, int n_pos, void *hip_stream) {
    return kv_load(kv, path, n_pos, (hipStream_t)hip_stream);
}

int ppx_kv_save_tokens(const ppx_kv *kv, const char *path, int n_pos, const int32_t *tokens_host, void *hip_stream) {
    if (!tokens_host && n_pos > 0) return PPX_E_INVAL;
    return kv_save(kv, path, n_pos, (hipStream_t)hip_stream, tokens_host ? tokens_host : reinterpret_cast<const int32_t *>(""));
}

int ppx_kv_load_prefix(ppx_kv *kv, const char *path, const int32_t *tokens_host, int n_tokens, int *n_reused,
                       void *hip_stream) {
    return kv_load_prefix(kv, path, tokens_host, n_tokens, n_reused, (hipStream_t)hip_stream);
}

int ppx_kvfile_validate(const char *path, int n_layers, int kv_dim, int n_pos, int n_ctx, int *file_n_pos) {
    if (!path) return PPX_E_INVAL;
    return kvfile_check(path, n_layers, kv_dim, n_pos, n_ctx, file_n_pos);
}

size_t ppx_workspace_bytes(const ppx_model *m, int n_ubatch, int n_ctx) {
    if (!m || n_ubatch < 1 || n_ctx < 1) return 0;
    return ws_layout(m, n_ubatch, n_ctx, prefill_slots(m, n_ubatch, n_ctx)).total;
}

int ppx_prefill(ppx_model *m, ppx_kv *kv, const int32_t *tokens_host, int n_tokens, const ppx_prefill_params *p,
                void *ws_dev, size_t ws_bytes, float *logits_dev, void *hip_stream) {
    return prefill(m, kv, tokens_host, n_tokens, p, ws_dev, ws_bytes, logits_dev, (hipStream_t)hip_stream);
}

size_t ppx_workspace_bytes_multi(const ppx_model *m, int n_ubatch, int n_seq, long n_tokens_total, int n_ctx_max) {
    if (!m || n_ubatch < 1 || n_seq < 1 || n_seq > PPX_MAX_SEQ || n_tokens_total < 1 || n_ctx_max < 1) return 0;
    const size_t one = ws_layout(m, n_ubatch, n_ctx_max, prefill_slots(m, n_ubatch, n_ctx_max)).total;
    return std::max(one, multi_layout(m, n_ubatch, n_seq, n_tokens_total, n_ctx_max).total);
}

int ppx_prefill_multi(ppx_model *m, const ppx_seq *seqs, int n_seq, const ppx_prefill_params *p, void *ws_dev,
                      size_t ws_bytes, float *logits_dev, void *hip_stream) {
    return prefill_multi(m, seqs, n_seq, p, ws_dev, ws_bytes, logits_dev, (hipStream_t)hip_stream);
}

size_t ppx_kvu_bytes(const ppx_model *m, int n_cells) {
    if (!m || n_cells <= 0 || n_cells % kKvPage) return 0;
    const size_t ls = m->info.n_layer_kv_from_start, kvd = m->info.kv_dim;
    const size_t kbytes = (ls * (size_t)n_cells * kvd * 2 + 255) / 256 * 256;
    return kbytes + ls * kvd * (size_t)n_cells * 2;
}

int ppx_kvu_init(ppx_model *m, void *kv_dev, size_t bytes, int n_cells, int n_seq_max, ppx_kvu **out) {
    if (!m || !out) return PPX_E_INVAL;
    *out = nullptr;
    if (n_cells <= 0 || n_cells % kKvPage || n_seq_max < 1 || n_seq_max > 65536) return PPX_E_INVAL;
    const size_t need = ppx_kvu_bytes(m, n_cells);
    if (need && !kv_dev) return PPX_E_INVAL;
    if (bytes < need) return PPX_E_NOMEM;
    if ((reinterpret_cast<uintptr_t>(kv_dev) & 255) != 0) return PPX_E_INVAL;
    PPX_TRY(ensure_rope(m, n_cells));
    if (need && hipMemset(kv_dev, 0, need) != hipSuccess) return PPX_E_HIP;
    ppx_kvu *u = new ppx_kvu();
    u->m = m;
    const size_t kbytes = ((size_t)m->info.n_layer_kv_from_start * n_cells * m->info.kv_dim * 2 + 255) / 256 * 256;
    u->k = static_cast<__half *>(kv_dev);
    u->vt = reinterpret_cast<__half *>(static_cast<uint8_t *>(kv_dev) + kbytes);
    u->n_cells = n_cells;
    u->n_seq_max = n_seq_max;
    u->page_seq.assign(n_cells / kKvPage, -1);
    u->pages.resize(n_seq_max);
    u->n_pos.assign(n_seq_max, 0);
    *out = u;
    return PPX_OK;
}

void ppx_kvu_free(ppx_kvu *u) { delete u; }

int ppx_kvu_n_pos(const ppx_kvu *u, int seq_id) {
    if (!u || seq_id < 0 || seq_id >= u->n_seq_max) return PPX_E_INVAL;
    return u->n_pos[seq_id];
}

int ppx_kvu_free_cells(const ppx_kvu *u) {
    if (!u) return PPX_E_INVAL;
    return (int)std::count(u->page_seq.begin(), u->page_seq.end(), -1) * kKvPage;
}

int ppx_kvu_seq_rm(ppx_kvu *u, int seq_id) {
    if (!u || seq_id < 0 || seq_id >= u->n_seq_max) return PPX_E_INVAL;
    for (int32_t pg : u->pages[seq_id]) u->page_seq[pg] = -1;
    u->pages[seq_id].clear();
    u->n_pos[seq_id] = 0;
    return PPX_OK;
}

int ppx_kvu_cells(const ppx_kvu *u, int seq_id, int32_t *cells_host, int n) {
    if (!u || seq_id < 0 || seq_id >= u->n_seq_max || n < 0 || n > u->n_pos[seq_id] || (n && !cells_host))
        return PPX_E_INVAL;
    for (int p = 0; p < n; ++p) cells_host[p] = kv_cell(u->pages[seq_id].data(), p);
    return PPX_OK;
}

size_t ppx_workspace_bytes_unified(const ppx_model *m, int n_ubatch, int n_seq, long n_tokens_total, int n_cells) {
    if (!m || n_ubatch < 1 || n_seq < 1 || n_seq > PPX_MAX_SEQ || n_tokens_total < 1 || n_cells < kKvPage ||
        n_cells % kKvPage)
        return 0;
    return multi_layout(m, n_ubatch, n_seq, n_tokens_total, n_cells, n_cells / kKvPage).total;
}

int ppx_prefill_unified(ppx_model *m, ppx_kvu *u, const ppx_useq *seqs, int n_seq, const ppx_prefill_params *p,
                        void *ws_dev, size_t ws_bytes, float *logits_dev, void *hip_stream) {
    return prefill_unified(m, u, seqs, n_seq, p, ws_dev, ws_bytes, logits_dev, (hipStream_t)hip_stream);
}

int ppx_decode(ppx_model *m, ppx_kv *kv, int32_t token, void *ws_dev, size_t ws_bytes, float *logits_dev,
               void *hip_stream) {
    return decode(m, kv, token, ws_dev, ws_bytes, logits_dev, (hipStream_t)hip_stream);
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free decode
// The workspace of ppx_decode_static lives in a file-scope device array: each
// GPU that loads the library holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address of the current GPU's copy is looked up once per device
// with hipGetSymbolAddress and used everywhere instead.
constexpr size_t kStaticScratchBytes = 32ull << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of the current device's scratch array (looked up on the
// first call on that device), or null if the lookup fails.
void *static_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int ppx_decode_static(ppx_model *m, ppx_kv *kv, int32_t token, float *logits_dev, void *hip_stream) {
    if (!m || !kv) return PPX_E_INVAL;
    if (kv->m != m) return PPX_E_INVAL;
    if (ws_layout(m, 1, kv->n_ctx, 1).total > kStaticScratchBytes) return PPX_E_NOMEM;
    void *ws = static_scratch();
    if (!ws) return PPX_E_HIP;
    return decode(m, kv, token, ws, kStaticScratchBytes, logits_dev, (hipStream_t)hip_stream);
}

size_t ppx_decode_static_limit(void) { return kStaticScratchBytes; }

int ppx_prune_predicate(int n_layer, int n_layer_kv_from_start, int embeddings, int n_seq_max,
                        const uint8_t *embeddings_layer_inp, int crop_before_nextn) {
    return predicate(n_layer, n_layer_kv_from_start, embeddings, n_seq_max, embeddings_layer_inp, crop_before_nextn);
}

int ppx_op_dequant(const ppx_model *m, const char *tensor, float *out_dev, void *hip_stream) {
    int kind;
    const Q4R *w = find_q4(m, tensor, &kind);
    if (!w || !out_dev) return PPX_E_INVAL;
    return launch_dequant(*w, out_dev, (hipStream_t)hip_stream);
}

size_t ppx_op_gemm_workspace_bytes(const ppx_model *m, const char *tensor, int M) {
    int kind;
    const Q4R *w = find_q4(m, tensor, &kind);
    if (!w || M <= 0) return 0;
    return 4 * gemm_part_floats(M, w->N, w->K);
}

int ppx_op_gemm(const ppx_model *m, const char *tensor, const void *a_dev_f16, int M, float *c_dev, void *ws_dev,
                size_t ws_bytes, void *hip_stream) {
    int kind;
    const Q4R *w = find_q4(m, tensor, &kind);
    if (!w || !a_dev_f16 || !c_dev || M < 0) return PPX_E_INVAL;
    if (kind == 3) return PPX_E_INVAL;  // exact-weight tensors go through ppx_op_gemm_exact
    GemmArgs g;
    g.part = static_cast<float *>(ws_dev);
    g.part_floats = ws_dev ? ws_bytes / 4 : 0;
    g.A = static_cast<const __half *>(a_dev_f16);
    g.lda = w->K;
    g.M = M;
    g.W = *w;
    g.epi = EPI_F32;
    g.out_f32 = c_dev;
    return launch_gemm(g, (hipStream_t)hip_stream);
}

int ppx_op_gemm_glu(const ppx_model *m, const char *tensor, const void *a_dev_f16, int M, void *h_dev_f16,
                    void *ws_dev, size_t ws_bytes, void *hip_stream) {
    int kind;
    const Q4R *w = find_q4(m, tensor, &kind);
    if (!w || kind != 2 || !a_dev_f16 || !h_dev_f16 || M < 0) return PPX_E_INVAL;
    GemmArgs g;
    g.part = static_cast<float *>(ws_dev);
    g.part_floats = ws_dev ? ws_bytes / 4 : 0;
    g.A = static_cast<const __half *>(a_dev_f16);
    g.lda = w->K;
    g.M = M;
    g.W = *w;
    g.epi = EPI_GLU;
    g.out_f16 = static_cast<__half *>(h_dev_f16);
    g.act = m->info.act;
    return launch_gemm(g, (hipStream_t)hip_stream);
}

int ppx_op_stream_read(const void *src_dev, size_t bytes, uint32_t *xor_dev, int n_workgroups, void *hip_stream) {
    if (!src_dev || !xor_dev || bytes == 0 || bytes % 1024 || n_workgroups < 1 || n_workgroups > 65536 ||
        (reinterpret_cast<uintptr_t>(src_dev) & 15) != 0)
        return PPX_E_INVAL;
    return launch_stream_read(src_dev, bytes, xor_dev, n_workgroups, (hipStream_t)hip_stream);
}

int ppx_op_tile_f16(const void *src_dev, int M, int K, void *dst_dev, void *hip_stream) {
    if (!src_dev || !dst_dev || M < 0 || K <= 0) return PPX_E_INVAL;
    return launch_tile_f16(static_cast<const __half *>(src_dev), M, K, static_cast<__half *>(dst_dev),
                           (hipStream_t)hip_stream);
}

int ppx_op_gemm_exact(const ppx_model *m, const char *tensor, const void *a_hi, const void *a_lo, int M,
                      float *c_dev, void *hip_stream) {
    int kind;
    const Q4R *w = find_q4(m, tensor, &kind);
    if (!w || !a_hi || !a_lo || !c_dev || M < 0) return PPX_E_INVAL;
    GemmArgs g;
    g.A = static_cast<const __half *>(a_hi);
    g.A2 = static_cast<const __half *>(a_lo);
    g.lda = w->K;
    g.M = M;
    g.W = *w;
    g.epi = EPI_F32;
    g.out_f32 = c_dev;
    return launch_gemm_exact(g, (hipStream_t)hip_stream);
}

int ppx_op_gemv(const ppx_model *m, const char *tensor, const float *x_dev, float *y_dev, void *hip_stream) {
    int kind;
    const Q4R *w = find_q4(m, tensor, &kind);
    if (!w || !x_dev || !y_dev) return PPX_E_INVAL;
    GemvArgs a;
    a.x = x_dev;
    a.W = *w;
    a.epi = GV_F32;
    a.out = y_dev;
    return launch_gemv(a, (hipStream_t)hip_stream);
}

int ppx_op_attention(const ppx_model *m, const void *q_dev, const void *k_dev, const void *vt_dev, int vld, int M,
                     int pos0, void *o_dev, void *ws_dev, size_t ws_bytes, void *hip_stream) {
    if (!m || !q_dev || !k_dev || !vt_dev || !o_dev || !ws_dev || M < 1 || pos0 < 0 || M > PPX_MAX_UBATCH)
        return PPX_E_INVAL;
    if (vld % 64 || vld < pos0 + M) return PPX_E_INVAL;
    const WsLayout L = ws_layout(m, M, pos0 + M, 1);
    if (ws_bytes < L.total) return PPX_E_NOMEM;
    AttnArgs a;
    a.q = static_cast<const __half *>(q_dev);
    a.k = static_cast<const __half *>(k_dev);
    a.vt = static_cast<const __half *>(vt_dev);
    a.vld = vld;
    a.o = static_cast<__half *>(o_dev);
    a.M = M;
    a.H = m->info.n_head;
    a.KVH = m->info.n_kv_head;
    a.hd = m->info.head_dim;
    a.pos0 = pos0;
    a.part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws_dev) + L.ap_part);
    return launch_attn_prefill(a, (hipStream_t)hip_stream);
}

int ppx_op_attention_1row(const ppx_model *m, const float *q_dev, const void *k_dev, const void *vt_dev, int vld,
                          int pos, float *o_dev, void *ws_dev, size_t ws_bytes, void *hip_stream) {
    if (!m || !q_dev || !k_dev || !vt_dev || !o_dev || !ws_dev || pos < 0) return PPX_E_INVAL;
    if (vld % 64 || vld <= pos) return PPX_E_INVAL;
    const WsLayout L = ws_layout(m, 1, pos + 1, 1);
    if (ws_bytes < L.total) return PPX_E_NOMEM;
    uint8_t *ws = static_cast<uint8_t *>(ws_dev);
    hipStream_t s = (hipStream_t)hip_stream;
    Attn1Args a;
    a.q = q_dev;
    a.k = static_cast<const __half *>(k_dev);
    a.vt = static_cast<const __half *>(vt_dev);
    a.vld = vld;
    a.o = o_dev;
    a.H = m->info.n_head;
    a.KVH = m->info.n_kv_head;
    a.hd = m->info.head_dim;
    a.pos = pos;
    a.partial = reinterpret_cast<float *>(ws + L.at_part);
    return launch_attn_1row(a, s);
}

const char *ppx_status_str(int st) {
    switch (st) {
    case PPX_OK: return "ok";
    case PPX_E_INVAL: return "invalid argument";
    case PPX_E_TOKEN: return "token id out of range";
    case PPX_E_CTX: return "context length exceeded";
    case PPX_E_IO: return "i/o error";
    case PPX_E_FORMAT: return "bad file format";
    case PPX_E_MISMATCH: return "snapshot does not match the model";
    case PPX_E_UNSUPPORTED: return "unsupported shape or option";
    case PPX_E_HIP: return "HIP runtime error";
    case PPX_E_NOMEM: return "out of memory / buffer too small";
    case PPX_E_EMPTY: return "empty prompt";
    default: return "unknown status";
    }
}

}  // extern "C"
