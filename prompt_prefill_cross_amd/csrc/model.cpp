// Model container parsing, Q4_0 repacking and upload.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <memory>
#include <thread>
#include <string>
#include <vector>

#include "ppx_internal.h"

namespace ppx {

bool log_enabled() {
    static const bool on = std::getenv("PPX_LOG") != nullptr;
    return on;
}

namespace {

constexpr uint64_t kHeader = 128, kEntry = 96;

struct Parsed {
    int32_t h[12];
    float eps, base, escale;
    std::vector<int32_t> src;
    std::vector<float> ple_s;
    std::unordered_map<std::string, HostTensor> t;
};

int parse(const uint8_t *b, size_t n, Parsed &p) {
    if (n < kHeader || std::memcmp(b, "PPXM", 4) != 0) return PPX_E_FORMAT;
    uint32_t ver;
    std::memcpy(&ver, b + 4, 4);
    if (ver != 1) return PPX_E_FORMAT;
    std::memcpy(p.h, b + 8, sizeof(p.h));
    std::memcpy(&p.eps, b + 56, 4);
    std::memcpy(&p.base, b + 60, 4);
    std::memcpy(&p.escale, b + 64, 4);
    const int L = p.h[0], nt = p.h[11];
    if (L <= 0 || L > 4096 || nt <= 0 || nt > 1 << 20) return PPX_E_FORMAT;
    const uint64_t toff = (kHeader + 8ull * L + 63) / 64 * 64;
    if (toff + kEntry * (uint64_t)nt > n) return PPX_E_FORMAT;
    p.src.resize(L);
    p.ple_s.resize(L);
    std::memcpy(p.src.data(), b + kHeader, 4ull * L);
    std::memcpy(p.ple_s.data(), b + kHeader + 4ull * L, 4ull * L);
    for (int i = 0; i < nt; ++i) {
        const uint8_t *e = b + toff + kEntry * i;
        char name[65];
        std::memcpy(name, e, 64);
        name[64] = 0;
        HostTensor ht;
        uint32_t tt;
        std::memcpy(&tt, e + 64, 4);
        std::memcpy(&ht.rows, e + 72, 8);
        std::memcpy(&ht.cols, e + 80, 8);
        std::memcpy(&ht.offset, e + 88, 8);
        ht.type = (int)tt;
        if (tt > 1) return PPX_E_FORMAT;
        if (tt == 1 && ht.cols % 32) return PPX_E_FORMAT;
        // sizes in 64 bits without wrapping: a tensor must lie inside the container
        uint64_t nb = 0;
        const uint64_t per = tt == 0 ? 4 : 18, units = tt == 0 ? ht.cols : ht.cols / 32;
        if (__builtin_mul_overflow(ht.rows, units, &nb) || __builtin_mul_overflow(nb, per, &nb)) return PPX_E_FORMAT;
        if (ht.offset > n || nb > n - ht.offset) return PPX_E_FORMAT;
        p.t[name] = ht;
    }
    return PPX_OK;
}

// Device-side arena: sizes are planned first, then one allocation.
struct Arena {
    size_t used = 0;
    size_t take(size_t bytes) {
        const size_t off = used;
        used += (bytes + 255) / 256 * 256;
        return off;
    }
};

// A repack job: output rows of a Q4R matrix, each taken from a raw source row.
struct RepackJob {
    std::vector<const uint8_t *> rows;  // raw Q4_0 row (first block) per output row
    int N = 0, K = 0;
    size_t nib_off = 0, scl_off = 0;
};

template <typename F>
void parallel_rows(int n, F &&f) {
    const int nt = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    if (n < 256 || nt == 1) {
        f(0, n);
        return;
    }
    std::vector<std::thread> th;
    const int per = (n + nt - 1) / nt;
    for (int t = 0; t < nt; ++t) {
        const int a = t * per, b = std::min(n, a + per);
        if (a < b) th.emplace_back([&f, a, b] { f(a, b); });
    }
    for (auto &x : th) x.join();
}

void repack_rows(const RepackJob &j, uint8_t *host) {
    uint32_t *nib = reinterpret_cast<uint32_t *>(host + j.nib_off);
    uint16_t *scl = reinterpret_cast<uint16_t *>(host + j.scl_off);
    const int kblocks = j.K / 32, kch = j.K / 64;
    parallel_rows(j.N, [&](int n0, int n1) {
    for (int n = n0; n < n1; ++n) {
        const uint8_t *row = j.rows[n];
        const int grp = n >> 4, col = n & 15;
        for (int kb = 0; kb < kblocks; ++kb) {
            const uint8_t *blk = row + (size_t)kb * 18;
            const int kc = kb >> 1, s = kb & 1;
            const size_t base = (size_t)grp * kch + kc;
            scl[(base * 16 + col) * 2 + s] = (uint16_t)(blk[0] | (blk[1] << 8));
            uint8_t codes[32];
            for (int q = 0; q < 16; ++q) {
                codes[q] = blk[2 + q] & 15;
                codes[q + 16] = blk[2 + q] >> 4;
            }
            for (int g = 0; g < 4; ++g) {
                uint32_t w = 0;
                for (int e = 0; e < 8; ++e) {
                    const int sh = (e & 1) ? 16 + 4 * (e >> 1) : 4 * (e >> 1);
                    w |= (uint32_t)codes[8 * g + e] << sh;
                }
                nib[(base * 64 + g * 16 + col) * 2 + s] = w;
            }
        }
    }
    });
}

}  // namespace

// weights_dev: caller-owned device memory of weights_bytes bytes for the
// repacked weights (null: the library allocates it).  With out == null only
// the layout is planned and *need_bytes receives its size; nothing touches
// the GPU.
int model_load(const uint8_t *b, size_t n, hipStream_t stream, void *weights_dev, size_t weights_bytes,
               size_t *need_bytes, ppx_model **out) {
    Parsed p;
    int st = parse(b, n, p);
    if (st) return st;
    std::unique_ptr<ppx_model> m(new ppx_model());
    ppx_model_info &I = m->info;
    I.n_layer = p.h[0];
    I.n_layer_kv_from_start = p.h[1];
    I.d_model = p.h[2];
    I.n_head = p.h[3];
    I.n_kv_head = p.h[4];
    I.head_dim = p.h[5];
    I.n_ff = p.h[6];
    I.n_vocab = p.h[7];
    I.ple_dim = p.h[8];
    I.act = p.h[9];
    // every dimension is bounded before any product of them is formed
    for (int k = 1; k <= 8; ++k)
        if (p.h[k] < 0 || p.h[k] > (1 << 20)) return PPX_E_FORMAT;
    if ((int64_t)p.h[3] * p.h[5] > (1 << 24) || (int64_t)p.h[4] * p.h[5] > (1 << 24) ||
        (int64_t)p.h[0] * p.h[8] > (1 << 24))
        return PPX_E_FORMAT;
    I.kv_dim = I.n_kv_head * I.head_dim;
    m->tied = p.h[10];
    m->eps = p.eps;
    m->rope_base = p.base;
    m->embd_scale = p.escale;
    const int L = I.n_layer, Ls = I.n_layer_kv_from_start, d = I.d_model, hd = I.head_dim;
    const int qd = I.n_head * hd, kvd = I.kv_dim, F = I.n_ff, E = I.ple_dim, V = I.n_vocab;
    if (Ls < 0 || Ls > L || d <= 0 || I.n_head <= 0 || I.n_kv_head <= 0 || V <= 0 || F <= 0 || E < 0 ||
        I.act < 0 || I.act > 1)
        return PPX_E_FORMAT;
    if (d % 256 || qd % 256 || F % 256 || E % 256 || (hd != 64 && hd != 128 && hd != 256) ||
        I.n_head % I.n_kv_head || V % 32 || (I.n_head / I.n_kv_head) > 8 || kvd % 32)
        return PPX_E_UNSUPPORTED;
    for (int il = 0; il < L; ++il) {
        const int s = p.src[il];
        if (il < Ls ? s != il : (s < 0 || s >= Ls)) return PPX_E_FORMAT;
    }

    auto need = [&](const std::string &name, int type, uint64_t rows, uint64_t cols) -> const HostTensor * {
        auto it = p.t.find(name);
        if (it == p.t.end()) return nullptr;
        const HostTensor &t = it->second;
        if (t.type != type || t.rows != rows || t.cols != cols) return nullptr;
        return &t;
    };
    auto rowp = [&](const HostTensor *t, uint64_t r) { return b + t->offset + r * (t->cols / 32) * 18; };

    Arena ar;
    std::vector<RepackJob> jobs;
    struct F32Slot { const float **dst; size_t off; const HostTensor *t; };
    std::vector<F32Slot> f32s;
    struct Slot { Q4R *q; size_t job; };
    std::vector<Slot> slots;

    auto plan_q4 = [&](Q4R &q, RepackJob &&j) {
        j.nib_off = ar.take((size_t)j.N * j.K / 2);
        j.scl_off = ar.take((size_t)j.N * j.K / 32 * 2);
        q.N = j.N;
        q.K = j.K;
        jobs.push_back(std::move(j));
        slots.push_back({&q, jobs.size() - 1});
    };
    auto plain = [&](Q4R &q, const HostTensor *t) -> int {
        if (!t) return PPX_E_FORMAT;
        RepackJob j;
        j.N = (int)t->rows;
        j.K = (int)t->cols;
        j.rows.resize(j.N);
        for (int r = 0; r < j.N; ++r) j.rows[r] = rowp(t, r);
        plan_q4(q, std::move(j));
        return PPX_OK;
    };
    auto plan_f32 = [&](const float *&ptr, const HostTensor *t) -> int {
        if (!t) return PPX_E_FORMAT;
        f32s.push_back({&ptr, ar.take(t->cols * 4), t});
        return PPX_OK;
    };
    // rope-pair order: 16-row blocks alternate first-half / second-half of each head
    auto rope_row = [&](int r) {
        const int h = r / hd, rr = r % hd;
        const int blk = rr / 16, c = rr % 16;
        return h * hd + (blk & 1) * (hd / 2) + (blk >> 1) * 16 + c;
    };

    const HostTensor *tok = need("tok_embd", 1, V, d);
    if ((st = plain(m->tok, tok))) return st;
    const HostTensor *outw = nullptr;
    if (!m->tied) {
        outw = need("output", 1, V, d);
        if ((st = plain(m->out, outw))) return st;
    }
    if ((st = plan_f32(m->out_norm, need("output_norm", 0, 1, d)))) return st;
    if (p.t.count("nextn_norm")) {
        if ((st = plan_f32(m->nextn_norm, need("nextn_norm", 0, 1, d)))) return st;
        I.has_nextn = 1;
    }
    size_t ple_off = 0;
    const HostTensor *ple = nullptr;
    if (E) {
        ple = need("ple_table", 1, V, (uint64_t)L * E);
        if (!ple) return PPX_E_FORMAT;
        ple_off = ar.take((size_t)V * (L * E / 32) * 18);
    }
    m->layers.resize(L);
    for (int il = 0; il < L; ++il) {
        LayerW &lw = m->layers[il];
        const std::string pf = "blk." + std::to_string(il) + ".";
        lw.own = il < Ls;
        lw.src = p.src[il];
        lw.ple_s = p.ple_s[il];
        if ((st = plan_f32(lw.attn_norm, need(pf + "attn_norm", 0, 1, d)))) return st;
        if ((st = plan_f32(lw.ffn_norm, need(pf + "ffn_norm", 0, 1, d)))) return st;
        const HostTensor *wq = need(pf + "wq", 1, qd, d);
        if (!wq) return PPX_E_FORMAT;
        RepackJob jq;
        jq.K = d;
        for (int r = 0; r < qd; ++r) jq.rows.push_back(rowp(wq, rope_row(r)));
        jq.N = qd;
        plan_q4(lw.wq, std::move(jq));
        if (lw.own) {
            const HostTensor *wk = need(pf + "wk", 1, kvd, d), *wv = need(pf + "wv", 1, kvd, d);
            if (!wk || !wv) return PPX_E_FORMAT;
            RepackJob jk;
            jk.K = d;
            for (int r = 0; r < kvd; ++r) jk.rows.push_back(rowp(wk, rope_row(r)));
            for (int r = 0; r < kvd; ++r) jk.rows.push_back(rowp(wv, r));
            jk.N = 2 * kvd;
            plan_q4(lw.wkv, std::move(jk));
        } else if (p.t.count(pf + "wk") || p.t.count(pf + "wv")) {
            return PPX_E_FORMAT;
        }
        if ((st = plain(lw.wo, need(pf + "wo", 1, d, qd)))) return st;
        const HostTensor *wg = need(pf + "ffn_gate", 1, F, d), *wu = need(pf + "ffn_up", 1, F, d);
        if (!wg || !wu) return PPX_E_FORMAT;
        RepackJob jg;
        jg.K = d;
        jg.N = 2 * F;
        // every 16-row group: gate rows 8t..8t+7, then the matching up rows
        for (int r = 0; r < 2 * F; ++r) {
            const int blk = r / 8, c = r % 8;
            jg.rows.push_back(rowp((blk & 1) ? wu : wg, (blk >> 1) * 8 + c));
        }
        plan_q4(lw.wgu, std::move(jg));
        if ((st = plain(lw.wdown, need(pf + "ffn_down", 1, d, F)))) return st;
        if (E) {
            if ((st = plan_f32(lw.ple_norm, need(pf + "ple_norm", 0, 1, d)))) return st;
            if ((st = plain(lw.wpg, need(pf + "ple_gate", 1, E, d)))) return st;
            if ((st = plain(lw.wpu, need(pf + "ple_up", 1, d, E)))) return st;
        }
    }

    if (need_bytes) *need_bytes = ar.used;
    if (!out) return PPX_OK;
    if (weights_dev && ((reinterpret_cast<uintptr_t>(weights_dev) & 255) != 0)) return PPX_E_INVAL;
    if (weights_dev && weights_bytes < ar.used) return PPX_E_NOMEM;

    // ---- build the host image and upload it
    std::vector<uint8_t> host(ar.used);
    for (const RepackJob &j : jobs) repack_rows(j, host.data());
    for (auto &f : f32s) std::memcpy(host.data() + f.off, b + f.t->offset, f.t->cols * 4);
    if (E) std::memcpy(host.data() + ple_off, b + ple->offset, (size_t)V * (L * E / 32) * 18);

    if (weights_dev) {
        m->dev = weights_dev;
        m->dev_owned = false;
    } else {
        if (hipMalloc(&m->dev, ar.used) != hipSuccess) {
            (void)hipGetLastError();
            return PPX_E_NOMEM;
        }
        m->dev_owned = true;
    }
    m->dev_bytes = ar.used;
    if (hipMemcpyAsync(m->dev, host.data(), ar.used, hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        if (m->dev_owned) (void)hipFree(m->dev);
        m->dev = nullptr;
        return PPX_E_HIP;
    }
    uint8_t *dev = static_cast<uint8_t *>(m->dev);
    for (const Slot &s : slots) {
        const RepackJob &j = jobs[s.job];
        s.q->nib = reinterpret_cast<const uint32_t *>(dev + j.nib_off);
        s.q->scl = reinterpret_cast<const __half *>(dev + j.scl_off);
    }
    for (auto &f : f32s) *f.dst = reinterpret_cast<const float *>(dev + f.off);
    if (E) m->ple_raw = dev + ple_off;
    if (m->tied) m->out = m->tok;

    // named views for the kernel-level entry points
    m->q4["tok_embd"] = m->tok;
    if (!m->tied) m->q4["output"] = m->out;
    for (int il = 0; il < L; ++il) {
        const std::string pf = "blk." + std::to_string(il) + ".";
        const LayerW &lw = m->layers[il];
        m->q4[pf + "wq"] = lw.wq;
        m->q4_kind[pf + "wq"] = 1;
        if (lw.own) {
            m->q4[pf + "wk"] = lw.wkv;
            m->q4_kind[pf + "wk"] = 3;
        }
        m->q4[pf + "wo"] = lw.wo;
        m->q4[pf + "ffn_gate"] = lw.wgu;
        m->q4_kind[pf + "ffn_gate"] = 2;
        m->q4[pf + "ffn_down"] = lw.wdown;
        if (E) {
            m->q4[pf + "ple_gate"] = lw.wpg;
            m->q4[pf + "ple_up"] = lw.wpu;
        }
    }
    if (log_enabled())
        std::fprintf(stderr, "[ppx] model loaded: %d layers (%d own KV), d=%d, %.1f MiB on device\n", L, Ls, d,
                     ar.used / 1048576.0);
    *out = m.release();
    return PPX_OK;
}

void drop_graphs(ppx_model *m) {
    for (auto &g : m->graphs) (void)hipGraphExecDestroy(g.exec);
    for (auto &g : m->keyed_graphs) (void)hipGraphExecDestroy(g.exec);
    m->graphs.clear();
    m->keyed_graphs.clear();
}

int ensure_rope(ppx_model *m, int n_ctx) {
    if (m->rope_n >= n_ctx) return PPX_OK;
    const int half = m->info.head_dim / 2, hd = m->info.head_dim;
    std::vector<float2> tab((size_t)n_ctx * half);
    for (int i = 0; i < half; ++i) {
        const double th = std::pow((double)m->rope_base, -2.0 * i / hd);
        for (int p = 0; p < n_ctx; ++p) {
            const double a = (double)p * th;
            tab[(size_t)p * half + i] = make_float2((float)std::cos(a), (float)std::sin(a));
        }
    }
    float2 *dev = nullptr;
    if (hipMalloc(&dev, tab.size() * sizeof(float2)) != hipSuccess) {
        (void)hipGetLastError();
        return PPX_E_NOMEM;
    }
    if (hipMemcpy(dev, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(dev);
        return PPX_E_HIP;
    }
    if (m->rope) {
        // Recorded launch sequences hold the old table's address in their RoPE
        // epilogues: they are dropped with it and recorded again on next use.
        (void)hipDeviceSynchronize();
        drop_graphs(m);
        (void)hipFree(m->rope);
    }
    m->rope = dev;
    m->rope_n = n_ctx;
    return PPX_OK;
}

void model_free(ppx_model *m) {
    if (!m) return;
    (void)hipDeviceSynchronize();
    if (m->dev && m->dev_owned) (void)hipFree(m->dev);
    if (m->rope) (void)hipFree(m->rope);
    for (hipEvent_t e : m->events) (void)hipEventDestroy(e);
    drop_graphs(m);
    if (m->capture_stream) (void)hipStreamDestroy(m->capture_stream);
    if (m->stage_host) (void)hipHostFree(m->stage_host);
    if (m->stage_event) (void)hipEventDestroy(m->stage_event);
    delete m;
}

}  // namespace ppx
