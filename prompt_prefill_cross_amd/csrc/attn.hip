// Causal prefill attention (MFMA, flash-style online softmax) and the
// single-query attention of the pruned KV-shared layers.
//
// Cache layout: K is [pos][kv_head][head_dim]; V is kept transposed,
// [kv_head][head_dim][vld] with vld >= n_ctx a multiple of 64, so that the
// values of consecutive keys for one dimension are contiguous.
//
// Prefill: the query heads that share one KV head are packed together, so a
// key/value tile serves all of them (GQA/MQA).  A workgroup owns 64 query
// columns -- (row, head-in-group) pairs -- of one KV head and one chunk of
// keys; each of its four waves owns 16 columns.  The kernel computes
// S^T = K Q^T, so the 16x16 accumulator of a wave holds keys down and query
// columns across.  Inside each 32-key step the keys are taken in the order
// that puts keys 8g..8g+7 of the step in lane group g of the accumulator;
// then a lane's probabilities are exactly its B operand of O^T = V^T P^T, and
// its V^T A operand is one 16-byte read of the transposed cache.  Tiles are
// aligned to absolute key positions, so a row's result does not depend on
// how the prompt was split into ubatches.  When the keys are split over
// several workgroups, each writes (max, sum, unnormalised output) and a merge
// kernel combines the chunks in chunk order.
#include "ppx_dev.h"

namespace ppx {

namespace {

constexpr int KT = 32;  // keys per pipeline stage
static_assert(kKvPage % KT == 0, "a stage's keys lie in one page of a unified cache");

typedef __attribute__((address_space(3))) void lds_t;

__device__ __forceinline__ void adma16(const void *src, h8 *dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_t *)dst, 16, 0, 0);
}
__device__ __forceinline__ int attn_wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Workgroup barrier without the fences of __syncthreads (which would drain
// the producers' outstanding DMA).
__device__ __forceinline__ void attn_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Max / sum over the four lanes of one query column (l, l ^ 16, l ^ 32,
// l ^ 48), as (x_l op x_l^16) op (the same at l ^ 32), on VALU: the step's
// K and V^T fragment reads fill the LDS queue that a permute would wait in.
__device__ __forceinline__ float attn_col_max(float v) {
    LanePair p = swap16(v);
    p = swap32(fmaxf(p.a, p.b));
    return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float attn_col_sum(float v) {
    LanePair p = swap16(v);
    p = swap32(p.a + p.b);
    return p.a + p.b;
}

template <int N>
__device__ __forceinline__ void attn_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// NC compute waves of CPW groups of 16 query columns and NP producer waves;
// a ring of DEPTH stages of KT keys each: the K fragments [d step][16-key
// block][lane] and the V^T fragments [16-dim subtile][lane] of the stage.
template <int HD_, int CPW_, int NC_, int NP_, int DEPTH_>
struct ACfg {
    static constexpr int HD = HD_, CPW = CPW_, NC = NC_, NP = NP_, DEPTH = DEPTH_;
    static constexpr int KB = HD / 32;           // 32-wide d steps of S
    static constexpr int DT = HD / 16;           // 16-row d subtiles of O^T
    static constexpr int K_UNITS = KB * 2 * 64;  // 16-byte units
    static constexpr int V_UNITS = DT * 64;
    static constexpr int STAGE_UNITS = K_UNITS + V_UNITS;
    static constexpr int DMA_STAGE = KB * 2 + DT;
    static constexpr int PER = (DMA_STAGE + NP - 1) / NP;
    static constexpr int NT = 64 * (NC + NP);
    static constexpr int CB = 16 * CPW * NC;     // query columns per workgroup
    static_assert(DEPTH >= 2 && (DEPTH - 2) * PER <= 63, "vmcnt range");
    static_assert(DEPTH * STAGE_UNITS * 16 <= 160 * 1024, "LDS");
};

// The workgroup's share of one unit: its column block, rows and cache.
struct AttnSeg {
    int cb, M, pos0, row0, vld;
    const __half *kp, *vtp;
    const int32_t *page;  // unified cache: the sequence's page table (else null)
    int pend;             // last key any column here can see
    int plast;            // last key written before this launch reads the cache
    int kbeg, kend;       // the key chunk, clipped to pend
};

// false: the workgroup has nothing to do (past the unit's columns, its
// workgroup table or its keys)
template <int CB>
__device__ __forceinline__ bool attn_seg(const AttnArgs &a, int ck, int G, AttnSeg &s) {
    // the workgroup's rows: [row0, row0 + M) of the launch, one sequence's
    // positions pos0 .. pos0 + M - 1, read against that sequence's cache
    s.cb = blockIdx.x;
    s.M = a.M;
    s.pos0 = a.pos0;
    s.row0 = 0;
    s.vld = a.vld;
    s.kp = a.k;
    s.vtp = a.vt;
    s.page = nullptr;
    if (a.wg) {
        if ((int)blockIdx.x >= a.nwg) return false;
        const AttnWg &d = a.wg[blockIdx.x];
        s.cb = d.cb;
        s.M = d.M;
        s.pos0 = d.pos0;
        s.row0 = d.row0;
        const KVRef &ref = a.seq_kv[d.seq];
        s.kp = ref.k;
        s.vtp = ref.vt;
        s.vld = ref.vld;
        s.page = ref.page;
    } else if (s.cb * CB >= s.M * G) {
        return false;
    }
    const int tmax = min(s.M - 1, (s.cb * CB + CB - 1) / G);
    s.pend = s.pos0 + tmax;
    s.plast = s.pos0 + s.M - 1;
    s.kbeg = ck * a.kc;
    if (s.kbeg > s.pend) return false;
    s.kend = min(s.kbeg + a.kc, s.pend + 1);
    return true;
}

// Running state of a compute wave's CPW groups of 16 query columns.
template <int HD, int CPW>
struct AttnRun {
    static constexpr int KB = HD / 32, DT = HD / 16;
    h8 qf[CPW][KB];
    f4 oacc[CPW][DT];
    float mrun[CPW], lrun[CPW];
    int qpos[CPW];
};

// the unit's query column of the wave's group c (row col / G, head
// kvh * G + col % G)
template <int CB, int CPW>
__device__ __forceinline__ int attn_col(int cb, int wave, int c, int lc) {
    return cb * CB + wave * 16 * CPW + c * 16 + lc;
}

template <int HD, int CB, int CPW>
__device__ __forceinline__ void attn_begin(const AttnArgs &a, const AttnSeg &g, int wave, int kvh, int G, int lc,
                                           int lg, AttnRun<HD, CPW> &R) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int col = attn_col<CB, CPW>(g.cb, wave, c, lc);
        const int t = col / G, h = kvh * G + col % G;
        R.qpos[c] = g.pos0 + (t < g.M ? t : 0);
#pragma unroll
        for (int kb = 0; kb < HD / 32; ++kb)
            R.qf[c][kb] = *reinterpret_cast<const h8 *>(a.q + ((size_t)(g.row0 + min(t, g.M - 1)) * a.H + h) * HD +
                                                        kb * 32 + lg * 8);
#pragma unroll
        for (int i = 0; i < HD / 16; ++i) R.oacc[c][i] = f4{0.f, 0.f, 0.f, 0.f};
        R.mrun[c] = -INFINITY;
        R.lrun[c] = 0.f;
    }
}

// One step of 32 keys t0 .. t0 + 31.  kfrag(kb, j) is the K fragment of d
// step kb and 16-key block j, in which lane l holds the key of accumulator
// row 8 (r / 4) + 4 j + r % 4, r = l % 16, and dims kb*32 + 8 (l / 16) ..;
// vfrag(i) is the V^T fragment of dims 16 i .. 16 i + 15, in which lane l
// holds dim 16 i + l % 16, keys 8 (l / 16) .. + 7.
//
// The kernel computes S^T = K Q^T, so a wave's 16x16 accumulator holds keys
// down and query columns across; with the keys in that order a lane's
// probabilities are exactly its B operand of O^T = V^T P^T.
//
// Online softmax in the exp2 domain against a reference max m per column
// (mrun): p = 2^(s log2(e) / sqrt(hd) - m), l = sum p, O = sum p v.  Any m
// gives the same O / l; m only has to keep p finite in fp16, so it moves
// (and O and l are rescaled by 2^(m_old - m_new)) only when a score
// exceeds it by more than ATTN_LAZY: then p <= 2^ATTN_LAZY.  The first
// visible key of a column always sets m.
//
// edge (uniform): some key of the step lies past some column's position
// (the causal mask applies) or past the last written key (stale values are
// zeroed); other steps skip both.
constexpr float ATTN_LAZY = 8.0f;

template <int HD, int CPW, class KF, class VF>
__device__ __forceinline__ void attn_step32(const KF &kfrag, const VF &vfrag, int t0, int plast, int lg, bool edge,
                                            AttnRun<HD, CPW> &R) {
    constexpr int KB = HD / 32, DT = HD / 16;
    const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
    // S^T = K Q^T: s[c][j][r] is key t0 + 8 lg + 4 j + r, query column lc of group c
    // in groups of four fragments (d steps 2q and 2q + 1 of both key
    // blocks), the next group's reads issued before this group's products,
    // which alternate between the two key blocks' accumulators
    static_assert(KB % 2 == 0, "fragment groups");
    f4 s[CPW][2];
#pragma unroll
    for (int c = 0; c < CPW; ++c) s[c][0] = s[c][1] = f4{0.f, 0.f, 0.f, 0.f};
    h8 ka[4], kn[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) ka[u] = kfrag(u >> 1, u & 1);
#pragma unroll
    for (int q = 0; q < KB / 2; ++q) {
        if (q + 1 < KB / 2) {
#pragma unroll
            for (int u = 0; u < 4; ++u) kn[u] = kfrag(2 * (q + 1) + (u >> 1), u & 1);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < CPW; ++c) s[c][u & 1] = mfma16(ka[u], R.qf[c][2 * q + (u >> 1)], s[c][u & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) ka[u] = kn[u];
    }
    h8 pf[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        // masked scores are -inf; the max is taken on the raw scores (sl2 > 0)
        if (edge) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (t0 + 8 * lg + 4 * j + r > R.qpos[c]) s[c][j][r] = -INFINITY;
        }
        float tmx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) tmx = fmaxf(tmx, s[c][j][r]);
        tmx = attn_col_max(tmx) * sl2;
        // move m only past the margin (or at the first visible key); 2^-inf
        // = 0 covers masked keys and a column with no visible key yet, whose
        // m stays -inf and which subtracts 0 instead
        const bool move = tmx > R.mrun[c] + ATTN_LAZY;
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float mnew = move ? tmx : R.mrun[c];
            // 1 where m stays; against 0 while m is -inf (O and l are 0 then), never 2^(-inf + inf)
            const float alpha = __builtin_amdgcn_exp2f(R.mrun[c] - (mnew == -INFINITY ? 0.f : mnew));
            R.lrun[c] *= alpha;
#pragma unroll
            for (int i = 0; i < DT; ++i) R.oacc[c][i] *= alpha;
            R.mrun[c] = mnew;
        }
        const float msub = R.mrun[c] == -INFINITY ? 0.f : R.mrun[c];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][j][r], sl2, -msub));
                psum += p;
                pf[c][4 * j + r] = (_Float16)p;
            }
        R.lrun[c] += attn_col_sum(psum);
    }
    // O^T += V^T P^T over the step's 32 keys (8 lg .. 8 lg + 7 in lane group lg).
    // Values of keys past the last written position may be stale (a cache
    // cleared or reloaded to fewer positions keeps its old contents): they
    // are zeroed, so a non-finite stale value cannot meet a zero weight.
    // Groups of four fragments: the next group's reads are issued before
    // this group's products, so eight reads at most are in flight (more
    // would take the registers of the wave's Q fragments), and the zeroing
    // of a tail step is one test per group, not a branch per fragment.
    const bool tail = edge && t0 + 31 > plast;  // uniform over the workgroup
    const int vlim = plast - (t0 + 8 * lg);     // elements e <= vlim are written keys
    static_assert(DT % 4 == 0, "fragment groups");
    h8 va[4], vb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) va[u] = vfrag(u);
#pragma unroll
    for (int q = 0; q < DT / 4; ++q) {
        if (q + 1 < DT / 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) vb[u] = vfrag(4 * (q + 1) + u);
        }
        if (tail) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (e > vlim) va[u][e] = (_Float16)0.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < CPW; ++c) R.oacc[c][4 * q + u] = mfma16(va[u], pf[c], R.oacc[c][4 * q + u]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) va[u] = vb[u];
    }
}

// A step is an edge step when one of its keys may be masked for a column of
// the workgroup (qmin: the smallest position of its columns) or lies past
// the last written key (plast >= every column's position).
__device__ __forceinline__ bool attn_edge(int t0, int qmin) { return t0 + 31 > qmin; }

// The chunk's result of each valid column: the normalised output when the
// keys are not split, else the chunk's own normalised output in fp16 (a
// convex combination of value rows, so bounded by them) with its max and
// exp-sum in fp32; a row that sees no key of the chunk writes zeros, never read.
template <int HD, int CB, int CPW>
__device__ __forceinline__ void attn_finish(const AttnArgs &a, const AttnSeg &g, int ck, int wave, int kvh, int G,
                                            int lc, int lg, const AttnRun<HD, CPW> &R) {
    constexpr int DT = HD / 16;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int col = attn_col<CB, CPW>(g.cb, wave, c, lc);
        const int t = col / G, h = kvh * G + col % G;
        if (t >= g.M) continue;
        if (a.nkc == 1) {
            const float inv = 1.0f / R.lrun[c];
            const int od = a.H * HD;
#pragma unroll
            for (int i = 0; i < DT; ++i) {
                const int d = i * 16 + lg * 4;  // four consecutive columns: 8 contiguous bytes of the tiled layout
                h4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = (_Float16)(R.oacc[c][i][r] * inv);
                *reinterpret_cast<h4 *>(a.o + tiled_index(g.row0 + t, h * HD + d, od)) = v;
            }
        } else {
            const size_t slot = ((size_t)ck * a.M + g.row0 + t) * a.H + h;
            const float inv = R.lrun[c] > 0.f ? 1.0f / R.lrun[c] : 0.f;
            _Float16 *po = reinterpret_cast<_Float16 *>(a.part) + slot * HD;
#pragma unroll
            for (int i = 0; i < DT; ++i) {
                h4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = (_Float16)(R.oacc[c][i][r] * inv);
                *reinterpret_cast<h4 *>(po + i * 16 + lg * 4) = v;
            }
            if (lg == 0) {
                // (max, sum) pairs of one (row, head) are contiguous over the chunks
                float *pm = a.part + (size_t)a.nkc * a.M * a.H * (HD / 2) +
                            (((size_t)(g.row0 + t) * a.H + h) * a.nkc + ck) * 2;
                pm[0] = R.mrun[c];
                pm[1] = R.lrun[c];
            }
        }
    }
}

// Grid (column blocks, key chunks, KV heads x units): unit z / KVH of the
// group, KV head z % KVH; a unit with fewer column blocks or key chunks than
// the launch's largest leaves the surplus workgroups idle.
//
// Fragment-ordered staging: every copy instruction fills one MFMA fragment
// (16 keys x 64 bytes of K, or 16 dims x 64 bytes of V^T), so the compute
// waves read the ring in lane order.
template <class C>
__global__ __launch_bounds__(C::NT) void k_attn_prefill(const AttnGroup grp) {
    constexpr int HD = C::HD, KB = C::KB, CPW = C::CPW;
    __shared__ h8 ring[C::DEPTH * C::STAGE_UNITS];

    const AttnArgs &a = grp.u[blockIdx.z / grp.u[0].KVH];
    const int lane = threadIdx.x & 63, wave = attn_wave_id();
    const int G = a.H / a.KVH;
    const int ck = blockIdx.y, kvh = blockIdx.z % a.KVH;
    if (ck >= a.nkc) return;  // the whole workgroup
    const int lc = lane & 15, lg = lane >> 4;
    AttnSeg g;
    if (!attn_seg<C::CB>(a, ck, G, g)) return;  // the whole workgroup
    const int nst = (g.kend - g.kbeg + KT - 1) / KT;

    if (wave >= C::NC) {
        // ---- producers: wave NC + p issues DMAs p, p + NP, ... of every stage.
        // K rows past the last written position repeat it (their scores are
        // masked); V^T reads stay inside the row (vld is a multiple of 64).
        const int pw = C::NP == 1 ? 0 : wave - C::NC;
        auto entry = [&](int t) { return min(t * C::NP + pw, C::DMA_STAGE - 1); };
        int koff[C::PER];  // K: key within the stage; V^T: element offset within the row block
#pragma unroll
        for (int t = 0; t < C::PER; ++t) {
            const int e = entry(t);
            if (e < 2 * KB) {
                const int j = e & 1;
                koff[t] = 8 * ((lane & 15) >> 2) + 4 * j + (lane & 3);
            } else {
                // V^T subtile i: lane l holds dim 16 i + l % 16, keys 8 (l / 16) .. + 7
                const int i = e - 2 * KB;
                koff[t] = (kvh * HD + i * 16 + (lane & 15)) * g.vld + 8 * (lane >> 4);
            }
        }
        auto issue = [&](int sb) {
            h8 *st = ring + (sb % C::DEPTH) * C::STAGE_UNITS;
            const int t0 = g.kbeg + min(sb, nst - 1) * KT;  // past the end: repeats keep the count uniform
            // the stage's keys t0 .. t0 + KT - 1 (and the clamp target plast >= t0)
            // lie in one page: cells c0 + (key - t0)
            const int c0 = kv_cell(g.page, t0);
#pragma unroll
            for (int t = 0; t < C::PER; ++t) {
                const int e = entry(t);
                if (e < 2 * KB) {
                    const int kb = e >> 1;
                    const int key = min(t0 + koff[t], g.plast);
                    adma16(g.kp + ((size_t)(c0 + key - t0) * a.KVH + kvh) * HD + kb * 32 + 8 * (lane >> 4),
                           st + e * 64);
                } else {
                    adma16(g.vtp + (size_t)koff[t] + c0, st + C::K_UNITS + (e - 2 * KB) * 64);
                }
            }
        };
#pragma unroll
        for (int s = 0; s < C::DEPTH - 1; ++s) issue(s);
        for (int s = 0; s < nst; ++s) {
            attn_wait_vm<(C::DEPTH - 2) * C::PER>();  // this wave's share of stage s has landed
            attn_barrier();
            issue(s + C::DEPTH - 1);  // into the buffer of stage s - 1, already consumed
        }
        attn_wait_vm<0>();
        attn_barrier();
        return;
    }

    // ---- compute waves: CPW groups of 16 query columns; every K / V^T
    // fragment read from LDS feeds one MFMA per group
    AttnRun<HD, CPW> R;
    attn_begin<HD, C::CB, CPW>(a, g, wave, kvh, G, lc, lg, R);
    const int qmin = g.pos0 + g.cb * C::CB / G;
    for (int it = 0; it < nst; ++it) {
        attn_barrier();  // stage it has landed
        const h8 *st = ring + (it % C::DEPTH) * C::STAGE_UNITS + lane;
        const int t0 = g.kbeg + it * KT;
        auto kfrag = [&](int kb, int j) { return st[(kb * 2 + j) * 64]; };
        auto vfrag = [&](int i) { return st[C::K_UNITS + i * 64]; };
        attn_step32<HD, CPW>(kfrag, vfrag, t0, g.plast, lg, attn_edge(t0, qmin), R);
    }
    attn_barrier();  // matches the producers' last barrier
    attn_finish<HD, C::CB, CPW>(a, g, ck, wave, kvh, G, lc, lg, R);
}

// Line-wide staging (written for head_dim 128 and 256; launched at 256).  A
// copy instruction that fills a fragment reads 16 pieces of 64 bytes, and
// the vector memory path serves such pieces at about a third of the rate of
// whole 128-byte lines (16 against 44-56 bytes per clock per CU, measured);
// here every 1 KB copy instruction reads whole lines instead: 512 / head_dim
// whole K rows, or 8 V^T rows of one stage's 64 keys (128 bytes each, a
// line: cells of a stage are 64-aligned).  The ring holds the rows as they
// are, in 16-byte slots permuted by an XOR with a function of the row, so
// that the MFMA fragment reads (16 lanes on distinct rows at one slot) run
// at the rate of contiguous reads -- both permutations were picked by timing
// ds_read_b128 patterns on the chip (rows of 128 bytes at one slot, or with
// the slot XORed by (row & 7) ^ (row >> 3 & 1), read at two thirds of it):
//   K row k (key t0 + k), slot s holds the row's slot s ^ sigma(k),
//       sigma(k) = (k & 3) | ((k >> 3) & 3) << 2;
//   V^T row d (dim d), slot s holds keys t0 + 8 (s ^ tau(d)) .. + 7,
//       tau(d) = d & 7.
// A stage is 64 keys (two steps of 32); two stages fill the ring.  NC
// compute waves of CPW groups of 16 query columns; NP producer waves, or
// none (NP = 0): the compute waves then issue the copies themselves (with
// eight compute waves 11-15 % slower than two or four producers, measured).
template <int HD_, int NC_, int CPW_, int NP_>
struct WCfg {
    static constexpr int HD = HD_, NC = NC_, CPW = CPW_, NP = NP_, DEPTH = 2, KS = 64;
    static constexpr int ROW = HD / 8;                // 16-byte slots per K row
    static constexpr int K_UNITS = KS * ROW;          // 16-byte units
    static constexpr int V_UNITS = HD * (KS / 8);
    static constexpr int STAGE_UNITS = K_UNITS + V_UNITS;
    static constexpr int K_INSTR = K_UNITS / 64, V_INSTR = V_UNITS / 64;
    static constexpr int DMA_STAGE = K_INSTR + V_INSTR;
    static constexpr int NI = NP ? NP : NC;  // waves that issue the copies
    static constexpr int PER = DMA_STAGE / NI;
    static constexpr int NT = 64 * (NC + NP);
    static constexpr int CB = 16 * CPW * NC;
    static_assert(ROW >= 16 && 64 % ROW == 0, "whole K rows per copy instruction; sigma < ROW");
    static_assert(DMA_STAGE % NI == 0 && PER <= 63, "copies per issuing wave");
    static_assert(DEPTH * STAGE_UNITS * 16 <= 160 * 1024, "LDS");
    static_assert(kKvPage % KS == 0, "a stage's keys lie in one page of a unified cache");
};

__device__ __forceinline__ int attn_sigma(int k) { return (k & 3) | (((k >> 3) & 3) << 2); }
__device__ __forceinline__ int attn_tau(int d) { return d & 7; }

template <class C>
__global__ __launch_bounds__(C::NT) void k_attn_prefill_w(const AttnGroup grp) {
    constexpr int HD = C::HD, ROW = C::ROW, KS = C::KS;
    __shared__ h8 ring[C::DEPTH * C::STAGE_UNITS];

    const AttnArgs &a = grp.u[blockIdx.z / grp.u[0].KVH];
    const int lane = threadIdx.x & 63, wave = attn_wave_id();
    const int G = a.H / a.KVH;
    const int ck = blockIdx.y, kvh = blockIdx.z % a.KVH;
    if (ck >= a.nkc) return;  // the whole workgroup
    const int lc = lane & 15, lg = lane >> 4;
    AttnSeg g;
    if (!attn_seg<C::CB>(a, ck, G, g)) return;  // the whole workgroup
    const int nst = (g.kend - g.kbeg + KS - 1) / KS;

    // ---- copies: issuing wave p (producer NC + p, or compute wave p when NP
    // = 0) issues copies p, p + NI, ... of every stage (K instructions first,
    // then V^T).  K rows past the last written position repeat it (their
    // scores are masked); V^T reads stay inside the row (vld is a multiple of 64).
    const int pw = C::NP ? wave - C::NC : wave;
    const int kx = lane / ROW, ks = lane % ROW;  // K: row within the instruction, slot
    const int vr = lane >> 3, vs = lane & 7;     // V^T: row within the instruction, slot
    // Copy t of an issuing wave is e = t NI + pw: a K copy for t < PK (K_INSTR
    // is a multiple of NI), known when the loop is unrolled.  What the copies
    // read from the arguments is held in registers here: the barriers'
    // memory clobbers would otherwise have it re-read before every copy.
    static_assert(C::K_INSTR % C::NI == 0, "K copies per issuing wave");
    constexpr int PK = C::K_INSTR / C::NI;
    // Within a stage the offsets fit in 32 bits: K rows (key - t0) * KVH * HD
    // with key - t0 < 64, V^T rows d * vld with d < HD.
    const int kcell = a.KVH * HD;  // elements from one cell's K rows to the next's
    const __half *const kbase = g.kp + (size_t)kvh * HD;
    const __half *const vbase = g.vtp + (size_t)kvh * HD * g.vld;
    const int vld = g.vld, plast = g.plast, kbeg = g.kbeg;
    auto issue = [&](int sb) {
        h8 *st = ring + (sb % C::DEPTH) * C::STAGE_UNITS;
        const int t0 = kbeg + min(sb, nst - 1) * KS;  // past the end: repeats keep the count uniform
        // the stage's keys t0 .. t0 + 63 (and the clamp target plast >= t0)
        // lie in one page: cells c0 + (key - t0)
        const int c0 = kv_cell(g.page, t0);
        const __half *const ks0 = kbase + (size_t)c0 * kcell;
        const __half *const vs0 = vbase + c0;
        const int klim = plast - t0;  // keys past plast repeat it
#pragma unroll
        for (int t = 0; t < C::PER; ++t) {
            const int e = t * C::NI + pw;
            if (t < PK) {
                const int k = e * (64 / ROW) + kx;
                adma16(ks0 + (unsigned)(min(k, klim) * kcell + 8 * (ks ^ attn_sigma(k))), st + e * 64);
            } else {
                const int d = (e - C::K_INSTR) * 8 + vr;
                adma16(vs0 + (unsigned)(d * vld + 8 * (vs ^ attn_tau(d))), st + e * 64);
            }
        }
    };
    if (C::NP > 0 && wave >= C::NC) {
        // ---- producers
#pragma unroll
        for (int s = 0; s < C::DEPTH - 1; ++s) issue(s);
        for (int s = 0; s < nst; ++s) {
            attn_wait_vm<(C::DEPTH - 2) * C::PER>();  // this wave's share of stage s has landed
            attn_barrier();
            issue(s + C::DEPTH - 1);  // into the buffer of stage s - 1, already consumed
        }
        attn_wait_vm<0>();
        attn_barrier();
        return;
    }

    // ---- compute waves: CPW groups of 16 query columns each
    constexpr int CPW = C::CPW;
    AttnRun<HD, CPW> R;
    attn_begin<HD, C::CB, CPW>(a, g, wave, kvh, G, lc, lg, R);
    // the lane's ring offsets: K block j (keys 8 (r / 4) + 4 j + r % 4 of a
    // step, r = lane % 16) at d step kb reads row slot (4 kb + lg) ^ sigma,
    // = 16 (kb / 4) + kofs[j][kb % 4] within the row (sigma < 16 leaves bit 2
    // of kb alone); V^T subtile i reads row 16 i + lc at slot (4 h + lg) ^ tau
    // for step h, = 128 i + vofs[h] (tau(16 i + lc) = tau(lc)).  What varies
    // with kb / 4, i and h goes into the read's immediate offset.
    int kofs[2][4], vofs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int k = 8 * (lc >> 2) + 4 * j + (lc & 3), sg = attn_sigma(k);
#pragma unroll
        for (int b = 0; b < 4; ++b) kofs[j][b] = k * ROW + 4 * (b ^ (sg >> 2)) + (lg ^ (sg & 3));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) vofs[h] = C::K_UNITS + lc * 8 + ((4 * h + lg) ^ attn_tau(lc));
    const int qmin = g.pos0 + g.cb * C::CB / G;
    static_assert(C::NP > 0 || C::DEPTH == 2, "compute waves that copy keep one stage in flight");
    if (C::NP == 0) issue(0);
    for (int it = 0; it < nst; ++it) {
        if (C::NP == 0) attn_wait_vm<0>();  // this wave's copies of stage it have landed
        attn_barrier();  // stage it has landed (and stage it - 1 is consumed)
        if (C::NP == 0 && it + 1 < nst) issue(it + 1);  // into stage it - 1's buffer
        const h8 *st = ring + (it % C::DEPTH) * C::STAGE_UNITS;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t0 = g.kbeg + it * KS + 32 * h;
            if (t0 > g.pend) break;  // every key of the step is masked for every column: no change
            auto kfrag = [&](int kb, int j) { return st[kofs[j][kb & 3] + 16 * (kb >> 2) + 32 * h * ROW]; };
            auto vfrag = [&](int i) { return st[vofs[h] + 128 * i]; };
            attn_step32<HD, CPW>(kfrag, vfrag, t0, g.plast, lg, attn_edge(t0, qmin), R);
        }
    }
    attn_barrier();  // matches the producers' last barrier
    attn_finish<HD, C::CB, CPW>(a, g, ck, wave, kvh, G, lc, lg, R);
}

// Combine the key chunks of row t, head h: chunks 0..floor(pos/kc) hold keys
// the row can see.  Chunk c contributes its normalised output with weight
// l_c 2^(m_c - M), M = max_c m_c (the exp2 domain of the kernel); the chunks
// are summed in chunk order.  One workgroup per row of a unit (grid (rows,
// units)): thread i takes head hb + i / TPH of each pass and dims 8 (i % TPH)
// .. + 7 (TPH = HD / 8 threads per head), so the row's whole output is one
// pass of 16-byte reads; each thread requests the slices of its first
// MERGE_CU chunks before it reads the chunks' (max, sum) pairs.
constexpr int MERGE_CU = 8;
template <int HD>
__global__ __launch_bounds__(256) void k_attn_prefill_merge(const AttnGroup grp) {
    constexpr int TPH = HD / 8, HPP = 256 / TPH;  // threads per head, heads per pass
    const AttnArgs &a = grp.u[blockIdx.y];
    const int t = blockIdx.x;
    if (t >= a.M) return;  // past this unit's rows (the whole workgroup)
    const int nch = (a.row_pos ? a.row_pos[t] : a.pos0 + t) / a.kc + 1;
    const size_t cstride = (size_t)a.M * a.H * HD;  // fp16 elements per chunk
    const int dh = (threadIdx.x % TPH) * 8;
    for (int hb = 0; hb < a.H; hb += HPP) {
        const int h = hb + (int)threadIdx.x / TPH;
        if (h >= a.H) break;
        const size_t w = (size_t)t * a.H + h;
        const float *pm = a.part + (size_t)a.nkc * a.M * a.H * (HD / 2) + w * a.nkc * 2;
        const _Float16 *base = reinterpret_cast<const _Float16 *>(a.part) + w * HD + dh;
        h8 x[MERGE_CU];
        auto load = [&](int c0) {
            // chunks past the last repeat it (weight 0 below), so every load issues at once
#pragma unroll
            for (int u = 0; u < MERGE_CU; ++u)
                x[u] = *reinterpret_cast<const h8 *>(base + (size_t)min(c0 + u, nch - 1) * cstride);
        };
        load(0);
        float M = -INFINITY;
        for (int c = 0; c < nch; ++c) M = fmaxf(M, pm[2 * c]);
        float O[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, L = 0.f;
        for (int c0 = 0; c0 < nch; c0 += MERGE_CU) {
            if (c0) load(c0);
#pragma unroll
            for (int u = 0; u < MERGE_CU; ++u) {
                const int c = min(c0 + u, nch - 1);
                const float wg = c0 + u < nch ? exp2f(pm[2 * c] - M) * pm[2 * c + 1] : 0.f;
                L += wg;
#pragma unroll
                for (int e = 0; e < 8; ++e) O[e] += wg * (float)x[u][e];
            }
        }
        const float inv = 1.0f / L;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            h4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = (_Float16)(O[4 * q + e] * inv);
            // four consecutive dims: 8 contiguous bytes of the tiled layout
            *reinterpret_cast<h4 *>(a.o + tiled_index(t, h * HD + dh + 4 * q, a.H * HD)) = r;
        }
    }
}

// ------------------------------------------------------------------ single query
// One query row (all heads) over cache positions 0..pos, in two launches.
// k_attn_1row: grid (chunks of CH keys, KVH); the G <= 8 heads of a KV head
// share a workgroup and both products run on MFMA at ~fp32 accuracy: the fp32
// operand (q, then the probabilities) is split into fp16 hi and lo parts that
// fill columns 0..7 and 8..15 of the B operand, against exact fp16 keys and
// values, so a result is the sum of its two columns.
//   scores  S[key][g] = K[key] . q_g         (A = 16 keys x 32 dims per step)
//   softmax of the chunk per head (max, exp-sum)
//   P.V     O[d][g] = sum_key V^T[d][key] P[g][key]   (A = 16 dims x 32 keys)
// Each chunk writes per head its max, exp-sum and unnormalised output;
// k_attn_merge combines the chunks in chunk order.
constexpr int CH = 32;
static_assert(kKvPage % CH == 0, "a chunk's keys lie in one page of a unified cache");

template <int HD>
__global__ __launch_bounds__(256) void k_attn_1row(Attn1Args a) {
    __shared__ float sl[8][CH];  // scores, then probabilities

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.H / a.KVH;  // <= 8
    const int kvh = blockIdx.y, chunk = blockIdx.x, nchunks = gridDim.x;
    const int k0 = chunk * CH;
    const int nk = min(CH, a.pos + 1 - k0);
    const float scale = 1.0f / sqrtf((float)HD);
    const int c = lane & 15, g = c & 7, lg = lane >> 4;
    const bool lo = c >= 8;

    if (wave < CH / 16) {
        const int key = wave * 16 + c;
        const int kr = k0 + min(key, nk - 1);  // masked keys re-read a valid row
        const __half *krow = a.k + ((size_t)kr * a.KVH + kvh) * HD + lg * 8;
        const float *qrow = a.q + (size_t)(kvh * G + min(g, G - 1)) * HD + lg * 8;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < HD / 32; ++ks) {
            const h8 av = *reinterpret_cast<const h8 *>(krow + ks * 32);
            const float4 q0 = *reinterpret_cast<const float4 *>(qrow + ks * 32);
            const float4 q1 = *reinterpret_cast<const float4 *>(qrow + ks * 32 + 4);
            const float qe[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            h8 bv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const _Float16 h = (_Float16)qe[e];
                bv[e] = g < G ? (lo ? (_Float16)(qe[e] - (float)h) : h) : (_Float16)0.0f;
            }
            acc = mfma16(av, bv, acc);
        }
        // acc[r] = C[key 4*lg + r of the tile][column c]; S = column g + column g + 8
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = acc[r] + row_ror<8>(acc[r]);
            const int kt = wave * 16 + 4 * lg + r;
            if (c < G) sl[c][kt] = kt < nk ? v * scale : -INFINITY;
        }
    }
    // the wave's value tiles (t = wave, wave + 4, ...) do not depend on the
    // scores: requested here, so they arrive during the softmax
    constexpr int NTW = HD / 16 / 4;
    h8 vpre[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int d = (wave + 4 * i) * 16 + c;
        vpre[i] = *reinterpret_cast<const h8 *>(a.vt + ((size_t)kvh * HD + d) * a.vld + k0 + lg * 8);
    }
    __syncthreads();

    // softmax of the chunk: wave w takes heads w, w+4; lane = key
    for (int h = wave; h < G; h += 4) {
        const float sc = lane < CH ? sl[h][lane] : -INFINITY;
        const float m = wave_max(sc);
        const float p = (lane < nk) ? expf(sc - m) : 0.f;
        const float l = wave_sum(p);
        if (lane < CH) sl[h][lane] = p;
        if (lane == 0) {
            float *st = a.partial + ((size_t)(kvh * G + h) * nchunks + chunk) * 2;
            st[0] = m;
            st[1] = l;
        }
    }
    __syncthreads();

    // unnormalised P.V, 16 dimensions per MFMA tile; wave w takes tiles w, w+4, ...
    float *po = a.partial + (size_t)a.H * nchunks * 2;
    h8 bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = lg * 8 + e;
        const float p = g < G ? sl[g][j] : 0.f;
        const _Float16 h = (_Float16)p;
        bv[e] = lo ? (_Float16)(p - (float)h) : h;
    }
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int t = wave + 4 * i;
        h8 av = vpre[i];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (lg * 8 + e >= nk) av[e] = (_Float16)0.0f;
        const f4 acc = mfma16(av, bv, f4{0.f, 0.f, 0.f, 0.f});
        // acc[r] = C[dimension t*16 + 4*lg + r][column c]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = acc[r] + row_ror<8>(acc[r]);
            if (c < G) po[((size_t)(kvh * G + c) * nchunks + chunk) * HD + t * 16 + 4 * lg + r] = v;
        }
    }
}

// o[h][d] = sum_c e^(m_c - M) o_c[d] / sum_c e^(m_c - M) l_c.  One workgroup
// per head: thread (s, q) owns dims 4q .. 4q+3 and the chunks c = s (mod NS),
// NS = 1024 / hd subsets, four chunks' loads in flight at a time; the subsets
// are then added in subset order, so the result is deterministic.
__global__ __launch_bounds__(256) void k_attn_merge(Attn1Args a, int nchunks) {
    __shared__ float wl[1024];
    __shared__ float red[8];
    __shared__ f4 part[256];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hd = a.hd, nq = hd >> 2, ns = 256 / nq;
    const float *st = a.partial + (size_t)h * nchunks * 2;
    const float *po = a.partial + (size_t)a.H * nchunks * 2 + (size_t)h * nchunks * hd;
    const int q = tid % nq, sub = tid / nq;  // ns * nq = 256: every thread has a slice
    // the thread's first MERGE1_PRE batches of partial outputs (chunks sub +
    // 4 ns b + ns u) do not depend on the weights: requested before the
    // (max, sum) pass; past the last chunk the reads repeat it (weight 0)
    constexpr int MERGE1_PRE = 4;
    f4 xp[MERGE1_PRE][4];
#pragma unroll
    for (int b = 0; b < MERGE1_PRE; ++b)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = min(sub + 4 * ns * b + u * ns, nchunks - 1);
            xp[b][u] = *reinterpret_cast<const f4 *>(po + (size_t)c * hd + 4 * q);
        }
    float M = -INFINITY;
    for (int c = tid; c < nchunks; c += 256) M = fmaxf(M, st[2 * c]);
    M = wave_max(M);
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float L = 0.f;
    for (int c = tid; c < nchunks; c += 256) {
        const float w = expf(st[2 * c] - M);
        if (c < 1024) wl[c] = w;
        L += w * st[2 * c + 1];
    }
    L = wave_sum(L);
    if (lane == 0) red[4 + wave] = L;
    __syncthreads();
    L = red[4] + red[5] + red[6] + red[7];
    f4 o = {0.f, 0.f, 0.f, 0.f};
    // chunks in the order c0 = sub, sub + 4 ns, ...; u = 0..3 within each
    auto batch = [&](int c0, const f4 (&x)[4]) {
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = min(c0 + u * ns, nchunks - 1);
            w[u] = c0 + u * ns < nchunks ? (c < 1024 ? wl[c] : expf(st[2 * c] - M)) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) o += w[u] * x[u];
    };
#pragma unroll
    for (int b = 0; b < MERGE1_PRE; ++b)
        if (sub + 4 * ns * b < nchunks) batch(sub + 4 * ns * b, xp[b]);
    for (int c0 = sub + 4 * ns * MERGE1_PRE; c0 < nchunks; c0 += 4 * ns) {
        f4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = min(c0 + u * ns, nchunks - 1);
            x[u] = *reinterpret_cast<const f4 *>(po + (size_t)c * hd + 4 * q);
        }
        batch(c0, x);
    }
    part[tid] = o;
    __syncthreads();
    if (tid < nq) {
        f4 r = part[tid];
        for (int s2 = 1; s2 < ns; ++s2) r += part[s2 * nq + tid];
        const float inv = 1.0f / L;
        *reinterpret_cast<f4 *>(a.o + (size_t)h * hd + 4 * tid) = r * inv;
    }
}

// ------------------------------------------------------------------ exact rows
// Causal attention of M rows at ~fp32 accuracy.  Workgroup (row r, KV head):
// the G <= 8 query heads of the KV head take columns 0..7 (high part) and
// 8..15 (low part) of the MFMA B operand, as in the single-query kernel, and
// the keys 0..pos are taken 32 at a time with an online softmax in fp32:
//   scores  S[key][g] = K[key] . q_g          (waves 0, 1: 16 keys each)
//   softmax update per head: running max m, sum l, rescale factor alpha
//   O[d][g] = alpha O[d][g] + sum_key V^T[d][key] p[g][key]  (all waves)
// The output o = O / l leaves as fp16 high and low parts, fragment-tiled.
template <int HD>
__global__ __launch_bounds__(256) void k_attn_rows_exact(AttnArgs a) {
    constexpr int NJ = HD / 64;  // 16-dim output tiles per wave
    __shared__ float sl[8][CH];
    __shared__ float mrun[8], lrun[8], alf[8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x, kvh = blockIdx.y;
    const int G = a.H / a.KVH;
    const int pos = a.row_pos ? a.row_pos[r] : a.pos0 + r;
    const __half *kp = a.k, *vtp = a.vt;
    const int32_t *page = nullptr;
    int vld = a.vld;
    if (a.seq_kv) {
        const KVRef &ref = a.seq_kv[a.row_seq[r]];
        kp = ref.k;
        vtp = ref.vt;
        vld = ref.vld;
        page = ref.page;
    }
    const int c = lane & 15, g = c & 7, lg = lane >> 4;
    const bool lo = c >= 8;
    const float scale = 1.0f / sqrtf((float)HD);
    // the B operand of the scores: q of head g (high or low part), dims ks*32 + 8 lg ..
    h8 qb[HD / 32];
    {
        const float *qrow = a.q32 + ((size_t)r * a.H + kvh * G + min(g, G - 1)) * HD + lg * 8;
#pragma unroll
        for (int ks = 0; ks < HD / 32; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = qrow[ks * 32 + e];
                const _Float16 h = (_Float16)v;
                qb[ks][e] = g < G ? (lo ? (_Float16)(v - (float)h) : h) : (_Float16)0.0f;
            }
        }
    }
    if (tid < 8) {
        mrun[tid] = -INFINITY;
        lrun[tid] = 0.f;
    }
    f4 oacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) oacc[j] = f4{0.f, 0.f, 0.f, 0.f};
    const int nch = (pos + CH) / CH;
    for (int ch = 0; ch < nch; ++ch) {
        const int k0 = ch * CH, nk = min(CH, pos + 1 - k0);
        const int c0 = kv_cell(page, k0);  // the chunk's keys lie in one page: cells c0 ..
        if (wave < CH / 16) {
            const int kt = wave * 16 + c;
            const int kr = min(kt, nk - 1);  // masked keys re-read a valid row
            const __half *krow = kp + ((size_t)(c0 + kr) * a.KVH + kvh) * HD + lg * 8;
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < HD / 32; ++ks)
                acc = mfma16(*reinterpret_cast<const h8 *>(krow + ks * 32), qb[ks], acc);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float v = acc[q] + row_ror<8>(acc[q]);
                const int kk = wave * 16 + 4 * lg + q;
                if (c < G) sl[c][kk] = kk < nk ? v * scale : -INFINITY;
            }
        }
        __syncthreads();
        for (int h = wave; h < G; h += 4) {
            const float sc = lane < CH ? sl[h][lane] : -INFINITY;
            const float mx = wave_max(sc);
            const float mold = mrun[h];
            const float mnew = fmaxf(mold, mx);
            const float p = lane < nk ? expf(sc - mnew) : 0.f;
            const float l = wave_sum(p);
            if (lane < CH) sl[h][lane] = p;
            if (lane == 0) {
                const float al = expf(mold - mnew);  // 0 for the first chunk (mold = -inf)
                alf[h] = al;
                lrun[h] = lrun[h] * al + l;
                mrun[h] = mnew;
            }
        }
        __syncthreads();
        h8 bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = g < G ? sl[g][lg * 8 + e] : 0.f;
            const _Float16 h = (_Float16)p;
            bv[e] = lo ? (_Float16)(p - (float)h) : h;
        }
        const float al = g < G ? alf[g] : 1.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int d = (wave + 4 * j) * 16 + c;
            h8 av = *reinterpret_cast<const h8 *>(vtp + ((size_t)kvh * HD + d) * vld + c0 + lg * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (lg * 8 + e >= nk) av[e] = (_Float16)0.0f;
            oacc[j] = mfma16(av, bv, oacc[j] * al);
        }
        __syncthreads();  // sl and alf are rewritten by the next chunk
    }
    const int od = a.H * HD;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float v = oacc[j][q] + row_ror<8>(oacc[j][q]);
            if (c < G) {
                const int h = kvh * G + c, d = (wave + 4 * j) * 16 + 4 * lg + q;
                const float o = v / lrun[c];
                const _Float16 hv = (_Float16)o;
                const size_t idx = tiled_index(r, h * HD + d, od);
                a.o[idx] = hv;
                a.o_lo[idx] = (_Float16)(o - (float)hv);
            }
        }
    }
}

int ok() { return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP; }

}  // namespace

// Eight compute waves of one group of 16 query columns: 128 columns per
// workgroup, two compute waves per SIMD.
constexpr int ATTN_CPW = 1, ATTN_NC = 8, ATTN_CB = 16 * ATTN_CPW * ATTN_NC;
constexpr int ATTN_MIN_KC = 64;  // keys per chunk at least, one 64-key stage (a 512-token prompt: 1 % faster than 128)

AttnSplit attn_split_cols(int colblocks, int KVH, int P) {
    int want = (256 + colblocks * KVH - 1) / (colblocks * KVH);
    want = std::max(1, std::min(want, ATTN_MAX_CHUNKS));
    int kc = (P + want - 1) / want;
    kc = std::max(ATTN_MIN_KC, (kc + 63) / 64 * 64);
    AttnSplit sp;
    sp.kc = kc;
    sp.nkc = (P + kc - 1) / kc;
    return sp;
}

// Key split of a launch's only unit, whose column blocks and KV heads number
// tot_cb: chunks enough for about ATTN_WG_TARGET workgroups (a launch of
// several units takes attn_common_kc).
constexpr int ATTN_WG_TARGET = 256;
AttnSplit attn_split_group(int P, int tot_cb) {
    int want = (ATTN_WG_TARGET + tot_cb - 1) / tot_cb;
    want = std::max(1, std::min(want, ATTN_MAX_CHUNKS));
    int kc = (P + want - 1) / want;
    kc = std::max(ATTN_MIN_KC, (kc + 63) / 64 * 64);
    AttnSplit sp;
    sp.kc = kc;
    sp.nkc = (P + kc - 1) / kc;
    return sp;
}

// One key-chunk length for every unit of a launch: the shortest (a multiple
// of 64, at least ATTN_MIN_KC) whose chunks over all the units' column
// blocks number at most ATTN_WG_TARGET workgroups, each unit at most
// ATTN_MAX_CHUNKS chunks.  A workgroup then never holds more keys than
// that length, so the units further into the prompt (more keys) take more
// workgroups rather than longer ones; splitting each unit into the same
// number of chunks instead let the last unit's workgroups run up to four
// times as long as the first unit's.  A launch of one unit gets the split
// of attn_split_group.  cb[i], P[i]: column blocks (KV heads included) and
// keys of unit i.
int attn_common_kc(const int *cb, const int *P, int n) {
    int pmax = ATTN_MIN_KC;
    for (int i = 0; i < n; ++i) pmax = std::max(pmax, P[i]);
    const int top = (pmax + 63) / 64 * 64;
    for (int kc = ATTN_MIN_KC; kc < top; kc += 64) {
        long wgs = 0;
        bool fits = true;
        for (int i = 0; i < n && fits; ++i) {
            const int nk = (P[i] + kc - 1) / kc;
            fits = nk <= ATTN_MAX_CHUNKS;
            wgs += (long)cb[i] * nk;
        }
        if (fits && wgs <= ATTN_WG_TARGET) return kc;
    }
    return top;
}

int attn_prefill_cols_per_wg(int hd) {
    (void)hd;
    return ATTN_CB;
}
size_t attn_prefill_scratch_floats(int M, int H, int hd, int n_ctx) {
    const int nkc = std::min(ATTN_MAX_CHUNKS, (n_ctx + ATTN_MIN_KC - 1) / ATTN_MIN_KC);
    return (size_t)nkc * M * H * (hd / 2 + 2);  // fp16 chunk outputs, then fp32 (max, sum) pairs
}

int launch_attn_prefill_group(const AttnArgs *units, int n, hipStream_t s) {
    if (n < 1 || n > kMaxUnits) return PPX_E_INVAL;
    AttnGroup g;
    int nx = 0, ny = 0;
    // the common key-chunk length of the single-sequence units
    int ucb[kMaxUnits], uP[kMaxUnits], nu = 0;
    for (int i = 0; i < n; ++i)
        if (units[i].M > 0 && !units[i].wg && units[i].KVH > 0) {
            ucb[nu] = (units[i].M * (units[i].H / units[i].KVH) + ATTN_CB - 1) / ATTN_CB * units[i].KVH;
            uP[nu++] = units[i].pos0 + units[i].M;
        }
    const int kc_all = nu > 1 ? attn_common_kc(ucb, uP, nu) : 0;
    for (int i = 0; i < n; ++i) {
        AttnArgs a = units[i];
        if (a.M <= 0) continue;
        const int G = a.H / a.KVH;
        if (a.H % a.KVH || 64 % G) return PPX_E_UNSUPPORTED;
        if (g.n && (a.H != g.u[0].H || a.KVH != g.u[0].KVH || a.hd != g.u[0].hd || !a.wg != !g.u[0].wg))
            return PPX_E_INVAL;
        int x;
        if (a.wg) {
            // several sequences: the caller built the workgroup table and the split
            if (a.nwg < 1 || !a.seq_kv || !a.row_pos || a.kc < ATTN_MIN_KC || a.kc % 64 || a.nkc < 1 ||
                a.nkc > ATTN_MAX_CHUNKS)
                return PPX_E_INVAL;
            x = a.nwg;
        } else {
            if (a.vld % 64 || a.pos0 + a.M > a.vld) return PPX_E_UNSUPPORTED;
            if (kc_all) {
                a.kc = kc_all;
                a.nkc = (a.pos0 + a.M + kc_all - 1) / kc_all;
            } else {
                const AttnSplit sp = attn_split_group(a.pos0 + a.M, std::max(nu ? ucb[0] : 1, 1));
                a.kc = sp.kc;
                a.nkc = sp.nkc;
            }
            x = (a.M * G + ATTN_CB - 1) / ATTN_CB;
        }
        if (a.nkc > 1 && !a.part) return PPX_E_INVAL;
        nx = std::max(nx, x);
        ny = std::max(ny, a.nkc);
        g.u[g.n++] = a;
    }
    if (!g.n) return PPX_OK;
    const AttnArgs &a0 = g.u[0];
    dim3 grid(nx, ny, a0.KVH * g.n);
    switch (a0.hd) {
#define PPX_ATTN(hd_, np_, depth_)                                                                   \
    case hd_: {                                                                                      \
        using C = ACfg<hd_, ATTN_CPW, ATTN_NC, np_, depth_>;                                         \
        hipLaunchKernelGGL((k_attn_prefill<C>), grid, dim3(C::NT), 0, s, g);                         \
        break;                                                                                       \
    }
#define PPX_ATTN_W(hd_, nc_, cpw_, np_)                                                              \
    case hd_: {                                                                                      \
        using C = WCfg<hd_, nc_, cpw_, np_>;                                                         \
        static_assert(C::CB == ATTN_CB, "query columns per workgroup");                              \
        hipLaunchKernelGGL((k_attn_prefill_w<C>), grid, dim3(C::NT), 0, s, g);                       \
        break;                                                                                       \
    }
        PPX_ATTN(64, 1, 8)
        PPX_ATTN(128, 2, 6)
        PPX_ATTN_W(256, 8, 1, 4)
#undef PPX_ATTN
#undef PPX_ATTN_W
    default: return PPX_E_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return PPX_E_HIP;
    // the key-chunk merge, for the units whose keys were split
    AttnGroup mg;
    int mrows = 0;
    for (int i = 0; i < g.n; ++i)
        if (g.u[i].nkc > 1) {
            mg.u[mg.n++] = g.u[i];
            mrows = std::max(mrows, g.u[i].M);
        }
    if (!mg.n) return PPX_OK;
    const dim3 mgrid(mrows, mg.n);  // one workgroup per row
    switch (a0.hd) {
    case 64: hipLaunchKernelGGL(k_attn_prefill_merge<64>, mgrid, dim3(256), 0, s, mg); break;
    case 128: hipLaunchKernelGGL(k_attn_prefill_merge<128>, mgrid, dim3(256), 0, s, mg); break;
    default: hipLaunchKernelGGL(k_attn_prefill_merge<256>, mgrid, dim3(256), 0, s, mg); break;
    }
    return ok();
}

int launch_attn_prefill(const AttnArgs &a, hipStream_t s) { return launch_attn_prefill_group(&a, 1, s); }

int launch_attn_rows_exact(const AttnArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    const int G = a.KVH > 0 ? a.H / a.KVH : 0;
    if (!a.q32 || !a.o || !a.o_lo || G < 1 || G > 8 || a.H % a.KVH) return PPX_E_UNSUPPORTED;
    if (a.seq_kv ? (!a.row_pos || !a.row_seq) : (!a.k || !a.vt || a.vld % 64 || a.pos0 + a.M > a.vld))
        return PPX_E_UNSUPPORTED;
    dim3 grid(a.M, a.KVH);
    switch (a.hd) {
    case 64: hipLaunchKernelGGL(k_attn_rows_exact<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn_rows_exact<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(k_attn_rows_exact<256>, grid, dim3(256), 0, s, a); break;
    default: return PPX_E_UNSUPPORTED;
    }
    return ok();
}

size_t attn1_scratch_floats(int H, int hd, int n_pos) {
    const int chunks = (n_pos + CH - 1) / CH;
    return (size_t)chunks * H * (hd + 2);
}

int launch_attn_1row(const Attn1Args &a, hipStream_t s) {
    const int G = a.H / a.KVH;
    if (a.H % a.KVH || G > 8 || a.pos < 0 || !a.partial || a.vld % 64 || a.pos >= a.vld)
        return PPX_E_UNSUPPORTED;
    const int chunks = (a.pos + 1 + CH - 1) / CH;
    dim3 grid(chunks, a.KVH);
    switch (a.hd) {
    case 64: hipLaunchKernelGGL(k_attn_1row<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn_1row<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(k_attn_1row<256>, grid, dim3(256), 0, s, a); break;
    default: return PPX_E_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return PPX_E_HIP;
    hipLaunchKernelGGL(k_attn_merge, dim3(a.H), dim3(256), 0, s, a, chunks);
    return ok();
}

}  // namespace ppx
