// Internal declarations shared by the engine's host code and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/ppx.h"

namespace ppx {

// Repacked Q4_0 matrix W[N][K] (N % 16 == 0, K % 64 == 0).
//
// The MFMA v_mfma_f32_16x16x32_f16 B operand gives lane l the column
// n = l % 16 and eight consecutive k's of a 32-wide block, k = 8*(l/16)+0..7.
// One Q4_0 block is exactly one such K step.  For every 16-column group and
// every 64-wide K chunk (two blocks) the repacked layout stores, per lane, two
// 32-bit words (block 0, block 1) holding that lane's eight 4-bit codes,
// arranged so that (w >> 4i) & 0x000F000F yields the codes of k = 2i and
// 2i+1 in the two 16-bit halves; and per column its two fp16 block scales.
//   nib[((g * (K/64) + c) * 64 + lane) * 2 + s]   uint32
//   scl[((g * (K/64) + c) * 16 + col) * 2 + s]    fp16
// with g = n / 16, c = k / 64, s = (k / 32) % 2.  The decoded weight is
// d * (code - 8), identical to the container's Q4_0 block.
struct Q4R {
    const uint32_t *nib = nullptr;
    const __half *scl = nullptr;
    int N = 0, K = 0;
};

enum Act { ACT_GEGLU = 0, ACT_SWIGLU = 1 };

struct LayerW {
    bool own = false;
    int src = 0;        // KV source layer (own: itself)
    float ple_s = 0.f;  // per-layer embedding scale
    const float *attn_norm = nullptr, *ffn_norm = nullptr, *ple_norm = nullptr;
    Q4R wq;    // [qd][d], rows in rope-pair order
    Q4R wkv;   // own only: [2 kvd][d] rows K (rope-pair order) | V; run on the exact-weight path
    Q4R wo;    // [d][qd]
    Q4R wgu;   // [2F][d]: 8-row blocks alternate gate, up
    Q4R wdown; // [d][F]
    Q4R wpg;   // [E][d]
    Q4R wpu;   // [d][E]
};

struct HostTensor {
    int type;  // 0 f32, 1 q4_0
    uint64_t rows, cols, offset;
};

}  // namespace ppx

struct ppx_model {
    ppx_model_info info{};
    int tied = 1;
    float eps = 1e-6f, rope_base = 10000.f, embd_scale = 1.f;
    std::vector<ppx::LayerW> layers;
    ppx::Q4R tok, out;  // out == tok when tied
    const float *out_norm = nullptr;
    const float *nextn_norm = nullptr;  // the next-n head's gain (has_nextn)
    const uint8_t *ple_raw = nullptr;  // raw Q4_0 blocks [V][L*E/32][18]
    void *dev = nullptr;               // one allocation for all weights
    size_t dev_bytes = 0;
    bool dev_owned = true;             // false: the caller's memory (ppx_model_load_into)
    float2 *rope = nullptr;            // [rope_n][head_dim/2] (cos, sin)
    int rope_n = 0;
    // named tensors for the kernel-level entry points
    std::unordered_map<std::string, ppx::Q4R> q4;
    std::unordered_map<std::string, int> q4_kind;  // 0 plain, 1 qkv, 2 gate|up
    std::vector<hipEvent_t> events;                // reusable pool for per-phase timing
    // Recorded prefill launch sequences (HIP graphs), keyed by everything the
    // kernels' arguments depend on; token ids are read from device memory.
    struct Graph {
        const void *kv_k = nullptr, *kv_vt = nullptr, *ws = nullptr, *logits = nullptr, *nextn = nullptr;
        int n_ctx = 0, n = 0, p0 = 0, ub = 0, prune = 0, exact = 0;
        hipGraphExec_t exec = nullptr;
        unsigned long long last_use = 0;
    };
    std::vector<Graph> graphs;
    // recorded multi-sequence launch sequences, keyed by their shape
    struct KeyedGraph {
        std::vector<long long> key;
        hipGraphExec_t exec = nullptr;
        unsigned long long last_use = 0;
    };
    std::vector<KeyedGraph> keyed_graphs;
    unsigned long long graph_clock = 0;
    hipStream_t capture_stream = nullptr;  // recording only; graphs run on the caller's stream
    // pinned host staging of the per-row tables of a multi-sequence prefill;
    // stage_event marks the end of the last copy out of it
    void *stage_host = nullptr;
    size_t stage_bytes = 0;
    hipEvent_t stage_event = nullptr;
};

// A unified cache: one buffer for every sequence.  Cells are handed out in
// pages of kKvPage consecutive positions of one sequence; page_seq holds each
// page's sequence (-1: free), pages[s] sequence s's pages in position order.
struct ppx_kvu {
    const ppx_model *m = nullptr;
    __half *k = nullptr;   // [Ls][n_cells][kv_dim]
    __half *vt = nullptr;  // [Ls][kv_dim][n_cells]: V transposed, as in ppx_kv
    int n_cells = 0, n_seq_max = 0;
    std::vector<int32_t> page_seq;
    std::vector<std::vector<int32_t>> pages;
    std::vector<int> n_pos;
};

struct ppx_kv {
    const ppx_model *m = nullptr;
    __half *k = nullptr;   // [Ls][n_ctx][kv_dim]
    __half *vt = nullptr;  // [Ls][kv_dim][vld]: V transposed, row d = kv_head * head_dim + dim
    int n_ctx = 0, n_pos = 0;
    int vld = 0;           // n_ctx rounded up to a multiple of 64
};

namespace ppx {

// ---------------------------------------------------------------- launchers

// GEMM epilogues
enum GemmEpi {
    EPI_F32 = 0,  // C -> fp32 out[M][N]
    EPI_ADD = 1,  // resid[M][N] += C
    EPI_QKV = 2,  // rope(Q) -> q16, rope(K), V -> fp16 cache rows
    EPI_GLU = 3,  // act(gate) * up -> fp16 h[M][F]; in every 16-column group of the fused
                  // weight, columns 0-7 are gate rows 8t..8t+7 and columns 8-15 the up rows
    EPI_PLE = 4,  // gelu(C) * s * deq(ple_table[tok]) -> fp16 [M][E]
};

// One sequence's cache of one layer, for row batches that span several
// sequences.  Split caches: the sequence's own buffer, position p in row p.
// Unified cache: the one buffer of all sequences, position p in cell
// page[p / kKvPage] * kKvPage + p % kKvPage (kv_cell).
struct KVRef {
    __half *k = nullptr;           // [n_ctx][kv_dim]  (unified: [n_cells][kv_dim])
    __half *vt = nullptr;          // [kv_dim][vld]    (unified: vld = n_cells)
    const int32_t *page = nullptr; // null: split; else the sequence's page table
    int vld = 0;
    int pad = 0;
};

// Cells per page of a unified cache: a page holds consecutive positions of
// one sequence, so every 32-key stage of the attention kernels lies in one page.
constexpr int kKvPage = 64;
__host__ __device__ inline int kv_cell(const int32_t *page, int p) {
    return page ? page[p / kKvPage] * kKvPage + p % kKvPage : p;
}

struct GemmArgs {
    const __half *A = nullptr;  // [M][K] fp16, fragment-tiled (the high part on the exact-weight path)
    const __half *A2 = nullptr; // [M][K] fp16 low part a - fp16(a), tiled (exact-weight path only)
    int lda = 0;                // unused: the tiled layout's row stride is K
    int M = 0;
    Q4R W;
    int epi = EPI_F32;
    float *out_f32 = nullptr;   // EPI_F32 (ld = N), EPI_ADD residual (ld = N)
    __half *out_f16 = nullptr;  // EPI_QKV q16 [M][qd] row-major; EPI_GLU h [M][F], EPI_PLE [M][E] tiled
    // exact-precision outputs (the exact-weight kernel only): EPI_QKV writes Q
    // in fp32 to q32 [M][qd] row-major instead of q16; EPI_GLU / EPI_PLE also
    // write the low part fp16(v - fp16(v)) to out_lo, tiled as out_f16
    float *q32 = nullptr;
    __half *out_lo = nullptr;
    // rope / cache (EPI_QKV)
    int qd = 0, kvd = 0, hd = 0;
    int pos0 = 0;               // position of row 0
    const float2 *rope = nullptr;
    __half *kc = nullptr;       // K cache of this layer [n_ctx][kvd]
    __half *vc = nullptr;       // V cache of this layer, transposed [kvd][vld]
    int vld = 0;
    int act = ACT_GEGLU;
    // per-layer embedding (EPI_PLE)
    const uint8_t *ple_raw = nullptr;
    const int32_t *tok = nullptr;  // [M] token ids of the rows
    int ple_row_blocks = 0;        // L*E/32
    int ple_col0 = 0;              // il*E
    float ple_s = 0.f;
    // EPI_QKV rows of several sequences (null: one sequence, row r at pos0 + r
    // in kc / vc): row r's position, and for the K|V projection its sequence,
    // whose cache of this layer is seq_kv[row_seq[r]].
    const int32_t *row_pos = nullptr;
    const int32_t *row_seq = nullptr;
    const KVRef *seq_kv = nullptr;
    // the gathered output rows of several sequences: tiles chosen by row count
    // (other calls use plans that do not depend on M)
    bool few_rows = false;
    // K split over workgroups: fp32 partial tiles, summed in split order by a
    // second kernel that applies the epilogue.  Null: no split.
    float *part = nullptr;
    size_t part_floats = 0;
    // EPI_ADD only: after the residual update, RMS-normalise the updated rows with
    // gain norm_g into norm_out (fp16, fragment-tiled) -- fused into the split-K
    // reduction when the K split is used, a separate pass otherwise.  Null: none.
    const float *norm_g = nullptr;
    float norm_eps = 0.f;
    __half *norm_out = nullptr;
};
int launch_gemm(const GemmArgs &a, hipStream_t s);

// Ubatches in flight at once in a prefill: each step runs every in-flight
// ubatch through its next row-batched layer, and the step's identical
// operations run as one launch over the units (ubatch, layer).
constexpr int kMaxUnits = 8;
struct GemmGroup {
    int n = 0;
    GemmArgs u[kMaxUnits];
};
// One launch of the same product (same N, K, epilogue) for n <= kMaxUnits
// units with their own operands, rows (M) and outputs.
int launch_gemm_group(const GemmArgs *units, int n, hipStream_t s);
int launch_gemm_exact_group(const GemmArgs *units, int n, hipStream_t s);
// fp32 words of split-K partials launch_gemm would use for an M x N x K GEMM
// (0: that shape is not split).
size_t gemm_part_floats(int M, int N, int K);
// Exact-weight variant: B = (code - 8) exactly in fp16, A = A + A2 (split fp16),
// block scales applied to each 32-wide partial in fp32.  Used for K and V.
int launch_gemm_exact(const GemmArgs &a, hipStream_t s);

enum GemvEpi {
    GV_F32 = 0,   // y -> out[N]
    GV_ADD = 1,   // resid[N] += y
    GV_QROPE = 2, // rope(Q part) -> out fp32 [qd] (natural order), pos
    GV_GLU = 3,   // act(gate)*up -> out fp32 [F]
    GV_PLE = 4,   // gelu(y) * s * deq(ple row) -> out fp32 [E]
    GV_KV = 5,    // fused K|V weight: rope(K) and V -> fp16 cache at pos (K rows, V^T columns)
};
struct GemvArgs {
    const float *x = nullptr;  // [K]
    const float *norm_g = nullptr;  // if set: x is RMS-normalised with this gain first
    float eps = 0.f;
    Q4R W;
    int epi = GV_F32;
    float *out = nullptr;
    int hd = 0, pos = 0;
    const float2 *rope = nullptr;
    int act = ACT_GEGLU;
    const uint8_t *ple_raw = nullptr;
    const int32_t *tok = nullptr;  // device pointer to the row's token id
    int ple_row_blocks = 0, ple_col0 = 0;
    float ple_s = 0.f;
    __half *kc = nullptr;   // GV_KV: K cache of the layer [n_ctx][kvd]
    __half *vt = nullptr;   // GV_KV: V cache of the layer, transposed [kvd][vld]
    int kvd = 0, vld = 0;
    // Optional second matrix over the same (normalised) row, finished with
    // epi2 (the K|V projection beside Q in one launch): its units follow W's.
    // Both epilogues must take the same column pairing.  W2.N == 0: none.
    Q4R W2;
    int epi2 = GV_F32;
};
int launch_gemv(const GemvArgs &a, hipStream_t s);

constexpr int ATTN_MAX_CHUNKS = 16;
struct AttnSplit {
    int kc = 0, nkc = 1;  // keys per chunk (multiple of 64), chunks
};
// The same rule for a launch of `colblocks` workgroup column blocks per KV
// head whose longest sequence segment ends at position P - 1.
AttnSplit attn_split_cols(int colblocks, int KVH, int P);
// Query columns ((row, head-in-group) pairs) one prefill attention workgroup owns.
int attn_prefill_cols_per_wg(int hd);

// A workgroup of a row-batched attention launch over several sequences: rows
// [row0, row0 + M) of the launch are one sequence's positions pos0 .. pos0+M-1,
// and the workgroup owns column block cb of them.
struct AttnWg {
    int row0, M, pos0, seq, cb;
    int pad[3];
};
size_t attn_prefill_scratch_floats(int M, int H, int hd, int n_ctx);

struct AttnArgs {
    const __half *q = nullptr;   // [M][H][hd]
    const __half *k = nullptr;   // K cache of the source layer [P][KVH][hd]
    const __half *vt = nullptr;  // V cache of the source layer, transposed [KVH][hd][vld]
    int vld = 0;                 // multiple of 64, >= pos0 + M
    __half *o = nullptr;         // [M][H*hd], fragment-tiled (the O projection's A operand)
    int M = 0, H = 0, KVH = 0, hd = 0, pos0 = 0;
    int kc = 0, nkc = 1;         // key split (set by the launcher)
    float *part = nullptr;       // scratch of attn_prefill_scratch_floats(M, H, hd, pos0 + M) floats
    // Rows of several sequences (null wg: one sequence, k / vt / pos0 above):
    // workgroup x of the launch is wg[x]; sequence s reads the cache seq_kv[s];
    // row r is at position row_pos[r].  kc / nkc are then set by the caller
    // (attn_split_cols), every segment satisfies pos0 + M <= its vld.
    const AttnWg *wg = nullptr;
    int nwg = 0;
    const KVRef *seq_kv = nullptr;
    const int32_t *row_pos = nullptr;
    // exact precision: q32 fp32 [M][H][hd] replaces q; the output goes to o
    // (high part) and o_lo (fp16(v - fp16(v))), both fragment-tiled; with
    // rows of several sequences row r reads the cache seq_kv[row_seq[r]]
    const float *q32 = nullptr;
    __half *o_lo = nullptr;
    const int32_t *row_seq = nullptr;
};
int launch_attn_prefill(const AttnArgs &a, hipStream_t s);
// The per-layer-embedding block of one unit (rows of one ubatch and layer):
// x[M][d] += (gelu(a wg^T) * s * deq(ple_table[tok][ple_col0 + j])) wu^T,
// a the fp16 fragment-tiled RMSNorm of x with the block's gain.
struct PleArgs {
    const __half *a = nullptr;
    float *x = nullptr;
    Q4R wg, wu;                    // [E][d] and [d][E]
    const uint8_t *ple_raw = nullptr;
    const int32_t *tok = nullptr;  // [M]
    int ple_row_blocks = 0, ple_col0 = 0, M = 0;
    float ple_s = 0.f;
};
struct PleGroup {
    PleArgs u[kMaxUnits];
    int n = 0;
};
bool ple_fused_supported(int E, int d);
int launch_ple_group(const PleArgs *units, int n, hipStream_t s);

struct AttnGroup {
    int n = 0;
    AttnArgs u[kMaxUnits];
};
// Prefill attention of n units (same H, KVH, hd; their own queries, caches,
// positions and outputs) in one launch, each with its own key split.
int launch_attn_prefill_group(const AttnArgs *units, int n, hipStream_t s);
// Causal attention of M rows at ~fp32 accuracy (exact precision): one
// workgroup per (row, KV head) runs an online softmax over 32-key chunks with
// both products on MFMA, every fp32 operand split into fp16 high and low parts
// against the exact fp16 keys and values.  Needs a.q32 and a.o_lo; a.part is
// not used.
int launch_attn_rows_exact(const AttnArgs &a, hipStream_t s);

struct Attn1Args {
    const float *q = nullptr;  // [H][hd]
    const __half *k = nullptr;   // [P][KVH][hd]
    const __half *vt = nullptr;  // [KVH][hd][vld]
    int vld = 0;
    float *o = nullptr;        // [H*hd]
    int H = 0, KVH = 0, hd = 0, pos = 0;
    float *partial = nullptr;  // scratch of attn1_scratch_floats(H, hd, pos + 1) floats
};
int launch_attn_1row(const Attn1Args &a, hipStream_t s);
size_t attn1_scratch_floats(int H, int hd, int n_pos);

int launch_embed(const Q4R &tok, const int32_t *ids, int M, float scale, float *x, hipStream_t s);
int launch_stream_read(const void *src, size_t bytes, uint32_t *out, int grid, hipStream_t s);
int launch_embed_add(const Q4R &tok, const int32_t *id, float scale, const float *base, float *x, hipStream_t s);
// y = rmsnorm(x) * g -> fp16 in the fragment-tiled layout (the GEMM A operand).
int launch_rmsnorm_f16(const float *x, const float *g, float eps, int M, int d, __half *out,
                       hipStream_t s);
// The RMSNorm of n units' rows in one launch: unit i normalises x[i] (M[i]
// rows of d) with gain g[i] into hi[i] (and lo[i] when lo is set).
struct NormUnit {
    const float *x = nullptr;
    const float *g = nullptr;
    __half *hi = nullptr, *lo = nullptr;
    int M = 0;
};
struct NormGroup {
    int n = 0;
    NormUnit u[kMaxUnits];
};
int launch_rmsnorm_group(const NormUnit *units, int n, float eps, int d, bool lo, hipStream_t s);
// As launch_rmsnorm_f16, also writing lo = fp16(y - fp16(y)), tiled the same way.
int launch_rmsnorm_split(const float *x, const float *g, float eps, int M, int d, __half *hi, __half *lo,
                         hipStream_t s);
int launch_rmsnorm_f32(const float *x, const float *g, float eps, int M, int d, float *out,
                       hipStream_t s);
int launch_dequant(const Q4R &w, float *out, hipStream_t s);
// Row-major fp16 [M][K] -> fragment-tiled (K % 32 == 0).
int launch_tile_f16(const __half *src, int M, int K, __half *dst, hipStream_t s);
int launch_copy_f32(const float *src, float *dst, int n, hipStream_t s);
int launch_fill_u32(uint32_t *p, uint32_t v, size_t n, hipStream_t s);
// dst row pairs[i].y = src row pairs[i].x (fp32 rows of d values), i < n.
int launch_gather_rows(const float *src, int d, const int2 *pairs, int n, float *dst, hipStream_t s);
// dst[c * ld + r] = src[r * lds + c] (16-bit values, rows x cols).
int launch_transpose_u16(const uint16_t *src, int rows, int cols, size_t lds, uint16_t *dst, size_t ld,
                         hipStream_t s);

}  // namespace ppx
