// Q4_0 dequant-fused GEMM on CDNA4 MFMA (v_mfma_f32_16x16x32_f16).
//
//   C[M][N] = A[M][K] (fp16 activations, fragment-tiled) x W[N][K]^T (Q4_0),
//   fp32 accumulate, with the layer's elementwise work fused into the epilogue.
//
// Two kernels share the epilogue:
//
// k_q4gemm_p -- the row-batched projections (fast mode).  A workgroup holds
// NWN x KS compute waves and NP producer waves and computes a BM x BN tile
// over a K range (the whole K, or one of S ranges when the K split goes
// across workgroups).  Compute wave (w, g) owns columns [w*WN, (w+1)*WN) for
// all BM rows (TM x TN MFMA tiles of 16 x 16) over the g-th of KS slices of
// the range.
//   * The producer waves stream everything a stage needs into a ring of DEPTH
//     LDS stages with global_load_lds DMA: per K group one 64-wide K step of
//     A (1 KB fragments, contiguous in the fragment-tiled layout, landing in
//     A-operand order) and the repacked weight codes and block scales of the
//     workgroup's columns, each wave an equal share.  Stage s is handed over at
//     barrier s once every producer's outstanding-DMA count says its share of
//     stage s has landed, so DEPTH - 1 stages are in flight behind the one in
//     use.  (DMA lives in waves of its own because the
//     compiler makes any LDS read that follows an LDS DMA in the same wave wait
//     for all DMA; one wave issues DMA at only a fraction of what the CU can
//     take in, so wide tiles use several.)
//   * Compute waves never touch global memory in the main loop: per stage they
//     read A fragments and the stage's codes from LDS and decode the codes (a
//     shift, a mask, an OR with the fp16 exponent of 1024, a subtract and a
//     multiply per pair); with two compute waves per SIMD one wave's decode
//     runs beside the other's MFMAs.  (Decoding the next stage's codes during
//     this stage's MFMAs instead kept one stage fewer in flight: measured
//     slower, 26.7 vs 25.7 us for the E2B-like gate|up at M = 512.)
//   * The KS partial tiles meet in LDS in slice order; the waves of up to KS
//     groups then finish TM/KS row tiles each, spreading the epilogue.
//   * With a K split across S workgroups, each writes its fp32 partial tile;
//     k_gemm_reduce sums the S partials in split order and runs the epilogue.
//   Every summation order is fixed, so results are deterministic.
//
// k_q4gemm -- the exact-weight mode (the K|V projection): B = code - 8
// (exact in fp16), A = hi + lo (two fp16 arrays), each 32-wide block's partial
// scaled by its fp32 block scale before it is added -- only fp32 accumulation
// rounds, so the cache holds values accurate to the fp16 store itself.  Its
// weights stream from global memory into registers, four K steps ahead.
//
// Fast-mode B = fp16(d * (code - 8)): one rounding per weight.
#include "ppx_dev.h"

namespace ppx {

namespace {

typedef __attribute__((address_space(3))) void lds_t;

// DMA of 16 / 4 bytes per lane from global memory to LDS; lane l's bytes land
// at dst + size * l (dst is wave-uniform).
__device__ __forceinline__ void dma16(const void *src, h8 *dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_t *)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *src, h8 *dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_t *)dst, 4, 0, 0);
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Workgroup barrier without the memory fences of __syncthreads (which would
// drain every outstanding DMA); the empty asm statements keep memory accesses
// on their side of it in the compiler.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N), expcnt and lgkmcnt untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// The value of lane (l + 8) mod 16 within each 16-lane row (DPP row rotate).
__device__ __forceinline__ float row_swap8(float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

// Epilogue of one wave tile: acc[i][j][r] = C[r0 + 16i + 4(lane/16) + r][c0 + 16j + lane%16].
template <int TM, int TN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &a, const f4 (&acc)[TM][TN], int r0, int c0, int lane,
                                              _Float16 *stage = nullptr) {
    const int lc = lane & 15, lr = (lane >> 4) * 4;
    const int N = a.W.N;
    if (a.epi == EPI_F32 || a.epi == EPI_ADD) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = r0 + i * 16 + lr + r;
                    const int col = c0 + j * 16 + lc;
                    if (row < a.M) {
                        float *p = a.out_f32 + (size_t)row * N + col;
                        if (a.epi == EPI_ADD) *p += acc[i][j][r];
                        else *p = acc[i][j][r];
                    }
                }
    } else if (a.epi == EPI_PLE) {
        // gelu(C) * s * deq(ple_table[token][il*E + col]) -> fp16, fragment-tiled [M][E]
        const int E = N;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = r0 + i * 16 + lr + r;
                if (row >= a.M) continue;
                const uint8_t *prow = a.ple_raw + (size_t)a.tok[row] * a.ple_row_blocks * 18;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = c0 + j * 16 + lc;
                    const float P = a.ple_s * q4_raw_weight(prow, a.ple_col0 + col);
                    const float v = gelu_tanh_f(acc[i][j][r]) * P;
                    const _Float16 hv = (_Float16)v;
                    a.out_f16[tiled_index(row, col, E)] = hv;
                    if (a.out_lo) a.out_lo[tiled_index(row, col, E)] = (_Float16)(v - (float)hv);
                }
            }
    } else if (a.epi == EPI_GLU) {
        // lane c < 8 of a 16-lane row holds gate f = 8t + c of 16-column group t,
        // lane c + 8 the matching up: after a swap of the two halves of the row,
        // lanes c < 8 finish the first two of the lane group's four rows and
        // lanes c >= 8 the last two.
        const int F = N >> 1;
        const bool lo = lc < 8;
        if (stage) {
            // through this wave's LDS staging area (TM x TN x 16 units of 16 bytes:
            // eight consecutive f of one row), so that the tiled output is written
            // one 16-byte unit per lane
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float v0 = acc[i][j][2 * h], v1 = acc[i][j][2 * h + 1];
                        const float p0 = row_swap8(v0), p1 = row_swap8(v1);
                        if (lo == (h == 0)) {
                            const float g0 = lo ? v0 : p0, u0 = lo ? p0 : v0;
                            const float g1 = lo ? v1 : p1, u1 = lo ? p1 : v1;
                            _Float16 *u = stage + ((i * TN + j) * 16 + lr + 2 * h) * 8 + (lc & 7);
                            u[0] = (_Float16)(act_f(a.act, g0) * u0);
                            u[8] = (_Float16)(act_f(a.act, g1) * u1);
                        }
                    }
#pragma unroll
            for (int u = lane; u < TM * TN * 16; u += 64) {
                const int i = u / (TN * 16), j = (u / 16) % TN, rr = u % 16;
                const int row = r0 + i * 16 + rr;
                const h8 v = *reinterpret_cast<const h8 *>(stage + u * 8);
                if (row < a.M) *reinterpret_cast<h8 *>(a.out_f16 + tiled_index(row, ((c0 >> 4) + j) * 8, F)) = v;
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int f = ((c0 >> 4) + j) * 8 + (lc & 7);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float v0 = acc[i][j][2 * h], v1 = acc[i][j][2 * h + 1];
                    const float p0 = row_swap8(v0), p1 = row_swap8(v1);
                    if (lo == (h == 0)) {
                        const float g0 = lo ? v0 : p0, u0 = lo ? p0 : v0;
                        const float g1 = lo ? v1 : p1, u1 = lo ? p1 : v1;
                        const int row = r0 + i * 16 + lr + 2 * h;
                        const float y0 = act_f(a.act, g0) * u0, y1 = act_f(a.act, g1) * u1;
                        const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
                        if (row < a.M) a.out_f16[tiled_index(row, f, F)] = h0;
                        if (row + 1 < a.M) a.out_f16[tiled_index(row + 1, f, F)] = h1;
                        if (a.out_lo) {
                            if (row < a.M) a.out_lo[tiled_index(row, f, F)] = (_Float16)(y0 - (float)h0);
                            if (row + 1 < a.M) a.out_lo[tiled_index(row + 1, f, F)] = (_Float16)(y1 - (float)h1);
                        }
                    }
                }
            }
    } else {
        // EPI_QKV: 16-column groups (2p, 2p+1) of the wave tile hold the first and
        // second RoPE half of 16 dimensions.  Columns [0,qd) Q, [qd,qd+kvd) K,
        // [qd+kvd, qd+2kvd) V.  Rows of several sequences take their position
        // and their sequence's cache from the per-row tables.
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
            const int colA = c0 + p * 32 + lc;  // first member; second = colA + 16
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = r0 + i * 16 + lr + r;
                    if (row >= a.M) continue;
                    const float va = acc[i][2 * p][r], vb = acc[i][2 * p + 1][r];
                    const int hd = a.hd, half = hd >> 1;
                    const int pos = a.row_pos ? a.row_pos[row] : a.pos0 + row;
                    if (colA < a.qd + a.kvd) {
                        const bool isq = colA < a.qd;
                        const int c = isq ? colA : colA - a.qd;
                        const int h = c / hd, rr = c % hd;
                        const int ii = (rr >> 5) * 16 + lc;  // dimension in the first half
                        const float2 cs = a.rope[(size_t)pos * half + ii];
                        const float ra = va * cs.x - vb * cs.y;
                        const float rb = va * cs.y + vb * cs.x;
                        if (isq && a.q32) {
                            float *q = a.q32 + (size_t)row * a.qd + h * hd;
                            q[ii] = ra;
                            q[ii + half] = rb;
                        } else if (isq) {
                            __half *q = a.out_f16 + (size_t)row * a.qd + h * hd;
                            q[ii] = __float2half(ra);
                            q[ii + half] = __float2half(rb);
                        } else {
                            __half *kc = a.kc;
                            int cell = pos;
                            if (a.seq_kv) {
                                const KVRef &ref = a.seq_kv[a.row_seq[row]];
                                kc = ref.k;
                                cell = kv_cell(ref.page, pos);
                            }
                            __half *k = kc + (size_t)cell * a.kvd + h * hd;
                            k[ii] = __float2half(ra);
                            k[ii + half] = __float2half(rb);
                        }
                    } else {
                        const int c = colA - a.qd - a.kvd;
                        __half *vc = a.vc;
                        int vld = a.vld, cell = pos;
                        if (a.seq_kv) {
                            const KVRef &ref = a.seq_kv[a.row_seq[row]];
                            vc = ref.vt;
                            vld = ref.vld;
                            cell = kv_cell(ref.page, pos);
                        }
                        vc[(size_t)c * vld + cell] = __float2half(va);  // V^T
                        vc[(size_t)(c + 16) * vld + cell] = __float2half(vb);
                    }
                }
        }
    }
}

// ------------------------------------------------------------ pipelined kernel

template <int TM_, int TN_, int NWN_, int KS_, int DEPTH_, int NP_ = 1>
struct PCfg {
    static constexpr int TM = TM_, TN = TN_, NWN = NWN_, KS = KS_, DEPTH = DEPTH_, NP = NP_;
    static constexpr int NCW = NWN * KS;             // compute waves
    static constexpr int NT = 64 * (NCW + NP);
    static constexpr int BM = 16 * TM, WN = 16 * TN, BN = NWN * WN;
    static constexpr int AFR = 2 * TM;               // A fragments per K group and stage
    static constexpr int NB = NWN * TN * KS;         // weight blocks (16 columns x 64 k) per stage
    static constexpr int NBP = (NB + 1) / 2 * 2, NSP = (NB + 3) / 4 * 4;
    static constexpr int A_UNITS = KS * AFR * 64;    // 16-byte units of a stage
    static constexpr int B_UNITS = NBP * 32;         // 512 B of codes per block
    static constexpr int S_UNITS = NSP * 4;          // 64 B of scales per block
    static constexpr int STAGE_UNITS = A_UNITS + B_UNITS + S_UNITS;
    // DMAs of a stage: A fragments, code pairs, scale quads; each producer wave
    // issues PER of them (the last one repeated where the count does not divide)
    static constexpr int A_TOT = KS * AFR, B_TOT = NBP / 2, S_TOT = NSP / 4;
    static constexpr int DMA_STAGE = A_TOT + B_TOT + S_TOT;
    static constexpr int PER = (DMA_STAGE + NP - 1) / NP;
    // K groups that finish rows (NFG), TMS row tiles each
    static constexpr int NFG = (TM % KS == 0) ? KS : 1;
    static constexpr int TMS = TM / NFG;
    static constexpr int SLOT_FLOATS = TMS * TN * 4 * 64;
    static constexpr int XCH_FLOATS = (KS * NFG - NFG) * NWN * SLOT_FLOATS;
    static constexpr int STAGE_HALVES = TMS * TN * 16 * 8;  // epilogue staging per compute wave
    static_assert(NT <= 1024, "workgroup size");
    static_assert(DEPTH >= 3 && (DEPTH - 2) * PER <= 63, "ring depth / vmcnt range");
    static_assert(DEPTH * STAGE_UNITS * 16 <= 160 * 1024, "LDS");
    static_assert(XCH_FLOATS * 4 + NCW * STAGE_HALVES * 2 <= DEPTH * STAGE_UNITS * 16, "exchange + staging space");
    // exchange slot of the rows K group gs hands to finishing group gd (gs != gd)
    __device__ static constexpr int slot(int gs, int gd) {
        return gs * NFG - (gs < NFG ? gs : NFG) + gd - ((gs < NFG && gd > gs) ? 1 : 0);
    }
};

// Row tiles [G*TMS, (G+1)*TMS) of the wave's accumulators, summed over the K
// groups in group order (the wave's own partial in its place), then finished:
// the epilogue, or the fp32 partial of this workgroup's K range.
template <class C, int G>
__device__ __forceinline__ void finish_rows(const GemmArgs &a, const f4 (&acc)[C::TM][C::TN], const float *xch,
                                            int wn, int m0, int n0, int lane, _Float16 *stage, int split, int S,
                                            int Mt) {
    f4 sum[C::TMS][C::TN];
#pragma unroll
    for (int i = 0; i < C::TMS; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) sum[i][j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gs = 0; gs < C::KS; ++gs) {
        if (gs == G) {
#pragma unroll
            for (int i = 0; i < C::TMS; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j) sum[i][j] += acc[G * C::TMS + i][j];
        } else {
            const float *src = xch + (size_t)(C::slot(gs, G) * C::NWN + wn) * C::SLOT_FLOATS + lane;
#pragma unroll
            for (int i = 0; i < C::TMS; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sum[i][j][r] += src[((i * C::TN + j) * 4 + r) * 64];
        }
    }
    const int r0 = m0 + G * C::TMS * 16, c0 = n0 + wn * C::WN;
    if (S == 1) {
        gemm_epilogue<C::TMS, C::TN>(a, sum, r0, c0, lane, stage);
    } else {
        // partial tile layout: [split][row tile][16-column group][r][lane]
        const int Nt = a.W.N >> 4;
        float *dst = a.part + (size_t)split * Mt * Nt * 256;
#pragma unroll
        for (int i = 0; i < C::TMS; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                float *p = dst + ((size_t)((r0 >> 4) + i) * Nt + (c0 >> 4) + j) * 256 + lane;
#pragma unroll
                for (int r = 0; r < 4; ++r) p[r * 64] = sum[i][j][r];
            }
    }
}

template <class C, int G>
__device__ __forceinline__ void finish_group(const GemmArgs &a, const f4 (&acc)[C::TM][C::TN], const float *xch,
                                             int g, int wn, int m0, int n0, int lane, _Float16 *stage, int split,
                                             int S, int Mt) {
    if constexpr (G < C::NFG) {
        if (g == G) finish_rows<C, G>(a, acc, xch, wn, m0, n0, lane, stage, split, S, Mt);
        else finish_group<C, G + 1>(a, acc, xch, g, wn, m0, n0, lane, stage, split, S, Mt);
    }
}

// A launch covers grp.n units (the same product for different ubatches and
// layers: same N, K and epilogue, their own operands and outputs); z =
// unit * S + split.  Mt: row tiles of the split-K partial layout.
template <class C>
__global__ __launch_bounds__(C::NT) void k_q4gemm_p(const GemmGroup grp, int S, int Mt) {
    __shared__ h8 ring[C::DEPTH * C::STAGE_UNITS];
    const int unit = blockIdx.z / S, split = blockIdx.z % S;
    const GemmArgs &a = grp.u[unit];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int n0 = blockIdx.x * C::BN, m0 = blockIdx.y * C::BM;
    if (m0 >= a.M) return;  // a unit with fewer rows than the launch's tallest (the whole workgroup)
    const int kch = a.W.K >> 6;
    const int nkg = kch / (S * C::KS);  // 64-wide K steps per K group
    const int kz = split * C::KS * nkg;  // first K step of this workgroup
    const int ktiles = a.W.K >> 5;

    if (wave >= C::NCW) {
        // ---- producer waves: wave NCW + p issues DMAs p, p + NP, p + 2 NP, ... of
        // each stage (A fragments, then code pairs, then scale quads)
        const int pw = C::NP == 1 ? 0 : wave - C::NCW;
        const int last_tr = (a.M - 1) >> 4;
        const int gbase = n0 >> 4;
        // the wave's t-th DMA of a stage: e = t * NP + pw (the last one repeated past the end)
        auto entry = [&](int t) { return min(t * C::NP + pw, C::DMA_STAGE - 1); };
        const char *src[C::PER];
#pragma unroll
        for (int t = 0; t < C::PER; ++t) {
            const int e = entry(t);
            if (e < C::A_TOT) {
                // K group gk, fragment f = kb * TM + i: rows of tile i, the kb-th 32-wide half of the step
                const int gk = e / C::AFR, f = e % C::AFR;
                const int kb = f / C::TM, i = f % C::TM;
                const int tr = min((m0 >> 4) + i, last_tr);  // rows past M repeat the last tile
                src[t] = reinterpret_cast<const char *>(
                    a.A + (((size_t)tr * ktiles + 2 * (kz + gk * nkg) + kb) * 64 + lane) * 8);
            } else if (e < C::A_TOT + C::B_TOT) {
                // codes of weight blocks 2i and 2i+1, block b = (K group gk, column group cg)
                const int i = e - C::A_TOT;
                const int b = min(2 * i + (lane >> 5), C::NB - 1);
                const int gk = b / (C::NWN * C::TN), cg = b % (C::NWN * C::TN);
                src[t] = reinterpret_cast<const char *>(reinterpret_cast<const uint4 *>(a.W.nib) +
                                                        ((size_t)(gbase + cg) * kch + kz + gk * nkg) * 32 + (lane & 31));
            } else {
                // scales of weight blocks 4i .. 4i+3
                const int i = e - C::A_TOT - C::B_TOT;
                const int b = min(4 * i + (lane >> 4), C::NB - 1);
                const int gk = b / (C::NWN * C::TN), cg = b % (C::NWN * C::TN);
                src[t] = reinterpret_cast<const char *>(reinterpret_cast<const uint32_t *>(a.W.scl) +
                                                        ((size_t)(gbase + cg) * kch + kz + gk * nkg) * 16 + (lane & 15));
            }
        }
        auto issue = [&](int sb) {
            h8 *st = ring + (sb % C::DEPTH) * C::STAGE_UNITS;
            const size_t s = (size_t)min(sb, nkg - 1);  // past the end: repeats keep the DMA count uniform
#pragma unroll
            for (int t = 0; t < C::PER; ++t) {
                const int e = entry(t);
                if (e < C::A_TOT) {
                    dma16(src[t] + s * 2048, st + e * 64);
                } else if (e < C::A_TOT + C::B_TOT) {
                    dma16(src[t] + s * 512, st + C::A_UNITS + (e - C::A_TOT) * 64);
                } else {
                    dma4(src[t] + s * 64, st + C::A_UNITS + C::B_UNITS + (e - C::A_TOT - C::B_TOT) * 16);
                }
            }
        };
#pragma unroll
        for (int s = 0; s < C::DEPTH - 1; ++s) issue(s);
        for (int s = 0; s < nkg; ++s) {
            wait_vm<(C::DEPTH - 2) * C::PER>();  // this wave's share of stages <= s has landed
            lds_barrier();
            issue(s + C::DEPTH - 1);  // into the buffer of stage s - 1, which nobody reads any more
        }
        wait_vm<0>();
        lds_barrier();  // the ring is free once every DMA has landed
        return;
    }

    // ---- compute waves
    const int wn = wave % C::NWN, g = wave / C::NWN;
    f4 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    const int b0 = g * C::NWN * C::TN + wn * C::TN;
    auto decode = [&](const h8 *st, h8 (&bf)[2][C::TN]) {
        const uint2 *bws = reinterpret_cast<const uint2 *>(st + C::A_UNITS) + b0 * 64 + lane;
        const uint32_t *bss =
            reinterpret_cast<const uint32_t *>(st + C::A_UNITS + C::B_UNITS) + b0 * 16 + (lane & 15);
        uint2 bw[C::TN];
        uint32_t bs[C::TN];
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            bw[j] = bws[j * 64];
            bs[j] = bss[j * 16];
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const h2 d = __builtin_bit_cast(h2, bs[j]);
            bf[0][j] = q4_word_to_h8(bw[j].x, d[0]);
            bf[1][j] = q4_word_to_h8(bw[j].y, d[1]);
        }
    };
    // stage s: its codes decoded, then its MFMAs
    auto step = [&](int s) {
        const h8 *st = ring + (s % C::DEPTH) * C::STAGE_UNITS;
        const h8 *as = st + g * C::AFR * 64 + lane;
        h8 af[C::TM];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) af[i] = as[i * 64];
        h8 bc[2][C::TN];
        decode(st, bc);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            h8 an[C::TM];
            if (kb == 0) {
#pragma unroll
                for (int i = 0; i < C::TM; ++i) an[i] = as[(C::TM + i) * 64];
            }
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma16(af[i], bc[kb][j], acc[i][j]);
            if (kb == 0) {
#pragma unroll
                for (int i = 0; i < C::TM; ++i) af[i] = an[i];
            }
        }
        if (s + 1 < nkg) lds_barrier();
    };
    lds_barrier();  // stage 0 has landed
    for (int s = 0; s < nkg; ++s) step(s);
    lds_barrier();  // matches the producer's last barrier: the ring is free

    float *xch = reinterpret_cast<float *>(ring);
    if constexpr (C::KS > 1) {
        // hand the row tiles of the other finishing groups over, then sum in group order
#pragma unroll
        for (int gd = 0; gd < C::NFG; ++gd) {
            if (gd == g) continue;
            float *dst = xch + (size_t)(C::slot(g, gd) * C::NWN + wn) * C::SLOT_FLOATS + lane;
#pragma unroll
            for (int i = 0; i < C::TMS; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[((i * C::TN + j) * 4 + r) * 64] = acc[gd * C::TMS + i][j][r];
        }
        __syncthreads();  // compute waves only: the producers have returned
    }
    // each compute wave's epilogue staging area follows the exchange space
    _Float16 *stage = reinterpret_cast<_Float16 *>(xch + C::XCH_FLOATS) + (size_t)wave * C::STAGE_HALVES;
    finish_group<C, 0>(a, acc, xch, g, wn, m0, n0, lane, stage, split, S, Mt);
}

// Sum of the S split partials in split order, then the epilogue; one wave per
// 16 rows x (16 * TNR) columns.
template <int TNR>
__global__ __launch_bounds__(256) void k_gemm_reduce(const GemmGroup grp, int S, int Mt) {
    const GemmArgs &a = grp.u[blockIdx.y];
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int Nt = a.W.N >> 4, ncb = Nt / TNR;
    const int rt = w / ncb, cb = w % ncb;
    if (rt >= Mt || rt * 16 >= a.M) return;
    f4 acc[1][TNR];
#pragma unroll
    for (int j = 0; j < TNR; ++j) acc[0][j] = f4{0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < S; ++z) {
        const float *src = a.part + ((size_t)z * Mt * Nt + (size_t)rt * Nt + cb * TNR) * 256 + lane;
#pragma unroll
        for (int j = 0; j < TNR; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[0][j][r] += src[j * 256 + r * 64];
    }
    gemm_epilogue<1, TNR>(a, acc, rt * 16, cb * TNR * 16, lane);
}

// x[row] += the S split partials of its tile (summed in split order, as
// k_gemm_reduce does), then the RMSNorm of the updated row with gain g into
// the fp16 fragment-tiled norm_out.  One workgroup per row; thread t owns the
// eight-float chunks t, t + 256, ...; every split's loads issue together.
constexpr int RAN_MAX_CHUNKS = 2;  // d <= 2 * 8 * 256
constexpr int RAN_MAX_SPLIT = 8;
__global__ __launch_bounds__(256) void k_reduce_add_norm(const GemmGroup grp, int S, int Mt) {
    __shared__ float red[4];
    const GemmArgs &a = grp.u[blockIdx.y];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x;
    if (row >= a.M) return;
    const int d = a.W.N, Nt = d >> 4, nch = d >> 3;
    const int rt = row >> 4, rr = row & 15;
    const int sub = (rr & 3) * 64 + (rr >> 2) * 16;  // r * 64 + lane group * 16 in the partial tile
    float *xr = a.out_f32 + (size_t)row * d;
    float4 v[RAN_MAX_CHUNKS][2];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < RAN_MAX_CHUNKS; ++c) {
        const int ch = tid + 256 * c;
        if (ch < nch) {
            float4 p[RAN_MAX_SPLIT][2];
#pragma unroll
            for (int z = 0; z < RAN_MAX_SPLIT; ++z) {
                if (z < S) {
                    const float *src = a.part + (((size_t)z * Mt + rt) * Nt + (ch >> 1)) * 256 + sub + (ch & 1) * 8;
                    p[z][0] = *reinterpret_cast<const float4 *>(src);
                    p[z][1] = *reinterpret_cast<const float4 *>(src + 4);
                }
            }
            float4 x0 = *reinterpret_cast<const float4 *>(xr + ch * 8);
            float4 x1 = *reinterpret_cast<const float4 *>(xr + ch * 8 + 4);
            float4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int z = 0; z < RAN_MAX_SPLIT; ++z) {
                if (z < S) {
                    s0.x += p[z][0].x; s0.y += p[z][0].y; s0.z += p[z][0].z; s0.w += p[z][0].w;
                    s1.x += p[z][1].x; s1.y += p[z][1].y; s1.z += p[z][1].z; s1.w += p[z][1].w;
                }
            }
            x0.x += s0.x; x0.y += s0.y; x0.z += s0.z; x0.w += s0.w;
            x1.x += s1.x; x1.y += s1.y; x1.z += s1.z; x1.w += s1.w;
            *reinterpret_cast<float4 *>(xr + ch * 8) = x0;
            *reinterpret_cast<float4 *>(xr + ch * 8 + 4) = x1;
            v[c][0] = x0;
            v[c][1] = x1;
            ss += x0.x * x0.x + x0.y * x0.y + x0.z * x0.z + x0.w * x0.w;
            ss += x1.x * x1.x + x1.y * x1.y + x1.z * x1.z + x1.w * x1.w;
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    const float r = 1.0f / sqrtf(ss / (float)d + a.norm_eps);
#pragma unroll
    for (int c = 0; c < RAN_MAX_CHUNKS; ++c) {
        const int ch = tid + 256 * c;
        if (ch < nch) {
            const float4 g0 = *reinterpret_cast<const float4 *>(a.norm_g + ch * 8);
            const float4 g1 = *reinterpret_cast<const float4 *>(a.norm_g + ch * 8 + 4);
            const float y[8] = {v[c][0].x * r * g0.x, v[c][0].y * r * g0.y, v[c][0].z * r * g0.z, v[c][0].w * r * g0.w,
                                v[c][1].x * r * g1.x, v[c][1].y * r * g1.y, v[c][1].z * r * g1.z, v[c][1].w * r * g1.w};
            h8 yh;
#pragma unroll
            for (int e = 0; e < 8; ++e) yh[e] = (_Float16)y[e];
            *reinterpret_cast<h8 *>(a.norm_out + tiled_index(row, ch * 8, d)) = yh;
        }
    }
}

// ------------------------------------------------------- exact-weight kernel

template <int TM_, int TN_, int NWN_, int KS_, int DEPTH_>
struct Cfg {
    static constexpr int TM = TM_, TN = TN_, NWN = NWN_, KS = KS_, DEPTH = DEPTH_;
    static constexpr int NCW = NWN * KS;             // compute waves
    static constexpr int NT = 64 * (NCW + 1);
    static constexpr int BM = 16 * TM, WN = 16 * TN, BN = NWN * WN;
    static constexpr int AFR = 4 * TM;               // hi and lo fragments per chunk
    static constexpr int DMAS = AFR * KS;            // per stage
    static constexpr int STAGE_UNITS = DMAS * 64;
    static constexpr int PB = 4;
    static constexpr int RED_FLOATS = (KS - 1) * NWN * TM * TN * 4 * 64;
    static_assert(NT <= 1024, "workgroup size");
    static_assert(DEPTH >= 2 && (DEPTH - 2) * DMAS <= 63, "vmcnt range");
    static_assert(DEPTH * STAGE_UNITS * 16 <= 160 * 1024, "LDS");
    static_assert(RED_FLOATS * 4 <= DEPTH * STAGE_UNITS * 16, "reduction space");
};

template <class C>
__global__ __launch_bounds__(C::NT) void k_q4gemm(const GemmGroup units) {
    __shared__ h8 ring[C::DEPTH * C::STAGE_UNITS];
    const GemmArgs &a = units.u[blockIdx.z];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int n0 = blockIdx.x * C::BN, m0 = blockIdx.y * C::BM;
    if (m0 >= a.M) return;  // a unit with fewer rows than the launch's tallest
    const int kch = a.W.K >> 6;
    const int nkg = kch / C::KS;  // chunks per group
    const int ktiles = a.W.K >> 5;

    if (wave == C::NCW) {
        const int last_tr = (a.M - 1) >> 4;
        const __half *asrc[C::AFR];
#pragma unroll
        for (int f = 0; f < C::AFR; ++f) {
            const int p = f / (2 * C::TM), kb = (f / C::TM) & 1, i = f % C::TM;
            const int tr = min((m0 >> 4) + i, last_tr);
            asrc[f] = (p ? a.A2 : a.A) + (((size_t)tr * ktiles + kb) * 64 + lane) * 8;
        }
        auto issue = [&](int sb) {
            h8 *st = ring + (sb % C::DEPTH) * C::STAGE_UNITS;
            const int s = min(sb, nkg - 1);
#pragma unroll
            for (int g = 0; g < C::KS; ++g)
#pragma unroll
                for (int f = 0; f < C::AFR; ++f)
                    dma16(asrc[f] + (size_t)(g * nkg + s) * 1024, st + (g * C::AFR + f) * 64);
        };
#pragma unroll
        for (int s = 0; s < C::DEPTH - 1; ++s) issue(s);
        for (int s = 0; s < nkg; ++s) {
            wait_vm<(C::DEPTH - 2) * C::DMAS>();
            lds_barrier();
            issue(s + C::DEPTH - 1);
        }
        wait_vm<0>();
        if constexpr (C::KS > 1) lds_barrier();  // matches the compute waves' barrier before the reduction
        return;
    }

    const int wn = wave % C::NWN, grp = wave / C::NWN;
    const int g0 = (n0 >> 4) + wn * C::TN;
    const int cbase = grp * nkg;
    const uint2 *nib[C::TN];
    const uint32_t *scl[C::TN];
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
        nib[j] = reinterpret_cast<const uint2 *>(a.W.nib) + ((size_t)(g0 + j) * kch + cbase) * 64 + lane;
        scl[j] = reinterpret_cast<const uint32_t *>(a.W.scl) + ((size_t)(g0 + j) * kch + cbase) * 16 + (lane & 15);
    }
    uint2 bw[C::PB][C::TN];
    uint32_t bs[C::PB][C::TN];
    auto loadb = [&](int slot, int s) {
        const int sc = min(s, nkg - 1);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            bw[slot][j] = nib[j][(size_t)sc * 64];
            bs[slot][j] = scl[j][(size_t)sc * 16];
        }
    };
    f4 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < C::PB - 1; ++p) loadb(p, p);
    for (int s0 = 0; s0 < nkg; s0 += C::PB) {
#pragma unroll
        for (int u = 0; u < C::PB; ++u) {
            const int s = s0 + u;
            loadb((u + C::PB - 1) % C::PB, s + C::PB - 1);
            lds_barrier();
            const h8 *st = ring + (s % C::DEPTH) * C::STAGE_UNITS + grp * C::AFR * 64;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                h8 af[C::TM], al[C::TM];
#pragma unroll
                for (int i = 0; i < C::TM; ++i) {
                    af[i] = st[(kb * C::TM + i) * 64 + lane];
                    al[i] = st[((2 + kb) * C::TM + i) * 64 + lane];
                }
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const h8 bq = q4_word_codes(kb ? bw[u][j].y : bw[u][j].x);
                    const float dj = (float)__builtin_bit_cast(h2, bs[u][j])[kb];
#pragma unroll
                    for (int i = 0; i < C::TM; ++i) {
                        f4 t = mfma16(af[i], bq, f4{0.f, 0.f, 0.f, 0.f});
                        t = mfma16(al[i], bq, t);
                        acc[i][j] += dj * t;
                    }
                }
            }
        }
    }
    if constexpr (C::KS > 1) {
        // every wave is past its last ring read once this barrier completes
        lds_barrier();
        float *red = reinterpret_cast<float *>(ring);
        if (grp > 0) {
            float *dst = red + ((size_t)((grp - 1) * C::NWN + wn) * C::TM * C::TN * 4) * 64;
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[((i * C::TN + j) * 4 + r) * 64 + lane] = acc[i][j][r];
        }
        __syncthreads();  // compute waves only: the producer has returned
        if (grp > 0) return;
#pragma unroll
        for (int g = 1; g < C::KS; ++g) {
            const float *src = red + ((size_t)((g - 1) * C::NWN + wn) * C::TM * C::TN * 4) * 64;
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] += src[((i * C::TN + j) * 4 + r) * 64 + lane];
        }
    }
    gemm_epilogue<C::TM, C::TN>(a, acc, m0, n0 + wn * C::WN, lane);
}

// ------------------------------------------------------------------ launchers

// Rows of the launch: the tallest unit's (shorter units' surplus workgroups return at once).
int max_rows(const GemmGroup &g) {
    int M = 0;
    for (int i = 0; i < g.n; ++i) M = std::max(M, g.u[i].M);
    return M;
}

template <class C>
int launch_p(const GemmGroup &g, int S, hipStream_t s) {
    const GemmArgs &a = g.u[0];
    const int kch = a.W.K >> 6;
    if (S < 1 || a.W.N % C::BN || kch % (S * C::KS)) return PPX_E_UNSUPPORTED;
    if (a.epi == EPI_QKV && C::TN % 2) return PPX_E_UNSUPPORTED;
    const int mb = (max_rows(g) + C::BM - 1) / C::BM;
    const int Mt = mb * C::TM;
    for (int i = 0; i < g.n && S > 1; ++i)
        if (!g.u[i].part || (size_t)S * Mt * 16 * a.W.N > g.u[i].part_floats) return PPX_E_UNSUPPORTED;
    hipLaunchKernelGGL((k_q4gemm_p<C>), dim3(a.W.N / C::BN, mb, S * g.n), dim3(C::NT), 0, s, g, S, Mt);
    if (hipGetLastError() != hipSuccess) return PPX_E_HIP;
    if (S > 1) {
        if (a.norm_out && S <= RAN_MAX_SPLIT) {
            hipLaunchKernelGGL(k_reduce_add_norm, dim3(max_rows(g), g.n), dim3(256), 0, s, g, S, Mt);
        } else {
            const int waves = Mt * (a.W.N / 32);
            hipLaunchKernelGGL((k_gemm_reduce<2>), dim3((waves + 3) / 4, g.n), dim3(256), 0, s, g, S, Mt);
        }
        if (hipGetLastError() != hipSuccess) return PPX_E_HIP;
    }
    return PPX_OK;
}

template <class C>
int launch_cfg(const GemmGroup &g, hipStream_t s) {
    const GemmArgs &a = g.u[0];
    if (a.W.N % C::BN || (a.W.K >> 6) % (C::PB * C::KS)) return PPX_E_UNSUPPORTED;
    if (a.epi == EPI_QKV && C::TN % 2) return PPX_E_UNSUPPORTED;  // RoPE pairs are adjacent groups of one wave
    dim3 grid(a.W.N / C::BN, (max_rows(g) + C::BM - 1) / C::BM, g.n);
    hipLaunchKernelGGL((k_q4gemm<C>), grid, dim3(C::NT), 0, s, g);
    return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP;
}

// Fast-mode configurations: id, TM, TN, NWN, KS, DEPTH, NP (producer waves);
// workgroup tile (16 TM) x (16 TN NWN), K split over KS wave groups.
#define PPX_GEMM_CONFIGS(X) \
    X(0, 8, 3, 4, 2, 3, 1)  \
    X(1, 8, 2, 4, 2, 3, 1)  \
    X(2, 4, 3, 4, 2, 4, 4)  \
    X(3, 4, 2, 4, 2, 4, 4)  \
    X(4, 2, 2, 4, 2, 4, 4)  \
    X(5, 2, 2, 4, 2, 4, 1)  \
    X(6, 1, 2, 4, 2, 4, 4)  \
    X(7, 1, 1, 1, 4, 4, 1)  \
    X(8, 1, 2, 1, 4, 4, 1)

int launch_plan(const GemmGroup &g, int cfg, int S, hipStream_t s) {
    switch (cfg) {
#define PPX_CASE(id, tm, tn, nwn, ks, depth, np) \
    case id:                                     \
        return launch_p<PCfg<tm, tn, nwn, ks, depth, np>>(g, S, s);
        PPX_GEMM_CONFIGS(PPX_CASE)
#undef PPX_CASE
    default: return PPX_E_UNSUPPORTED;
    }
}

int tile_rows(int cfg) {
    switch (cfg) {
#define PPX_CASE(id, tm, tn, nwn, ks, depth, np) \
    case id:                                     \
        return 16 * tm;
        PPX_GEMM_CONFIGS(PPX_CASE)
#undef PPX_CASE
    default: return 16;
    }
}

struct Plan {
    int cfg, S;
};
#define PLAN_QO 4
#define PLAN_KSMALL 4

// Measured on the E2B-like shapes at M = 512 (one MI355X): wide outputs
// (gate|up) take the tallest wave tiles; the long-K down projection splits K
// four ways over workgroups; Q and O use 32-row tiles with four producer
// waves; narrow outputs (N <= 512) single 16 x 16 tiles with K split four
// ways inside the workgroup, so that 512 short chains run instead of 64 long
// ones; K = 256 the 32-row tiles of Q and O.  Otherwise the plan does not
// depend on M, so a row's result does not depend on the ubatch size.  The
// gathered output rows of several sequences (at most 64, GemmArgs::few_rows)
// take the single 16 x 16 tiles whatever the shape (16 x 32 where the RoPE
// epilogue needs column pairs), so the weights stream over N / 16 workgroups
// per 16 rows instead of a few dozen tall tiles with idle rows; measured
// 0.4-0.5 ms faster on multi-sequence prefills of 2048 tokens in 2 to 32
// prompts.
Plan plan_for(int M, int N, int K, bool few = false, int units = 1) {
    if (few && M <= 64) return {7, K >= 4096 ? 4 : 1};  // a few gathered rows: 16-row tiles, many workgroups
    if (N >= 8192) return {N % 192 == 0 ? 0 : 1, 1};
    if (K >= 4096) {
        // 128-row tiles once they still give every CU a workgroup (eight
        // 512-row ubatches in a launch: 1.6 % off the 8192-token prefill;
        // with four, half the CUs would idle: 5 % slower); both split K the
        // same way, so a row's sums do not change
        if (N % 192 == 0 && (long)units * ((M + 127) / 128) * (N / 192) >= 256) return {0, 1};
        return {N % 192 == 0 ? 2 : 3, units >= 4 ? 1 : units >= 2 ? 2 : 4};
    }
    if (N <= 512) return {7, 1};
    if (K <= 256) return {PLAN_KSMALL, 1};
    return {PLAN_QO, 1};
}

}  // namespace

size_t gemm_part_floats(int M, int N, int K) {
    const Plan p = plan_for(M, N, K);
    if (p.S <= 1) return 0;
    const int bm = tile_rows(p.cfg);
    return (size_t)p.S * ((M + bm - 1) / bm * bm) * N;
}

int launch_gemm_group(const GemmArgs *units, int n, hipStream_t s) {
    if (n < 1 || n > kMaxUnits) return PPX_E_INVAL;
    GemmGroup g;
    g.n = 0;
    for (int i = 0; i < n; ++i)
        if (units[i].M > 0) g.u[g.n++] = units[i];
    if (!g.n) return PPX_OK;
    const GemmArgs &a = g.u[0];
    for (int i = 1; i < g.n; ++i)
        if (g.u[i].W.N != a.W.N || g.u[i].W.K != a.W.K || g.u[i].epi != a.epi || g.u[i].few_rows != a.few_rows ||
            !g.u[i].norm_out != !a.norm_out)
            return PPX_E_INVAL;
    if (a.W.N % 128 || a.W.K % 256) return PPX_E_UNSUPPORTED;
    for (int i = 0; i < g.n; ++i) {
        const GemmArgs &u = g.u[i];
        if (!u.A) return PPX_E_UNSUPPORTED;
        if (u.norm_out && (u.epi != EPI_ADD || !u.norm_g || u.W.N > RAN_MAX_CHUNKS * 8 * 256)) return PPX_E_UNSUPPORTED;
    }
    const int M = max_rows(g);
    Plan p = plan_for(M, a.W.N, a.W.K, a.few_rows, g.n);
    if (a.few_rows && M <= 64 && a.epi == EPI_QKV) p = {8, 1};  // RoPE pairs need two column groups per wave
    int st = launch_plan(g, p.cfg, p.S, s);
    bool normed = st == PPX_OK && p.S > 1 && p.S <= RAN_MAX_SPLIT && a.norm_out;  // the split's reduction normalised too
    if (st == PPX_E_UNSUPPORTED && p.S > 1) st = launch_plan(g, p.cfg, 1, s);  // no split workspace given
    if (st == PPX_E_UNSUPPORTED) st = launch_plan(g, 5, 1, s);                 // N % 128, K % 256: always fits
    if (st == PPX_OK && a.norm_out && !normed) {
        NormUnit nu[kMaxUnits];
        for (int i = 0; i < g.n; ++i) {
            nu[i].x = g.u[i].out_f32;
            nu[i].g = g.u[i].norm_g;
            nu[i].hi = g.u[i].norm_out;
            nu[i].M = g.u[i].M;
        }
        st = launch_rmsnorm_group(nu, g.n, a.norm_eps, a.W.N, false, s);
    }
    return st;
}

int launch_gemm(const GemmArgs &a, hipStream_t s) { return launch_gemm_group(&a, 1, s); }

int launch_gemm_exact_group(const GemmArgs *units, int n, hipStream_t s) {
    if (n < 1 || n > kMaxUnits) return PPX_E_INVAL;
    GemmGroup g;
    g.n = 0;
    for (int i = 0; i < n; ++i)
        if (units[i].M > 0) g.u[g.n++] = units[i];
    if (!g.n) return PPX_OK;
    const GemmArgs &a = g.u[0];
    for (int i = 0; i < g.n; ++i) {
        const GemmArgs &u = g.u[i];
        if (u.W.N != a.W.N || u.W.K != a.W.K || u.epi != a.epi) return PPX_E_INVAL;
        if (!u.A || !u.A2) return PPX_E_UNSUPPORTED;
    }
    if (a.W.N % 64 || a.W.K % 256) return PPX_E_UNSUPPORTED;
    // 16 x 128 tiles, eight compute waves: against 16 x 64 tiles, half the
    // workgroups stream each weight column block (same-box runs: 2 % off the
    // 2048- and 8192-token prefills, where this is the K|V product; 32- or
    // 64-row and 256-column tiles were slower)
    if ((a.W.K >> 6) % 8 == 0 && a.W.N % 128 == 0) return launch_cfg<Cfg<1, 2, 4, 2, 6>>(g, s);
    if ((a.W.K >> 6) % 8 == 0) return launch_cfg<Cfg<1, 2, 2, 2, 6>>(g, s);
    return launch_cfg<Cfg<1, 2, 2, 1, 6>>(g, s);
}

int launch_gemm_exact(const GemmArgs &a, hipStream_t s) { return launch_gemm_exact_group(&a, 1, s); }

}  // namespace ppx
