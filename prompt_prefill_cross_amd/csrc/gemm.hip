// Q4_0 dequant-fused GEMM on CDNA4 MFMA (v_mfma_f32_16x16x32_f16).
//
//   C[M][N] = A[M][K] (fp16 activations, fragment-tiled) x W[N][K]^T (Q4_0),
//   fp32 accumulate, with the layer's elementwise work fused into the epilogue.
//
// A workgroup holds NWN x KS compute waves and one producer wave and computes
// a BM x BN tile; compute wave (w, g) owns columns [w*WN, (w+1)*WN) for all BM
// rows (TM x TN MFMA tiles of 16 x 16) over the g-th of KS equal slices of K;
// the KS partial tiles meet in LDS, in slice order, before the epilogue.
//   * A (shared by the compute waves) reaches LDS without passing through
//     registers: the producer wave fills a ring of DEPTH stages, one 64-wide
//     K step of every slice each, with global_load_lds DMA of 1 KB fragments -- contiguous in
//     the fragment-tiled activation layout, one 16-byte piece per lane straight
//     into A-operand order -- and hands a stage over with a workgroup barrier
//     once its own outstanding-DMA count says the stage has landed.
//   * W (private to each compute wave: its own columns) streams straight into
//     registers, PB stages ahead: per lane and 64-wide K step one 8-byte word
//     pair of repacked codes and one fp16 block-scale pair per 16-column group.
//     Compute waves decode in registers (a shift, a mask, an OR with the fp16
//     exponent of 1024, a subtract and a multiply per pair) and multiply.
// Keeping DMA in its own wave keeps the compiler from making LDS reads wait on
// DMA aimed at other stages.  The decode is paid once per wave for TM row
// tiles, so taller wave tiles amortise it; LDS carries only A.
//
// Two arithmetic modes:
//  * fast (EXACT = false): B = fp16(d * (code - 8)), one rounding per weight;
//  * exact (EXACT = true): B = code - 8 (exact in fp16), A = hi + lo (two
//    fp16 arrays), each 32-wide block's partial scaled by its fp32 block scale
//    before it is added -- only fp32 accumulation rounds.  The K|V projection
//    uses it, so the cache holds values accurate to the fp16 store itself.
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

// Epilogue of one wave tile: acc[i][j][r] = C[r0 + 16i + 4(lane/16) + r][c0 + 16j + lane%16].
template <int TM, int TN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &a, const f4 (&acc)[TM][TN], int r0, int c0, int lane) {
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
                    a.out_f16[tiled_index(row, col, E)] = (_Float16)(gelu_tanh_f(acc[i][j][r]) * P);
                }
            }
    } else {
        // paired epilogues: 16-column groups (2p, 2p+1) of the wave tile hold the
        // two members of a pair (gate, up) or (first, second RoPE half)
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
                    if (a.epi == EPI_GLU) {
                        // act(gate) * up -> fp16, fragment-tiled [M][F]
                        const int F = N >> 1;
                        const int f = (colA >> 5) * 16 + lc;
                        a.out_f16[tiled_index(row, f, F)] = (_Float16)(act_f(a.act, va) * vb);
                    } else {  // EPI_QKV: columns [0,qd) Q, [qd,qd+kvd) K, [qd+kvd, qd+2kvd) V
                        const int hd = a.hd, half = hd >> 1;
                        const int pos = a.pos0 + row;
                        if (colA < a.qd + a.kvd) {
                            const bool isq = colA < a.qd;
                            const int c = isq ? colA : colA - a.qd;
                            const int h = c / hd, rr = c % hd;
                            const int ii = (rr >> 5) * 16 + lc;  // dimension in the first half
                            const float2 cs = a.rope[(size_t)pos * half + ii];
                            const float ra = va * cs.x - vb * cs.y;
                            const float rb = va * cs.y + vb * cs.x;
                            if (isq) {
                                __half *q = a.out_f16 + (size_t)row * a.qd + h * hd;
                                q[ii] = __float2half(ra);
                                q[ii + half] = __float2half(rb);
                            } else {
                                __half *k = a.kc + (size_t)pos * a.kvd + h * hd;
                                k[ii] = __float2half(ra);
                                k[ii + half] = __float2half(rb);
                            }
                        } else {
                            const int c = colA - a.qd - a.kvd;
                            a.vc[(size_t)c * a.vld + pos] = __float2half(va);  // V^T
                            a.vc[(size_t)(c + 16) * a.vld + pos] = __float2half(vb);
                        }
                    }
                }
        }
    }
}

template <int TM_, int TN_, int NWN_, int KS_, int DEPTH_, bool EXACT_>
struct Cfg {
    static constexpr int TM = TM_, TN = TN_, NWN = NWN_, KS = KS_, DEPTH = DEPTH_;
    static constexpr bool EXACT = EXACT_;
    static constexpr int NCW = NWN * KS;             // compute waves
    static constexpr int NT = 64 * (NCW + 1);
    static constexpr int BM = 16 * TM, WN = 16 * TN, BN = NWN * WN;
    static constexpr int NA = EXACT ? 2 : 1;
    static constexpr int AFR = 2 * TM * NA;          // fragments per chunk
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
__global__ __launch_bounds__(C::NT) void k_q4gemm(GemmArgs a) {
    __shared__ h8 ring[C::DEPTH * C::STAGE_UNITS];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int n0 = blockIdx.x * C::BN, m0 = blockIdx.y * C::BM;
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
                h8 af[C::TM];
#pragma unroll
                for (int i = 0; i < C::TM; ++i) af[i] = st[(kb * C::TM + i) * 64 + lane];
                if constexpr (C::EXACT) {
                    h8 al[C::TM];
#pragma unroll
                    for (int i = 0; i < C::TM; ++i) al[i] = st[((2 + kb) * C::TM + i) * 64 + lane];
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
                } else {
                    h8 bf[C::TN];
#pragma unroll
                    for (int j = 0; j < C::TN; ++j)
                        bf[j] = q4_word_to_h8(kb ? bw[u][j].y : bw[u][j].x, __builtin_bit_cast(h2, bs[u][j])[kb]);
#pragma unroll
                    for (int i = 0; i < C::TM; ++i)
#pragma unroll
                        for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
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

template <class C>
int launch_cfg(const GemmArgs &a, hipStream_t s) {
    if (a.W.N % C::BN || (a.W.K >> 6) % (C::PB * C::KS)) return PPX_E_UNSUPPORTED;
    dim3 grid(a.W.N / C::BN, (a.M + C::BM - 1) / C::BM);
    hipLaunchKernelGGL((k_q4gemm<C>), grid, dim3(C::NT), 0, s, a);
    return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP;
}

}  // namespace

// Tile shapes measured on the E2B-like shapes at M = 512 (one MI355X):
//  * wide outputs (gate|up, N >= 8192): 64 x 128 tiles, four compute waves;
//  * long K (down, K >= 4096): 64 x 64 tiles, K split over four wave groups;
//  * narrow outputs (N <= 512): 16 x 128 tiles, K split over two groups;
//  * the rest (Q, O, PLE up): 32 x 128 tiles, K split over two groups.
// The exact-weight K|V projection: 16 x 64 tiles, K split over two groups.
// A split needs K/64 to be a multiple of 4 x KS; narrower splits are used
// where it is not.
template <int TM, int TN, int NWN, int KS, int DEPTH, bool EXACT>
int launch_split(const GemmArgs &a, hipStream_t s) {
    if constexpr (KS > 1) {
        if ((a.W.K >> 6) % (4 * KS)) return launch_split<TM, TN, NWN, KS / 2, DEPTH, EXACT>(a, s);
    }
    return launch_cfg<Cfg<TM, TN, NWN, KS, DEPTH, EXACT>>(a, s);
}

int launch_gemm(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    if (a.W.N % 128 || a.W.K % 256 || !a.A) return PPX_E_UNSUPPORTED;
    if (a.W.N >= 8192) return launch_split<4, 2, 4, 1, 4, false>(a, s);
    if (a.W.K >= 4096) return launch_split<4, 2, 2, 4, 3, false>(a, s);
    if (a.W.N <= 512) return launch_split<1, 2, 4, 2, 6, false>(a, s);
    return launch_split<2, 2, 4, 2, 4, false>(a, s);
}

int launch_gemm_exact(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    if (a.W.N % 64 || a.W.K % 256 || !a.A || !a.A2) return PPX_E_UNSUPPORTED;
    return launch_split<1, 2, 2, 2, 6, true>(a, s);
}

}  // namespace ppx
