// Q4_0 dequant-fused GEMM on CDNA4 MFMA (v_mfma_f32_16x16x32_f16).
//
//   C[M][N] = A[M][K] (fp16 activations, fragment-tiled) x W[N][K]^T (Q4_0),
//   fp32 accumulate, with the layer's elementwise work fused into the epilogue.
//
// A workgroup holds NWN compute waves and one producer wave and computes a
// BM x BN tile; compute wave w owns columns [w*WN, (w+1)*WN) for all BM rows
// (TM x TN MFMA tiles of 16 x 16).  Operands reach LDS without passing through
// registers: the producer wave fills a ring of DEPTH stages, one K step of 64
// each, with global_load_lds DMA --
//   * A: 1 KB fragments, contiguous in the fragment-tiled activation layout,
//     one 16-byte piece per lane straight into A-operand order;
//   * W: for every compute wave, its columns' repacked Q4_0 codes (16 bytes per
//     lane = two lanes' words, two 16-column groups per instruction) and fp16
//     block-scale pairs (4 bytes per lane, four groups per instruction).
// The producer waits for a stage by counting its own outstanding DMA
// instructions, then joins the workgroup barrier that hands the stage over;
// compute waves only read LDS, decode weights in registers (a shift, a mask,
// an OR with the fp16 exponent of 1024, a subtract and a multiply per pair)
// and multiply.  Keeping the roles in different waves keeps the compiler from
// making LDS reads wait on DMA aimed at other stages.
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

template <int TM_, int TN_, int NWN_, int DEPTH_, bool EXACT_>
struct Cfg {
    static constexpr int TM = TM_, TN = TN_, NWN = NWN_, DEPTH = DEPTH_;
    static constexpr bool EXACT = EXACT_;
    static constexpr int NT = 64 * (NWN + 1);
    static constexpr int BM = 16 * TM, WN = 16 * TN, BN = NWN * WN;
    static constexpr int NA = EXACT ? 2 : 1;              // A parts (hi, lo)
    static constexpr int AFR = 2 * TM * NA;                // 1 KB A fragments per stage
    static constexpr int CPW = TN / 2;                     // code DMAs per compute wave
    static constexpr int SPW = (TN + 3) / 4;               // scale DMAs per compute wave
    static constexpr int DMAS = AFR + NWN * (CPW + SPW);   // producer instructions per stage
    // LDS, in 16-byte units
    static constexpr int A_UNITS = AFR * 64;
    static constexpr int C_UNITS = TN * 32;                // codes: 512 B per group
    static constexpr int S_UNITS = SPW * 16;               // scales: 256 B per four groups
    static constexpr int W_UNITS = C_UNITS + S_UNITS;
    static constexpr int STAGE_UNITS = A_UNITS + NWN * W_UNITS;
    static_assert(TN % 2 == 0 && TN >= 2 && TN <= 4, "wave tile columns");
    static_assert(DEPTH >= 2 && (DEPTH - 2) * DMAS <= 63, "vmcnt range");
    static_assert(DEPTH * STAGE_UNITS * 16 <= 160 * 1024, "LDS");
};

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

template <class C>
__global__ __launch_bounds__(C::NT) void k_q4gemm(GemmArgs a) {
    __shared__ h8 ring[C::DEPTH * C::STAGE_UNITS];

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int n0 = blockIdx.x * C::BN, m0 = blockIdx.y * C::BM;
    const int kch = a.W.K >> 6;  // K steps of 64
    const int ktiles = a.W.K >> 5;

    if (wave == C::NWN) {
        // ------------------------------------------------------ producer wave
        // A fragment (part p, kb, i) of stage s: tile row m0/16 + i (clamped to
        // the last tile row; rows past M are computed and discarded), tile
        // column 2s + kb; stage layout [p][kb][i] x 1 KB
        const int last_tr = (a.M - 1) >> 4;
        const __half *asrc[C::AFR];
#pragma unroll
        for (int f = 0; f < C::AFR; ++f) {
            const int p = f / (2 * C::TM), kb = (f / C::TM) & 1, i = f % C::TM;
            const int tr = min((m0 >> 4) + i, last_tr);
            asrc[f] = (p ? a.A2 : a.A) + (((size_t)tr * ktiles + kb) * 64 + lane) * 8;
        }
        const uint32_t *csrc[C::NWN][C::CPW];
        const uint32_t *ssrc[C::NWN][C::SPW];
#pragma unroll
        for (int w = 0; w < C::NWN; ++w) {
            const int g0 = (n0 >> 4) + w * C::TN;
#pragma unroll
            for (int p = 0; p < C::CPW; ++p)
                csrc[w][p] = a.W.nib + ((size_t)(g0 + 2 * p + (lane >> 5)) * kch * 64 + (lane & 31) * 2) * 2;
#pragma unroll
            for (int q = 0; q < C::SPW; ++q) {
                const int j = min(4 * q + (lane >> 4), C::TN - 1);
                ssrc[w][q] = reinterpret_cast<const uint32_t *>(a.W.scl) + ((size_t)(g0 + j) * kch * 16 + (lane & 15));
            }
        }
        // DMA of stage min(sb, kch-1) into the buffer of stage sb
        auto issue = [&](int sb) {
            h8 *st = ring + (sb % C::DEPTH) * C::STAGE_UNITS;
            const int s = min(sb, kch - 1);
#pragma unroll
            for (int f = 0; f < C::AFR; ++f) dma16(asrc[f] + (size_t)s * 1024, st + f * 64);
#pragma unroll
            for (int w = 0; w < C::NWN; ++w) {
                h8 *wst = st + C::A_UNITS + w * C::W_UNITS;
#pragma unroll
                for (int p = 0; p < C::CPW; ++p) dma16(csrc[w][p] + (size_t)s * 128, wst + p * 64);
#pragma unroll
                for (int q = 0; q < C::SPW; ++q) dma4(ssrc[w][q] + (size_t)s * 16, wst + C::C_UNITS + q * 16);
            }
        };
        // Stages 0 .. DEPTH-2 up front; stage s + DEPTH - 1 right after the
        // barrier that hands stage s over (every compute wave has then finished
        // reading stage s - 1, whose buffer it refills).  Past the end the same
        // number of instructions is issued -- reloads of the last stage into
        // buffers of stages no one reads again -- so the count stays exact.
#pragma unroll
        for (int s = 0; s < C::DEPTH - 1; ++s) issue(s);
        for (int s = 0; s < kch; ++s) {
            wait_vm<(C::DEPTH - 2) * C::DMAS>();
            lds_barrier();
            issue(s + C::DEPTH - 1);
        }
        wait_vm<0>();
        return;
    }

    // ---------------------------------------------------------- compute waves
    f4 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < kch; ++s) {
        lds_barrier();
        const h8 *st = ring + (s % C::DEPTH) * C::STAGE_UNITS;
        const h8 *wst = st + C::A_UNITS + wave * C::W_UNITS;
        const uint2 *codes = reinterpret_cast<const uint2 *>(wst);
        const uint32_t *scales = reinterpret_cast<const uint32_t *>(wst + C::C_UNITS);
        uint2 bw[C::TN];
        h2 bs[C::TN];
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            bw[j] = codes[j * 64 + lane];
            bs[j] = __builtin_bit_cast(h2, scales[j * 16 + (lane & 15)]);
        }
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
                    const h8 bq = q4_word_codes(kb ? bw[j].y : bw[j].x);
                    const float dj = (float)bs[j][kb];
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
                for (int j = 0; j < C::TN; ++j) bf[j] = q4_word_to_h8(kb ? bw[j].y : bw[j].x, bs[j][kb]);
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
#pragma unroll
                    for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
            }
        }
    }
    gemm_epilogue<C::TM, C::TN>(a, acc, m0, n0 + wave * C::WN, lane);
}

template <class C>
int launch_cfg(const GemmArgs &a, hipStream_t s) {
    if (a.W.N % C::BN) return PPX_E_UNSUPPORTED;
    dim3 grid(a.W.N / C::BN, (a.M + C::BM - 1) / C::BM);
    hipLaunchKernelGGL((k_q4gemm<C>), grid, dim3(C::NT), 0, s, a);
    return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP;
}

}  // namespace

// Tile shapes measured on the E2B-like shapes at M = 512 (one MI355X):
//  * wide outputs (gate|up, N >= 8192): 64 x 128 tiles, a three-stage ring
//    (39 KB of LDS: four workgroups per CU);
//  * narrow outputs (N <= 512): 32 x 64 tiles with two compute waves, for
//    enough workgroups;
//  * the rest (Q, O, down, PLE up): 32 x 128 tiles.
int launch_gemm(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    if (a.W.N % 128 || a.W.K % 64 || !a.A) return PPX_E_UNSUPPORTED;
    if (a.W.N >= 8192) return launch_cfg<Cfg<4, 2, 4, 3, false>>(a, s);
    if (a.W.N <= 512) return launch_cfg<Cfg<2, 2, 2, 4, false>>(a, s);
    return launch_cfg<Cfg<2, 2, 4, 4, false>>(a, s);
}

int launch_gemm_exact(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    if (a.W.N % 128 || a.W.K % 64 || !a.A || !a.A2) return PPX_E_UNSUPPORTED;
    return launch_cfg<Cfg<1, 2, 4, 4, true>>(a, s);
}

}  // namespace ppx
