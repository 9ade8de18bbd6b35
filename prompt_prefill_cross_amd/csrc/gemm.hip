// Q4_0 dequant-fused GEMM on CDNA4 MFMA (v_mfma_f32_16x16x32_f16).
//
//   C[M][N] = A[M][K] (fp16 activations) x W[N][K]^T (Q4_0), fp32 accumulate.
//
// A workgroup of four waves computes a BM x BN tile; the waves form a 2 x 2
// grid of (BM/2) x (BN/2) wave tiles.  K advances 64 (two Q4_0 blocks) per
// stage through double-buffered LDS.  A is staged as fp16 in the MFMA A
// fragment order; W is read as repacked codes + fp16 block scales, decoded in
// registers and written to LDS in B fragment order, so a tile's weights are
// decoded once per workgroup.  Epilogues work on the accumulator registers
// directly; weights whose outputs are combined in pairs (RoPE halves,
// gate/up) are stored with the two members of a pair in adjacent 16-column
// groups, so both values of a pair sit in the same lane.
//
// Two arithmetic modes share the kernel:
//  * fast (EXACT = false): B = fp16(d * (code - 8)), one rounding per weight;
//  * exact (EXACT = true): B = code - 8 (exact in fp16), A = hi + lo split in
//    two fp16 operands, and each 32-wide block's partial sum is scaled by its
//    fp32 block scale before it is added -- only fp32 accumulation rounds.
//    The K and V projections use it, so the cache holds values accurate to
//    the fp16 store itself.
#include "ppx_dev.h"

namespace ppx {

namespace {

constexpr int KSTEP = 64;

template <int BM, int BN, bool EXACT>
struct GemmShape {
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int TM = WM / 16, TN = WN / 16;
    static constexpr int A_UNITS = 2 * (BM / 16) * 64;  // 16-byte units per stage (per A part)
    static constexpr int B_UNITS = 2 * (BN / 16) * 64;
    static constexpr int NA = EXACT ? 2 : 1;             // A parts staged
    static constexpr int S_FLOATS = EXACT ? 2 * BN : 0;  // block scales per stage
    static constexpr int STAGE_UNITS = NA * A_UNITS + B_UNITS + S_FLOATS / 4;
    static constexpr int A_LOADS = BM * 8 / 256;         // A units per thread per stage
    static constexpr int B_LOADS = BN * 4 / 256;         // B lane slots per thread per stage
    static_assert(BM % 32 == 0 && BN % 64 == 0, "tile");
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small for 256 threads");
};

// (code - 8) exactly, as fp16, for the eight codes of a repacked word.
__device__ __forceinline__ h8 q4_word_to_h8_codes(uint32_t w) {
    h8 r;
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t t = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
        h2 v = __builtin_bit_cast(h2, t) - bias;
        r[2 * i] = v[0];
        r[2 * i + 1] = v[1];
    }
    return r;
}

template <int BM, int BN, bool EXACT>
struct Stage {
    using S = GemmShape<BM, BN, EXACT>;
    h8 ar[S::NA][S::A_LOADS];
    uint2 br[S::B_LOADS];
    uint32_t sr[S::B_LOADS];

    __device__ __forceinline__ void load(const GemmArgs &a, int m0, int n0, int kc) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < S::A_LOADS; ++i) {
            const int u = tid + i * 256;
            const int row = u >> 3, k8 = u & 7;
            const int gr = m0 + row;
#pragma unroll
            for (int p = 0; p < S::NA; ++p) {
                const __half *src = p ? a.A2 : a.A;
                if (gr < a.M)
                    ar[p][i] = *reinterpret_cast<const h8 *>(src + (size_t)gr * a.lda + kc * KSTEP + k8 * 8);
                else
                    ar[p][i] = h8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        const int kchunks = a.W.K >> 6;
#pragma unroll
        for (int i = 0; i < S::B_LOADS; ++i) {
            const int sl = tid + i * 256;
            const int grp = sl >> 6, ln = sl & 63;
            const size_t base = (size_t)((n0 >> 4) + grp) * kchunks + kc;
            br[i] = *reinterpret_cast<const uint2 *>(a.W.nib + (base * 64 + ln) * 2);
            sr[i] = *reinterpret_cast<const uint32_t *>(a.W.scl + (base * 16 + (ln & 15)) * 2);
        }
    }

    __device__ __forceinline__ void store(h8 *lds) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < S::A_LOADS; ++i) {
            const int u = tid + i * 256;
            const int row = u >> 3, k8 = u & 7;
            const int kb = k8 >> 2, g = k8 & 3;
#pragma unroll
            for (int p = 0; p < S::NA; ++p)
                lds[p * S::A_UNITS + kb * (BM / 16) * 64 + (row >> 4) * 64 + g * 16 + (row & 15)] = ar[p][i];
        }
        h8 *lb = lds + S::NA * S::A_UNITS;
        float *ls = reinterpret_cast<float *>(lb + S::B_UNITS);
#pragma unroll
        for (int i = 0; i < S::B_LOADS; ++i) {
            const int sl = tid + i * 256;
            const int grp = sl >> 6, ln = sl & 63;
            const h2 d2 = __builtin_bit_cast(h2, sr[i]);
            if constexpr (EXACT) {
                lb[0 * (BN / 16) * 64 + grp * 64 + ln] = q4_word_to_h8_codes(br[i].x);
                lb[1 * (BN / 16) * 64 + grp * 64 + ln] = q4_word_to_h8_codes(br[i].y);
                if (ln < 16) {
                    ls[grp * 16 + ln] = (float)d2[0];
                    ls[BN + grp * 16 + ln] = (float)d2[1];
                }
            } else {
                lb[0 * (BN / 16) * 64 + grp * 64 + ln] = q4_word_to_h8(br[i].x, d2[0]);
                lb[1 * (BN / 16) * 64 + grp * 64 + ln] = q4_word_to_h8(br[i].y, d2[1]);
            }
        }
    }
};

template <int BM, int BN, bool EXACT>
__global__ __launch_bounds__(256) void k_q4gemm(GemmArgs a) {
    using S = GemmShape<BM, BN, EXACT>;
    __shared__ h8 lds[2][S::STAGE_UNITS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int wm = (wave >> 1) * S::WM, wn = (wave & 1) * S::WN;
    const int lc = lane & 15, lr = (lane >> 4) * 4;

    f4 acc[S::TM][S::TN];
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
        for (int j = 0; j < S::TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    Stage<BM, BN, EXACT> st;
    const int nk = a.W.K / KSTEP;
    st.load(a, m0, n0, 0);
    st.store(lds[0]);
    __syncthreads();

    for (int kc = 0; kc < nk; ++kc) {
        const int cur = kc & 1;
        if (kc + 1 < nk) st.load(a, m0, n0, kc + 1);
        const h8 *la = lds[cur];
        const h8 *lb = lds[cur] + S::NA * S::A_UNITS;
        const float *ls = reinterpret_cast<const float *>(lb + S::B_UNITS);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            h8 af[S::TM], bf[S::TN];
#pragma unroll
            for (int i = 0; i < S::TM; ++i) af[i] = la[kb * (BM / 16) * 64 + ((wm >> 4) + i) * 64 + lane];
#pragma unroll
            for (int j = 0; j < S::TN; ++j) bf[j] = lb[kb * (BN / 16) * 64 + ((wn >> 4) + j) * 64 + lane];
            if constexpr (EXACT) {
                h8 af2[S::TM];
#pragma unroll
                for (int i = 0; i < S::TM; ++i)
                    af2[i] = la[S::A_UNITS + kb * (BM / 16) * 64 + ((wm >> 4) + i) * 64 + lane];
#pragma unroll
                for (int j = 0; j < S::TN; ++j) {
                    const float dsc = ls[kb * BN + wn + j * 16 + lc];
#pragma unroll
                    for (int i = 0; i < S::TM; ++i) {
                        f4 p = mfma16(af[i], bf[j], f4{0.f, 0.f, 0.f, 0.f});
                        p = mfma16(af2[i], bf[j], p);
                        acc[i][j] += dsc * p;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < S::TM; ++i)
#pragma unroll
                    for (int j = 0; j < S::TN; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
            }
        }
        if (kc + 1 < nk) st.store(lds[cur ^ 1]);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // acc[i][j][r] = C[row][col], row = m0+wm+16i+4*(lane/16)+r, col = n0+wn+16j+lane%16
    const int N = a.W.N;
    if (a.epi == EPI_F32 || a.epi == EPI_ADD) {
#pragma unroll
        for (int i = 0; i < S::TM; ++i)
#pragma unroll
            for (int j = 0; j < S::TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + wm + i * 16 + lr + r;
                    const int col = n0 + wn + j * 16 + lc;
                    if (row < a.M) {
                        float *p = a.out_f32 + (size_t)row * N + col;
                        if (a.epi == EPI_ADD) *p += acc[i][j][r];
                        else *p = acc[i][j][r];
                    }
                }
    } else if (a.epi == EPI_PLE) {
        const int E = N;
#pragma unroll
        for (int i = 0; i < S::TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + i * 16 + lr + r;
                if (row >= a.M) continue;
                const uint8_t *prow = a.ple_raw + (size_t)a.tok[row] * a.ple_row_blocks * 18;
#pragma unroll
                for (int j = 0; j < S::TN; ++j) {
                    const int col = n0 + wn + j * 16 + lc;
                    const float P = a.ple_s * q4_raw_weight(prow, a.ple_col0 + col);
                    a.out_f16[(size_t)row * E + col] = (_Float16)(gelu_tanh_f(acc[i][j][r]) * P);
                }
            }
    } else {
        // paired epilogues: subtiles (2p, 2p+1) of the wave tile
#pragma unroll
        for (int p = 0; p < S::TN / 2; ++p) {
            const int colA = n0 + wn + p * 32 + lc;  // first member; second = colA + 16
#pragma unroll
            for (int i = 0; i < S::TM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + wm + i * 16 + lr + r;
                    if (row >= a.M) continue;
                    const float va = acc[i][2 * p][r], vb = acc[i][2 * p + 1][r];
                    if (a.epi == EPI_GLU) {
                        const int F = N >> 1;
                        const int f = (colA >> 5) * 16 + lc;
                        a.out_f16[(size_t)row * F + f] = (_Float16)(act_f(a.act, va) * vb);
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
                            __half *v = a.vc + (size_t)pos * a.kvd;
                            v[c] = __float2half(va);
                            v[c + 16] = __float2half(vb);
                        }
                    }
                }
        }
    }
}

template <int BM, int BN, bool EXACT>
int launch_tile(const GemmArgs &a, hipStream_t s) {
    dim3 grid(a.W.N / BN, (a.M + BM - 1) / BM);
    hipLaunchKernelGGL((k_q4gemm<BM, BN, EXACT>), grid, dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP;
}

}  // namespace

int launch_gemm(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    if (a.W.N % 64 || a.W.K % 64 || a.lda % 8 || !a.A) return PPX_E_UNSUPPORTED;
    const long tiles128 = (long)(a.W.N / 128) * ((a.M + 127) / 128);
    if (a.W.N % 128 == 0 && tiles128 >= 192) return launch_tile<128, 128, false>(a, s);
    if (a.W.N % 128 == 0 && (long)(a.W.N / 128) * ((a.M + 63) / 64) >= 128) return launch_tile<64, 128, false>(a, s);
    return launch_tile<64, 64, false>(a, s);
}

int launch_gemm_exact(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    if (a.W.N % 64 || a.W.K % 64 || a.lda % 8 || !a.A || !a.A2) return PPX_E_UNSUPPORTED;
    return launch_tile<64, 64, true>(a, s);
}

}  // namespace ppx
