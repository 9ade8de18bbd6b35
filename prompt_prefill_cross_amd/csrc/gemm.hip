// Q4_0 dequant-fused GEMM on CDNA4 MFMA (v_mfma_f32_16x16x32_f16).
//
//   C[M][N] = A[M][K] (fp16 activations) x W[N][K]^T (Q4_0), fp32 accumulate.
//
// A workgroup of WGM x WGN waves computes a BM x BN tile, each wave a
// (BM/WGM) x (BN/WGN) block of 16x16 MFMA tiles.  K advances 64 (two Q4_0
// blocks) per stage through two LDS buffers; global loads run two stages ahead
// of the MFMAs (two register sets, the loop unrolled by two), so a stage's
// memory latency overlaps two stages of matrix work.  A is staged as fp16 in
// the MFMA A fragment order -- one wave store fills one 1 KB fragment, lane by
// lane -- and W is read as repacked codes + fp16 block scales, decoded in
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

template <int BM_, int BN_, int WGM_, int WGN_, bool EXACT_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
    static constexpr bool EXACT = EXACT_;
    static constexpr int NT = 64 * WGM * WGN;            // threads
    static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
    static constexpr int TM = WM / 16, TN = WN / 16;
    static constexpr int A_UNITS = 2 * (BM / 16) * 64;   // 16-byte units per stage, per A part
    static constexpr int B_UNITS = 2 * (BN / 16) * 64;
    static constexpr int NA = EXACT ? 2 : 1;             // A parts staged
    static constexpr int S_FLOATS = EXACT ? 2 * BN : 0;  // block scales per stage
    static constexpr int STAGE_UNITS = NA * A_UNITS + B_UNITS + S_FLOATS / 4;
    static constexpr int A_LOADS = A_UNITS / NT;         // per thread, per part
    static constexpr int B_SLOTS = (BN / 16) * 64 / NT;  // lane slots per thread
    static_assert(TM >= 1 && TN >= 2 && TN % 2 == 0, "wave tile");
    static_assert(A_UNITS % NT == 0 && A_LOADS >= 1, "A staging");
    static_assert((BN / 16) * 64 % NT == 0 && B_SLOTS >= 1, "B staging");
};

// One stage of operands held in registers between its global load and its LDS store.
template <class C>
struct Stage {
    h8 ar[C::NA][C::A_LOADS];
    uint2 br[C::B_SLOTS];
    uint32_t sr[C::B_SLOTS];

    // Loads are branch-free (rows past M are clamped, then zeroed by a select),
    // so the compiler can count outstanding loads exactly and keep the next
    // stage's loads in flight across this stage's store.
    __device__ __forceinline__ void load(const GemmArgs &a, int m0, int n0, int kc) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
            // unit u = [kb][16-row subtile][lane]; lane l holds row 16*sub + l%16, k = 32*kb + 8*(l/16)
            const int u = tid + i * C::NT;
            const int kb = u / ((C::BM / 16) * 64), rem = u % ((C::BM / 16) * 64);
            const int row = m0 + (rem >> 6) * 16 + (rem & 15);
            const unsigned off = (unsigned)(min(row, a.M - 1) * a.lda + kc * KSTEP + kb * 32 + ((rem >> 4) & 3) * 8);
#pragma unroll
            for (int p = 0; p < C::NA; ++p) {
                const __half *src = p ? a.A2 : a.A;
                ar[p][i] = *reinterpret_cast<const h8 *>(src + off);
            }
        }
        const unsigned kchunks = (unsigned)a.W.K >> 6;
#pragma unroll
        for (int i = 0; i < C::B_SLOTS; ++i) {
            const unsigned sl = tid + i * C::NT;
            const unsigned grp = sl >> 6, ln = sl & 63;
            const unsigned base = (((unsigned)n0 >> 4) + grp) * kchunks + kc;
            br[i] = *reinterpret_cast<const uint2 *>(a.W.nib + (base * 64 + ln) * 2);
            sr[i] = *reinterpret_cast<const uint32_t *>(a.W.scl + (base * 16 + (ln & 15)) * 2);
        }
    }

    __device__ __forceinline__ void store(h8 *lds, int m0, int M) const {
        const int tid = threadIdx.x;
        if (m0 + C::BM <= M) {  // uniform: the whole tile is inside the matrix
#pragma unroll
            for (int i = 0; i < C::A_LOADS; ++i)
#pragma unroll
                for (int p = 0; p < C::NA; ++p) lds[p * C::A_UNITS + tid + i * C::NT] = ar[p][i];
        } else {
#pragma unroll
            for (int i = 0; i < C::A_LOADS; ++i) {
                const int rem = (tid + i * C::NT) % ((C::BM / 16) * 64);
                const bool valid = m0 + (rem >> 6) * 16 + (rem & 15) < M;  // rows past M were clamped
#pragma unroll
                for (int p = 0; p < C::NA; ++p)
                    lds[p * C::A_UNITS + tid + i * C::NT] = valid ? ar[p][i] : h8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        h8 *lb = lds + C::NA * C::A_UNITS;
        float *ls = reinterpret_cast<float *>(lb + C::B_UNITS);
#pragma unroll
        for (int i = 0; i < C::B_SLOTS; ++i) {
            const int sl = tid + i * C::NT;
            const int grp = sl >> 6, ln = sl & 63;
            const h2 d2 = __builtin_bit_cast(h2, sr[i]);
            if constexpr (C::EXACT) {
                lb[0 * (C::BN / 16) * 64 + grp * 64 + ln] = q4_word_codes(br[i].x);
                lb[1 * (C::BN / 16) * 64 + grp * 64 + ln] = q4_word_codes(br[i].y);
                if (ln < 16) {
                    ls[grp * 16 + ln] = (float)d2[0];
                    ls[C::BN + grp * 16 + ln] = (float)d2[1];
                }
            } else {
                lb[0 * (C::BN / 16) * 64 + grp * 64 + ln] = q4_word_to_h8(br[i].x, d2[0]);
                lb[1 * (C::BN / 16) * 64 + grp * 64 + ln] = q4_word_to_h8(br[i].y, d2[1]);
            }
        }
    }
};

// The fragments of one stage, read from LDS before the next stage is stored,
// so that the MFMAs of this stage overlap the decode and LDS stores of the next.
template <class C>
struct Frags {
    h8 af[2][C::TM], bf[2][C::TN];
    h8 af2[2][C::EXACT ? C::TM : 1];
    float dsc[2][C::EXACT ? C::TN : 1];

    __device__ __forceinline__ void read(const h8 *lds, int wm, int wn, int lane) {
        const h8 *la = lds;
        const h8 *lb = lds + C::NA * C::A_UNITS;
        const float *ls = reinterpret_cast<const float *>(lb + C::B_UNITS);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < C::TM; ++i) af[kb][i] = la[kb * (C::BM / 16) * 64 + ((wm >> 4) + i) * 64 + lane];
#pragma unroll
            for (int j = 0; j < C::TN; ++j) bf[kb][j] = lb[kb * (C::BN / 16) * 64 + ((wn >> 4) + j) * 64 + lane];
            if constexpr (C::EXACT) {
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
                    af2[kb][i] = la[C::A_UNITS + kb * (C::BM / 16) * 64 + ((wm >> 4) + i) * 64 + lane];
#pragma unroll
                for (int j = 0; j < C::TN; ++j) dsc[kb][j] = ls[kb * C::BN + wn + j * 16 + (lane & 15)];
            }
        }
    }

    __device__ __forceinline__ void mma(f4 (&acc)[C::TM][C::TN]) const {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if constexpr (C::EXACT) {
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int i = 0; i < C::TM; ++i) {
                        f4 p = mfma16(af[kb][i], bf[kb][j], f4{0.f, 0.f, 0.f, 0.f});
                        p = mfma16(af2[kb][i], bf[kb][j], p);
                        acc[i][j] += dsc[kb][j] * p;
                    }
            } else {
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
#pragma unroll
                    for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma16(af[kb][i], bf[kb][j], acc[i][j]);
            }
        }
    }
};

template <class C>
__global__ __launch_bounds__(C::NT) void k_q4gemm(GemmArgs a) {
    using S = C;
    __shared__ h8 lds[2][C::STAGE_UNITS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * C::BN, m0 = blockIdx.y * C::BM;
    const int wm = (wave / C::WGN) * C::WM, wn = (wave % C::WGN) * C::WN;
    const int lc = lane & 15, lr = (lane >> 4) * 4;

    f4 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    // stage s lives in register set (s % 2) between its load and its store
    Stage<C> r0, r1;
    const int nk = a.W.K / KSTEP;
    // nk is even (K % 128 == 0).  Every load, store and MFMA is unconditional:
    // past the last stage the load index is clamped and the duplicate lands in
    // a buffer that is not read again; no branch splits the accumulators'
    // live ranges, so they stay in place across iterations.
    const int last = nk - 1;
    r0.load(a, m0, n0, 0);
    r0.store(lds[0], m0, a.M);
    r1.load(a, m0, n0, 1);
    r0.load(a, m0, n0, min(2, last));
    __syncthreads();
    Frags<C> f;
    for (int kc = 0; kc < nk; kc += 2) {
        f.read(lds[0], wm, wn, lane);  // stage kc
        r1.store(lds[1], m0, a.M);     // stage kc + 1 (lds[1] was last read before the previous barrier)
        f.mma(acc);
        __syncthreads();
        r1.load(a, m0, n0, min(kc + 3, last));
        f.read(lds[1], wm, wn, lane);  // stage kc + 1
        r0.store(lds[0], m0, a.M);     // stage kc + 2
        f.mma(acc);
        __syncthreads();
        r0.load(a, m0, n0, min(kc + 4, last));
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
                            a.vc[(size_t)c * a.vld + pos] = __float2half(va);  // V^T
                            a.vc[(size_t)(c + 16) * a.vld + pos] = __float2half(vb);
                        }
                    }
                }
        }
    }
}

template <class C>
int launch_cfg(const GemmArgs &a, hipStream_t s) {
    dim3 grid(a.W.N / C::BN, (a.M + C::BM - 1) / C::BM);
    hipLaunchKernelGGL((k_q4gemm<C>), grid, dim3(C::NT), 0, s, a);
    return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP;
}

long tiles(const GemmArgs &a, int bm, int bn) {
    return a.W.N % bn ? 0 : (long)(a.W.N / bn) * ((a.M + bm - 1) / bm);
}

}  // namespace

int launch_gemm(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    if (a.W.N % 64 || a.W.K % 128 || a.lda % 8 || !a.A) return PPX_E_UNSUPPORTED;
    // measured on the E2B-like shapes at M = 512: wide outputs (gate|up) run best
    // as 128x256 tiles of eight 64x64 wave tiles; everything narrower as 64x64
    // tiles, which give the most workgroups
    if (a.W.N >= 8192 && tiles(a, 128, 256) >= 128) return launch_cfg<Cfg<128, 256, 2, 4, false>>(a, s);
    return launch_cfg<Cfg<64, 64, 2, 2, false>>(a, s);
}

int launch_gemm_exact(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    if (a.W.N % 64 || a.W.K % 128 || a.lda % 8 || !a.A || !a.A2) return PPX_E_UNSUPPORTED;
    return launch_cfg<Cfg<64, 64, 2, 2, true>>(a, s);
}

}  // namespace ppx
