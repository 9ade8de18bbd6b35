// The per-layer-embedding block of the row-batched layers in one kernel.
//
// For 16 rows of one unit:
//   c = the rows' RMSNorm with the block's gain (fp16, fragment-tiled; the
//       down projection's epilogue wrote it),
//   p = gelu(c Wg^T) * s * deq(ple_table[token][il*E + j])      [16 x E]
//   x += p Wu^T                                                 [16 x d]
// p never leaves the workgroup: it is rounded to fp16 into LDS in the
// A-operand order of v_mfma_f32_16x16x32_f16 and read back as the A operand of
// the second product.  Two launches (a GEMM whose epilogue forms p, another
// that adds p Wu^T) become one, and p's round trip through memory goes away.
//
// Eight waves.  Phase 1: wave (kq, ch) = (wave / 2, wave % 2) takes gate
// columns [128 ch, 128 ch + 128) over the kq-th quarter of K = d; all of its
// A fragments and weight codes are requested at once, so the wave waits for
// one memory round trip instead of one per K step.  The four quarters' partial
// sums meet in LDS and are added in quarter order by the wave that forms p for
// columns [32 w, 32 w + 32) (its per-layer-embedding values were requested
// when the kernel started).  Phase 2: the workgroup's share of the d outputs
// (all of them, or one half when two workgroups split the columns of a row
// tile to fill the chip; each then forms p itself) in 16-column groups w,
// w + 8, ..., K = E from LDS, weight codes again requested at once.
#include "ppx_dev.h"

namespace ppx {

namespace {

constexpr int PLE_WAVES = 8;
constexpr int PLE_KQ = 6;   // 64-wide K steps per quarter: d = 4 * 64 * 6
constexpr int PLE_CG = 8;   // phase-1 column groups per wave: E = 2 * 8 * 16

// P2: phase-2 column groups per wave (d / 16 / 8 / halves)
template <int E, int P2>
__global__ __launch_bounds__(64 * PLE_WAVES) void k_ple_fused(const PleGroup grp, int halves) {
    static_assert(E == 2 * PLE_CG * 16, "gate width");
    constexpr int KS2 = E / 32, KC2 = E / 64;     // phase-2 K steps (32 and 64 wide)
    __shared__ h8 pl[KS2 * 64];                   // p of the 16 rows, A-fragment order
    __shared__ float xch[4][2 * PLE_CG][4][64];   // partial sums [quarter][column group][r][lane]
    const PleArgs &a = grp.u[blockIdx.z];
    const int row0 = blockIdx.x * 16;
    if (row0 >= a.M) return;  // past this unit's rows (the whole workgroup)
    const int half = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int kq = wave >> 1, ch = wave & 1;
    const int lc = lane & 15, lr = (lane >> 4) * 4;
    const int d = a.wu.N, kch = d >> 6;

    // token ids of the lane's rows first: the per-layer-embedding values need them
    int tk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) tk[r] = a.tok[min(row0 + lr + r, a.M - 1)];

    // the per-layer-embedding factors of this wave's p columns 32 w + 16 j + lc,
    // requested before the products' operands: both columns of
    // a row sit in one 32-wide Q4_0 block of its table row (the low and high
    // nibble of code byte lc), so a row takes one scale and one code byte
    uint16_t dbits[4];
    uint8_t code[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint8_t *b = a.ple_raw + (size_t)tk[r] * a.ple_row_blocks * 18 +
                           (size_t)((a.ple_col0 + 32 * wave) >> 5) * 18;
        dbits[r] = *reinterpret_cast<const uint16_t *>(b);
        code[r] = b[2 + lc];
    }

    // ---- phase 1: gate columns of groups 8 ch .. 8 ch + 7 over K steps [6 kq, 6 kq + 6)
    {
        const h8 *A = reinterpret_cast<const h8 *>(a.a) + (size_t)(row0 >> 4) * (d >> 5) * 64 + lane;
        const uint2 *gn = reinterpret_cast<const uint2 *>(a.wg.nib) + lane;
        const uint32_t *gs = reinterpret_cast<const uint32_t *>(a.wg.scl) + lc;
        h8 af[PLE_KQ][2];
        uint2 bw[PLE_KQ][PLE_CG];
        uint32_t bs[PLE_KQ][PLE_CG];
#pragma unroll
        for (int t = 0; t < PLE_KQ; ++t) {
            const int k = kq * PLE_KQ + t;
            af[t][0] = A[(size_t)(2 * k) * 64];
            af[t][1] = A[(size_t)(2 * k + 1) * 64];
#pragma unroll
            for (int j = 0; j < PLE_CG; ++j) {
                const size_t base = (size_t)(ch * PLE_CG + j) * kch + k;
                bw[t][j] = gn[base * 64];
                bs[t][j] = gs[base * 16];
            }
        }
        f4 acc[PLE_CG];
#pragma unroll
        for (int j = 0; j < PLE_CG; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < PLE_KQ; ++t)
#pragma unroll
            for (int j = 0; j < PLE_CG; ++j) {
                const h2 dd = __builtin_bit_cast(h2, bs[t][j]);
                acc[j] = mfma16(af[t][0], q4_word_to_h8(bw[t][j].x, dd[0]), acc[j]);
                acc[j] = mfma16(af[t][1], q4_word_to_h8(bw[t][j].y, dd[1]), acc[j]);
            }
#pragma unroll
        for (int j = 0; j < PLE_CG; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) xch[kq][ch * PLE_CG + j][r][lane] = acc[j][r];
    }
    // (the table bytes were requested before the operands, so they have landed)
    float pf32[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float dv = row0 + lr + r < a.M ? a.ple_s * __half2float(__ushort_as_half(dbits[r])) : 0.f;
        pf32[0][r] = dv * (float)((int)(code[r] & 15) - 8);
        pf32[1][r] = dv * (float)((int)(code[r] >> 4) - 8);
    }

    // phase 2's weight codes do not depend on p: request them now
    const int ngrp = d >> 4, per = ngrp / halves;
    const int g0 = half * per + wave;  // groups g0 + 8 i, i < P2 = per / 8
    const uint2 *un = reinterpret_cast<const uint2 *>(a.wu.nib) + lane;
    const uint32_t *us = reinterpret_cast<const uint32_t *>(a.wu.scl) + lc;
    uint2 cw[P2][KC2];
    uint32_t cs[P2][KC2];
    float xv[P2][4];  // the residual rows this wave adds to, read up front too
#pragma unroll
    for (int i = 0; i < P2; ++i) {
        const int g = g0 + PLE_WAVES * i;
#pragma unroll
        for (int k = 0; k < KC2; ++k) {
            const size_t base = (size_t)g * KC2 + k;
            cw[i][k] = un[base * 64];
            cs[i][k] = us[base * 16];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = min(row0 + lr + r, a.M - 1);
            xv[i][r] = a.x[(size_t)row * d + g * 16 + lc];
        }
    }
    __syncthreads();

    // p = gelu(g) * s * deq(ple row) for column groups 2 w, 2 w + 1: the four
    // quarters summed in order, fp16 into LDS at the A-operand position of
    // (row, column); rows past M hold zeros (their results are never stored)
    {
        _Float16 *pp = reinterpret_cast<_Float16 *>(pl);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int cg = 2 * wave + j;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gsum = ((xch[0][cg][r][lane] + xch[1][cg][r][lane]) + xch[2][cg][r][lane]) +
                                   xch[3][cg][r][lane];
                pp[tiled_index(lr + r, cg * 16 + lc, E)] = (_Float16)(gelu_tanh_f(gsum) * pf32[j][r]);
            }
        }
    }
    __syncthreads();

    // ---- phase 2: x[rows][n] += p . Wu[n], 16-column groups g0, g0 + 8, ... < g1
    h8 pf[KS2];
#pragma unroll
    for (int k = 0; k < KS2; ++k) pf[k] = pl[k * 64 + lane];
#pragma unroll
    for (int i = 0; i < P2; ++i) {
        const int g = g0 + PLE_WAVES * i;
        f4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KC2; ++k) {
            const h2 dd = __builtin_bit_cast(h2, cs[i][k]);
            y = mfma16(pf[2 * k], q4_word_to_h8(cw[i][k].x, dd[0]), y);
            y = mfma16(pf[2 * k + 1], q4_word_to_h8(cw[i][k].y, dd[1]), y);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = row0 + lr + r;
            if (row < a.M) a.x[(size_t)row * d + g * 16 + lc] = xv[i][r] + y[r];
        }
    }
}

}  // namespace

// E = 256 and d = 4 quarters of PLE_KQ 64-wide K steps (1536)
bool ple_fused_supported(int E, int d) { return E == 256 && d == 4 * 64 * PLE_KQ; }

int launch_ple_group(const PleArgs *units, int n, hipStream_t s) {
    if (n < 1 || n > kMaxUnits) return PPX_E_INVAL;
    PleGroup g;
    int mt = 0;
    for (int i = 0; i < n; ++i) {
        const PleArgs &u = units[i];
        if (u.M <= 0) continue;
        if (!u.a || !u.x || !u.ple_raw || !u.tok) return PPX_E_INVAL;
        if (!ple_fused_supported(u.wg.N, u.wu.N) || u.wg.K != u.wu.N || u.wu.K != u.wg.N) return PPX_E_UNSUPPORTED;
        if (g.n && (u.wg.N != g.u[0].wg.N || u.wu.N != g.u[0].wu.N)) return PPX_E_INVAL;
        g.u[g.n++] = u;
        mt = std::max(mt, (u.M + 15) / 16);
    }
    if (!g.n) return PPX_OK;
    // two workgroups per row tile (each forms p, then adds half of the columns)
    // when one per tile would leave most of the chip idle
    const int halves = mt * g.n >= 256 ? 1 : 2;
    // d = 1536: 96 column groups, 12 or 6 per wave
    if (halves == 1) hipLaunchKernelGGL((k_ple_fused<256, 12>), dim3(mt, 1, g.n), dim3(64 * PLE_WAVES), 0, s, g, 1);
    else hipLaunchKernelGGL((k_ple_fused<256, 6>), dim3(mt, 2, g.n), dim3(64 * PLE_WAVES), 0, s, g, 2);
    return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP;
}

}  // namespace ppx
