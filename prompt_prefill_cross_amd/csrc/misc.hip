// Elementwise, gather and single-row (HBM-bound) kernels of the prefill path.
#include "ppx_dev.h"

namespace ppx {

namespace {

// x[t][k] = scale * W[id_t][k]: token-embedding gather from the repacked table.
__global__ __launch_bounds__(256) void k_embed(Q4R w, const int32_t *ids, float scale, float *x) {
    const int t = blockIdx.x;
    const int id = ids[t];
    for (int k = threadIdx.x; k < w.K; k += 256) x[(size_t)t * w.K + k] = scale * q4r_weight(w, id, k);
}

__device__ __forceinline__ float block_sum_256(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// out[t] = x[t] / sqrt(mean(x[t]^2) + eps) * g, one workgroup per row.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(const float *x, const float *g, float eps, int d, T *out) {
    __shared__ float red[4];
    const float *xr = x + (size_t)blockIdx.x * d;
    float ss = 0.f;
    for (int k = threadIdx.x; k < d; k += 256) ss += xr[k] * xr[k];
    ss = block_sum_256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    T *o = out + (size_t)blockIdx.x * d;
    for (int k = threadIdx.x; k < d; k += 256) o[k] = (T)(xr[k] * r * g[k]);
}

// y = rmsnorm(x) -> fp16 in the fragment-tiled layout, one wave per row; with
// LO, also lo = fp16(y - fp16(y)) (the split operand of the exact-weight
// GEMM).  Lane l handles the 8-column chunks l, l+64, ... of its row, kept in
// registers between the sum of squares and the scaling.
constexpr int NORM_MAX_CHUNKS = 8;  // d <= 8 * 8 * 64 = 4096
template <bool LO>
__global__ __launch_bounds__(256) void k_rmsnorm_tiled(const float *x, const float *g, float eps, int M, int d,
                                                       __half *hi, __half *lo) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const float *xr = x + (size_t)row * d;
    const int nch = d >> 3;
    float4 v[NORM_MAX_CHUNKS][2];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NORM_MAX_CHUNKS; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
            v[c][0] = *reinterpret_cast<const float4 *>(xr + ch * 8);
            v[c][1] = *reinterpret_cast<const float4 *>(xr + ch * 8 + 4);
            ss += v[c][0].x * v[c][0].x + v[c][0].y * v[c][0].y + v[c][0].z * v[c][0].z + v[c][0].w * v[c][0].w;
            ss += v[c][1].x * v[c][1].x + v[c][1].y * v[c][1].y + v[c][1].z * v[c][1].z + v[c][1].w * v[c][1].w;
        }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int c = 0; c < NORM_MAX_CHUNKS; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
            const float4 g0 = *reinterpret_cast<const float4 *>(g + ch * 8);
            const float4 g1 = *reinterpret_cast<const float4 *>(g + ch * 8 + 4);
            const float y[8] = {v[c][0].x * r * g0.x, v[c][0].y * r * g0.y, v[c][0].z * r * g0.z, v[c][0].w * r * g0.w,
                                v[c][1].x * r * g1.x, v[c][1].y * r * g1.y, v[c][1].z * r * g1.z, v[c][1].w * r * g1.w};
            h8 yh, yl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                yh[e] = (_Float16)y[e];
                if (LO) yl[e] = (_Float16)(y[e] - (float)yh[e]);
            }
            const size_t o = tiled_index(row, ch * 8, d);
            *reinterpret_cast<h8 *>(hi + o) = yh;
            if (LO) *reinterpret_cast<h8 *>(lo + o) = yl;
        }
    }
}

// Row-major fp16 [M][K] -> fragment-tiled.
__global__ void k_tile_f16(const __half *src, int M, int K, __half *dst) {
    const int nch = K >> 3;
    const size_t total = (size_t)M * nch;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const int r = (int)(i / nch), ch = (int)(i % nch);
        *reinterpret_cast<h8 *>(dst + tiled_index(r, ch * 8, K)) =
            *reinterpret_cast<const h8 *>(src + (size_t)r * K + ch * 8);
    }
}

__global__ void k_dequant(Q4R w, float *out) {
    const size_t total = (size_t)w.N * w.K;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const int n = (int)(i / w.K), k = (int)(i % w.K);
        out[i] = q4r_weight(w, n, k);
    }
}

__global__ void k_fill_u32(uint32_t *p, uint32_t v, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void k_copy_f32(const float *src, float *dst, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) dst[i] = src[i];
}

int ok() { return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP; }

// ------------------------------------------------------------------ GEMV
// y[n] = sum_k W[n][k] x[k] for one fp32 row (the pruned layers and the head).
// The row runs through the MFMA as two rows of the A operand: row 0 holds
// fp16(x) and row 1 holds fp16(x - fp16(x)), so their sum carries x to ~22
// bits; B holds (code - 8) exactly, and each block's partial is scaled by its
// fp32 block scale -- only fp32 accumulation rounds.
// A workgroup owns one pair of 16-row groups (RoPE and gate/up partners sit in
// such a pair); KW waves per group split K, and their partial sums meet in LDS
// in wave order, so the result is deterministic and no workgroup waits for
// another.
template <int KW>
__global__ __launch_bounds__(128 * KW) void k_q4gemv(GemvArgs a) {
    __shared__ float red[2][KW][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = wave / KW, kw = wave % KW;
    const int grp = 2 * blockIdx.x + half;
    const int kch = a.W.K >> 6;
    const int per = (kch + KW - 1) / KW;
    const int c0 = kw * per, c1 = min(kch, c0 + per);
    const int col = lane & 15, g = lane >> 4;
    const bool arow = col < 2;  // A rows 0 (hi) and 1 (lo) carry x

    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint2 *nib = reinterpret_cast<const uint2 *>(a.W.nib) + (size_t)grp * kch * 64 + lane;
    const uint32_t *scl = reinterpret_cast<const uint32_t *>(a.W.scl) + (size_t)grp * kch * 16 + col;
#pragma unroll 2
    for (int kc = c0; kc < c1; ++kc) {
        const uint2 w = nib[(size_t)kc * 64];
        const h2 d = __builtin_bit_cast(h2, scl[(size_t)kc * 16]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            h8 af = h8{0, 0, 0, 0, 0, 0, 0, 0};
            if (arow) {
                const float4 *xv = reinterpret_cast<const float4 *>(a.x + kc * 64 + s * 32 + g * 8);
                const float4 x0 = xv[0], x1 = xv[1];
                const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const _Float16 hi = (_Float16)xs[e];
                    af[e] = col == 0 ? hi : (_Float16)(xs[e] - (float)hi);
                }
            }
            const h8 bf = q4_word_codes(s ? w.y : w.x);
            const f4 p = mfma16(af, bf, f4{0.f, 0.f, 0.f, 0.f});
            acc += (float)d[s] * p;
        }
    }
    // lanes 0..15 hold rows 0 and 1 (hi and lo parts) of column `col`
    if (lane < 16) red[half][kw][lane] = acc[0] + acc[1];
    __syncthreads();
    if (threadIdx.x >= 16) return;
    const int c = threadIdx.x;
    float ya = 0.f, yb = 0.f;
#pragma unroll
    for (int i = 0; i < KW; ++i) {
        ya += red[0][i][c];
        yb += red[1][i][c];
    }
    const int n0 = blockIdx.x * 32;
    switch (a.epi) {
    case GV_F32:
        a.out[n0 + c] = ya;
        a.out[n0 + 16 + c] = yb;
        break;
    case GV_ADD:
        a.out[n0 + c] += ya;
        a.out[n0 + 16 + c] += yb;
        break;
    case GV_QROPE: {
        const int hd = a.hd, hh = hd >> 1;
        const int h = n0 / hd, rr = n0 % hd;
        const int ii = (rr >> 5) * 16 + c;
        const float2 cs = a.rope[(size_t)a.pos * hh + ii];
        a.out[h * hd + ii] = ya * cs.x - yb * cs.y;
        a.out[h * hd + ii + hh] = ya * cs.y + yb * cs.x;
        break;
    }
    case GV_GLU:
        a.out[blockIdx.x * 16 + c] = act_f(a.act, ya) * yb;
        break;
    case GV_PLE: {
        const uint8_t *prow = a.ple_raw + (size_t)a.tok * a.ple_row_blocks * 18;
        a.out[n0 + c] = gelu_tanh_f(ya) * (a.ple_s * q4_raw_weight(prow, a.ple_col0 + n0 + c));
        a.out[n0 + 16 + c] = gelu_tanh_f(yb) * (a.ple_s * q4_raw_weight(prow, a.ple_col0 + n0 + 16 + c));
        break;
    }
    }
}

// waves per 16-row group: enough waves in flight to cover memory latency,
// at least two 64-wide K chunks per wave
int gemv_kw(int N, int K) {
    const int groups = N / 16, kch = K / 64;
    int kw = 1;
    while (kw < 8 && groups * kw < 2048 && kch / (2 * kw) >= 2) kw *= 2;
    return kw;
}

}  // namespace

int launch_gemv(const GemvArgs &a, hipStream_t s) {
    if (a.W.N % 32 || a.W.K % 64 || !a.x || !a.out) return PPX_E_UNSUPPORTED;
    const dim3 grid(a.W.N / 32);
    switch (gemv_kw(a.W.N, a.W.K)) {
    case 1: hipLaunchKernelGGL(k_q4gemv<1>, grid, dim3(128), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_q4gemv<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_q4gemv<4>, grid, dim3(512), 0, s, a); break;
    default: hipLaunchKernelGGL(k_q4gemv<8>, grid, dim3(1024), 0, s, a); break;
    }
    return ok();
}

int launch_embed(const Q4R &tok, const int32_t *ids, int M, float scale, float *x, hipStream_t s) {
    if (M <= 0) return PPX_OK;
    hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, s, tok, ids, scale, x);
    return ok();
}

int launch_rmsnorm_f16(const float *x, const float *g, float eps, int M, int d, __half *out, hipStream_t s) {
    if (M <= 0) return PPX_OK;
    if (d % 32 || d > NORM_MAX_CHUNKS * 8 * 64) return PPX_E_UNSUPPORTED;
    hipLaunchKernelGGL((k_rmsnorm_tiled<false>), dim3((M + 3) / 4), dim3(256), 0, s, x, g, eps, M, d, out, nullptr);
    return ok();
}

int launch_rmsnorm_split(const float *x, const float *g, float eps, int M, int d, __half *hi, __half *lo,
                         hipStream_t s) {
    if (M <= 0) return PPX_OK;
    if (d % 32 || d > NORM_MAX_CHUNKS * 8 * 64) return PPX_E_UNSUPPORTED;
    hipLaunchKernelGGL((k_rmsnorm_tiled<true>), dim3((M + 3) / 4), dim3(256), 0, s, x, g, eps, M, d, hi, lo);
    return ok();
}

int launch_tile_f16(const __half *src, int M, int K, __half *dst, hipStream_t s) {
    if (M <= 0) return PPX_OK;
    if (K % 32) return PPX_E_UNSUPPORTED;
    const size_t n = (size_t)M * (K >> 3);
    hipLaunchKernelGGL(k_tile_f16, dim3((unsigned)std::min<size_t>((n + 255) / 256, 4096)), dim3(256), 0, s, src, M, K,
                       dst);
    return ok();
}

int launch_rmsnorm_f32(const float *x, const float *g, float eps, int M, int d, float *out, hipStream_t s) {
    if (M <= 0) return PPX_OK;
    hipLaunchKernelGGL((k_rmsnorm<float>), dim3(M), dim3(256), 0, s, x, g, eps, d, out);
    return ok();
}

int launch_dequant(const Q4R &w, float *out, hipStream_t s) {
    hipLaunchKernelGGL(k_dequant, dim3(2048), dim3(256), 0, s, w, out);
    return ok();
}

int launch_fill_u32(uint32_t *p, uint32_t v, size_t n, hipStream_t s) {
    if (!n) return PPX_OK;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, s, p, v, n);
    return ok();
}

int launch_copy_f32(const float *src, float *dst, int n, hipStream_t s) {
    if (n <= 0) return PPX_OK;
    hipLaunchKernelGGL(k_copy_f32, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, s, src,
                       dst, n);
    return ok();
}

}  // namespace ppx
