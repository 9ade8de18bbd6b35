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

// y = rmsnorm(x) split into hi = fp16(y) and lo = fp16(y - hi).
__global__ __launch_bounds__(256) void k_rmsnorm_split(const float *x, const float *g, float eps, int d,
                                                       __half *hi, __half *lo) {
    __shared__ float red[4];
    const float *xr = x + (size_t)blockIdx.x * d;
    float ss = 0.f;
    for (int k = threadIdx.x; k < d; k += 256) ss += xr[k] * xr[k];
    ss = block_sum_256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    const size_t o = (size_t)blockIdx.x * d;
    for (int k = threadIdx.x; k < d; k += 256) {
        const float y = xr[k] * r * g[k];
        const __half h = __float2half(y);
        hi[o + k] = h;
        lo[o + k] = __float2half(y - __half2float(h));
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

// ------------------------------------------------------------------ GEMV
// y[n] = sum_k W[n][k] x[k] for one fp32 row, weights decoded exactly in fp32.
// Grid: (N/32 column pairs, ksplit).  A workgroup (4 waves) owns one pair of
// 16-column groups and a contiguous range of 64-wide K chunks; lane l covers
// column l%16 and the eight k's 8*(l/16)..+7 of each block.  Partial sums of
// the ksplit workgroups of a pair go to scratch; the last one to arrive (an
// integer counter) adds them in split order and applies the epilogue, so
// the result does not depend on arrival order.
__global__ __launch_bounds__(256) void k_q4gemv(GemvArgs a) {
    __shared__ float red[4][2][16];
    __shared__ int last;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pair = blockIdx.x, split = blockIdx.y;
    const int kch = a.W.K >> 6;
    const int per = (kch + a.ksplit - 1) / a.ksplit;
    const int c0 = split * per, c1 = min(kch, c0 + per);
    const int col = lane & 15, g = lane >> 4;

    float acc0 = 0.f, acc1 = 0.f;
    for (int kc = c0 + wave; kc < c1; kc += 4) {
        const size_t b0 = (size_t)(2 * pair) * kch + kc;
        const size_t b1 = (size_t)(2 * pair + 1) * kch + kc;
        const uint2 w0 = *reinterpret_cast<const uint2 *>(a.W.nib + (b0 * 64 + lane) * 2);
        const uint2 w1 = *reinterpret_cast<const uint2 *>(a.W.nib + (b1 * 64 + lane) * 2);
        const h2 d0 = __builtin_bit_cast(h2, *reinterpret_cast<const uint32_t *>(a.W.scl + (b0 * 16 + col) * 2));
        const h2 d1 = __builtin_bit_cast(h2, *reinterpret_cast<const uint32_t *>(a.W.scl + (b1 * 16 + col) * 2));
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float *xv = a.x + kc * 64 + s * 32 + g * 8;
            const float4 xa = *reinterpret_cast<const float4 *>(xv);
            const float4 xb = *reinterpret_cast<const float4 *>(xv + 4);
            const float xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            const uint32_t u0 = s ? w0.y : w0.x, u1 = s ? w1.y : w1.x;
            const float dd0 = (float)d0[s], dd1 = (float)d1[s];
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p0 += (float)(q4_word_code(u0, e) - 8) * xs[e];
                p1 += (float)(q4_word_code(u1, e) - 8) * xs[e];
            }
            acc0 += dd0 * p0;
            acc1 += dd1 * p1;
        }
    }
    acc0 += __shfl_xor(acc0, 16, 64);
    acc0 += __shfl_xor(acc0, 32, 64);
    acc1 += __shfl_xor(acc1, 16, 64);
    acc1 += __shfl_xor(acc1, 32, 64);
    if (lane < 16) {
        red[wave][0][lane] = acc0;
        red[wave][1][lane] = acc1;
    }
    __syncthreads();
    const int N = a.W.N;
    const int n0 = pair * 32;
    if (a.ksplit > 1) {
        if (threadIdx.x < 32) {
            const int t = threadIdx.x >> 4, c = threadIdx.x & 15;
            const float v = red[0][t][c] + red[1][t][c] + red[2][t][c] + red[3][t][c];
            a.partial[(size_t)split * N + n0 + t * 16 + c] = v;
        }
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t prev = atomicAdd(a.counter + pair, 1u);
            last = (prev == (uint32_t)(a.ksplit - 1));
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
        if (threadIdx.x < 32) {
            const int t = threadIdx.x >> 4, c = threadIdx.x & 15;
            float v = 0.f;
            for (int sp = 0; sp < a.ksplit; ++sp)
                v += __builtin_nontemporal_load(a.partial + (size_t)sp * N + n0 + t * 16 + c);
            red[0][t][c] = v;
        }
        if (threadIdx.x == 0) a.counter[pair] = 0u;
        __syncthreads();
    } else {
        if (threadIdx.x < 32) {
            const int t = threadIdx.x >> 4, c = threadIdx.x & 15;
            red[0][t][c] = red[0][t][c] + red[1][t][c] + red[2][t][c] + red[3][t][c];
        }
        __syncthreads();
    }
    if (threadIdx.x >= 16) return;
    const int c = threadIdx.x;
    const float ya = red[0][0][c], yb = red[0][1][c];
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
        const int hd = a.hd, half = hd >> 1;
        const int h = n0 / hd, rr = n0 % hd;
        const int ii = (rr >> 5) * 16 + c;
        const float2 cs = a.rope[(size_t)a.pos * half + ii];
        a.out[h * hd + ii] = ya * cs.x - yb * cs.y;
        a.out[h * hd + ii + half] = ya * cs.y + yb * cs.x;
        break;
    }
    case GV_GLU:
        a.out[pair * 16 + c] = act_f(a.act, ya) * yb;
        break;
    case GV_PLE: {
        const uint8_t *prow = a.ple_raw + (size_t)a.tok * a.ple_row_blocks * 18;
        a.out[n0 + c] = gelu_tanh_f(ya) * (a.ple_s * q4_raw_weight(prow, a.ple_col0 + n0 + c));
        a.out[n0 + 16 + c] = gelu_tanh_f(yb) * (a.ple_s * q4_raw_weight(prow, a.ple_col0 + n0 + 16 + c));
        break;
    }
    }
}

int ok() { return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP; }

int gemv_splits(int N, int K) {
    const int pairs = N / 32, kch = K / 64;
    int s = 1;
    while (pairs * s < 1024 && s * 2 <= kch / 4) s *= 2;
    return s;
}

}  // namespace

size_t gemv_scratch_floats(int N, int K) { return (size_t)gemv_splits(N, K) * N; }

int launch_gemv(const GemvArgs &a0, hipStream_t s) {
    GemvArgs a = a0;
    if (a.W.N % 32 || a.W.K % 64) return PPX_E_UNSUPPORTED;
    a.ksplit = gemv_splits(a.W.N, a.W.K);
    if (a.ksplit > 1 && (!a.partial || !a.counter)) return PPX_E_INVAL;
    hipLaunchKernelGGL(k_q4gemv, dim3(a.W.N / 32, a.ksplit), dim3(256), 0, s, a);
    return ok();
}

int launch_embed(const Q4R &tok, const int32_t *ids, int M, float scale, float *x, hipStream_t s) {
    if (M <= 0) return PPX_OK;
    hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, s, tok, ids, scale, x);
    return ok();
}

int launch_rmsnorm_f16(const float *x, const float *g, float eps, int M, int d, __half *out, hipStream_t s) {
    if (M <= 0) return PPX_OK;
    hipLaunchKernelGGL((k_rmsnorm<__half>), dim3(M), dim3(256), 0, s, x, g, eps, d, out);
    return ok();
}

int launch_rmsnorm_split(const float *x, const float *g, float eps, int M, int d, __half *hi, __half *lo,
                         hipStream_t s) {
    if (M <= 0) return PPX_OK;
    hipLaunchKernelGGL(k_rmsnorm_split, dim3(M), dim3(256), 0, s, x, g, eps, d, hi, lo);
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
