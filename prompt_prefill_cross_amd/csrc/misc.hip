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

// x[k] = base[k] + scale * deq(w[*id])[k]: one row (the next-n head's input)
__global__ __launch_bounds__(256) void k_embed_add(Q4R w, const int32_t *id, float scale, const float *base,
                                                   float *x) {
    const int t = *id;
    for (int k = threadIdx.x; k < w.K; k += 256) x[k] = base[k] + scale * q4r_weight(w, t, k);
}

typedef __attribute__((address_space(3))) void lds_t;

// Reads nchunks 1 KB chunks through LDS DMA (global_load_lds, 16 bytes per
// lane: the instruction and the per-wave 1 KB pattern of the GEMM's producer
// waves) and XORs the 32-bit words read; workgroup w writes its XOR to
// out[w].  Four waves, one 1 KB LDS slot each.
__global__ __launch_bounds__(256) void k_stream_read(const uint8_t *src, size_t nchunks, uint32_t *out) {
    __shared__ uint4 slot[4][64];
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = 0;
    for (size_t c = (size_t)blockIdx.x * 4 + wave; c < nchunks; c += (size_t)gridDim.x * 4) {
        __builtin_amdgcn_global_load_lds(src + c * 1024 + lane * 16, (lds_t *)&slot[wave][0], 16, 0, 0);
        __builtin_amdgcn_s_waitcnt(0);  // the wave's own DMA has landed in its slot
        const uint4 v = slot[wave][lane];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
        __builtin_amdgcn_s_waitcnt(0);  // the read is done before the next DMA reuses the slot
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
    if (lane == 0) red[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
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

// y = rmsnorm(x) -> fp16 in the fragment-tiled layout; with LO, also
// lo = fp16(y - fp16(y)) (the split operand of the exact-weight GEMM).
constexpr int NORM_MAX_CHUNKS = 2;  // d <= 2 * 8 * 256
constexpr int NORM_WAVE_CHUNKS = 8;  // one wave per row: d <= 8 * 8 * 64

// One wave per row, four rows per workgroup: lane l owns the eight-float
// chunks l, l + 64, ... of its row, held in registers between the sum of
// squares and the scaling; no workgroup barrier.  Grid (row quads, units).
template <bool LO>
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const NormGroup grp, float eps, int d) {
    const NormUnit &u = grp.u[blockIdx.y];
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= u.M) return;  // the whole wave
    const float *xr = u.x + (size_t)row * d;
    const int nch = d >> 3;
    float4 v[NORM_WAVE_CHUNKS][2], gv[NORM_WAVE_CHUNKS][2];
    // the row and the gain are requested together: the gain does not wait for the sum
#pragma unroll
    for (int c = 0; c < NORM_WAVE_CHUNKS; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
            v[c][0] = *reinterpret_cast<const float4 *>(xr + ch * 8);
            v[c][1] = *reinterpret_cast<const float4 *>(xr + ch * 8 + 4);
            gv[c][0] = *reinterpret_cast<const float4 *>(u.g + ch * 8);
            gv[c][1] = *reinterpret_cast<const float4 *>(u.g + ch * 8 + 4);
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NORM_WAVE_CHUNKS; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
            ss += v[c][0].x * v[c][0].x + v[c][0].y * v[c][0].y + v[c][0].z * v[c][0].z + v[c][0].w * v[c][0].w;
            ss += v[c][1].x * v[c][1].x + v[c][1].y * v[c][1].y + v[c][1].z * v[c][1].z + v[c][1].w * v[c][1].w;
        }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int c = 0; c < NORM_WAVE_CHUNKS; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
            const float4 g0 = gv[c][0], g1 = gv[c][1];
            const float y[8] = {v[c][0].x * r * g0.x, v[c][0].y * r * g0.y, v[c][0].z * r * g0.z, v[c][0].w * r * g0.w,
                                v[c][1].x * r * g1.x, v[c][1].y * r * g1.y, v[c][1].z * r * g1.z, v[c][1].w * r * g1.w};
            h8 yh, yl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                yh[e] = (_Float16)y[e];
                if (LO) yl[e] = (_Float16)(y[e] - (float)yh[e]);
            }
            const size_t o = tiled_index(row, ch * 8, d);
            *reinterpret_cast<h8 *>(u.hi + o) = yh;
            if (LO) *reinterpret_cast<h8 *>(u.lo + o) = yl;
        }
    }
}

// One workgroup per row (rows wider than the wave kernel takes): thread t
// owns the eight-float chunks t, t + 256; the gain is loaded before the row's
// reduction, which it does not need.  Grid (rows, units).
template <bool LO>
__global__ __launch_bounds__(256) void k_rmsnorm_tiled(const NormGroup grp, float eps, int d) {
    __shared__ float red[4];
    const NormUnit &u = grp.u[blockIdx.y];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x;
    if (row >= u.M) return;
    const float *g = u.g;
    __half *hi = u.hi, *lo = u.lo;
    const float *xr = u.x + (size_t)row * d;
    const int nch = d >> 3;
    float4 v[NORM_MAX_CHUNKS][2], gv[NORM_MAX_CHUNKS][2];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NORM_MAX_CHUNKS; ++c) {
        const int ch = tid + 256 * c;
        if (ch < nch) {
            v[c][0] = *reinterpret_cast<const float4 *>(xr + ch * 8);
            v[c][1] = *reinterpret_cast<const float4 *>(xr + ch * 8 + 4);
            gv[c][0] = *reinterpret_cast<const float4 *>(g + ch * 8);
            gv[c][1] = *reinterpret_cast<const float4 *>(g + ch * 8 + 4);
            ss += v[c][0].x * v[c][0].x + v[c][0].y * v[c][0].y + v[c][0].z * v[c][0].z + v[c][0].w * v[c][0].w;
            ss += v[c][1].x * v[c][1].x + v[c][1].y * v[c][1].y + v[c][1].z * v[c][1].z + v[c][1].w * v[c][1].w;
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int c = 0; c < NORM_MAX_CHUNKS; ++c) {
        const int ch = tid + 256 * c;
        if (ch < nch) {
            const float4 g0 = gv[c][0], g1 = gv[c][1];
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

// dst[c * ld + r] = src[r * lds + c] for a rows x cols array of 16-bit
// values, through 32 x 32 LDS tiles (both sides touch memory in rows).
__global__ __launch_bounds__(256) void k_transpose_u16(const uint16_t *src, int rows, int cols, size_t lds,
                                                      uint16_t *dst, size_t ld) {
    __shared__ uint16_t t[32][33];
    const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int i = ty; i < 32; i += 8) {
        const int r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) t[i][tx] = src[(size_t)r * lds + c];
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
        const int c = c0 + i, r = r0 + tx;
        if (r < rows && c < cols) dst[(size_t)c * ld + r] = t[tx][i];
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

// One workgroup per pair: dst row pairs[i].y = src row pairs[i].x (the
// output rows of several sequences, gathered before the KV-shared layers).
__global__ __launch_bounds__(256) void k_gather_rows(const float *src, int d, const int2 *pairs, float *dst) {
    const int2 pr = pairs[blockIdx.x];
    const float *x = src + (size_t)pr.x * d;
    float *y = dst + (size_t)pr.y * d;
    for (int i = threadIdx.x; i < d; i += 256) y[i] = x[i];
}

int ok() { return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP; }

// ------------------------------------------------------------------ GEMV
// y[n] = sum_k W[n][k] v[k] for one fp32 row (the pruned layers and the head),
// v = x, or v = x / sqrt(mean(x^2) + eps) * g when a norm gain is given (the
// RMSNorm that precedes the projection, fused).
// The row runs through the MFMA as two rows of the A operand: row 0 holds
// fp16(v) and row 1 holds fp16(v - fp16(v)), so their sum carries v to ~22
// bits; B holds (code - 8) exactly, and each block's partial is scaled by its
// fp32 block scale -- only fp32 accumulation rounds.
// A workgroup owns G groups of 16 columns (G = 2 when the epilogue combines
// the two RoPE halves of Q or K); KW waves per group take interleaved 64-wide K
// chunks with UNR weight loads in flight.  v is staged once per workgroup in
// LDS as hi/lo fp16 arrays, so a lane's A-operand piece is one 16-byte read.
// Partial sums meet in LDS in wave order: the result is deterministic and no
// workgroup waits for another.
constexpr int GEMV_UNR = 4;

// The finished unit: thread c < 16 sums column c of each group over the KW
// waves (in wave order) and applies the epilogue.
template <int KW, int G>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs &a, const float *red, int unit, int c, int epi) {
    float yv[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        float y = 0.f;
#pragma unroll
        for (int i = 0; i < KW; ++i) y += red[(q * KW + i) * 16 + c];
        yv[q] = y;
    }
    const int n0 = unit * 16 * G;
    switch (epi) {
    case GV_F32:
#pragma unroll
        for (int q = 0; q < G; ++q) a.out[n0 + 16 * q + c] = yv[q];
        break;
    case GV_ADD:
#pragma unroll
        for (int q = 0; q < G; ++q) a.out[n0 + 16 * q + c] += yv[q];
        break;
    case GV_QROPE:
        if (G == 2) {
            const int hd = a.hd, hh = hd >> 1;
            const int h = n0 / hd, rr = n0 % hd;
            const int ii = (rr >> 5) * 16 + c;
            const float2 cs = a.rope[(size_t)a.pos * hh + ii];
            a.out[h * hd + ii] = yv[0] * cs.x - yv[G - 1] * cs.y;
            a.out[h * hd + ii + hh] = yv[0] * cs.y + yv[G - 1] * cs.x;
        }
        break;
    case GV_KV:
        if (G == 2) {
            if (n0 < a.kvd) {
                // K: groups (2p, 2p+1) hold the first and second RoPE half of 16 dims
                const int hd = a.hd, hh = hd >> 1;
                const int h = n0 / hd, rr = n0 % hd;
                const int ii = (rr >> 5) * 16 + c;
                const float2 cs = a.rope[(size_t)a.pos * hh + ii];
                __half *k = a.kc + (size_t)a.pos * a.kvd + h * hd;
                k[ii] = __float2half(yv[0] * cs.x - yv[G - 1] * cs.y);
                k[ii + hh] = __float2half(yv[0] * cs.y + yv[G - 1] * cs.x);
            } else {
#pragma unroll
                for (int q = 0; q < G; ++q)
                    a.vt[(size_t)(n0 - a.kvd + 16 * q + c) * a.vld + a.pos] = __float2half(yv[q]);
            }
        }
        break;
    case GV_GLU:
        // columns 0-7 of the group are gate rows 8t..8t+7, columns 8-15 their up rows
        if (c < 8) {
            float u = 0.f;
#pragma unroll
            for (int i = 0; i < KW; ++i) u += red[i * 16 + c + 8];
            a.out[unit * 8 + c] = act_f(a.act, yv[0]) * u;
        }
        break;
    case GV_PLE: {
        const uint8_t *prow = a.ple_raw + (size_t)a.tok[0] * a.ple_row_blocks * 18;
#pragma unroll
        for (int q = 0; q < G; ++q)
            a.out[n0 + 16 * q + c] = gelu_tanh_f(yv[q]) * (a.ple_s * q4_raw_weight(prow, a.ple_col0 + n0 + 16 * q + c));
        break;
    }
    }
}

template <int KW, int G>
__global__ __launch_bounds__(64 * KW * G) void k_q4gemv(GemvArgs a) {
    extern __shared__ float gemv_lds[];  // red[G][KW][16] floats, then hi[K], lo[K] fp16
    constexpr int NT = 64 * KW * G;
    const int K = a.W.K, kch = K >> 6;
    const int n1 = a.W.N / (16 * G);       // a unit: the G groups of one workgroup pass
    const int nunits = n1 + a.W2.N / (16 * G);  // then the second matrix's units
    float *red = gemv_lds;
    _Float16 *xh = reinterpret_cast<_Float16 *>(gemv_lds + G * KW * 16);
    _Float16 *xl = xh + K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gi = wave / KW, kw = wave % KW;
    const int col = lane & 15, g8 = (lane >> 4) * 8;

    // weight batches: UNR chunks kc = base + u KW of group G unit + gi (clamped, so no branch)
    uint2 w[GEMV_UNR];
    uint32_t sc[GEMV_UNR];
    auto load = [&](int unit, int base, uint2 (&wd)[GEMV_UNR], uint32_t (&sd)[GEMV_UNR]) {
        const bool sec = unit >= n1;
        const uint2 *nib0 = reinterpret_cast<const uint2 *>(sec ? a.W2.nib : a.W.nib) + lane;
        const uint32_t *scl0 = reinterpret_cast<const uint32_t *>(sec ? a.W2.scl : a.W.scl) + col;
        const size_t grp = (size_t)(G * (sec ? unit - n1 : unit) + gi) * kch;
#pragma unroll
        for (int u = 0; u < GEMV_UNR; ++u) {
            const size_t kc = grp + min(base + u * KW, kch - 1);
            wd[u] = nib0[kc * 64];
            sd[u] = scl0[kc * 16];
        }
    };
    // the first batch does not depend on v: it is in flight during the norm and staging
    int unit = blockIdx.x;
    load(unit, kw, w, sc);

    // stage v (normalised if asked) as hi / lo halves
    float r = 1.f;
    if (a.norm_g) {
        float ss = 0.f;
        for (int k = tid; k < K; k += NT) ss += a.x[k] * a.x[k];
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        ss = 0.f;
        for (int i = 0; i < NT / 64; ++i) ss += red[i];
        r = 1.0f / sqrtf(ss / (float)K + a.eps);
        __syncthreads();
    }
    for (int k = tid; k < K; k += NT) {
        const float v = a.norm_g ? a.x[k] * r * a.norm_g[k] : a.x[k];
        const _Float16 h = (_Float16)v;
        xh[k] = h;
        xl[k] = (_Float16)(v - (float)h);
    }
    __syncthreads();

    // Rows 0 and 1 of the A operand carry hi and lo; the other rows repeat
    // them (their results, rows 2..15 of the product, are never read), so no
    // lane masks its fragment.
    const _Float16 *xsrc = (col & 1) ? xl : xh;
    for (; unit < nunits; unit += gridDim.x) {
        float acc0 = 0.f, acc1 = 0.f;
        for (int base = kw; base < kch; base += KW * GEMV_UNR) {
            // the next batch (this unit's, else the next unit's first) while this one is used
            uint2 wn[GEMV_UNR];
            uint32_t sn[GEMV_UNR];
            const int nb = base + KW * GEMV_UNR;
            const int nu = nb < kch ? unit : unit + gridDim.x;
            if (nu < nunits) load(nu, nb < kch ? nb : kw, wn, sn);
#pragma unroll
            for (int u = 0; u < GEMV_UNR; ++u) {
                const int kc = base + u * KW;
                if (kc >= kch) break;  // uniform across the wave
                const h2 d = __builtin_bit_cast(h2, sc[u]);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const h8 af = *reinterpret_cast<const h8 *>(xsrc + kc * 64 + s * 32 + g8);
                    const f4 p = mfma16(af, q4_word_codes(s ? w[u].y : w[u].x), f4{0.f, 0.f, 0.f, 0.f});
                    const float ds = (float)d[s];
                    acc0 += ds * p[0];  // rows 0 and 1 of the 16 x 16 product
                    acc1 += ds * p[1];
                }
            }
#pragma unroll
            for (int u = 0; u < GEMV_UNR; ++u) {
                w[u] = wn[u];
                sc[u] = sn[u];
            }
        }
        // lanes 0..15 hold rows 0 and 1 (hi and lo parts) of column `col`
        if (lane < 16) red[(gi * KW + kw) * 16 + lane] = acc0 + acc1;
        __syncthreads();
        if (tid < 16) {
            if (unit < n1) gemv_epilogue<KW, G>(a, red, unit, tid, a.epi);
            else gemv_epilogue<KW, G>(a, red, unit - n1, tid, a.epi2);
        }
        __syncthreads();  // red is reused by the next unit
    }
}

constexpr int kGemvMaxGrid = 2048;

// waves per group: aim for ~4096 waves in flight with >= 1 chunk per wave
// (at least two per wave: 1.3 % slower decode, 0.3 % slower prefill;
// 2048 or 8192 waves: slower too)
int gemv_kw(int groups, int kch) {
    int kw = 1;
    while (kw < 16 && groups * kw < 4096 && kch / (2 * kw) >= 1) kw *= 2;
    return kw;
}

}  // namespace

int launch_gemv(const GemvArgs &a, hipStream_t s) {
    if (a.W.N % 32 || a.W.K % 64 || !a.x) return PPX_E_UNSUPPORTED;
    auto bad_epi = [&](int epi, const Q4R &W) {
        return epi == GV_KV ? (!a.kc || !a.vt || a.kvd % 32 || 2 * a.kvd != W.N) : !a.out;
    };
    if (bad_epi(a.epi, a.W)) return PPX_E_UNSUPPORTED;
    const bool paired = a.epi == GV_QROPE || a.epi == GV_KV;
    if (a.W2.N) {
        const bool paired2 = a.epi2 == GV_QROPE || a.epi2 == GV_KV;
        if (a.W2.K != a.W.K || a.W2.N % 32 || paired2 != paired || bad_epi(a.epi2, a.W2)) return PPX_E_UNSUPPORTED;
    }
    const int G = paired ? 2 : 1;
    const int units = (a.W.N + a.W2.N) / (16 * G);
    // wide outputs (the vocabulary head): a capped grid of workgroups that each
    // stage v once and loop over their units, four waves per unit
    const bool looped = units > kGemvMaxGrid;
    const int kw = looped ? 4 : std::min(gemv_kw((a.W.N + a.W2.N) / 16, a.W.K / 64), 16 / G);
    const dim3 grid(looped ? kGemvMaxGrid : units);
    const size_t lds = sizeof(float) * G * kw * 16 + 4ull * a.W.K;
    if (lds > 64 * 1024) return PPX_E_UNSUPPORTED;
#define PPX_GEMV(KW_, G_) hipLaunchKernelGGL((k_q4gemv<KW_, G_>), grid, dim3(64 * KW_ * G_), lds, s, a)
    if (G == 2) {
        switch (kw) {
        case 1: PPX_GEMV(1, 2); break;
        case 2: PPX_GEMV(2, 2); break;
        case 4: PPX_GEMV(4, 2); break;
        default: PPX_GEMV(8, 2); break;
        }
    } else {
        switch (kw) {
        case 1: PPX_GEMV(1, 1); break;
        case 2: PPX_GEMV(2, 1); break;
        case 4: PPX_GEMV(4, 1); break;
        case 8: PPX_GEMV(8, 1); break;
        default: PPX_GEMV(16, 1); break;
        }
    }
#undef PPX_GEMV
    return ok();
}

int launch_embed(const Q4R &tok, const int32_t *ids, int M, float scale, float *x, hipStream_t s) {
    if (M <= 0) return PPX_OK;
    hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, s, tok, ids, scale, x);
    return ok();
}

int launch_stream_read(const void *src, size_t bytes, uint32_t *out, int grid, hipStream_t s) {
    hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, s, static_cast<const uint8_t *>(src), bytes >> 10,
                       out);
    return ok();
}

int launch_embed_add(const Q4R &tok, const int32_t *id, float scale, const float *base, float *x, hipStream_t s) {
    hipLaunchKernelGGL(k_embed_add, dim3(1), dim3(256), 0, s, tok, id, scale, base, x);
    return ok();
}

int launch_rmsnorm_group(const NormUnit *units, int n, float eps, int d, bool lo, hipStream_t s) {
    if (n < 1 || n > kMaxUnits) return PPX_E_INVAL;
    if (d % 32 || d > NORM_MAX_CHUNKS * 8 * 256) return PPX_E_UNSUPPORTED;
    NormGroup g;
    int M = 0;
    for (int i = 0; i < n; ++i) {
        if (units[i].M <= 0) continue;
        if (!units[i].x || !units[i].g || !units[i].hi || (lo && !units[i].lo)) return PPX_E_INVAL;
        g.u[g.n++] = units[i];
        M = std::max(M, units[i].M);
    }
    if (!g.n) return PPX_OK;
    if (d <= NORM_WAVE_CHUNKS * 8 * 64) {
        if (lo) hipLaunchKernelGGL((k_rmsnorm_rows<true>), dim3((M + 3) / 4, g.n), dim3(256), 0, s, g, eps, d);
        else hipLaunchKernelGGL((k_rmsnorm_rows<false>), dim3((M + 3) / 4, g.n), dim3(256), 0, s, g, eps, d);
    } else if (lo) {
        hipLaunchKernelGGL((k_rmsnorm_tiled<true>), dim3(M, g.n), dim3(256), 0, s, g, eps, d);
    } else {
        hipLaunchKernelGGL((k_rmsnorm_tiled<false>), dim3(M, g.n), dim3(256), 0, s, g, eps, d);
    }
    return ok();
}

int launch_rmsnorm_f16(const float *x, const float *g, float eps, int M, int d, __half *out, hipStream_t s) {
    NormUnit u;
    u.x = x;
    u.g = g;
    u.hi = out;
    u.M = M;
    return launch_rmsnorm_group(&u, 1, eps, d, false, s);
}

int launch_rmsnorm_split(const float *x, const float *g, float eps, int M, int d, __half *hi, __half *lo,
                         hipStream_t s) {
    NormUnit u;
    u.x = x;
    u.g = g;
    u.hi = hi;
    u.lo = lo;
    u.M = M;
    return launch_rmsnorm_group(&u, 1, eps, d, true, s);
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

int launch_transpose_u16(const uint16_t *src, int rows, int cols, size_t lds, uint16_t *dst, size_t ld,
                         hipStream_t s) {
    if (rows <= 0 || cols <= 0) return PPX_OK;
    hipLaunchKernelGGL(k_transpose_u16, dim3((cols + 31) / 32, (rows + 31) / 32), dim3(256), 0, s, src, rows, cols,
                       lds, dst, ld);
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

int launch_gather_rows(const float *src, int d, const int2 *pairs, int n, float *dst, hipStream_t s) {
    if (n <= 0) return PPX_OK;
    if (!src || !pairs || !dst || d <= 0) return PPX_E_INVAL;
    hipLaunchKernelGGL(k_gather_rows, dim3(n), dim3(256), 0, s, src, d, pairs, dst);
    return ok();
}

}  // namespace ppx
