// Causal prefill attention (MFMA, flash-style online softmax) and the
// single-query attention of the pruned KV-shared layers.
//
// Prefill: the query heads that share one KV head are packed together, so a
// key/value tile read from the cache serves all of them (GQA/MQA).  A
// workgroup owns 64 query columns -- (row, head-in-group) pairs -- of one KV
// head; each of its four waves owns 16.  The kernel computes S^T = K Q^T so
// that the 16x16 accumulator of a wave holds keys down and query columns
// across; after the online-softmax update the probabilities in a lane are
// exactly the B operand of O^T = V^T P^T for that lane (the MFMA pairs A and
// B by lane group and element, so any common order of the 32 keys of a step
// is valid).  V is staged transposed in LDS to serve as the A operand.
// Tiles are aligned to absolute key positions, so a row's result does not
// depend on how the prompt was split into ubatches.
#include "ppx_dev.h"

namespace ppx {

namespace {

constexpr int KT = 64;       // keys per tile
constexpr int VT_LD = 68;    // LDS row stride (halves) of V^T

template <int HD>
__global__ __launch_bounds__(256) void k_attn_prefill(AttnArgs a) {
    constexpr int KB = HD / 32;  // 32-wide d steps
    constexpr int DT = HD / 16;  // 16-row d subtiles of O^T
    __shared__ h8 ks[KB * 4 * 64];             // K tile, A-fragment order [kb][key16][lane]
    __shared__ _Float16 vt[HD * VT_LD];        // V^T tile [d][key]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.H / a.KVH;
    const int kvh = blockIdx.y;
    const int cbase = blockIdx.x * 64;
    const int lc = lane & 15, lg = lane >> 4;

    // this lane's query column
    const int col = cbase + wave * 16 + lc;
    const int t = col / G, hg = col % G;
    const bool valid = t < a.M;
    const int h = kvh * G + hg;
    const int qpos = a.pos0 + (valid ? t : 0);

    // Q^T fragments (B operand): column = query, k = d
    h8 qf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        if (valid)
            qf[kb] = *reinterpret_cast<const h8 *>(a.q + ((size_t)t * a.H + h) * HD + kb * 32 + lg * 8);
        else
            qf[kb] = h8{0, 0, 0, 0, 0, 0, 0, 0};
    }

    f4 oacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] = f4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    const float sl2 = 1.4426950408889634f / sqrtf((float)HD);

    // last position any column of this workgroup needs
    const int tmax = min(a.M - 1, (cbase + 63) / G);
    const int pend = a.pos0 + tmax;  // inclusive
    const int ntiles = pend / KT + 1;

    for (int tile = 0; tile < ntiles; ++tile) {
        const int k0 = tile * KT;
        // ---- stage K (fragment order) and V^T
        for (int u = tid; u < KT * HD / 8; u += 256) {
            const int key = u / (HD / 8), d8 = u % (HD / 8);
            const int kp = k0 + key;
            h8 kv = h8{0, 0, 0, 0, 0, 0, 0, 0}, vv = h8{0, 0, 0, 0, 0, 0, 0, 0};
            if (kp <= pend) {
                const size_t off = ((size_t)kp * a.KVH + kvh) * HD + d8 * 8;
                kv = *reinterpret_cast<const h8 *>(a.k + off);
                vv = *reinterpret_cast<const h8 *>(a.v + off);
            }
            const int kb = d8 >> 2, g = d8 & 3;
            ks[(kb * 4 + (key >> 4)) * 64 + g * 16 + (key & 15)] = kv;
#pragma unroll
            for (int e = 0; e < 8; ++e) vt[(d8 * 8 + e) * VT_LD + key] = vv[e];
        }
        __syncthreads();

        // ---- S^T = K Q^T for 64 keys x 16 query columns
        f4 s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s[j] = mfma16(ks[(kb * 4 + j) * 64 + lane], qf[kb], s[j]);
        }
        // ---- online softmax (per query column; a column lives in lanes lc, lc+16, lc+32, lc+48)
        float tmx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kp = k0 + j * 16 + lg * 4 + r;
                const float v = (kp <= qpos) ? s[j][r] * sl2 : -INFINITY;
                s[j][r] = v;
                tmx = fmaxf(tmx, v);
            }
        tmx = fmaxf(tmx, __shfl_xor(tmx, 16, 64));
        tmx = fmaxf(tmx, __shfl_xor(tmx, 32, 64));
        const float mnew = fmaxf(mrun, tmx);
        const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(mrun - mnew);
        float psum = 0.f;
        h8 pf[2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = (s[j][r] == -INFINITY) ? 0.f : exp2f(s[j][r] - mnew);
                psum += p;
                pf[j >> 1][(j & 1) * 4 + r] = (_Float16)p;
            }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        lrun = lrun * alpha + psum;
        mrun = mnew;
#pragma unroll
        for (int i = 0; i < DT; ++i) oacc[i] *= alpha;

        // ---- O^T += V^T P^T; step kb2 covers keys 32kb2 + {4lg+r, 16+4lg+r}
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int i = 0; i < DT; ++i) {
                const _Float16 *vr = vt + (i * 16 + lc) * VT_LD + kb2 * 32 + lg * 4;
                const h4 lo = *reinterpret_cast<const h4 *>(vr);
                const h4 hi = *reinterpret_cast<const h4 *>(vr + 16);
                const h8 va = h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[i] = mfma16(va, pf[kb2], oacc[i]);
            }
        }
        __syncthreads();
    }

    if (!valid) return;
    const float inv = 1.0f / lrun;
    __half *o = a.o + ((size_t)t * a.H + h) * HD;
#pragma unroll
    for (int i = 0; i < DT; ++i) {
        const int d = i * 16 + lg * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[d + r] = __float2half(oacc[i][r] * inv);
    }
}
// ------------------------------------------------------------------ single query
// One query row (all heads, fp32) over cache positions 0..pos, in two launches.
// k_attn_1row: grid (chunks of CH keys, KVH); a workgroup stages its keys and
// values in LDS with 16-byte loads, scores them against the G heads of its KV
// head (one wave per head group of 64 keys), and writes per head the chunk's
// max, exp-sum and unnormalised output.  k_attn_merge: one workgroup per head
// combines the chunks in chunk order.
constexpr int CH = 64;

template <int HD>
__global__ __launch_bounds__(256) void k_attn_1row(Attn1Args a) {
    constexpr int KLD = HD + 2;  // padded K rows (halves): row r starts at bank r
    __shared__ _Float16 kl[CH * KLD];
    __shared__ _Float16 vl[CH * HD];
    __shared__ float ql[8 * HD];
    __shared__ float pl[8 * CH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.H / a.KVH;  // <= 8
    const int kvh = blockIdx.y, chunk = blockIdx.x, nchunks = gridDim.x;
    const int k0 = chunk * CH;
    const int nk = min(CH, a.pos + 1 - k0);
    const float scale = 1.0f / sqrtf((float)HD);

    for (int u = tid; u < G * HD; u += 256) ql[u] = a.q[(size_t)kvh * G * HD + u];
    for (int u = tid; u < CH * HD / 8; u += 256) {
        const int key = u / (HD / 8), d8 = u % (HD / 8);
        h8 kv = h8{0, 0, 0, 0, 0, 0, 0, 0}, vv = kv;
        if (key < nk) {
            const size_t off = ((size_t)(k0 + key) * a.KVH + kvh) * HD + d8 * 8;
            kv = *reinterpret_cast<const h8 *>(a.k + off);
            vv = *reinterpret_cast<const h8 *>(a.v + off);
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) *reinterpret_cast<h2 *>(kl + key * KLD + d8 * 8 + e) = h2{kv[e], kv[e + 1]};
        *reinterpret_cast<h8 *>(vl + key * HD + d8 * 8) = vv;
    }
    __syncthreads();

    // scores: wave w takes heads w, w+4; lane = key
    for (int g = wave; g < G; g += 4) {
        float s = -INFINITY;
        if (lane < nk) {
            const _Float16 *kr = kl + lane * KLD;
            const float *qr = ql + g * HD;
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
            for (int d = 0; d < HD; d += 2) {
                const h2 kk = *reinterpret_cast<const h2 *>(kr + d);
                acc0 += qr[d] * (float)kk[0];
                acc1 += qr[d + 1] * (float)kk[1];
            }
            s = (acc0 + acc1) * scale;
        }
        const float m = wave_max(s);
        const float p = lane < nk ? expf(s - m) : 0.f;
        const float l = wave_sum(p);
        pl[g * CH + lane] = p;
        if (lane == 0) {
            float *st = a.partial + ((size_t)(kvh * G + g) * nchunks + chunk) * 2;
            st[0] = m;
            st[1] = l;
        }
    }
    __syncthreads();
    // unnormalised P.V: thread d (HD <= 256 threads), every head of the group
    float *po = a.partial + (size_t)a.H * nchunks * 2;
    for (int d = tid; d < HD; d += 256) {
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < nk; ++j) {
            const float v = (float)vl[j * HD + d];
#pragma unroll
            for (int g = 0; g < 8; ++g)
                if (g < G) o[g] += pl[g * CH + j] * v;
        }
#pragma unroll
        for (int g = 0; g < 8; ++g)
            if (g < G) po[((size_t)(kvh * G + g) * nchunks + chunk) * HD + d] = o[g];
    }
}

// o[h][d] = sum_c e^(m_c - M) o_c[d] / sum_c e^(m_c - M) l_c, chunks in order.
__global__ __launch_bounds__(256) void k_attn_merge(Attn1Args a, int nchunks) {
    __shared__ float wl[1024];
    __shared__ float red[4];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int hd = a.hd;
    const float *st = a.partial + (size_t)h * nchunks * 2;
    const float *po = a.partial + (size_t)a.H * nchunks * 2 + (size_t)h * nchunks * hd;
    float M = -INFINITY;
    for (int c = tid; c < nchunks; c += 256) M = fmaxf(M, st[2 * c]);
    M = wave_max(M);
    if ((tid & 63) == 0) red[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float L = 0.f;
    for (int c = tid; c < nchunks; c += 256) {
        const float w = expf(st[2 * c] - M);
        if (c < 1024) wl[c] = w;
        L += w * st[2 * c + 1];
    }
    __syncthreads();
    L = wave_sum(L);
    if ((tid & 63) == 0) red[tid >> 6] = L;
    __syncthreads();
    L = red[0] + red[1] + red[2] + red[3];
    for (int d = tid; d < hd; d += 256) {
        float o = 0.f;
        for (int c = 0; c < nchunks; ++c) {
            const float w = c < 1024 ? wl[c] : expf(st[2 * c] - M);
            o += w * po[(size_t)c * hd + d];
        }
        a.o[(size_t)h * hd + d] = o / L;
    }
}

int ok() { return hipGetLastError() == hipSuccess ? PPX_OK : PPX_E_HIP; }

}  // namespace

int launch_attn_prefill(const AttnArgs &a, hipStream_t s) {
    if (a.M <= 0) return PPX_OK;
    const int G = a.H / a.KVH;
    if (a.H % a.KVH || 64 % G) return PPX_E_UNSUPPORTED;
    dim3 grid((a.M * G + 63) / 64, a.KVH);
    switch (a.hd) {
    case 64: hipLaunchKernelGGL(k_attn_prefill<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn_prefill<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(k_attn_prefill<256>, grid, dim3(256), 0, s, a); break;
    default: return PPX_E_UNSUPPORTED;
    }
    return ok();
}

size_t attn1_scratch_floats(int H, int hd, int n_pos) {
    const int chunks = (n_pos + CH - 1) / CH;
    return (size_t)chunks * H * (hd + 2);
}

int launch_attn_1row(const Attn1Args &a, hipStream_t s) {
    const int G = a.H / a.KVH;
    if (a.H % a.KVH || G > 8 || a.pos < 0 || !a.partial) return PPX_E_UNSUPPORTED;
    const int chunks = (a.pos + 1 + CH - 1) / CH;
    dim3 grid(chunks, a.KVH);
    switch (a.hd) {
    case 64: hipLaunchKernelGGL(k_attn_1row<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn_1row<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(k_attn_1row<256>, grid, dim3(256), 0, s, a); break;
    default: return PPX_E_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return PPX_E_HIP;
    hipLaunchKernelGGL(k_attn_merge, dim3(a.H), dim3(256), 0, s, a, chunks);
    return ok();
}

}  // namespace ppx
