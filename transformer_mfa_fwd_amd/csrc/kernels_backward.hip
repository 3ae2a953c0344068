// kernels_backward.hip -- gradients of the attention forward with respect to
// Q, K and V, in fp32 arithmetic for every dtype.
//
// With P the softmax weights recomputed from the saved LSE (p = exp(s - LSE)),
// Z the dropout factors and dO the upstream gradient (vision_rs
// flash_attn2.rs, backward kernels; ferrotensor attention.rs, backward with
// the same options and mask as the forward):
//     Delta_i = <dO_i, O_i>                         (bwd_delta_kernel)
//     g_ij    = P_ij (Z_ij <dO_i, V_j> - Delta_i) * ds_ij / d<Q_i, K_j>
//     dQ_i    = sum_j g_ij K_j                      (bwd_dq_kernel, per query tile)
//     dK_j    = sum_i g_ij Q_i,  dV_j = sum_i P_ij Z_ij dO_i
//                                                   (bwd_dkdv_kernel, per key tile,
//                                                    over every query head of the group)
// ds/d<Q, K> is scale, times 1 - tanh^2 under the soft-cap; the additive mask
// takes no gradient.  Each output element is written by exactly one
// workgroup, with no atomics, so results are deterministic.
#include "mfa_internal.h"

#include <math.h>

namespace mfa {
namespace {

constexpr int QT = 64;      // query rows per dQ workgroup (4 waves x 16)
constexpr int KT = 64;      // keys per dQ step (one per lane)
constexpr int DK_KEYS = 32; // keys per dK/dV workgroup (4 waves x 8)
constexpr int DK_ROWS = 64; // query rows per dK/dV step (one per lane)

template <typename T>
__device__ inline float f32(T x) { return static_cast<float>(x); }

// Logit of score (b, hq, i, j) from the raw dot product, and d logit / d dot.
__device__ inline float logit(const FwdArgs& a, float dot, int b, int hq, int i, int j, float& dl) {
    const float t = dot * a.scale;
    float x = t;
    dl = a.scale;
    if (a.softcap > 0.0f) {
        const float th = tanhf(t / a.softcap);
        x = a.softcap * th;
        dl = a.scale * (1.0f - th * th);
    }
    if (a.bias)
        x += a.bias[b * a.bias_stride[0] + hq * a.bias_stride[1] + i * a.bias_stride[2] + j * a.bias_stride[3]];
    return x;
}

__device__ inline bool key_kept(const FwdArgs& a, int b, int j) {
    return j < a.Lk && (!a.key_mask || a.key_mask[(int64_t)b * a.Lk + j] > 0.5f);
}

// Delta of every query row: the rows of [B, Lq, Hq, D] are taken in memory
// order, D/E lanes per row read 16 bytes (E elements) each of O and dO, and
// the row's lanes add their partial sums.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(FwdArgs a, const T* __restrict__ dout,
                                                        float* __restrict__ delta) {
    constexpr int E = 16 / (int)sizeof(T);    // elements per 16-byte chunk
    constexpr int LPR = D / E;                // lanes per row
    constexpr int RPB = 256 / LPR;            // rows per block
    static_assert(LPR <= 64 && (LPR & (LPR - 1)) == 0, "a row's lanes lie in one wave");
    const int64_t nrows = (int64_t)a.B * a.Lq * a.Hq;
    const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;   // (b * Lq + i) * Hq + hq
    const int c = threadIdx.x % LPR;
    float s = 0.0f;
    int64_t bi = 0;
    int hq = 0;
    if (r < nrows) {
        bi = r / a.Hq;
        hq = (int)(r - bi * a.Hq);
        const int64_t off = bi * a.o_stride + (int64_t)hq * D + c * E;
        const T* o = static_cast<const T*>(a.out) + off;
        const T* g = dout + off;
        T ov[E], gv[E];
        *reinterpret_cast<uint4*>(ov) = *reinterpret_cast<const uint4*>(o);
        *reinterpret_cast<uint4*>(gv) = *reinterpret_cast<const uint4*>(g);
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(f32(ov[e]), f32(gv[e]), s);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (r < nrows && c == 0) {
        const int64_t b = bi / a.Lq, i = bi - b * a.Lq;
        delta[(b * a.Hq + hq) * a.Lq + i] = s;
    }
}

template <typename T, int D>
hipError_t launch_delta(const FwdArgs& a, const T* dout, float* delta, hipStream_t s) {
    constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
    const int64_t blocks = ((int64_t)a.B * a.Lq * a.Hq + RPB - 1) / RPB;
    hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a, dout, delta);
    return hipGetLastError();
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(FwdArgs a, const T* __restrict__ dout,
                                                     const float* __restrict__ delta, T* __restrict__ dq) {
    __shared__ float sQ[QT][D + 4];
    __shared__ float sO[QT][D + 4];   // dO rows
    __shared__ float sK[KT][D + 4];
    __shared__ float sV[KT][D + 4];
    __shared__ float sG[4][16][KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = blockIdx.x * QT, hq = blockIdx.y, b = blockIdx.z;
    const int kvh = hq / a.group;
    const int i_end = min(i0 + QT, a.Lq);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);

    for (int x = tid; x < QT * D; x += 256) {
        const int r = x / D, d = x % D, i = i0 + r;
        const int64_t off = ((int64_t)b * a.Lq + i) * a.q_stride + (int64_t)hq * D + d;
        sQ[r][d] = i < a.Lq ? f32(q[off]) : 0.0f;
        sO[r][d] = i < a.Lq ? f32(dout[((int64_t)b * a.Lq + i) * a.o_stride + (int64_t)hq * D + d]) : 0.0f;
    }
    int lo_f, hi_f, lo_l, hi_l;
    row_key_range<false>(a, i0, lo_f, hi_f);
    row_key_range<false>(a, i_end - 1, lo_l, hi_l);
    int rlo[16], rhi[16];
    float lse[16], dl_[16], acc[16][D / 64];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int i = i0 + wave * 16 + rr;
        if (i < a.Lq) row_key_range<false>(a, i, rlo[rr], rhi[rr]);
        else { rlo[rr] = 1; rhi[rr] = 0; }
        lse[rr] = i < a.Lq ? a.lse[((int64_t)b * a.Hq + hq) * a.Lq + i] : -INFINITY;
        dl_[rr] = i < a.Lq ? delta[((int64_t)b * a.Hq + hq) * a.Lq + i] : 0.0f;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) acc[rr][c] = 0.0f;
    }

    if (lo_f <= hi_l) {
        for (int kt = lo_f / KT; kt <= hi_l / KT; ++kt) {
            __syncthreads();
            for (int x = tid; x < KT * D; x += 256) {
                const int j = x / D, d = x % D, key = kt * KT + j;
                const int64_t off = ((int64_t)b * a.Lk + key) * a.kv_stride + (int64_t)kvh * D + d;
                // a masked key's rows stay zero (whatever they hold cannot reach a gradient)
                const bool use = key_kept(a, b, key);
                sK[j][d] = use ? f32(k[off]) : 0.0f;
                sV[j][d] = use ? f32(v[off]) : 0.0f;
            }
            __syncthreads();
            const int key = kt * KT + lane;
            const bool kept = key_kept(a, b, key);
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int r = wave * 16 + rr, i = i0 + r;
                float dot = 0.0f, dov = 0.0f;
                for (int d = 0; d < D; d += 4) {
                    const float4 kk = *reinterpret_cast<const float4*>(&sK[lane][d]);
                    const float4 vv = *reinterpret_cast<const float4*>(&sV[lane][d]);
                    const float4 qq = *reinterpret_cast<const float4*>(&sQ[r][d]);
                    const float4 gg = *reinterpret_cast<const float4*>(&sO[r][d]);
                    dot = fmaf(qq.x, kk.x, fmaf(qq.y, kk.y, fmaf(qq.z, kk.z, fmaf(qq.w, kk.w, dot))));
                    dov = fmaf(gg.x, vv.x, fmaf(gg.y, vv.y, fmaf(gg.z, vv.z, fmaf(gg.w, vv.w, dov))));
                }
                float g = 0.0f;
                if (kept && key >= rlo[rr] && key <= rhi[rr] && lse[rr] != -INFINITY) {
                    float dl;
                    const float x = logit(a, dot, b, hq, i, key, dl);
                    const float p = __expf(x - lse[rr]);
                    float z = 1.0f;
                    if (a.drop_scale > 0.0f) z = dropout_keep(a, b, hq, i, key) ? a.drop_scale : 0.0f;
                    g = p * (z * dov - dl_[rr]) * dl;
                }
                sG[wave][rr][lane] = g;
            }
            __syncthreads();
            for (int j = 0; j < KT; ++j) {
                float kv[D / 64];
#pragma unroll
                for (int c = 0; c < D / 64; ++c) kv[c] = sK[j][lane + 64 * c];
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const float g = sG[wave][rr][j];
#pragma unroll
                    for (int c = 0; c < D / 64; ++c) acc[rr][c] = fmaf(g, kv[c], acc[rr][c]);
                }
            }
        }
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int i = i0 + wave * 16 + rr;
        if (i >= a.Lq) continue;
        T* row = dq + ((int64_t)b * a.Lq + i) * a.q_stride + (int64_t)hq * D;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) row[lane + 64 * c] = static_cast<T>(acc[rr][c]);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(FwdArgs a, const T* __restrict__ dout,
                                                       const float* __restrict__ delta, T* __restrict__ dk,
                                                       T* __restrict__ dv) {
    __shared__ float sK[DK_KEYS][D + 4];
    __shared__ float sV[DK_KEYS][D + 4];
    __shared__ float sQ[DK_ROWS][D + 4];
    __shared__ float sO[DK_ROWS][D + 4];   // dO rows
    __shared__ float sPZ[4][8][DK_ROWS];
    __shared__ float sG[4][8][DK_ROWS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j0 = blockIdx.x * DK_KEYS, kvh = blockIdx.y, b = blockIdx.z;
    const int j_last = min(j0 + DK_KEYS, a.Lk) - 1;
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);

    for (int x = tid; x < DK_KEYS * D; x += 256) {
        const int j = x / D, d = x % D, key = j0 + j;
        const int64_t off = ((int64_t)b * a.Lk + key) * a.kv_stride + (int64_t)kvh * D + d;
        const bool use = key_kept(a, b, key);   // a masked key's rows stay zero
        sK[j][d] = use ? f32(k[off]) : 0.0f;
        sV[j][d] = use ? f32(v[off]) : 0.0f;
    }
    float dka[8][D / 64], dva[8][D / 64];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int c = 0; c < D / 64; ++c) dka[kk][c] = dva[kk][c] = 0.0f;
    bool kept[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kept[kk] = key_kept(a, b, j0 + wave * 8 + kk);

    const int nqt = (a.Lq + DK_ROWS - 1) / DK_ROWS;
    for (int hq = kvh * a.group; hq < (kvh + 1) * a.group; ++hq) {
        for (int qt = 0; qt < nqt; ++qt) {
            const int i0 = qt * DK_ROWS, i_end = min(i0 + DK_ROWS, a.Lq);
            int lo_f, hi_f, lo_l, hi_l;
            row_key_range<false>(a, i0, lo_f, hi_f);
            row_key_range<false>(a, i_end - 1, lo_l, hi_l);
            if (lo_f > j_last || hi_l < j0 || lo_f > hi_l) continue;   // no row of the tile sees these keys
            __syncthreads();
            for (int x = tid; x < DK_ROWS * D; x += 256) {
                const int r = x / D, d = x % D, i = i0 + r;
                sQ[r][d] = i < a.Lq ? f32(q[((int64_t)b * a.Lq + i) * a.q_stride + (int64_t)hq * D + d]) : 0.0f;
                sO[r][d] = i < a.Lq ? f32(dout[((int64_t)b * a.Lq + i) * a.o_stride + (int64_t)hq * D + d]) : 0.0f;
            }
            __syncthreads();
            // lane = query row
            const int i = i0 + lane;
            int rlo = 1, rhi = 0;
            float lse = -INFINITY, dlt = 0.0f;
            if (i < a.Lq) {
                row_key_range<false>(a, i, rlo, rhi);
                lse = a.lse[((int64_t)b * a.Hq + hq) * a.Lq + i];
                dlt = delta[((int64_t)b * a.Hq + hq) * a.Lq + i];
            }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int jj = wave * 8 + kk, key = j0 + jj;
                float dot = 0.0f, dov = 0.0f;
                for (int d = 0; d < D; d += 4) {
                    const float4 kx = *reinterpret_cast<const float4*>(&sK[jj][d]);
                    const float4 vx = *reinterpret_cast<const float4*>(&sV[jj][d]);
                    const float4 qq = *reinterpret_cast<const float4*>(&sQ[lane][d]);
                    const float4 gg = *reinterpret_cast<const float4*>(&sO[lane][d]);
                    dot = fmaf(qq.x, kx.x, fmaf(qq.y, kx.y, fmaf(qq.z, kx.z, fmaf(qq.w, kx.w, dot))));
                    dov = fmaf(gg.x, vx.x, fmaf(gg.y, vx.y, fmaf(gg.z, vx.z, fmaf(gg.w, vx.w, dov))));
                }
                float pz = 0.0f, g = 0.0f;
                if (kept[kk] && key >= rlo && key <= rhi && lse != -INFINITY) {
                    float dl;
                    const float x = logit(a, dot, b, hq, i, key, dl);
                    const float p = __expf(x - lse);
                    float z = 1.0f;
                    if (a.drop_scale > 0.0f) z = dropout_keep(a, b, hq, i, key) ? a.drop_scale : 0.0f;
                    pz = p * z;
                    g = p * (z * dov - dlt) * dl;
                }
                sPZ[wave][kk][lane] = pz;
                sG[wave][kk][lane] = g;
            }
            __syncthreads();
            for (int r = 0; r < DK_ROWS; ++r) {
                float qv[D / 64], ov[D / 64];
#pragma unroll
                for (int c = 0; c < D / 64; ++c) { qv[c] = sQ[r][lane + 64 * c]; ov[c] = sO[r][lane + 64 * c]; }
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const float pz = sPZ[wave][kk][r], g = sG[wave][kk][r];
#pragma unroll
                    for (int c = 0; c < D / 64; ++c) {
                        dva[kk][c] = fmaf(pz, ov[c], dva[kk][c]);
                        dka[kk][c] = fmaf(g, qv[c], dka[kk][c]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const int key = j0 + wave * 8 + kk;
        if (key >= a.Lk) continue;
        const int64_t off = ((int64_t)b * a.Lk + key) * a.kv_stride + (int64_t)kvh * D;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
            dk[off + lane + 64 * c] = static_cast<T>(dka[kk][c]);
            dv[off + lane + 64 * c] = static_cast<T>(dva[kk][c]);
        }
    }
}

template <typename T, int D>
hipError_t launch_bwd_t(const FwdArgs& a, const void* dout, float* delta, void* dq, void* dk, void* dv,
                        hipStream_t s) {
    const T* g = static_cast<const T*>(dout);
    hipError_t e;
    if (a.Lq > 0) {   // with no query rows only the (zero) key gradients remain
        e = launch_delta<T, D>(a, g, delta, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3((a.Lq + QT - 1) / QT, a.Hq, a.B), dim3(256), 0, s, a, g,
                           delta, static_cast<T*>(dq));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D>), dim3((a.Lk + DK_KEYS - 1) / DK_KEYS, a.Hkv, a.B), dim3(256), 0,
                       s, a, g, delta, static_cast<T*>(dk), static_cast<T*>(dv));
    return hipGetLastError();
}

template <typename T>
hipError_t launch_delta_t(const FwdArgs& a, const void* dout, float* delta, hipStream_t s) {
    const T* g = static_cast<const T*>(dout);
    return a.D == 64 ? launch_delta<T, 64>(a, g, delta, s) : launch_delta<T, 128>(a, g, delta, s);
}

template <typename T>
hipError_t launch_bwd_d(const FwdArgs& a, const void* dout, float* delta, void* dq, void* dk, void* dv,
                        hipStream_t s) {
    return a.D == 64 ? launch_bwd_t<T, 64>(a, dout, delta, dq, dk, dv, s)
                     : launch_bwd_t<T, 128>(a, dout, delta, dq, dk, dv, s);
}

}  // namespace

hipError_t launch_backward(const FwdArgs& a, const void* dout, float* delta, void* dq, void* dk, void* dv,
                           int dtype, hipStream_t s) {
    if (bwd_mfma_supported(a, dtype)) {   // Delta here, the rest on the matrix cores
        hipError_t e = hipSuccess;
        if (a.Lq > 0) {
            e = dtype == kBF16 ? launch_delta_t<__bf16>(a, dout, delta, s) : launch_delta_t<_Float16>(a, dout, delta, s);
            if (e != hipSuccess) return e;
        }
        return launch_backward_mfma(a, dout, delta, dq, dk, dv, dtype, s);
    }
    switch (dtype) {
        case kF32: return launch_bwd_d<float>(a, dout, delta, dq, dk, dv, s);
        case kF16: return launch_bwd_d<_Float16>(a, dout, delta, dq, dk, dv, s);
        case kBF16: return launch_bwd_d<__bf16>(a, dout, delta, dq, dk, dv, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mfa
