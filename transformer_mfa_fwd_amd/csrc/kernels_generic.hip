// kernels_generic.hip -- fp32-arithmetic attention forward for every dtype,
// plus the key-mask bit-packing prepass.
//
// The generic kernel is the straightforward tiled form of the method (vision_rs
// flash_attn2.rs, forward kernel: running max, rescaled running sum and
// accumulator per query row, LSE = max + log(sum) at the end), written for
// clarity rather than speed.  It serves fp32 inputs (whose 1e-4 tolerance rules
// out 16-bit MFMA operands) and any shape the MFMA kernels decline.
//
// Work decomposition: one 256-thread workgroup per (64-query tile, q head,
// batch); each of its four waves owns 16 query rows.  K and V tiles of 64 keys
// are converted to fp32 in LDS.  For the scores, lane j of a wave owns key j of
// the tile; for P.V, lane c owns output columns c and c+64.
#include "mfa_internal.h"

#include <math.h>

namespace mfa {
namespace {

constexpr int GBN = 64;  // keys per tile

template <typename T>
__device__ inline float to_f32(T x) { return static_cast<float>(x); }

// RPW query rows per wave, 4 RPW per workgroup: 16 where the grid is large,
// 4 or 1 for small problems, which then spread over more workgroups.
template <typename T, int D, int RPW>
__global__ __launch_bounds__(256) void generic_fwd_kernel(FwdArgs a) {
    constexpr int ROWS_PER_WAVE = RPW;
    constexpr int GBM = 4 * RPW;   // query rows per workgroup
    __shared__ float sQ[GBM][D + 4];
    __shared__ float sK[GBN][D + 4];
    __shared__ float sV[GBN][D];
    __shared__ float sP[4][ROWS_PER_WAVE][GBN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int i0 = blockIdx.x * GBM;
    const int hq = blockIdx.y;
    const int b = blockIdx.z;
    const int kvh = hq / a.group;
    const int i_end = min(i0 + GBM, a.Lq);

    const T* __restrict__ q = static_cast<const T*>(a.q);
    const T* __restrict__ k = static_cast<const T*>(a.k);
    const T* __restrict__ v = static_cast<const T*>(a.v);
    T* __restrict__ out = static_cast<T*>(a.out);
    const int64_t q_row_stride = a.q_stride;
    const int64_t kv_row_stride = a.kv_stride;

    // keys any row of this tile can see
    int lo_first, hi_first, lo_last, hi_last;
    row_key_range(a, i0, lo_first, hi_first);
    row_key_range(a, i_end - 1, lo_last, hi_last);
    const int klo = lo_first, khi = hi_last;

    // K and V of key tile kt into registers (thread tid holds elements tid,
    // tid + 256, ... of the tile): the next tile's loads are in flight while
    // the current one is computed, and the first tile's beside Q's.  A masked
    // key's row stays zero: whatever it holds (NaN in never-written memory)
    // cannot reach O through its zero weight.
    constexpr int NPF = GBN * D / 256;
    float pk[NPF], pv[NPF];
    auto prefetch = [&](int kt) {
#pragma unroll
        for (int n = 0; n < NPF; ++n) {
            const int x = tid + 256 * n;
            const int j = x / D, d = x % D;
            const int key = kt * GBN + j;
            float kv = 0.0f, vv = 0.0f;
            if (key < a.Lk && (!a.key_mask || a.key_mask[(int64_t)b * a.Lk + key] > 0.5f)) {
                const int64_t off = ((int64_t)b * a.Lk + key) * kv_row_stride + (int64_t)kvh * D + d;
                kv = to_f32(k[off]);
                vv = to_f32(v[off]);
            }
            pk[n] = kv;
            pv[n] = vv;
        }
    };
    if (klo <= khi) prefetch(klo / GBN);

    for (int x = tid; x < GBM * D; x += 256) {
        const int r = x / D, d = x % D;
        const int i = i0 + r;
        sQ[r][d] = i < a.Lq ? to_f32(q[((int64_t)b * a.Lq + i) * q_row_stride + (int64_t)hq * D + d])
                            : 0.0f;
    }

    int rlo[ROWS_PER_WAVE], rhi[ROWS_PER_WAVE];
    float m[ROWS_PER_WAVE], l[ROWS_PER_WAVE], acc[ROWS_PER_WAVE][D / 64];
#pragma unroll
    for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
        const int i = i0 + wave * ROWS_PER_WAVE + rr;
        if (i < a.Lq) row_key_range(a, i, rlo[rr], rhi[rr]);
        else { rlo[rr] = 1; rhi[rr] = 0; }
        m[rr] = -INFINITY;
        l[rr] = 0.0f;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) acc[rr][c] = 0.0f;
    }

    if (klo <= khi) {
        for (int kt = klo / GBN; kt <= khi / GBN; ++kt) {
            __syncthreads();  // previous tile fully consumed (and sQ written)
#pragma unroll
            for (int n = 0; n < NPF; ++n) {
                const int x = tid + 256 * n;
                sK[x / D][x % D] = pk[n];
                sV[x / D][x % D] = pv[n];
            }
            if (kt < khi / GBN) prefetch(kt + 1);
            __syncthreads();

            const int key = kt * GBN + lane;
            bool key_ok = key < a.Lk;
            if (key_ok && a.key_mask) key_ok = a.key_mask[(int64_t)b * a.Lk + key] > 0.5f;

            float s[ROWS_PER_WAVE];
#pragma unroll
            for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) s[rr] = 0.0f;
#pragma unroll 4
            for (int d = 0; d < D; d += 4) {
                const float4 kk = *reinterpret_cast<const float4*>(&sK[lane][d]);
#pragma unroll
                for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
                    const float4 qq = *reinterpret_cast<const float4*>(&sQ[wave * ROWS_PER_WAVE + rr][d]);
                    s[rr] = fmaf(qq.x, kk.x, s[rr]);
                    s[rr] = fmaf(qq.y, kk.y, s[rr]);
                    s[rr] = fmaf(qq.z, kk.z, s[rr]);
                    s[rr] = fmaf(qq.w, kk.w, s[rr]);
                }
            }

#pragma unroll
            for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
                const int i = i0 + wave * ROWS_PER_WAVE + rr;
                float x = s[rr] * a.scale;
                if (a.softcap > 0.0f) x = a.softcap * tanhf(x / a.softcap);
                const bool vis = key_ok && key >= rlo[rr] && key <= rhi[rr];
                if (vis && a.bias)
                    x += a.bias[b * a.bias_stride[0] + hq * a.bias_stride[1] + i * a.bias_stride[2] +
                                key * a.bias_stride[3]];
                x = vis ? x : -INFINITY;

                float mx = x;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
                const float m_new = fmaxf(m[rr], mx);
                const float m_use = m_new == -INFINITY ? 0.0f : m_new;
                const float alpha = expf(m[rr] - m_use);
                const float p = expf(x - m_use);
                l[rr] = l[rr] * alpha + p;
                m[rr] = m_new;
                float pv = p;   // the weight that multiplies V: after dropout, the sum stays undropped
                if (a.drop_scale > 0.0f && p > 0.0f) {
                    pv = dropout_keep(a, b, hq, i, key) ? p * a.drop_scale : 0.0f;
                }
                sP[wave][rr][lane] = pv;
#pragma unroll
                for (int c = 0; c < D / 64; ++c) acc[rr][c] *= alpha;
            }
            __syncthreads();

            // (unrolled by 8: fully unrolled, the compiler hoists every LDS read
            // of the loop and runs out of registers)
#pragma unroll 8
            for (int j = 0; j < GBN; ++j) {
                float vv[D / 64];
#pragma unroll
                for (int c = 0; c < D / 64; ++c) vv[c] = sV[j][lane + 64 * c];
#pragma unroll
                for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
                    const float p = sP[wave][rr][j];
#pragma unroll
                    for (int c = 0; c < D / 64; ++c) acc[rr][c] = fmaf(p, vv[c], acc[rr][c]);
                }
            }
        }
    }

#pragma unroll
    for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
        const int i = i0 + wave * ROWS_PER_WAVE + rr;
        float lt = l[rr];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lt += __shfl_xor(lt, off);
        if (i >= a.Lq) continue;
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        T* orow = out + ((int64_t)b * a.Lq + i) * a.o_stride + (int64_t)hq * D;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) orow[lane + 64 * c] = static_cast<T>(acc[rr][c] * inv);
        if (a.lse && lane == 0)
            a.lse[((int64_t)b * a.Hq + hq) * a.Lq + i] = lt > 0.0f ? m[rr] + logf(lt) : -INFINITY;
    }
}

// words[b * W + w], bit t: key 64*w + t exists and its mask is > 0.5.
__global__ __launch_bounds__(64) void mask_words_kernel(const float* __restrict__ mask, int Lk, int W,
                                                        uint64_t* __restrict__ words) {
    const int w = blockIdx.x, b = blockIdx.y;
    const int key = w * 64 + threadIdx.x;
    const bool keep = key < Lk && mask[(int64_t)b * Lk + key] > 0.5f;
    const uint64_t bits = __ballot(keep);
    if (threadIdx.x == 0) words[(int64_t)b * W + w] = bits;
}

__device__ inline int clamp_to(int x, int hi) { return x < 0 ? 0 : (x > hi ? hi : x); }

// One thread per query row: the last sequence whose first row is at or
// before the row (binary search over the prefix sums), then its key bounds.
__global__ __launch_bounds__(256) void varlen_rows_kernel(const int* __restrict__ cu_q,
                                                          const int* __restrict__ cu_k, int batch, int Tq,
                                                          int Tk, int* __restrict__ row_pos,
                                                          int* __restrict__ seq_bounds) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= Tq) return;
    int lo = 0, hi = batch - 1;   // largest b with cu_q[b] <= i
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (clamp_to(cu_q[mid], Tq) <= i) lo = mid; else hi = mid - 1;
    }
    const int q0 = clamp_to(cu_q[lo], Tq), q1 = clamp_to(cu_q[lo + 1], Tq);
    int k0 = clamp_to(cu_k[lo], Tk), k1 = clamp_to(cu_k[lo + 1], Tk);
    if (!(q0 <= i && i < q1)) k0 = k1 = Tk;   // the row belongs to no sequence
    if (k1 < k0) k1 = k0;
    row_pos[i] = k0 + (i - q0);
    seq_bounds[2 * i] = k0;
    seq_bounds[2 * i + 1] = k1;
}

template <typename T, int RPW>
hipError_t launch_generic_r(const FwdArgs& a, hipStream_t s) {
    dim3 grid((a.Lq + 4 * RPW - 1) / (4 * RPW), a.Hq, a.B);
    if (a.D == 64)
        hipExtLaunchKernelGGL((generic_fwd_kernel<T, 64, RPW>), grid, dim3(256), 0, s, instr_event_begin(),
                              instr_event_end(), 0, a);
    else
        hipExtLaunchKernelGGL((generic_fwd_kernel<T, 128, RPW>), grid, dim3(256), 0, s, instr_event_begin(),
                              instr_event_end(), 0, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_generic_t(const FwdArgs& a, hipStream_t s) {
    // fewer 64-row workgroups than two per CU: 16-row workgroups instead, and
    // 4-row ones below a quarter of the CUs
    const int64_t wg64 = (int64_t)((a.Lq + 63) / 64) * a.Hq * a.B;
    if (wg64 < 64) return launch_generic_r<T, 1>(a, s);
    return wg64 < 512 ? launch_generic_r<T, 4>(a, s) : launch_generic_r<T, 16>(a, s);
}

}  // namespace

hipError_t launch_generic(const FwdArgs& a, int dtype, hipStream_t s) {
    switch (dtype) {
        case kF32: return launch_generic_t<float>(a, s);
        case kF16: return launch_generic_t<_Float16>(a, s);
        case kBF16: return launch_generic_t<__bf16>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_varlen_rows(const int* cu_q, const int* cu_k, int batch, int Tq, int Tk, int* row_pos,
                              int* seq_bounds, hipStream_t s) {
    hipLaunchKernelGGL(varlen_rows_kernel, dim3((Tq + 255) / 256), dim3(256), 0, s, cu_q, cu_k, batch, Tq,
                       Tk, row_pos, seq_bounds);
    return hipGetLastError();
}

hipError_t launch_mask_words(const FwdArgs& a, uint64_t* words, hipStream_t s) {
    dim3 grid(a.words_per_batch, a.B);
    hipLaunchKernelGGL(mask_words_kernel, grid, dim3(64), 0, s, a.key_mask, a.Lk, a.words_per_batch,
                       words);
    return hipGetLastError();
}

}  // namespace mfa
