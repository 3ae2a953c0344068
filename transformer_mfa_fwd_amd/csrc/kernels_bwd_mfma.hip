// kernels_bwd_mfma.hip -- the backward on the matrix cores for fp16/bf16
// inputs, with or without an additive mask and dropout.
//
// Same formulas as kernels_backward.hip (vision_rs flash_attn2.rs, backward
// kernels): P = exp(s - LSE) from the saved LSE, Delta = <dO, O>,
// dS = P (Z dO V^T - Delta) * d s / d<Q, K>, dQ = dS K, dK = dS^T Q,
// dV = (P Z)^T dO, with Z the dropout factors (keep / (1 - p), or 1) and the
// additive mask inside s.
// The dQ products are 32x32x16 MFMAs, the dK/dV products 16x16x32, all with
// fp32 accumulation; P and dS are rounded to the input type to serve as
// operands, as the forward rounds P.
//
//   bwd_dq_mfma_kernel    one wave per 32 query rows, walking 32-key tiles:
//       S^T  = K Q^T    (K rows from LDS, Q^T in registers)
//       dP^T = V dO^T   (V rows from LDS, dO^T in registers)
//       dQ^T += K^T dS^T (K^T by transposing LDS reads, dS^T straight from the
//                         accumulator of S^T)
//   bwd_dkdv16_kernel     one wave per 16 keys, walking the 32-row query tiles
//                         of every query head of its GQA group:
//       S  = Q K^T      (Q rows from LDS, K^T in registers)
//       dP = dO V^T
//       dV^T += dO^T P,  dK^T += Q^T dS   (transposing LDS reads of dO and Q)
// An accumulator's elements per lane serve as the B operand of the next
// product in the order the transposing reads deliver the A operand's rows, so
// no score crosses lanes.  Each gradient element has one writer (no atomics).
// The dK/dV kernel, and the dQ kernel of calls whose mask cannot be copied
// whole or whose dropout pattern is not stored (bwd_dq_pipe_mfma_kernel), run
// a software pipeline: the next tile's S and dP MFMAs beside the current
// tile's softmax, over three LDS buffers.
#include "mfa_device.h"
#include "mfa_internal.h"

#include <math.h>

namespace mfa {
namespace {

constexpr float BW_LOG2E = 1.4426950408889634f;

// A 32-row tile of D 16-bit columns, rows unpadded, the 16-byte chunks of row r
// permuted by XOR with swz(r).  Both read patterns then hit 64 distinct banks
// per pass: row reads (16 rows at one chunk: swz is a permutation over any 16
// consecutive rows at D = 128, over the 8 rows of each parity at D = 64) and
// transposing reads (4 consecutive rows x 4 chunks: the row's low bits move
// the chunk's high bits, the next two row bits its low bits).
template <int D>
struct BwLds {
    static constexpr int RS = D * 2;         // bytes per tile row
    static constexpr int TILE = 32 * RS;     // one 32-row tile
    static __device__ inline int swz(int r) {
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }
};

// A operand from a row-major 16-bit LDS tile: lane l takes row l % 32 and the
// eight elements from column c0 + 8 (l / 32).
template <typename T, int D>
__device__ inline typename Mfma<T>::v8 rows_a(const char* tile, int lane, int c0) {
    const int r = lane & 31;
    const char* p = tile + r * BwLds<D>::RS + (((c0 >> 3) + (lane >> 5)) ^ BwLds<D>::swz(r)) * 16;
    return bitcast<typename Mfma<T>::v8>(*reinterpret_cast<const u32x4_t*>(p));
}

// A operand = M^T for a row-major 16-bit LDS tile M[k][m]: k-step s (16 of the
// tile's 32 rows), m-block mb (32 columns).  Lane l takes column 32 mb + l % 32
// at rows 16 s + 8 (e / 4) + 4 (l / 32) + e % 4, e = 0..7: the rows that
// accumulator elements 8 s .. 8 s + 7 of lane l hold, so pack8_at(acc, 8 s) is
// the matching B operand.  Two transposing reads per operand (4 rows each).
template <typename T, int D>
__device__ inline typename Mfma<T>::v8 cols_a(const char* tile, int lane, int s, int mb) {
    const int g = lane >> 4, j = lane & 15;
    const int row = 16 * s + 4 * (g >> 1) + (j >> 2);
    const int col = 32 * mb + 16 * (g & 1) + 4 * (j & 3);
    const int c = col >> 3, w = (col & 7) * 2;
    const i16x4_t lo = lds_read_tr16(tile + row * BwLds<D>::RS + ((c ^ BwLds<D>::swz(row)) * 16) + w);
    const i16x4_t hi = lds_read_tr16(tile + (row + 8) * BwLds<D>::RS + ((c ^ BwLds<D>::swz(row + 8)) * 16) + w);
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return bitcast<typename Mfma<T>::v8>(v);
}

// A 32-row x D tile of a [rows, stride] 16-bit tensor moves in two halves:
// fetch_tile reads it into registers (thread tid holds 16-byte chunks tid and
// tid + 256; rows at or past `rows_valid` are zero) so that the next tile's
// global reads overlap the current tile's products, and store_tile writes the
// registers into the padded LDS tile.
template <int D>
struct TileRegs {
    static constexpr int N = 32 * (D / 8) / 256;   // chunks per thread: 1 (D = 64) or 2 (D = 128)
    u32x4_t v[N];
};
template <typename T, int D>
__device__ inline void fetch_tile(TileRegs<D>& t, const T* src, int64_t stride, int rows_valid, int tid,
                                  const float* keep = nullptr) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int n = 0; n < TileRegs<D>::N; ++n) {
        // rows past the end read the last valid row (rows_valid >= 1) and are
        // then zeroed: a select, not a branch; so are the rows of keys whose
        // mask value (keep[r], when given) drops them
        const int c = tid + 256 * n, r = c / CPR, k = c % CPR;
        const int rc = r < rows_valid ? r : rows_valid - 1;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + (int64_t)rc * stride + k * 8);
        const bool ok = r < rows_valid && (!keep || keep[rc] > 0.5f);
        t.v[n] = u32x4_t{ok ? v[0] : 0u, ok ? v[1] : 0u, ok ? v[2] : 0u, ok ? v[3] : 0u};
    }
}
template <int D>
__device__ inline void store_tile(char* tile, const TileRegs<D>& t, int tid) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int n = 0; n < TileRegs<D>::N; ++n) {
        const int c = tid + 256 * n, r = c / CPR, k = c % CPR;
        *reinterpret_cast<u32x4_t*>(tile + r * BwLds<D>::RS + (k ^ BwLds<D>::swz(r)) * 16) = t.v[n];
    }
}

// logit of a raw dot product (scale, optional soft-cap) minus the row's LSE,
// both in base-2 units, and d logit / d dot.  Without a cap that derivative is
// the constant scale, which the kernels apply once to dQ and dK at the end
// (dl = 1 here) and the logit is one fma.
template <bool CAP>
__device__ inline float logit2_minus(const FwdArgs& a, float dot, float lse2, float& dl) {
    if constexpr (CAP) {
        // tanh y = 1 - 2 / (e^(2 y) + 1) from the hardware exp2 and reciprocal
        // (saturates to +-1 for large |y|), as the forward forms its cap
        const float th = 1.0f - 2.0f * fast_rcp(fast_exp2(dot * (2.0f * BW_LOG2E) * a.scale / a.softcap) + 1.0f);
        dl = a.scale * (1.0f - th * th);
        return fmaf(a.softcap * BW_LOG2E, th, -lse2);
    } else {
        dl = 1.0f;
        return fmaf(dot, a.score_to_log2, -lse2);   // score_to_log2 = scale * log2(e) without a cap
    }
}


// dQ (two workgroups per CU but with a soft-cap at D = 128).  EXTRA: with an
// additive mask whose keys are contiguous (copied into LDS straight from
// global memory, one 128-row x 32-key tile ahead) and dropout whose pattern
// the dK/dV kernel stored; other mask or dropout calls take the pipelined
// kernel below.
template <typename T, int D, bool CAP, bool EXTRA>
__global__ __launch_bounds__(256, (CAP && EXTRA && D == 128) ? 1 : 2) void bwd_dq_mfma_kernel(FwdArgs a, const T* __restrict__ dout,
                                                             const float* __restrict__ delta, T* __restrict__ dq) {
    typedef typename Mfma<T>::v8 v8;
    constexpr int NKS = D / 16, NDB = D / 32;
    __shared__ __attribute__((aligned(16))) char sK[BwLds<D>::TILE];
    __shared__ __attribute__((aligned(16))) char sV[BwLds<D>::TILE];
    __shared__ float sM[32];   // 1: key kept (in range of the axis and of the key mask)
    // EXTRA: the additive mask of the tile's 128 rows x 32 keys, two buffers;
    // 16-byte chunk c of row r at chunk c ^ ((r / 2) % 8) of its 128-byte row
    __shared__ __attribute__((aligned(16))) float sB[EXTRA ? 2 : 1][EXTRA ? 128 * 32 : 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    // grid (Hq, B, query blocks), the latest query block first: under a causal
    // mask it walks the most key tiles
    const int hq = blockIdx.x, b = blockIdx.y, kvh = hq / a.group;
    const int i0 = (gridDim.z - 1 - blockIdx.z) * 128, i_last = min(i0 + 127, a.Lq - 1);
    const int row = i0 + 32 * wave + (lane & 31);
    const int rowc = row <= i_last ? row : i_last;
    const T* qb = static_cast<const T*>(a.q) + (int64_t)b * a.Lq * a.q_stride + (int64_t)hq * D;
    const T* gb = dout + (int64_t)b * a.Lq * a.o_stride + (int64_t)hq * D;
    const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Lk * a.kv_stride + (int64_t)kvh * D;
    const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Lk * a.kv_stride + (int64_t)kvh * D;

    v8 qop[NKS], gop[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        qop[ks] = bitcast<v8>(*reinterpret_cast<const u32x4_t*>(qb + (int64_t)rowc * a.q_stride + 16 * ks + 8 * h));
        gop[ks] = bitcast<v8>(*reinterpret_cast<const u32x4_t*>(gb + (int64_t)rowc * a.o_stride + 16 * ks + 8 * h));
    }
    int rlo = 1, rhi = 0;
    float lse2 = 0.0f, dlt = 0.0f;
    if (row <= i_last) {
        row_key_range<false>(a, row, rlo, rhi);
        const float l = a.lse[((int64_t)b * a.Hq + hq) * a.Lq + row];
        if (l == -INFINITY) { rlo = 1; rhi = 0; }   // no weight anywhere in the row
        lse2 = l == -INFINITY ? 0.0f : l * BW_LOG2E;   // finite: hidden logits are -inf
        dlt = delta[((int64_t)b * a.Hq + hq) * a.Lq + row];
    }
    int lo_blk, t0, t1, hi_blk;
    row_key_range<false>(a, i0, lo_blk, t0);
    row_key_range<false>(a, i_last, t1, hi_blk);
    // EXTRA: this (batch, query head)'s additive mask as a buffer of its whole
    // extent (copies past it read zeros), and the stored dropout pattern
    const float* bhead = nullptr;
    int bbytes = 0;
    if (EXTRA && a.bias) {
        bhead = a.bias + b * a.bias_stride[0] + hq * a.bias_stride[1];
        bbytes = (int)(((int64_t)(a.Lq - 1) * a.bias_stride[2] + a.Lk) * 4);
    }
    const int njb = (a.Lk + 15) >> 4;
    const uint16_t* keep_row = (EXTRA && a.drop_scale > 0.0f)
                                   ? a.keep_bits + ((int64_t)b * a.Hq + hq) * njb * a.Lq + rowc
                                   : nullptr;
    // copy of tile TL's mask into buffer BB: slot 256 j + tid holds row s / 8,
    // chunk (s % 8) ^ ((row / 2) % 8)
    auto bias_copy = [&](int TL, int BB) {
        if constexpr (EXTRA) {
            if (bhead) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int sl = 256 * j + tid, r = sl >> 3, c = (sl & 7) ^ ((r >> 1) & 7);
                    const int64_t off = ((int64_t)(i0 + r) * a.bias_stride[2] + 32 * TL + 4 * c) * 4;
                    buffer_copy16_to_lds(bhead, bbytes, &sB[BB][(256 * j + 64 * wave) * 4],
                                         off < bbytes ? (uint32_t)off : (uint32_t)bbytes);
                }
            }
        }
    };
    // the pattern words of this lane's row for tile TL: block 2 TL + h
    auto keep_load = [&](int TL) -> uint32_t {
        const int jb = 2 * TL + h;
        return (keep_row && row <= i_last && jb < njb) ? (uint32_t)keep_row[(int64_t)jb * a.Lq] : 0u;
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = 0.0f;

    if (lo_blk <= hi_blk) {
        const int t_first = lo_blk / 32, t_end = hi_blk / 32 + 1;
        TileRegs<D> rk, rv;
        float rm = 0.0f;
        // tile t's K, V and key-kept flags into registers
        auto fetch = [&](int t) {
            const int k0 = 32 * t;
            // a masked key's K and V rows stay zero (whatever they hold cannot reach dQ)
            const float* keep = a.key_mask ? a.key_mask + (int64_t)b * a.Lk + k0 : nullptr;
            fetch_tile<T, D>(rk, kb + (int64_t)k0 * a.kv_stride, a.kv_stride, a.Lk - k0, tid, keep);
            fetch_tile<T, D>(rv, vb + (int64_t)k0 * a.kv_stride, a.kv_stride, a.Lk - k0, tid, keep);
            if (tid < 32) {
                const int key = k0 + tid;
                rm = (key < a.Lk && (!a.key_mask || a.key_mask[(int64_t)b * a.Lk + key] > 0.5f)) ? 1.0f : 0.0f;
            }
        };
        fetch(t_first);
        bias_copy(t_first, 0);
        uint32_t kw_next = EXTRA ? keep_load(t_first) : 0u;
        for (int t = t_first; t < t_end; ++t) {
            const int k0 = 32 * t, bb = (t - t_first) & 1;
            __syncthreads();   // the previous tile is no longer read
            store_tile<D>(sK, rk, tid);
            store_tile<D>(sV, rv, tid);
            if (tid < 32) sM[tid] = rm;
            if constexpr (EXTRA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this tile's mask copies
            __syncthreads();
            const uint32_t kw = kw_next;
            if (t + 1 < t_end) {   // in flight during this tile's products
                fetch(t + 1);
                bias_copy(t + 1, bb ^ 1);
                if constexpr (EXTRA) kw_next = keep_load(t + 1);
            }
            // EXTRA: mask values and dropout keep bits of this lane's 16 scores
            // (score 4 G + e is key k0 + 8 G + 4 h + e); the tile's two 16-key
            // pattern words of this row are shared by lanes l and l ^ 32
            float bv[EXTRA ? 16 : 1];
            uint32_t keepm = 0xffffu;
            if constexpr (EXTRA) {
                if (bhead) {
                    const int rr = 32 * wave + (lane & 31);
#pragma unroll
                    for (int G = 0; G < 4; ++G) {
                        const float4 f = *reinterpret_cast<const float4*>(&sB[bb][(rr * 8 + ((2 * G + h) ^ ((rr >> 1) & 7))) * 4]);
                        bv[4 * G] = f.x; bv[4 * G + 1] = f.y; bv[4 * G + 2] = f.z; bv[4 * G + 3] = f.w;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) bv[r] = 0.0f;
                }
                if (keep_row) {
                    const uint32_t oth = (uint32_t)__shfl_xor((int)kw, 32);
                    const uint32_t m32 = h ? (oth | (kw << 16)) : (kw | (oth << 16));   // keys 0 .. 31
                    keepm = pack_even_nibbles(m32 >> (4 * h));
                }
            }
            (void)bv; (void)kw;
            f32x16_t s = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                s = Mfma<T>::mma32(rows_a<T, D>(sK, lane, 16 * ks), qop[ks], s);
                dp = Mfma<T>::mma32(rows_a<T, D>(sV, lane, 16 * ks), gop[ks], dp);
            }
            // element r of lane l: key k0 + 8 (r / 4) + 4 h + r % 4 of this lane's row
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = 8 * (r >> 2) + 4 * h + (r & 3), key = k0 + kk;
                // a hidden score's logit becomes -inf, so its weight is exactly 0
                // (a select on the logit, not a branch around the arithmetic)
                float dl;
                float x = logit2_minus<CAP>(a, s[r], lse2, dl);
                float dpz = dp[r];
                if constexpr (EXTRA) {
                    x = fmaf(bv[r], BW_LOG2E, x);
                    if (a.drop_scale > 0.0f) dpz = (keepm >> r) & 1u ? dpz * a.drop_scale : 0.0f;
                }
                x = ((key >= rlo) & (key <= rhi) & (sM[kk] != 0.0f)) ? x : -INFINITY;   // & : no short circuit
                const float p = fast_exp2(x);
                s[r] = CAP ? p * (dpz - dlt) * dl : p * (dpz - dlt);
            }
#pragma unroll
            for (int sx = 0; sx < 2; ++sx) {
                const v8 bop = pack8_at<T>(s, 8 * sx);
#pragma unroll
                for (int mb = 0; mb < NDB; ++mb) acc[mb] = Mfma<T>::mma32(cols_a<T, D>(sK, lane, sx, mb), bop, acc[mb]);
            }
        }
    }
    // acc[mb] element r: d = 32 mb + 8 (r / 4) + 4 h + r % 4 of this lane's row;
    // without a cap the scale (d logit / d dot) is applied here
    const float oscale = CAP ? 1.0f : a.scale;
    if (row <= i_last) {
        T* out = dq + ((int64_t)b * a.Lq + row) * a.q_stride + (int64_t)hq * D;
#pragma unroll
        for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                T v4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v4[i] = static_cast<T>(acc[mb][4 * j + i] * oscale);
                *reinterpret_cast<uint2*>(out + 32 * mb + 8 * j + 4 * h) = *reinterpret_cast<const uint2*>(v4);
            }
    }
}

// dQ with the additive mask and dropout: a software pipeline over three LDS
// buffers, as in the dK/dV kernel (one workgroup per CU at D = 128, where
// these calls' registers leave one anyway; the plain kernel above keeps two).
template <typename T, int D, bool CAP, bool EXTRA>
__global__ __launch_bounds__(256, 1) void bwd_dq_pipe_mfma_kernel(FwdArgs a, const T* __restrict__ dout,
                                                             const float* __restrict__ delta, T* __restrict__ dq) {
    typedef typename Mfma<T>::v8 v8;
    constexpr int NKS = D / 16, NDB = D / 32;
    // Three buffers of the per-tile data (K and V tiles, key-kept flags): tile
    // u lives in buffer u % 3, stored two tiles ahead; its S^T and dP^T are
    // formed one tile ahead, its softmax and dQ product in its own iteration.
    constexpr int NBUF = 3;
    __shared__ __attribute__((aligned(16))) char sK[NBUF][BwLds<D>::TILE];
    __shared__ __attribute__((aligned(16))) char sV[NBUF][BwLds<D>::TILE];
    __shared__ float sM[NBUF][32];   // 1: key kept (in range of the axis and of the key mask)
    // the additive mask of the tile's 128 rows x 32 keys (EXTRA): read from
    // global memory 32 keys of a row at a time and from here by each lane's
    // row; rows padded to 36 floats (16-byte reads of 16 rows hit different banks)
    constexpr int BRS = 36;
    __shared__ __attribute__((aligned(16))) float sB[EXTRA ? NBUF : 1][EXTRA ? 128 * BRS : 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    // grid (Hq, B, query blocks), the latest query block first: under a causal
    // mask it walks the most key tiles
    const int hq = blockIdx.x, b = blockIdx.y, kvh = hq / a.group;
    const int i0 = (gridDim.z - 1 - blockIdx.z) * 128, i_last = min(i0 + 127, a.Lq - 1);
    const int row = i0 + 32 * wave + (lane & 31);
    const int rowc = row <= i_last ? row : i_last;
    const T* qb = static_cast<const T*>(a.q) + (int64_t)b * a.Lq * a.q_stride + (int64_t)hq * D;
    const T* gb = dout + (int64_t)b * a.Lq * a.o_stride + (int64_t)hq * D;
    const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Lk * a.kv_stride + (int64_t)kvh * D;
    const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Lk * a.kv_stride + (int64_t)kvh * D;

    v8 qop[NKS], gop[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        qop[ks] = bitcast<v8>(*reinterpret_cast<const u32x4_t*>(qb + (int64_t)rowc * a.q_stride + 16 * ks + 8 * h));
        gop[ks] = bitcast<v8>(*reinterpret_cast<const u32x4_t*>(gb + (int64_t)rowc * a.o_stride + 16 * ks + 8 * h));
    }
    int rlo = 1, rhi = 0;
    float lse2 = 0.0f, dlt = 0.0f;
    if (row <= i_last) {
        row_key_range<false>(a, row, rlo, rhi);
        const float l = a.lse[((int64_t)b * a.Hq + hq) * a.Lq + row];
        if (l == -INFINITY) { rlo = 1; rhi = 0; }   // no weight anywhere in the row
        lse2 = l == -INFINITY ? 0.0f : l * BW_LOG2E;   // finite: hidden logits are -inf
        dlt = delta[((int64_t)b * a.Hq + hq) * a.Lq + row];
    }
    int lo_blk, t0, t1, hi_blk;
    row_key_range<false>(a, i0, lo_blk, t0);
    row_key_range<false>(a, i_last, t1, hi_blk);
    // additive mask of this (batch, query head) (EXTRA with a mask)
    const float* bhead = nullptr;
    if (EXTRA && a.bias) bhead = a.bias + b * a.bias_stride[0] + hq * a.bias_stride[1];

    f32x16_t acc[NDB];
#pragma unroll
    for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = 0.0f;

    if (lo_blk <= hi_blk) {
        const int t_first = lo_blk / 32, n_t = hi_blk / 32 + 1 - t_first;
        TileRegs<D> rk, rv;
        float rm = 0.0f;
        float rb[EXTRA ? 16 : 1];   // thread tid: key tid % 32 of rows tid / 32 + 8 j
        (void)rb;
        // tile t_first + u's K, V and key-kept flags into registers
        auto fetch = [&](int u) {
            const int k0 = 32 * (t_first + u);
            // a masked key's K and V rows stay zero (whatever they hold cannot reach dQ)
            const float* keep = a.key_mask ? a.key_mask + (int64_t)b * a.Lk + k0 : nullptr;
            fetch_tile<T, D>(rk, kb + (int64_t)k0 * a.kv_stride, a.kv_stride, a.Lk - k0, tid, keep);
            fetch_tile<T, D>(rv, vb + (int64_t)k0 * a.kv_stride, a.kv_stride, a.Lk - k0, tid, keep);
            if (tid < 32) {
                const int key = k0 + tid;
                rm = (key < a.Lk && (!a.key_mask || a.key_mask[(int64_t)b * a.Lk + key] > 0.5f)) ? 1.0f : 0.0f;
            }
            if constexpr (EXTRA) {
                if (bhead) {
                    const int key = k0 + (tid & 31);
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int r = i0 + (tid >> 5) + 8 * j;
                        rb[j] = (r < a.Lq && key < a.Lk)
                                    ? bhead[(int64_t)r * a.bias_stride[2] + (int64_t)key * a.bias_stride[3]]
                                    : 0.0f;
                    }
                }
            }
        };
        auto store = [&](int buf) {
            store_tile<D>(sK[buf], rk, tid);
            store_tile<D>(sV[buf], rv, tid);
            if (tid < 32) sM[buf][tid] = rm;
            if constexpr (EXTRA) {
                if (bhead) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) sB[buf][((tid >> 5) + 8 * j) * BRS + (tid & 31)] = rb[j];
                }
            }
        };
        // A operands of S^T and dP^T (K and V rows) of the tile in buffer BUF
        v8 ka[NKS], va[NKS];
        auto read_sdp = [&](int buf) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                ka[ks] = rows_a<T, D>(sK[buf], lane, 16 * ks);
                va[ks] = rows_a<T, D>(sV[buf], lane, 16 * ks);
            }
        };

        // prologue: tiles 0 and 1 stored, tile 2 fetched, S^T and dP^T of tile 0
        fetch(0);
        store(0);
        if (n_t > 1) { fetch(1); store(1); }
        if (n_t > 2) fetch(2);
        __syncthreads();
        f32x16_t sc = {}, dc = {};
        read_sdp(0);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            sc = Mfma<T>::mma32(ka[ks], qop[ks], sc);
            dc = Mfma<T>::mma32(va[ks], gop[ks], dc);
        }

        int buf = 0;   // buffer of tile u
        for (int u = 0; u < n_t; ++u) {
            const int bn = buf == 2 ? 0 : buf + 1, bn2 = bn == 2 ? 0 : bn + 1;
            const int k0 = 32 * (t_first + u);
            read_sdp(bn);   // tile u + 1 (stale after the last tile; discarded)
            // A operands of this tile's dQ product, k-half 0 now, k-half 1
            // halfway through the softmax
            v8 ck[2][NDB];
#pragma unroll
            for (int mb = 0; mb < NDB; ++mb) ck[0][mb] = cols_a<T, D>(sK[buf], lane, 0, mb);
            if (u + 2 < n_t) store(bn2);   // its buffer was last read by tile u - 1
            if (u + 3 < n_t) fetch(u + 3);

            // mask values and dropout keep bits of this lane's 16 scores: score
            // 4 G + e is key k0 + 8 G + 4 h + e
            float bv[EXTRA ? 16 : 1];
            uint32_t keepm = 0xffffu;
            if constexpr (EXTRA) {
                if (bhead) {
                    const float* br = &sB[buf][(32 * wave + (lane & 31)) * BRS + 4 * h];
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const float4 f = *reinterpret_cast<const float4*>(br + 8 * gq);
                        bv[4 * gq] = f.x; bv[4 * gq + 1] = f.y; bv[4 * gq + 2] = f.z; bv[4 * gq + 3] = f.w;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) bv[r] = 0.0f;
                }
                if (a.drop_scale > 0.0f) {
                    // the tile's 32 keys are two 16-key Philox blocks of this
                    // row, which lanes l and l ^ 32 share: each evaluates one
                    // (from the dK/dV kernel's buffer when it stored them)
                    const int jb = (k0 >> 4) + h;
                    const uint32_t own =
                        a.keep_bits ? (row < a.Lq && 16 * jb < a.Lk
                                           ? (uint32_t)a.keep_bits[(((int64_t)b * a.Hq + hq) * ((a.Lk + 15) >> 4) + jb) *
                                                                       a.Lq + row]
                                           : 0u)
                                    : dropout_keep16(a, b, hq, row, jb);
                    const uint32_t oth = (uint32_t)__shfl_xor((int)own, 32);
                    const uint32_t m32 = h ? (oth | (own << 16)) : (own | (oth << 16));   // keys 0 .. 31
                    keepm = pack_even_nibbles(m32 >> (4 * h));
                }
            }
            (void)bv;

            // S^T and dP^T of tile u + 1 beside the softmax of tile u: element r
            // of lane l is key k0 + 8 (r / 4) + 4 h + r % 4 of this lane's row
            f32x16_t sn = {}, dn = {};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if ((r & 1) == 0 && NKS == 8) {
                    sn = Mfma<T>::mma32(ka[r >> 1], qop[r >> 1], sn);
                    dn = Mfma<T>::mma32(va[r >> 1], gop[r >> 1], dn);
                }
                if ((r & 3) == 0 && NKS == 4) {
                    sn = Mfma<T>::mma32(ka[r >> 2], qop[r >> 2], sn);
                    dn = Mfma<T>::mma32(va[r >> 2], gop[r >> 2], dn);
                }
                if (r == 8) {
#pragma unroll
                    for (int mb = 0; mb < NDB; ++mb) ck[1][mb] = cols_a<T, D>(sK[buf], lane, 1, mb);
                }
                const int kk = 8 * (r >> 2) + 4 * h + (r & 3), key = k0 + kk;
                // a hidden score's logit becomes -inf, so its weight is exactly 0
                // (a select on the logit, not a branch around the arithmetic)
                float dl;
                float x = logit2_minus<CAP>(a, sc[r], lse2, dl);
                float dpz = dc[r];
                if constexpr (EXTRA) {
                    x = fmaf(bv[r], BW_LOG2E, x);
                    if (a.drop_scale > 0.0f) dpz = (keepm >> r) & 1u ? dpz * a.drop_scale : 0.0f;
                }
                x = ((key >= rlo) & (key <= rhi) & (sM[buf][kk] != 0.0f)) ? x : -INFINITY;   // & : no short circuit
                const float p = fast_exp2(x);
                sc[r] = CAP ? p * (dpz - dlt) * dl : p * (dpz - dlt);
            }
            // dQ^T += K^T dS^T of tile u
#pragma unroll
            for (int sx = 0; sx < 2; ++sx) {
                const v8 bop = pack8_at<T>(sc, 8 * sx);
#pragma unroll
                for (int mb = 0; mb < NDB; ++mb) acc[mb] = Mfma<T>::mma32(ck[sx][mb], bop, acc[mb]);
            }
            __syncthreads();   // tile u + 2 stored; tile u's buffer free for tile u + 3
            sc = sn;
            dc = dn;
            buf = bn;
        }
    }
    // acc[mb] element r: d = 32 mb + 8 (r / 4) + 4 h + r % 4 of this lane's row;
    // without a cap the scale (d logit / d dot) is applied here
    const float oscale = CAP ? 1.0f : a.scale;
    if (row <= i_last) {
        T* out = dq + ((int64_t)b * a.Lq + row) * a.q_stride + (int64_t)hq * D;
#pragma unroll
        for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                T v4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v4[i] = static_cast<T>(acc[mb][4 * j + i] * oscale);
                *reinterpret_cast<uint2*>(out + 32 * mb + 8 * j + 4 * h) = *reinterpret_cast<const uint2*>(v4);
            }
    }
}

// dK and dV: 16 keys per wave on 16x16x32 MFMAs, D / 16 waves (D keys) per
// workgroup.  At D = 128 the accumulators of 16 keys (2 x 32 registers) and
// their K and V operands (2 x 16) leave two waves per SIMD, where 32 keys per
// wave (2 x 64 accumulators) would leave one; at D = 64 (half of each) three.  Per 32-row step:
//   S  [32 rows x 16 keys] = Q  . K^T   (A: Q rows from LDS, B: K in registers)
//   dP [32 rows x 16 keys] = dO . V^T
//   dV^T [D x 16 keys] += dO^T . P      (A: transposing LDS reads, B: P itself)
//   dK^T [D x 16 keys] += Q^T . dS
// The products' k index e of lane group g (rows 8 g + e of the MFMA) is tile
// row 4 g + e for e < 4 and 16 + 4 g + e - 4 after: the rows that score
// elements (block 0, i) and (block 1, i) of the lane hold, so the packed
// weights are the B operand as they are, and the transposing reads of dO and
// Q take the same two groups of four rows.  Two LDS buffers: step u + 1 is
// stored while step u computes, and its global reads were issued a step
// earlier.
template <typename T, int D, bool CAP, bool EXTRA>
__global__ __launch_bounds__(4 * D, D == 128 ? 1 : ((CAP || EXTRA) ? 2 : 3)) void bwd_dkdv16_kernel(FwdArgs a, const T* __restrict__ dout,
                                                           const float* __restrict__ delta, T* __restrict__ dk,
                                                           T* __restrict__ dv) {
    typedef typename Mfma<T>::v8 v8;
    constexpr int NKS = D / 32, NDB = D / 16, CPR = D / 8, KW = D;   // KW: keys per workgroup
    typedef BwLds<D> L;
    // where 16-byte chunk c of row r sits.  D = 128: at c ^ swz(r), swz(r) =
    // 4 (r % 4) + the two bits of (r / 4) % 4 swapped, a permutation over any
    // 16 consecutive rows (the row reads), and the transposing reads of lane
    // groups 0 and 1 (rows 0..7 at two chunks) land on 16 different chunks, as
    // do those of groups 2 and 3.  D = 64 (8 chunks a row): c rotated right by
    // one bit, then xor (r / 2) % 8; found, like the D = 128 order, by
    // counting bank conflicts of both read patterns over candidate layouts
    auto pch = [](int r, int c) {
        if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 1) & 2) | ((r >> 3) & 1));
        else return (((c & 1) << 2) | (c >> 1)) ^ ((r >> 1) & 7);
    };
    constexpr int NBUF = 3;
    __shared__ __attribute__((aligned(16))) char sQ[NBUF][L::TILE];
    __shared__ __attribute__((aligned(16))) char sG[NBUF][L::TILE];   // dO rows
    __shared__ __attribute__((aligned(16))) float sL[NBUF][32];
    __shared__ __attribute__((aligned(16))) float sD[NBUF][32];
    __shared__ __attribute__((aligned(16))) int sLo[NBUF][32];
    __shared__ __attribute__((aligned(16))) int sHi[NBUF][32];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int kvh = blockIdx.x, b = blockIdx.y;
    const int j0 = blockIdx.z * KW, j_last = min(j0 + KW - 1, a.Lk - 1);
    const int key = j0 + 16 * wave + col;   // this lane's key (MFMA column)
    const int keyc = key <= j_last ? key : j_last;
    const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Lk * a.kv_stride + (int64_t)kvh * D;
    const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Lk * a.kv_stride + (int64_t)kvh * D;

    // B operands: at k-step ks lane l holds K and V of its key at d = (D / 4) g
    // + 8 ks .. +7 (the A operands read the same d: any order of d within the
    // products gives the same sums, and this one keeps the row reads free of
    // LDS bank conflicts); a masked key's rows stay zero (whatever they hold
    // cannot reach a gradient)
    const bool mask_ok = !a.key_mask || a.key_mask[(int64_t)b * a.Lk + keyc] > 0.5f;
    const bool kept = key <= j_last && mask_ok;
    v8 kop[NKS], vop[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        u32x4_t kx = *reinterpret_cast<const u32x4_t*>(kb + (int64_t)keyc * a.kv_stride + (D / 4) * grp + 8 * ks);
        u32x4_t vx = *reinterpret_cast<const u32x4_t*>(vb + (int64_t)keyc * a.kv_stride + (D / 4) * grp + 8 * ks);
        if (!mask_ok) kx = vx = u32x4_t{0u, 0u, 0u, 0u};
        kop[ks] = bitcast<v8>(kx);
        vop[ks] = bitcast<v8>(vx);
    }

    // dka / dva [db] element i: d = 16 db + 4 g + i of this lane's key
    f32x4_t dka[NDB], dva[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dka[db] = dva[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // the run of 32-row query tiles that can see a key of the block (both ends
    // of a row's key range are nondecreasing in the row)
    const int nqt = (a.Lq + 31) / 32;
    int qt_lo, qt_hi;
    {
        int lo = 0, hi = nqt;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            int l0, h0;
            row_key_range<false>(a, min(32 * mid + 31, a.Lq - 1), l0, h0);
            if (h0 >= j0) hi = mid; else lo = mid + 1;
        }
        qt_lo = lo;
        hi = nqt;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            int l0, h0;
            row_key_range<false>(a, 32 * mid, l0, h0);
            if (l0 > j_last) hi = mid; else lo = mid + 1;
        }
        qt_hi = lo - 1;
    }
    const int nv = qt_hi >= qt_lo ? qt_hi - qt_lo + 1 : 0, nsteps = a.group * nv;

    // step u's Q and dO rows (thread tid: row tid / 16, 16-byte chunk tid % 16)
    // and the LSE, Delta and key range of its rows, into registers
    u32x4_t rq, rg;
    int rlo_ = 1, rhi_ = 0;
    float rl_ = 0.0f, rd_ = 0.0f;
    const int fr = tid / CPR, fk = tid % CPR;
    auto fetch = [&](int u) {
        const int hq = kvh * a.group + u / nv, r0 = 32 * (qt_lo + u % nv);
        const T* qb = static_cast<const T*>(a.q) + (int64_t)b * a.Lq * a.q_stride + (int64_t)hq * D;
        const T* gb = dout + (int64_t)b * a.Lq * a.o_stride + (int64_t)hq * D;
        // a row past the end reads the last row and is zeroed: a select, not a branch
        const int valid = a.Lq - r0, rc = r0 + (fr < valid ? fr : valid - 1);
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + (int64_t)rc * a.q_stride + 8 * fk);
        const u32x4_t y = *reinterpret_cast<const u32x4_t*>(gb + (int64_t)rc * a.o_stride + 8 * fk);
        const bool ok = fr < valid;
        rq = u32x4_t{ok ? x[0] : 0u, ok ? x[1] : 0u, ok ? x[2] : 0u, ok ? x[3] : 0u};
        rg = u32x4_t{ok ? y[0] : 0u, ok ? y[1] : 0u, ok ? y[2] : 0u, ok ? y[3] : 0u};
        if (tid < 32) {
            const int r = r0 + tid;
            rlo_ = 1; rhi_ = 0; rl_ = 0.0f; rd_ = 0.0f;
            if (r < a.Lq) {
                row_key_range<false>(a, r, rlo_, rhi_);
                const float l = a.lse[((int64_t)b * a.Hq + hq) * a.Lq + r];
                if (l == -INFINITY) { rlo_ = 1; rhi_ = 0; }
                rl_ = l == -INFINITY ? 0.0f : l * BW_LOG2E;   // finite: hidden logits are -inf
                rd_ = delta[((int64_t)b * a.Hq + hq) * a.Lq + r];
            }
        }
    };
    auto store = [&](int buf) {
        *reinterpret_cast<u32x4_t*>(sQ[buf] + fr * L::RS + pch(fr, fk) * 16) = rq;
        *reinterpret_cast<u32x4_t*>(sG[buf] + fr * L::RS + pch(fr, fk) * 16) = rg;
        if (tid < 32) { sLo[buf][tid] = rlo_; sHi[buf][tid] = rhi_; sL[buf][tid] = rl_; sD[buf][tid] = rd_; }
    };
    // A operand of S / dP: row 16 blk + (l % 16) at d = (D / 4) g + 8 ks .. +7
    auto rows16 = [&](const char* tile, int blk, int ks) {
        const int r = 16 * blk + col;
        return bitcast<v8>(*reinterpret_cast<const u32x4_t*>(tile + r * L::RS + pch(r, NKS * grp + ks) * 16));
    };
    // A operand of dV / dK: the tile transposed, d = 16 db + (l % 16) at rows
    // 4 g + e and 16 + 4 g + e (e = 0..3); source lane j points at row 4 g +
    // j / 4 (+ 16), columns 16 db + 4 (j % 4) .. +3
    const int tr_r0 = 4 * grp + (col >> 2), tr_c = (col & 3) >> 1, tr_h = (col & 1) * 8;
    auto cols16 = [&](const char* tile, int db) {
        const int c = 2 * db + tr_c;
        const i16x4_t lo = lds_read_tr16(tile + tr_r0 * L::RS + pch(tr_r0, c) * 16 + tr_h);
        const i16x4_t hi = lds_read_tr16(tile + (tr_r0 + 16) * L::RS + pch(tr_r0 + 16, c) * 16 + tr_h);
        const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return bitcast<v8>(v);
    };

    // S and dP of the step in buffer BUF: element (blk, i) of lane l is row
    // 16 blk + 4 g + i at this lane's key
    auto sdp_mfma = [&](f32x4_t (&sv)[2], f32x4_t (&dpv)[2], int buf, int blk, int ks) {
        sv[blk] = Mfma<T>::mma16(rows16(sQ[buf], blk, ks), kop[ks], sv[blk]);
        dpv[blk] = Mfma<T>::mma16(rows16(sG[buf], blk, ks), vop[ks], dpv[blk]);
    };

    if (nsteps > 0) {
        // prologue: steps 0 and 1 stored, step 2 fetched, S and dP of step 0
        fetch(0);
        store(0);
        if (nsteps > 1) { fetch(1); store(1); }
        if (nsteps > 2) fetch(2);
        __syncthreads();
        f32x4_t sc[2], dc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            sc[blk] = dc[blk] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) sdp_mfma(sc, dc, 0, blk, ks);
        }
        int buf = 0;   // buffer of step it
        uint32_t mpair = 0u;   // dropout keep bits of two steps' rows (EXTRA)
        (void)mpair;
        for (int it = 0; it < nsteps; ++it) {
            const int bn = buf == 2 ? 0 : buf + 1, bn2 = bn == 2 ? 0 : bn + 1;   // steps it + 1, it + 2
            if (it + 2 < nsteps) store(bn2);   // its buffer was last read by step it - 1
            if (it + 3 < nsteps) fetch(it + 3);
            // The step in NSD + NC slots of one MFMA each, in a fixed order
            // (scheduling barriers between them), every LDS operand read LA
            // slots before its MFMA.  Slots 0..NSD-1: S and dP of step it + 1
            // (after the last step they read a stale buffer and are discarded),
            // with the softmax of step it, one score every SPS slots.  The NC
            // slots after them: dV and dK of step it.
            constexpr int NSD = 4 * NKS, NC = 2 * NDB, SPS = NSD / 8;
            constexpr int LA = EXTRA ? 3 : 4;   // (the mask and dropout registers leave room for three)
            // operand m of the first slots: block m / (2 NKS), k-step (m / 2) %
            // NKS, Q (m even) or dO rows; operand n of the others: d block n / 2
            // of dO^T (n even, dV) or Q^T
            auto read_a = [&](int m) { return rows16((m & 1) ? sG[bn] : sQ[bn], m / (2 * NKS), (m >> 1) % NKS); };
            auto read_c = [&](int n) { return cols16((n & 1) ? sQ[buf] : sG[buf], n >> 1); };
            v8 opa[NSD], opc[NC];
            f32x4_t sn[2], dn[2];
            sn[0] = sn[1] = dn[0] = dn[1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            float p[8], ds[8];
            // the step's additive mask values and dropout keep bits of this
            // lane's 8 scores (score e: row 16 (e / 4) + 4 g + e % 4).  The
            // wave's 16 keys are one 16-key Philox block of each row: lane L
            // evaluates the block of row L % 32, and each lane takes its key's
            // bit of its rows' blocks from the lanes that hold them.
            float bv[EXTRA ? 8 : 1];
            uint32_t keepm = 0xffu;
            if constexpr (EXTRA) {
                const int hq = kvh * a.group + it / nv, r0 = 32 * (qt_lo + it % nv);
                if (a.bias) {
                    const float* bk = a.bias + b * a.bias_stride[0] + hq * a.bias_stride[1] +
                                      (int64_t)keyc * a.bias_stride[3];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = r0 + 16 * (e >> 2) + 4 * grp + (e & 3);
                        bv[e] = row < a.Lq ? bk[(int64_t)row * a.bias_stride[2]] : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) bv[e] = 0.0f;
                }
                if (a.drop_scale > 0.0f) {
                    // a step needs 32 blocks: lanes 0..31 evaluate those of an
                    // even step and lanes 32..63 those of the step after it
                    if ((it & 1) == 0) {
                        const int u = min(it + (lane >> 5), nsteps - 1);
                        const int hqu = kvh * a.group + u / nv, rowu = 32 * (qt_lo + u % nv) + (lane & 31);
                        const int jb = (j0 + 16 * wave) >> 4;
                        mpair = dropout_keep16(a, b, hqu, rowu, jb);
                        // stored for the dQ kernel: every (row, block) with a visible
                        // weight is written here (its row's tile is in the run)
                        if (a.keep_bits && it + (lane >> 5) < nsteps && rowu < a.Lq && 16 * jb < a.Lk)
                            a.keep_bits[(((int64_t)b * a.Hq + hqu) * ((a.Lk + 15) >> 4) + jb) * a.Lq + rowu] =
                                (uint16_t)mpair;
                    }
                    keepm = 0u;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t ms =
                            (uint32_t)__shfl((int)mpair, 32 * (it & 1) + 16 * (e >> 2) + 4 * grp + (e & 3));
                        keepm |= ((ms >> col) & 1u) << e;
                    }
                }
            }
            (void)bv;
            int los[4], his[4];
            float ls[4], dd[4];
            // row data of block BLK of step it: rows 16 blk + 4 g .. +3
            auto read_rows = [&](int blk) {
                const int m0 = 16 * blk + 4 * grp;
                const int4 lo4 = *reinterpret_cast<const int4*>(&sLo[buf][m0]);
                const int4 hi4 = *reinterpret_cast<const int4*>(&sHi[buf][m0]);
                const float4 l4 = *reinterpret_cast<const float4*>(&sL[buf][m0]);
                const float4 d4 = *reinterpret_cast<const float4*>(&sD[buf][m0]);
                los[0] = lo4.x; los[1] = lo4.y; los[2] = lo4.z; los[3] = lo4.w;
                his[0] = hi4.x; his[1] = hi4.y; his[2] = hi4.z; his[3] = hi4.w;
                ls[0] = l4.x; ls[1] = l4.y; ls[2] = l4.z; ls[3] = l4.w;
                dd[0] = d4.x; dd[1] = d4.y; dd[2] = d4.z; dd[3] = d4.w;
            };
            read_rows(0);
#pragma unroll
            for (int m = 0; m < LA; ++m) opa[m] = read_a(m);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < NSD; ++m) {
                if (m + LA < NSD) opa[m + LA] = read_a(m + LA);
                else opc[m + LA - NSD] = read_c(m + LA - NSD);
                const int blk = m / (2 * NKS), ks = (m >> 1) % NKS;
                if (m & 1) dn[blk] = Mfma<T>::mma16(opa[m], vop[ks], dn[blk]);
                else sn[blk] = Mfma<T>::mma16(opa[m], kop[ks], sn[blk]);
                if (m % SPS == SPS - 1) {
                    // score e = m / SPS: row 16 (e / 4) + 4 g + e % 4 at this lane's key;
                    // a hidden score's logit becomes -inf, so its weight is exactly 0
                    const int e = m / SPS, eb = e >> 2, i = e & 3;
                    float dl;
                    float x = logit2_minus<CAP>(a, sc[eb][i], ls[i], dl);
                    float z = 1.0f;
                    if constexpr (EXTRA) {
                        x = fmaf(bv[e], BW_LOG2E, x);
                        if (a.drop_scale > 0.0f) z = (keepm >> e) & 1u ? a.drop_scale : 0.0f;
                    }
                    x = (kept & (key >= los[i]) & (key <= his[i])) ? x : -INFINITY;   // & : no short circuit
                    const float pe = fast_exp2(x);
                    // with dropout dV takes the kept, rescaled weights and dS
                    // the kept, rescaled dP
                    p[e] = EXTRA ? pe * z : pe;
                    const float dz = EXTRA ? dc[eb][i] * z : dc[eb][i];
                    ds[e] = CAP ? pe * (dz - dd[i]) * dl : pe * (dz - dd[i]);
                }
                if (m == 4 * SPS - 1) read_rows(1);   // block 0's row data is used up by this slot's score
                __builtin_amdgcn_sched_barrier(0);
            }
            const v8 pop = pack8<T>(p), dop = pack8<T>(ds);
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                if (n + LA < NC) opc[n + LA] = read_c(n + LA);
                if (n & 1) dka[n >> 1] = Mfma<T>::mma16(opc[n], dop, dka[n >> 1]);
                else dva[n >> 1] = Mfma<T>::mma16(opc[n], pop, dva[n >> 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();   // step it + 2 stored; step it's buffer free for step it + 3
            sc[0] = sn[0]; sc[1] = sn[1]; dc[0] = dn[0]; dc[1] = dn[1];
            buf = bn;
        }
    }
    // without a cap the scale (d logit / d dot) is applied to dK here
    const float oscale = CAP ? 1.0f : a.scale;
    if (key <= j_last) {
        T* ko = dk + ((int64_t)b * a.Lk + key) * a.kv_stride + (int64_t)kvh * D;
        T* vo = dv + ((int64_t)b * a.Lk + key) * a.kv_stride + (int64_t)kvh * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            T k4[4], v4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                k4[i] = static_cast<T>(dka[db][i] * oscale);
                v4[i] = static_cast<T>(dva[db][i]);
            }
            *reinterpret_cast<uint2*>(ko + 16 * db + 4 * grp) = *reinterpret_cast<const uint2*>(k4);
            *reinterpret_cast<uint2*>(vo + 16 * db + 4 * grp) = *reinterpret_cast<const uint2*>(v4);
        }
    }
}

template <typename T, int D, bool CAP, bool EXTRA>
hipError_t launch_bwd_mfma_t(const FwdArgs& a, const void* dout, const float* delta, void* dq, void* dk, void* dv,
                             hipStream_t s) {
    const T* g = static_cast<const T*>(dout);
    // dK/dV first: with dropout its kernel may store the keep bits that the
    // dQ kernel then reads (same stream)
    hipLaunchKernelGGL((bwd_dkdv16_kernel<T, D, CAP, EXTRA>), dim3(a.Hkv, a.B, (a.Lk + D - 1) / D), dim3(4 * D), 0, s,
                       a, g, delta, static_cast<T*>(dk), static_cast<T*>(dv));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.Lq <= 0) return e;
    // the unpipelined dQ kernel keeps two workgroups per CU; with a mask or
    // dropout it needs the mask's keys contiguous (copied 16 bytes at a time,
    // offsets within 32 bits) and the stored dropout pattern
    const bool direct = !EXTRA || ((!a.bias || (a.bias_stride[3] == 1 &&
                                                ((int64_t)(a.Lq - 1) * a.bias_stride[2] + a.Lk) * 4 < ((int64_t)1 << 31))) &&
                                   (!(a.drop_scale > 0.0f) || a.keep_bits));
    if (EXTRA && !direct)
        hipLaunchKernelGGL((bwd_dq_pipe_mfma_kernel<T, D, CAP, true>), dim3(a.Hq, a.B, (a.Lq + 127) / 128),
                           dim3(256), 0, s, a, g, delta, static_cast<T*>(dq));
    else
        hipLaunchKernelGGL((bwd_dq_mfma_kernel<T, D, CAP, EXTRA>), dim3(a.Hq, a.B, (a.Lq + 127) / 128), dim3(256), 0,
                           s, a, g, delta, static_cast<T*>(dq));
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_mfma_dd(const FwdArgs& a, const void* dout, const float* delta, void* dq, void* dk, void* dv,
                              hipStream_t s) {
    const bool cap = a.softcap > 0.0f, extra = a.bias != nullptr || a.drop_scale > 0.0f;
    if (extra)
        return cap ? launch_bwd_mfma_t<T, D, true, true>(a, dout, delta, dq, dk, dv, s)
                   : launch_bwd_mfma_t<T, D, false, true>(a, dout, delta, dq, dk, dv, s);
    return cap ? launch_bwd_mfma_t<T, D, true, false>(a, dout, delta, dq, dk, dv, s)
               : launch_bwd_mfma_t<T, D, false, false>(a, dout, delta, dq, dk, dv, s);
}

template <typename T>
hipError_t launch_bwd_mfma_d(const FwdArgs& a, const void* dout, const float* delta, void* dq, void* dk, void* dv,
                             hipStream_t s) {
    return a.D == 64 ? launch_bwd_mfma_dd<T, 64>(a, dout, delta, dq, dk, dv, s)
                     : launch_bwd_mfma_dd<T, 128>(a, dout, delta, dq, dk, dv, s);
}

}  // namespace

size_t bwd_keep_bits_bytes(const FwdArgs& a, int dtype) {
    if (!(a.drop_scale > 0.0f) || !bwd_mfma_supported(a, dtype) || a.B <= 0 ||
        a.Lq <= 0 || a.Lk <= 0)
        return 0;
    return (size_t)a.B * a.Hq * ((a.Lk + 15) / 16) * a.Lq * sizeof(uint16_t);
}

bool bwd_mfma_supported(const FwdArgs& a, int dtype) {
    return (dtype == kBF16 || dtype == kF16) && (a.D == 64 || a.D == 128) && !a.seq_bounds && !a.row_pos &&
           (a.Lq + 127) / 128 <= 65535 && (a.Lk + a.D - 1) / a.D <= 65535;   // grid z
}

hipError_t launch_backward_mfma(const FwdArgs& a, const void* dout, const float* delta, void* dq, void* dk, void* dv,
                                int dtype, hipStream_t s) {
    if (dtype == kBF16) return launch_bwd_mfma_d<__bf16>(a, dout, delta, dq, dk, dv, s);
    if (dtype == kF16) return launch_bwd_mfma_d<_Float16>(a, dout, delta, dq, dk, dv, s);
    return hipErrorInvalidValue;
}

}  // namespace mfa
