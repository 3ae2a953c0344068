// kernels_decode.hip -- single-query (Lq = 1) decode over a long KV cache:
// a split-over-keys partial kernel and a combine kernel.
//
// The key range of the query is cut into S splits (brotensor
// flash_attention.h, flash_attention_decode_len: the work divides the valid
// keys; different split points change only the rounding).  One wave handles
// one (split, kv head, batch) and serves all Hq/Hkv query heads that share the
// kv head, so every cache row is read from HBM once (same header: each cache
// row read once for all query rows; GQA without widening the kv heads).
//
// Per 32-key tile:
//   K, V rows  --coalesced 16-byte loads-->  registers  -->  swizzled LDS
//   S^T[16 keys x 16 q] = K . Q^T         MFMA 16x16x32, Q^T held in registers
//   online softmax per query column (running max m, rescaled sum l), base 2
//   O^T[16 d x 16 q] += V^T . P^T          MFMA 16x16x32; P^T is the score
//                                          accumulator itself, V^T comes from
//                                          transposing LDS reads; for bf16 the
//                                          weights go in as two operands, the
//                                          rounded weight and its rounded
//                                          residue (the loop is bound by HBM,
//                                          so the second product is free)
// Query heads beyond Hq/Hkv (columns g..15) compute on zeros and are dropped.
//
// With a device-held length (same header, flash_attention_decode_len) the
// kernel serves R query rows per batch, the columns being (row, head) pairs,
// R * Hq/Hkv <= 16: row r attends causally to the first len - R + 1 + r keys
// of the cache.  The length is read on the device and the splits divide its
// tiles, so the launch shape depends on the cache capacity only and rows past
// the length cost nothing.
//
// With a key mask over a fixed-capacity cache (same header,
// flash_attention_decode_masked) the single query sits at the batch's last
// valid key, found on the device from the packed mask words, and a window
// counts back from it; the splits divide the tiles of that range and tiles
// without a valid key are skipped before any K/V read, so the launch shape
// depends on the capacity only.
//
// Each split writes (m, l, O_unnormalised[D]) in base-2 units; the combine
// kernel merges them: M = max m_s, w_s = 2^(m_s - M), O = sum w_s O_s / sum
// w_s l_s, LSE = (M + log2 sum w_s l_s) ln 2.  Empty splits carry m = -inf,
// l = 0, O = 0; a query with no visible key ends with O = 0, LSE = -inf.
#include "mfa_device.h"
#include "mfa_internal.h"

#include <math.h>

#include <type_traits>

namespace mfa {
namespace {

constexpr int DT = 32;  // keys per tile

struct DecodeArgs {
    FwdArgs f;                // Lq = R query rows per batch; Lk = cache rows
    const int* d_len;         // [B] valid lengths on the device, or null (Lq = 1, key_range)
    int pos_from_mask;        // Lq = 1: the query sits at the batch's last valid key (needs the mask)
    int splits;
    float* part_ml;   // [B, R, Hq, S, 2]: m (base 2), l
    float* part_o;    // [B, R, Hq, S, D]
};

template <typename T, int D, bool CAP, bool MASK>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs da) {
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int RPL = 64 / CPR;       // rows per wave-wide load
    constexpr int NLD = DT / RPL;       // loads per tensor per tile
    constexpr int NDB = D / 16;         // 16-wide d blocks
    constexpr int NKS = D / 32;         // 32-wide k steps of Q.K
    constexpr bool SPLIT_P = std::is_same<T, __bf16>::value;   // weights as bf16 hi + lo
    typedef typename Mfma<T>::v8 v8;

    __shared__ u32x4_t sK[DT * CPR];
    __shared__ u32x4_t sV[DT * CPR];

    const FwdArgs& a = da.f;
    const int lane = threadIdx.x;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int g = a.group;
    const int col = lane & 15;          // query column of the MFMA tiles
    const int grp = lane >> 4;          // lane group 0..3
    const int R = a.Lq;
    const int crow = col / g;           // column -> (query row, head in the group)
    const int chead = col - crow * g;
    const bool real = crow < R;

    // Keys [lo, hi] of all columns, this column's last key hi_col and the last
    // key every column sees (hi_min), then this split's share of the tiles.
    const uint64_t* words = MASK ? a.mask_words + (int64_t)b * a.words_per_batch : nullptr;
    int lo, hi, hi_col, hi_min;
    if (MASK && da.pos_from_mask) {
        // the last valid key (highest set bit of the batch's mask words) is
        // the query's position; keys after position - window, up to it
        int p = -1;
        for (int w = lane; w < a.words_per_batch; w += 64) {
            const uint64_t x = words[w];
            if (x) p = w * 64 + 63 - __clzll((long long)x);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) p = max(p, __shfl_xor(p, off));
        lo = (p >= 0 && a.window > 0 && p - a.window + 1 > 0) ? p - a.window + 1 : 0;
        hi = p;
        hi_col = hi_min = hi;
    } else if (da.d_len) {
        int n = da.d_len[b];
        n = n < 0 ? 0 : (n > a.Lk ? a.Lk : n);
        lo = 0;
        hi = n - 1;
        hi_min = n - R;
        hi_col = n - R + (real ? crow : R - 1);
    } else {
        key_range(a.q_offset, a.Lk, a.causal, a.window, lo, hi);
        hi_col = hi_min = hi;
    }
    int t_begin = 0, t_end = 0;
    if (lo <= hi) {
        const int t_lo = lo / DT, n_t = hi / DT - t_lo + 1;
        t_begin = t_lo + (int)((int64_t)n_t * split / da.splits);
        t_end = t_lo + (int)((int64_t)n_t * (split + 1) / da.splits);
    }

    // Q^T operand: lane (col, grp) holds Q[row crow][head kvh*g + chead][32 ks + 8 grp .. +7]
    const T* __restrict__ qp = static_cast<const T*>(a.q);
    v8 qop[NKS];
    {
        const int hq = kvh * g + chead;
        const T* qrow = qp + (((int64_t)b * R + (real ? crow : 0)) * a.Hq + (real ? hq : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4_t raw = *reinterpret_cast<const u32x4_t*>(qrow + ks * 32 + grp * 8);
            if (!real) raw = u32x4_t{0u, 0u, 0u, 0u};
            qop[ks] = bitcast<v8>(raw);
        }
    }

    // Mask bits of tile t.  Lane l holds word wbase + l of the batch (a window
    // of 64 words, 128 tiles), reloaded when the tiles move past it, so the
    // choice of the next tile costs a cross-lane read instead of a memory
    // round trip before that tile's loads can issue.  Tiles only move forward.
    int wbase = -64;
    uint32_t wlo = 0u, whi = 0u;
    auto bits_of = [&](int t) -> uint32_t {
        const int w = t >> 1;
        if (w >= wbase + 64) {
            wbase = w & ~63;
            const int ww = wbase + lane;
            const uint64_t x = ww < a.words_per_batch ? words[ww] : 0ull;
            wlo = (uint32_t)x;
            whi = (uint32_t)(x >> 32);
        }
        return (uint32_t)__builtin_amdgcn_readlane((int)((t & 1) ? whi : wlo), w - wbase);
    };
    (void)bits_of;

    const T* __restrict__ kp = static_cast<const T*>(a.k);
    const T* __restrict__ vp = static_cast<const T*>(a.v);
    const int64_t row_stride = (int64_t)a.Hkv * D;
    const T* kbase = kp + (int64_t)b * a.Lk * row_stride + (int64_t)kvh * D;
    const T* vbase = vp + (int64_t)b * a.Lk * row_stride + (int64_t)kvh * D;
    const int ld_row = lane / CPR, ld_chunk = lane % CPR;

    u32x4_t kreg[NLD], vreg[NLD];
    f32x4_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;   // running max of this lane's query column (base 2)
    float l = 0.0f;        // this lane's share of the running sum

    const float two_log2e_over_cap = CAP ? 2.0f * 1.4426950408889634f / a.softcap : 0.0f;

    // bits_t: mask bits of tile t, read when t was chosen (the window may
    // have moved on to the next tile's words since)
    int t = t_begin;
    uint32_t bits_t = 0xffffffffu;
    if (MASK) while (t < t_end && (bits_t = bits_of(t)) == 0u) ++t;
    // Rows of tile tt into registers.  A row no query row can use (outside
    // [lo, hi], or masked) is not read: it becomes zeros, so whatever the
    // cache holds there (unwritten slots past the length, say) never meets a
    // zero weight in the products, and the skipped rows cost no bandwidth.
    auto load_tile = [&](int tt, uint32_t tbits) {
        // bit r: row r of the tile is used (wave-uniform, built on the scalar unit)
        const int l0 = lo - tt * DT, h0 = hi - tt * DT;
        uint32_t use = MASK ? tbits : 0xffffffffu;
        if (h0 < DT - 1) use &= h0 < 0 ? 0u : (0xffffffffu >> (DT - 1 - h0));
        if (l0 > 0) use &= l0 >= DT ? 0u : (0xffffffffu << l0);
        const uint32_t mine = use >> ld_row;   // bit i * RPL: this lane's row of load i
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            u32x4_t kx = u32x4_t{0u, 0u, 0u, 0u}, vx = u32x4_t{0u, 0u, 0u, 0u};
            if ((mine >> (i * RPL)) & 1u) {
                const int64_t off = (int64_t)(tt * DT + i * RPL + ld_row) * row_stride + ld_chunk * 8;
                kx = *reinterpret_cast<const u32x4_t*>(kbase + off);
                vx = *reinterpret_cast<const u32x4_t*>(vbase + off);
            }
            kreg[i] = kx;
            vreg[i] = vx;
        }
    };
    if (t < t_end) load_tile(t, bits_t);
    while (t < t_end) {
        // next tile with a visible key
        int tn = t + 1;
        uint32_t bits_n = 0xffffffffu;
        if (MASK) while (tn < t_end && (bits_n = bits_of(tn)) == 0u) ++tn;
        __syncthreads();  // LDS no longer read by the previous tile
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int r = i * RPL + ld_row;
            sK[r * CPR + swz_k<D>(r, ld_chunk)] = kreg[i];
            sV[r * CPR + swz_v<D>(r, ld_chunk)] = vreg[i];
        }
        if (tn < t_end) load_tile(tn, bits_n);
        __syncthreads();

        // scores: two 16-key blocks
        f32x4_t s[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            s[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const int r = blk * 16 + col;  // A operand row = key
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const v8 kop = bitcast<v8>(sK[r * CPR + swz_k<D>(r, ks * 4 + grp)]);
                s[blk] = Mfma<T>::mma16(kop, qop[ks], s[blk]);
            }
        }

        // transform, mask, running max
        const uint32_t bits = bits_t;
        const bool interior = t * DT >= lo && t * DT + DT - 1 <= hi_min && (!MASK || bits == 0xffffffffu);
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = s[blk][i];
                if (CAP) v = softcap_apply(v * a.scale, a.softcap, two_log2e_over_cap) * 1.4426950408889634f;
                else v = v * a.score_to_log2;
                if (!interior) {
                    const int kk = blk * 16 + grp * 4 + i;
                    const int key = t * DT + kk;
                    const bool vis = key >= lo && key <= hi_col && ((bits >> kk) & 1u);
                    v = vis ? v : -INFINITY;
                }
                x[blk * 4 + i] = v;
                tmax = fmax_fast(tmax, v);
            }
        }
        tmax = fmax_fast(tmax, __shfl_xor(tmax, 16));
        tmax = fmax_fast(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m - m_use);
        m = m_new;
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = fast_exp2(x[e] - m_use);
            psum += x[e];
        }
        l = l * alpha + psum;
        const v8 pop = pack8<T>(x);
        // bf16 keeps 8 significant bits of a weight; the rounding residue
        // x - bf16(x), itself rounded, is a second operand whose products
        // restore about 16 bits (fp16 weights already keep 11)
        v8 pop_lo;
        if constexpr (SPLIT_P) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pop_lo[e] = static_cast<T>(x[e] - static_cast<float>(pop[e]));
        }
        (void)pop_lo;

        // O^T += V^T P^T over the 32 keys of the tile
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[db][i] *= alpha;
            const int j = col;  // source lane within the 16-lane group
            const int chunk = db * 2 + ((j & 3) >> 1);
            const int half = j & 1;
            const int r0 = grp * 4 + (j >> 2);
            const int r1 = 16 + grp * 4 + (j >> 2);
            const char* p0 = reinterpret_cast<const char*>(sV) + (r0 * CPR + swz_v<D>(r0, chunk)) * 16 + half * 8;
            const char* p1 = reinterpret_cast<const char*>(sV) + (r1 * CPR + swz_v<D>(r1, chunk)) * 16 + half * 8;
            const i16x4_t lo4 = lds_read_tr16(p0);
            const i16x4_t hi4 = lds_read_tr16(p1);
            const i16x8_t vv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            oacc[db] = Mfma<T>::mma16(bitcast<v8>(vv), pop, oacc[db]);
            if constexpr (SPLIT_P) oacc[db] = Mfma<T>::mma16(bitcast<v8>(vv), pop_lo, oacc[db]);
        }
        t = tn;
        bits_t = bits_n;
    }

    // lane groups hold disjoint keys of the same query column: total the sum
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (real) {
        const int hq = kvh * g + chead;
        const int64_t slot = (((int64_t)b * R + crow) * a.Hq + hq) * da.splits + split;
        if (grp == 0) {
            da.part_ml[slot * 2 + 0] = m;
            da.part_ml[slot * 2 + 1] = l;
        }
        float* po = da.part_o + slot * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<float4*>(po + db * 16 + grp * 4) =
                make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs da) {
    const FwdArgs& a = da.f;
    const int bh = blockIdx.x;          // (b * R + r) * Hq + hq
    const int lane = threadIdx.x;
    const int S = da.splits;
    const float* ml = da.part_ml + (int64_t)bh * S * 2;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
    const float M_use = M == -INFINITY ? 0.0f : M;
    float L = 0.0f;
    float acc[D / 64];
#pragma unroll
    for (int c = 0; c < D / 64; ++c) acc[c] = 0.0f;
    const float* po = da.part_o + (int64_t)bh * S * D;
    for (int s = 0; s < S; ++s) {
        const float w = fast_exp2(ml[2 * s] - M_use);
        L += w * ml[2 * s + 1];
#pragma unroll
        for (int c = 0; c < D / 64; ++c) acc[c] += w * po[(int64_t)s * D + lane + 64 * c];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    T* out = static_cast<T*>(a.out) + (int64_t)bh * D;   // [B, R, Hq, D]
#pragma unroll
    for (int c = 0; c < D / 64; ++c) out[lane + 64 * c] = static_cast<T>(acc[c] * inv);
    if (a.lse && lane == 0) {
        const int hq = bh % a.Hq, br = bh / a.Hq;          // LSE is [B, Hq, R]
        const int r = br % a.Lq, b = br / a.Lq;
        a.lse[((int64_t)b * a.Hq + hq) * a.Lq + r] = L > 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
    }
}

template <typename T, int D, bool CAP, bool MASK>
hipError_t launch_t(const DecodeArgs& da, hipStream_t s) {
    const FwdArgs& a = da.f;
    // instrumentation events: start of the split kernel, end of the combine
    hipExtLaunchKernelGGL((decode_split_kernel<T, D, CAP, MASK>), dim3(da.splits, a.Hkv, a.B), dim3(64), 0, s,
                          instr_event_begin(), nullptr, 0, da);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipExtLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.B * a.Lq * a.Hq), dim3(64), 0, s, nullptr,
                          instr_event_end(), 0, da);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& da, hipStream_t s) {
    const bool cap = da.f.softcap > 0.0f, mask = da.f.key_mask != nullptr;
    if (cap) return mask ? launch_t<T, D, true, true>(da, s) : launch_t<T, D, true, false>(da, s);
    return mask ? launch_t<T, D, false, true>(da, s) : launch_t<T, D, false, false>(da, s);
}

}  // namespace

bool split_decode_supported(int dtype, int D, int Lq, int group) {
    return Lq == 1 && (dtype == kBF16 || dtype == kF16) && (D == 64 || D == 128) && group >= 1 &&
           group <= 16;
}

bool decode_len_supported(int dtype, int D, int R, int group) {
    return (dtype == kBF16 || dtype == kF16) && (D == 64 || D == 128) && R >= 1 && group >= 1 &&
           R * group <= 16;
}

// About three (split, kv head, batch) waves per CU of the 256-CU part, but at
// least 8 tiles (256 keys) per split.  Each wave keeps enough loads in flight
// to stream on its own: swept over batch 4 .. 64 of the long cache, the rate
// peaks at 512 - 768 waves and falls by 5 - 30 % at the 4096 - 16384 waves of
// more, shorter splits.
int split_decode_default_splits(int B, int Hkv, int Lk, int group) {
    (void)group;
    const int64_t streams = (int64_t)B * Hkv;
    const int64_t target_waves = 768;
    int64_t s = (target_waves + streams - 1) / streams;
    const int64_t tiles = (Lk + DT - 1) / DT;
    const int64_t max_s = tiles / 8 > 0 ? tiles / 8 : 1;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    if (s > 256) s = 256;
    return (int)s;
}

size_t split_decode_workspace_bytes(int B, int R, int Hq, int D, int splits) {
    const size_t slots = (size_t)B * R * Hq * splits;
    return slots * 2 * sizeof(float) + 256 + slots * D * sizeof(float);
}

hipError_t launch_split_decode(const FwdArgs& a, const int* d_len, int dtype, int splits, float* partials,
                               hipStream_t s, bool pos_from_mask) {
    if (pos_from_mask && (!a.key_mask || !a.mask_words || a.Lq != 1 || d_len)) return hipErrorInvalidValue;
    DecodeArgs da;
    da.f = a;
    da.d_len = d_len;
    da.pos_from_mask = pos_from_mask ? 1 : 0;
    da.splits = splits;
    const size_t slots = (size_t)a.B * a.Lq * a.Hq * splits;
    da.part_ml = partials;
    const size_t ml_bytes = (slots * 2 * sizeof(float) + 255) & ~size_t(255);
    da.part_o = reinterpret_cast<float*>(reinterpret_cast<char*>(partials) + ml_bytes);
    if (dtype == kBF16) return a.D == 64 ? launch_d<__bf16, 64>(da, s) : launch_d<__bf16, 128>(da, s);
    if (dtype == kF16) return a.D == 64 ? launch_d<_Float16, 64>(da, s) : launch_d<_Float16, 128>(da, s);
    return hipErrorInvalidValue;
}

}  // namespace mfa
