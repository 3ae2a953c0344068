// kernels_mfma.hip -- bf16/fp16 prefill forward on gfx950 matrix cores.
//
// The method is the tiled online softmax of vision_rs flash_attn2.rs (forward
// kernel): per query row a running max m, a running sum l rescaled by
// exp(m_old - m_new) and an accumulator rescaled the same way, finished as
// O = acc / l and LSE = m + log l.  Both contractions (Q.K^T and P.V) run on
// MFMA with fp32 accumulation (brotensor flash_attention.h: fp32
// accumulation); the softmax runs in fp32 in base 2.
//
// Work decomposition.  One 256-thread workgroup owns 128 query rows of one
// query head; its four waves own 32 rows each.  64-key tiles of K and V are
// staged, double buffered, in XOR-swizzled LDS through coalesced 16-byte
// loads.  Per wave and tile:
//   S^T[32 keys x 32 q] = K . Q^T            v_mfma_f32_32x32x16, Q^T in VGPRs
//     -> lane l holds 16 keys of query row (l % 32): the row max is an in-lane
//        max plus one exchange with lane l ^ 32
//   O^T[32 d x 32 q] += V^T . P^T            v_mfma_f32_32x32x16; P^T is the
//        score accumulator (rounded to the input type), V^T comes from the
//        transposing LDS read, so no score ever leaves the registers.
// Only tiles that intersect the key range of the workgroup's rows are visited
// (causal and window bounds), tiles whose key-mask word is zero are skipped
// without loading K or V, and per-element masking runs only on tiles that are
// not fully visible to every row of the wave.
//
// Scheduling.  Blocks are ordered so that the Hq/Hkv heads sharing a kv head
// and q tile are adjacent (they read the same K/V tiles together) and the
// heaviest causal tiles go first; the block id is remapped so that each of the
// 8 XCDs (round-robin dispatch, one L2 each) receives a contiguous range of
// that order.
#include "mfa_device.h"
#include "mfa_internal.h"

#include <math.h>

namespace mfa {
namespace {

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile

// Padded LDS rows.  K rows are D*2 + 16 bytes apart: the 32 lanes that read
// one 16-byte chunk from 32 consecutive rows start 4 banks apart, so each
// group of 16 rows covers all 64 banks once.  V rows are D*2 + 64 bytes apart:
// a transposing read takes 64 bytes from each of 4 consecutive rows per half
// wave, and those rows start 16 banks apart.  With padding (instead of an XOR
// swizzle) every LDS read is a per-lane base plus a compile-time offset.
template <int D> struct PfLds {
    static constexpr int KS = D * 2 + 16;         // K row stride, bytes
    static constexpr int VS = D * 2 + 64;         // V row stride, bytes
    static constexpr int KT = BN * KS;            // one K tile
    static constexpr int VT = BN * VS;            // one V tile
    static constexpr int BUF = KT + VT;           // one stage
    static constexpr int BYTES = 2 * BUF;         // double buffered
};

__device__ inline int remap_xcd(int p, int n) {
    const int per = n / 8;
    if (p < per * 8) return (p % 8) * per + p / 8;
    return p;
}

template <typename T, int D, bool CAP, bool MASK>
__global__ __launch_bounds__(256, 2) void prefill_kernel(FwdArgs a, int nqt) {
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int NKS = D / 16;             // k-steps of Q.K^T
    constexpr int NDB = D / 32;             // 32-wide d blocks of O
    constexpr int LPT = BN * CPR / 256;     // 16-byte loads per thread per tensor
    typedef typename Mfma<T>::v8 v8;
    constexpr float LOG2E = 1.4426950408889634f;

    typedef PfLds<D> L;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lq = lane & 31;               // query row within the wave
    const int h2 = lane >> 5;               // lane half

    // ---- block -> (batch, kv head, q tile, q head)
    const int n = remap_xcd(blockIdx.x, gridDim.x);
    const int g = a.group;
    const int per_group = g * nqt;
    const int bk = n / per_group;           // b * Hkv + kvh
    const int rem = n - bk * per_group;
    const int qt = nqt - 1 - rem / g;       // heaviest tile first
    const int b = bk / a.Hkv;
    const int kvh = bk - b * a.Hkv;
    const int hq = kvh * g + (rem % g);

    const int i0 = qt * BM;
    const int i_last = min(i0 + BM, a.Lq) - 1;
    const int w_first = i0 + wave * 32;
    const int w_last = min(w_first + 31, i_last);
    const int qrow = w_first + lq;

    // key ranges: workgroup (tiles to visit), wave (interior test), lane (mask)
    int lo_blk, hi_tmp, lo_tmp, hi_blk;
    key_range(i0 + a.q_offset, a.Lk, a.causal, a.window, lo_blk, hi_tmp);
    key_range(i_last + a.q_offset, a.Lk, a.causal, a.window, lo_tmp, hi_blk);
    int wlo_last = a.Lk, whi_first = -1;
    if (w_first <= i_last) {
        int t0, t1;
        key_range(w_first + a.q_offset, a.Lk, a.causal, a.window, t0, whi_first);
        key_range(w_last + a.q_offset, a.Lk, a.causal, a.window, wlo_last, t1);
    }
    int rlo = 1, rhi = 0;
    if (qrow <= i_last) key_range(qrow + a.q_offset, a.Lk, a.causal, a.window, rlo, rhi);

    const int64_t q_stride = (int64_t)a.Hq * D;
    const int64_t kv_stride = (int64_t)a.Hkv * D;
    const T* __restrict__ qbase = static_cast<const T*>(a.q) + (int64_t)b * a.Lq * q_stride + (int64_t)hq * D;
    const T* __restrict__ kbase = static_cast<const T*>(a.k) + (int64_t)b * a.Lk * kv_stride + (int64_t)kvh * D;
    const T* __restrict__ vbase = static_cast<const T*>(a.v) + (int64_t)b * a.Lk * kv_stride + (int64_t)kvh * D;
    const uint64_t* words = MASK ? a.mask_words + (int64_t)b * a.words_per_batch : nullptr;

    // ---- Q^T operand: lane holds Q[qrow][16 ks + 8 h2 .. +7]
    v8 qop[NKS];
    {
        const int r = qrow <= i_last ? qrow : i_last;
        const T* qp = qbase + (int64_t)r * q_stride + h2 * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qop[ks] = bitcast<v8>(*reinterpret_cast<const u32x4_t*>(qp + ks * 16));
    }

    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
    float m = -INFINITY;   // running max (base 2) of this lane's row
    float l = 0.0f;        // this lane's half of the running sum

    const float c_log2 = a.score_to_log2;                       // scale * log2(e)
    const float cap_arg = CAP ? 2.0f * LOG2E * a.scale / a.softcap : 0.0f;
    const float cap_l2 = CAP ? a.softcap * LOG2E : 0.0f;
    const float two_cap_l2 = 2.0f * cap_l2;

    int kt_lo = 0, kt_hi = -1;
    if (lo_blk <= hi_blk) { kt_lo = lo_blk / BN; kt_hi = hi_blk / BN; }

    // per-thread offsets of its LPT (row, chunk) pieces of a tile: in global
    // memory (elements, relative to the tile's first row) and in LDS (bytes)
    int ld_off[LPT], ld_row[LPT], st_k[LPT], st_v[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int idx = tid + 256 * i;
        const int r = idx / CPR, c = idx % CPR;
        ld_row[i] = r;
        ld_off[i] = r * (int)kv_stride + c * 8;
        st_k[i] = r * L::KS + c * 16;
        st_v[i] = L::KT + r * L::VS + c * 16;
    }
    // per-lane LDS read bases (bytes within a stage)
    //  K (A operand): row 32 kb + lq, chunk 2 ks + h2
    const int rd_k = lq * L::KS + h2 * 16;
    //  V (transposing read): rows 32 kb + 16 hh + 4 h2 + j/4 (+8), 16 d-columns
    //  32 db + 16 (group & 1) + 4 (j & 3) .. +3
    const int grp16 = lane >> 4, j16 = lane & 15;
    const int rd_v = L::KT + (h2 * 4 + (j16 >> 2)) * L::VS + (grp16 & 1) * 32 + (j16 & 3) * 8;

    u32x4_t kreg[LPT], vreg[LPT];
    int t = kt_lo;
    if (MASK) while (t <= kt_hi && words[t] == 0ull) ++t;

    if (t <= kt_hi) {
        // prologue: first tile into stage 0
        {
            const int64_t tb = (int64_t)t * BN * kv_stride;
            const bool full = t * BN + BN <= a.Lk;
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                int off = ld_off[i];
                if (!full && t * BN + ld_row[i] >= a.Lk) off -= (t * BN + ld_row[i] - (a.Lk - 1)) * (int)kv_stride;
                kreg[i] = *reinterpret_cast<const u32x4_t*>(kbase + tb + off);
                vreg[i] = *reinterpret_cast<const u32x4_t*>(vbase + tb + off);
            }
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                *reinterpret_cast<u32x4_t*>(smem + st_k[i]) = kreg[i];
                *reinterpret_cast<u32x4_t*>(smem + st_v[i]) = vreg[i];
            }
        }
        __syncthreads();

        int cur = 0;
        while (true) {
            int tn = t + 1;
            if (MASK) while (tn <= kt_hi && words[tn] == 0ull) ++tn;
            const bool more = tn <= kt_hi;
            if (more) {
                const int64_t tb = (int64_t)tn * BN * kv_stride;
                const bool full = tn * BN + BN <= a.Lk;
#pragma unroll
                for (int i = 0; i < LPT; ++i) {
                    int off = ld_off[i];
                    if (!full && tn * BN + ld_row[i] >= a.Lk)
                        off -= (tn * BN + ld_row[i] - (a.Lk - 1)) * (int)kv_stride;  // clamp; masked below
                    kreg[i] = *reinterpret_cast<const u32x4_t*>(kbase + tb + off);
                    vreg[i] = *reinterpret_cast<const u32x4_t*>(vbase + tb + off);
                }
            }
            const char* stage = smem + cur * L::BUF;

            const int k0 = t * BN;
            const uint64_t word = MASK ? words[t] : ~0ull;
            // uniform across the wave: every row of the wave sees every key of the tile
            const bool interior = __builtin_amdgcn_readfirstlane(
                (k0 >= wlo_last && k0 + BN - 1 <= whi_first && (!MASK || word == ~0ull)) ? 1 : 0);

            // ---- S^T = K Q^T for two 32-key blocks
            f32x16_t sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const v8 kop = bitcast<v8>(
                        *reinterpret_cast<const u32x4_t*>(stage + rd_k + kb * 32 * L::KS + ks * 32));
                    sacc[kb] = Mfma<T>::mma32(kop, qop[ks], sacc[kb]);
                }
            }

            // ---- scores: sacc[kb][4 j + i] is key k0 + 32 kb + 8 j + 4 h2 + i of row qrow.
            // Without a cap the base-2 logit is s * c_log2, folded into the exponent below;
            // with a cap it is cap*log2e - 2 cap*log2e / (2^(2 log2e s scale / cap) + 1).
            float x[32];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = sacc[kb][e];
                    if (CAP) v = cap_l2 - two_cap_l2 * fast_rcp(fast_exp2(v * cap_arg) + 1.0f);
                    x[kb * 16 + e] = v;
                }
            if (!interior) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int kk = kb * 32 + (e >> 2) * 8 + h2 * 4 + (e & 3);
                        const int key = k0 + kk;
                        bool vis = key >= rlo && key <= rhi;
                        if (MASK) vis = vis && ((word >> kk) & 1ull);
                        x[kb * 16 + e] = vis ? x[kb * 16 + e] : -INFINITY;
                    }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 32; e += 2) tmax = fmax_fast(fmax_fast(tmax, x[e]), x[e + 1]);
            tmax = fmax_fast(tmax, __shfl_xor(tmax, 32));
            const float tmax_l2 = CAP ? tmax : tmax * c_log2;   // base-2 logit units

            // Lazy rescale: the running max only moves when a tile's max exceeds
            // it by more than 8 (base 2), so every weight 2^(x - m) stays <= 256
            // and the accumulator is rescaled rarely.  Exact after O = acc / l.
            const bool grow = tmax_l2 > m + 8.0f;
            if (__any(grow)) {
                // rows that do not grow keep alpha = 1 (m may still be -inf there)
                const float alpha = grow ? fast_exp2(m - tmax_l2) : 1.0f;   // 0 when m = -inf
                m = grow ? tmax_l2 : m;
                l *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            }
            const float m_use = m == -INFINITY ? 0.0f : m;
            float psum = 0.0f;
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                x[e] = CAP ? fast_exp2(x[e] - m_use) : fast_exp2(fmaf(x[e], c_log2, -m_use));
                psum += x[e];
            }
            l += psum;

            // ---- O^T += V^T P^T, four 16-key steps
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int kb = st >> 1, hh = st & 1;
                float pv[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[i] = x[kb * 16 + (2 * hh) * 4 + i];
                    pv[4 + i] = x[kb * 16 + (2 * hh + 1) * 4 + i];
                }
                const v8 pop = pack8<T>(pv);
                const char* vb = stage + rd_v + (kb * 32 + hh * 16) * L::VS;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const i16x4_t lo4 = lds_read_tr16(vb + db * 64);
                    const i16x4_t hi4 = lds_read_tr16(vb + 8 * L::VS + db * 64);
                    const i16x8_t vv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                    oacc[db] = Mfma<T>::mma32(bitcast<v8>(vv), pop, oacc[db]);
                }
            }

            if (more) {
                char* nstage = smem + (cur ^ 1) * L::BUF;
#pragma unroll
                for (int i = 0; i < LPT; ++i) {
                    *reinterpret_cast<u32x4_t*>(nstage + st_k[i]) = kreg[i];
                    *reinterpret_cast<u32x4_t*>(nstage + st_v[i]) = vreg[i];
                }
            }
            __syncthreads();
            if (!more) break;
            cur ^= 1;
            t = tn;
        }
    }

    // ---- epilogue: normalise, round, store; LSE in natural log
    l += __shfl_xor(l, 32);
    if (qrow <= i_last) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        T* orow = static_cast<T*>(a.out) + ((int64_t)b * a.Lq + qrow) * q_stride + (int64_t)hq * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // oacc[db][4 j + i] is column d = 32 db + 8 j + 4 h2 + i
                T o4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = static_cast<T>(oacc[db][4 * j + i] * inv);
                *reinterpret_cast<uint2*>(orow + db * 32 + j * 8 + h2 * 4) = *reinterpret_cast<const uint2*>(o4);
            }
        }
        if (a.lse && h2 == 0)
            a.lse[((int64_t)b * a.Hq + hq) * a.Lq + qrow] =
                l > 0.0f ? (m + log2f(l)) * 0.6931471805599453f : -INFINITY;
    }
}

template <typename T, int D, bool CAP, bool MASK>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    const int nqt = (a.Lq + BM - 1) / BM;
    const int64_t blocks = (int64_t)a.B * a.Hq * nqt;
    hipLaunchKernelGGL((prefill_kernel<T, D, CAP, MASK>), dim3((unsigned)blocks), dim3(256), 0, s, a, nqt);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
    const bool cap = a.softcap > 0.0f, mask = a.key_mask != nullptr;
    if (cap) return mask ? launch_t<T, D, true, true>(a, s) : launch_t<T, D, true, false>(a, s);
    return mask ? launch_t<T, D, false, true>(a, s) : launch_t<T, D, false, false>(a, s);
}

}  // namespace

bool mfma_prefill_supported(int dtype, int D) {
    return (dtype == kBF16 || dtype == kF16) && (D == 64 || D == 128);
}

hipError_t launch_mfma_prefill(const FwdArgs& a, int dtype, hipStream_t s) {
    if ((int64_t)a.B * a.Hq * ((a.Lq + BM - 1) / BM) > 0x7fffffff) return hipErrorInvalidValue;
    if (dtype == kBF16) return a.D == 64 ? launch_d<__bf16, 64>(a, s) : launch_d<__bf16, 128>(a, s);
    if (dtype == kF16) return a.D == 64 ? launch_d<_Float16, 64>(a, s) : launch_d<_Float16, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace mfa
