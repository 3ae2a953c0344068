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

// swizzle of a [BN][D] tile for the K pattern (32 rows, same chunk) and the
// V pattern (transposing reads of 4 rows x 4 chunks per half wave)
template <int D>
__device__ inline int pf_swz_k(int row, int chunk) {
    return D == 128 ? (chunk ^ (row & 15)) : (chunk ^ ((row >> 1) & 7));
}
template <int D>
__device__ inline int pf_swz_v(int row, int chunk) {
    return D == 128 ? (chunk ^ ((row & 3) << 2)) : (chunk ^ (((row >> 1) & 1) << 2));
}

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

    __shared__ u32x4_t sK[2][BN * CPR];
    __shared__ u32x4_t sV[2][BN * CPR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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

    const float c_log2 = a.score_to_log2;
    const float two_log2e_over_cap = CAP ? 2.0f * LOG2E / a.softcap : 0.0f;

    int kt_lo = 0, kt_hi = -1;
    if (lo_blk <= hi_blk) { kt_lo = lo_blk / BN; kt_hi = hi_blk / BN; }

    u32x4_t kreg[LPT], vreg[LPT];
    int t = kt_lo;
    if (MASK) while (t <= kt_hi && words[t] == 0ull) ++t;

    // prologue: first tile into buffer 0
    if (t <= kt_hi) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / CPR, c = idx % CPR;
            int key = t * BN + r;
            key = key < a.Lk ? key : a.Lk - 1;
            const int64_t off = (int64_t)key * kv_stride + c * 8;
            kreg[i] = *reinterpret_cast<const u32x4_t*>(kbase + off);
            vreg[i] = *reinterpret_cast<const u32x4_t*>(vbase + off);
        }
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / CPR, c = idx % CPR;
            sK[0][r * CPR + pf_swz_k<D>(r, c)] = kreg[i];
            sV[0][r * CPR + pf_swz_v<D>(r, c)] = vreg[i];
        }
    }
    __syncthreads();

    int cur = 0;
    while (t <= kt_hi) {
        int tn = t + 1;
        if (MASK) while (tn <= kt_hi && words[tn] == 0ull) ++tn;
        const bool more = tn <= kt_hi;
        if (more) {
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const int idx = tid + 256 * i;
                const int r = idx / CPR, c = idx % CPR;
                int key = tn * BN + r;
                key = key < a.Lk ? key : a.Lk - 1;
                const int64_t off = (int64_t)key * kv_stride + c * 8;
                kreg[i] = *reinterpret_cast<const u32x4_t*>(kbase + off);
                vreg[i] = *reinterpret_cast<const u32x4_t*>(vbase + off);
            }
        }

        const int k0 = t * BN;
        const uint64_t word = MASK ? words[t] : ~0ull;
        const bool interior = k0 >= wlo_last && k0 + BN - 1 <= whi_first && (!MASK || word == ~0ull);

        // ---- S^T = K Q^T for two 32-key blocks
        f32x16_t sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
            const int r = kb * 32 + lq;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const v8 kop = bitcast<v8>(sK[cur][r * CPR + pf_swz_k<D>(r, ks * 2 + h2)]);
                sacc[kb] = Mfma<T>::mma32(kop, qop[ks], sacc[kb]);
            }
        }

        // ---- scores -> base-2 logits, masking, running max
        // sacc[kb][4 j + i] is key k0 + 32 kb + 8 j + 4 h2 + i of row qrow
        float x[32];
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float v = sacc[kb][e];
                if (CAP) v = softcap_apply(v * a.scale, a.softcap, two_log2e_over_cap) * LOG2E;
                else v = v * c_log2;
                if (!interior) {
                    const int kk = kb * 32 + (e >> 2) * 8 + h2 * 4 + (e & 3);
                    const int key = k0 + kk;
                    bool vis = key >= rlo && key <= rhi;
                    if (MASK) vis = vis && ((word >> kk) & 1ull);
                    v = vis ? v : -INFINITY;
                }
                x[kb * 16 + e] = v;
                tmax = fmaxf(tmax, v);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m - m_use);
        m = m_new;
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            x[e] = fast_exp2(x[e] - m_use);
            psum += x[e];
        }
        l = l * alpha + psum;
        // rescale the accumulator only when some row's max moved
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        }

        // ---- O^T += V^T P^T, four 16-key steps
        const int grp16 = lane >> 4;        // 16-lane group
        const int j16 = lane & 15;          // source lane within the group
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
            const int r0 = kb * 32 + hh * 16 + h2 * 4 + (j16 >> 2);
            const int r1 = r0 + 8;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int chunk = db * 4 + (grp16 & 1) * 2 + ((j16 & 3) >> 1);
                const int half = (j16 & 1) * 8;
                const char* p0 = reinterpret_cast<const char*>(&sV[cur][r0 * CPR + pf_swz_v<D>(r0, chunk)]) + half;
                const char* p1 = reinterpret_cast<const char*>(&sV[cur][r1 * CPR + pf_swz_v<D>(r1, chunk)]) + half;
                const i16x4_t lo4 = lds_read_tr16(p0);
                const i16x4_t hi4 = lds_read_tr16(p1);
                const i16x8_t vv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                oacc[db] = Mfma<T>::mma32(bitcast<v8>(vv), pop, oacc[db]);
            }
        }

        if (more) {
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const int idx = tid + 256 * i;
                const int r = idx / CPR, c = idx % CPR;
                sK[cur ^ 1][r * CPR + pf_swz_k<D>(r, c)] = kreg[i];
                sV[cur ^ 1][r * CPR + pf_swz_v<D>(r, c)] = vreg[i];
            }
        }
        __syncthreads();
        cur ^= 1;
        t = tn;
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
