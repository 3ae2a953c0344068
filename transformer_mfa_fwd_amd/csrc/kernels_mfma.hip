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
// copied straight from HBM into XOR-swizzled LDS (global_load_lds_dwordx4, no
// register staging), two stages each.  Per wave and tile:
//   S^T[32 keys x 32 q] = K . Q^T            v_mfma_f32_32x32x16, Q^T in VGPRs
//     -> lane l holds 16 keys of query row (l % 32): the row max is an in-lane
//        max plus one exchange with lane l ^ 32
//   O^T[32 d x 32 q] += V^T . P^T            v_mfma_f32_32x32x16; P^T is the
//        score accumulator (rounded to the input type), V^T comes from the
//        transposing LDS read, so no score ever leaves the registers.
// The next tile's copy is in flight while the current one is computed; the
// two workgroups resident per CU interleave softmax (VALU) with MFMA work.
//
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

// LDS layout of one stage: K tile then V tile, each [BN rows][D] of 16-bit
// elements stored as 16-byte chunks, row-major without padding (a direct
// global->LDS load writes 1 KiB contiguously per wave instruction).  The
// chunk index is XOR-swizzled with row bits:
//  - K: 32 lanes read one chunk from 32 consecutive rows; XOR with the row's
//    low bits spreads 16 rows over all 64 banks.
//  - V: a transposing read takes 64 bytes from each of 4 consecutive rows per
//    half wave; XOR moves those rows into different 64-byte bank groups.
template <int D> struct PfLds {
    static constexpr int CPR = D / 8;             // chunks per row
    static constexpr int RS = D * 2;              // row bytes
    static constexpr int TILE = BN * RS;          // one K or V tile
    static constexpr int KST = 0;                 // K stage s at KST + s * TILE
    static constexpr int VST = 2 * TILE;          // V stage s at VST + s * TILE
    static constexpr int BYTES = 4 * TILE;
    static __device__ inline int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
    static __device__ inline int swz_v(int row) { return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }
};

__device__ inline int remap_xcd(int p, int n) {
    const int per = n / 8;
    if (p < per * 8) return (p % 8) * per + p / 8;
    return p;
}

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int QK_LA = 4;  // K fragment reads in flight ahead of the MFMA

// fragment f = (key block f / nks, k-step f % nks); compile-time f after unrolling
template <int RS, int NKS>
__device__ inline void mfa_qk_issue(u32x4_t (&kf)[2 * NKS], const uint32_t (&ka)[NKS], int f) {
    const int kb = f / NKS, ks = f % NKS;
    if (kb == 0) lds_read_b128_asm<0>(kf[f], ka[ks]);
    else lds_read_b128_asm<32 * RS>(kf[f], ka[ks]);
}
template <int LA, int NF>
__device__ inline void mfa_qk_wait(u32x4_t (&kf)[NF], int f) {
    // reads issued so far: min(NF, f + LA); those after f may stay in flight
    const int after = (f + LA < NF ? f + LA : NF) - f - 1;
    switch (after) {
        case 0: lds_wait_b128<0>(kf[f]); break;
        case 1: lds_wait_b128<1>(kf[f]); break;
        case 2: lds_wait_b128<2>(kf[f]); break;
        default: lds_wait_b128<3>(kf[f]); break;
    }
}

template <typename T, int D, bool CAP, bool MASK>
__global__ __launch_bounds__(256, 2) void prefill_kernel(FwdArgs a, int nqt) {
    typedef PfLds<D> L;
    constexpr int CPR = L::CPR;
    constexpr int NKS = D / 16;             // k-steps of Q.K^T
    constexpr int NDB = D / 32;             // 32-wide d blocks of O
    constexpr int RPI = 64 / CPR;           // tile rows per DMA instruction
    constexpr int IPW = BN / RPI / 4;       // DMA instructions per wave per tile
    typedef typename Mfma<T>::v8 v8;
    constexpr float LOG2E = 1.4426950408889634f;

    __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lq = lane & 31;               // query row within the wave
    const int h2 = lane >> 5;               // lane half
    const int grp16 = lane >> 4, j16 = lane & 15;

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

    // ---- DMA: instruction i of this wave fills tile rows R..R+RPI-1,
    // R = (wave * IPW + i) * RPI; lane -> physical (row, chunk), fetching the
    // logical chunk that the swizzle stores there.
    int dma_row[IPW], dma_koff[IPW], dma_voff[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int r = (wave * IPW + i) * RPI + lane / CPR;
        const int pc = lane % CPR;
        dma_row[i] = r;
        dma_koff[i] = r * (int)kv_stride + (pc ^ L::swz_k(r)) * 8;
        dma_voff[i] = r * (int)kv_stride + (pc ^ L::swz_v(r)) * 8;
    }
    // per-lane LDS read offsets (bytes, within a K or V tile)
    //  K (A operand): row 32 kb + lq, logical chunk 2 ks + h2
    int rd_k[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) rd_k[ks] = lq * L::RS + (((2 * ks + h2) ^ L::swz_k(lq)) * 16);
    //  V (transposing read): rows 32 kb + 16 hh + 4 h2 + j/4 (and +8),
    //  d columns 32 db + 16 (group & 1) + 4 (j & 3) .. +3
    int rd_v[NDB];
    {
        const int r0 = h2 * 4 + (j16 >> 2);  // row within the 16-row step (low bits fix the swizzle)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int chunk = db * 4 + (grp16 & 1) * 2 + ((j16 & 3) >> 1);
            rd_v[db] = r0 * L::RS + ((chunk ^ L::swz_v(r0)) * 16) + (j16 & 1) * 8;
        }
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

// next tile at or after x that has a visible key
#define MFA_NEXT_TILE(x) ({ int _t = (x); if (MASK) while (_t <= kt_hi && words[_t] == 0ull) ++_t; _t; })

// copy K (and/or V) rows of tile TT into stage STG with direct global->LDS loads
#define MFA_DMA(TT, STG, DO_K, DO_V)                                                         \
    do {                                                                                     \
        const int _t = (TT);                                                                 \
        const int64_t _tb = (int64_t)_t * BN * kv_stride;                                    \
        const bool _full = _t * BN + BN <= a.Lk;                                             \
        _Pragma("unroll") for (int i = 0; i < IPW; ++i) {                                    \
            int _clamp = 0;                                                                  \
            if (!_full && _t * BN + dma_row[i] >= a.Lk)                                      \
                _clamp = (_t * BN + dma_row[i] - (a.Lk - 1)) * (int)kv_stride;               \
            char* _dst = smem + (wave * IPW + i) * 1024;                                     \
            if (DO_K)                                                                        \
                __builtin_amdgcn_global_load_lds((const void*)(kbase + _tb + dma_koff[i] - _clamp), \
                    (lds_void_t*)(_dst + L::KST + (STG) * L::TILE), 16, 0, 0);               \
            if (DO_V)                                                                        \
                __builtin_amdgcn_global_load_lds((const void*)(vbase + _tb + dma_voff[i] - _clamp), \
                    (lds_void_t*)(_dst + L::VST + (STG) * L::TILE), 16, 0, 0);               \
        }                                                                                    \
    } while (0)

// S^T = K Q^T for the two 32-key blocks of the K tile in stage STG.  The
// 2*NKS K fragments are read through a rolling window of QK_LA reads in
// flight, each MFMA waiting only for its own fragment.
#define MFA_QK(SACC, STG)                                                                    \
    do {                                                                                     \
        uint32_t _ka[NKS];                                                                   \
        _Pragma("unroll") for (int ks = 0; ks < NKS; ++ks)                                   \
            _ka[ks] = lds_base + L::KST + (STG) * L::TILE + rd_k[ks];                        \
        u32x4_t _kf[2 * NKS];                                                                \
        _Pragma("unroll") for (int f = 0; f < QK_LA; ++f) mfa_qk_issue<L::RS, NKS>(_kf, _ka, f); \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                     \
            _Pragma("unroll") for (int e = 0; e < 16; ++e) SACC[kb][e] = 0.0f;              \
        _Pragma("unroll") for (int f = 0; f < 2 * NKS; ++f) {                                \
            mfa_qk_wait<QK_LA, 2 * NKS>(_kf, f);                                             \
            if (f + QK_LA < 2 * NKS) mfa_qk_issue<L::RS, NKS>(_kf, _ka, f + QK_LA);         \
            SACC[f / NKS] = Mfma<T>::mma32(bitcast<v8>(_kf[f]), qop[f % NKS], SACC[f / NKS]); \
        }                                                                                    \
    } while (0)

// transposing reads of V for 16-key step S (rows 16 S .. 16 S + 15 of the tile)
#define MFA_TR_ISSUE(S, LO, HI)                                                              \
    do {                                                                                     \
        if constexpr (NDB == 4)                                                              \
            lds_read_tr16_pair4<(S) * 16 * L::RS, (S) * 16 * L::RS + 8 * L::RS>(vaddr, LO, HI); \
        else                                                                                 \
            lds_read_tr16_pair2<(S) * 16 * L::RS, (S) * 16 * L::RS + 8 * L::RS>(vaddr, LO, HI); \
    } while (0)

    const uint32_t lds_base = lds_offset(smem);
    int tcur = MFA_NEXT_TILE(kt_lo);
    if (tcur <= kt_hi) {
        // prologue: K,V of the first tile into stage 0
        MFA_DMA(tcur, 0, true, true);
        __syncthreads();

        int st = 0;       // stage of tile tcur
        while (true) {
            const int tnext = MFA_NEXT_TILE(tcur + 1);
            const bool more = tnext <= kt_hi;
            // DMA: K,V of the next tile into the other stage (read two steps ago)
            if (more) MFA_DMA(tnext, st ^ 1, true, true);

            f32x16_t scur[2];
            MFA_QK(scur, st);

            // ---- scores -> weights (VALU)
            const int k0 = tcur * BN;
            const uint64_t word = MASK ? words[tcur] : ~0ull;
            const bool interior = __builtin_amdgcn_readfirstlane(
                (k0 >= wlo_last && k0 + BN - 1 <= whi_first && (!MASK || word == ~0ull)) ? 1 : 0);

            // scur[kb][4 j + i] is key k0 + 32 kb + 8 j + 4 h2 + i of row qrow.
            // Without a cap the base-2 logit is s * c_log2, folded into the
            // exponent below; with a cap it is
            // cap*log2e - 2 cap*log2e / (2^(2 log2e s scale / cap) + 1).
            float x[32];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = scur[kb][e];
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

            // ---- O^T += V^T P^T, four 16-key steps over V stage st.  The
            // transposing reads of step s+1 are in flight while step s runs on
            // the matrix cores.
            {
                uint32_t vaddr[NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db) vaddr[db] = lds_base + L::VST + st * L::TILE + rd_v[db];
                i16x4_t vlo[2][NDB], vhi[2][NDB];
                MFA_TR_ISSUE(0, vlo[0], vhi[0]);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int kb = s4 >> 1, hh = s4 & 1;
                    float pv[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pv[i] = x[kb * 16 + (2 * hh) * 4 + i];
                        pv[4 + i] = x[kb * 16 + (2 * hh + 1) * 4 + i];
                    }
                    const v8 pop = pack8<T>(pv);
                    lds_wait<NDB>(vlo[s4 & 1], vhi[s4 & 1]);
                    if (s4 == 0) MFA_TR_ISSUE(1, vlo[1], vhi[1]);
                    if (s4 == 1) MFA_TR_ISSUE(2, vlo[0], vhi[0]);
                    if (s4 == 2) MFA_TR_ISSUE(3, vlo[1], vhi[1]);
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const i16x4_t lo4 = vlo[s4 & 1][db], hi4 = vhi[s4 & 1][db];
                        const i16x8_t vv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                        oacc[db] = Mfma<T>::mma32(bitcast<v8>(vv), pop, oacc[db]);
                    }
                }
            }

            __syncthreads();  // DMA of this step landed; stage st free for reuse
            if (!more) break;
            tcur = tnext;
            st ^= 1;
        }
    }
#undef MFA_NEXT_TILE
#undef MFA_DMA
#undef MFA_QK
#undef MFA_TR_ISSUE

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
