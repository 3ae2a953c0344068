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
//
// Software pipeline.  Iteration j of a wave issues the Q.K^T MFMAs of tile
// j+1 and, between them, the softmax of tile j (masking, row max, rescale,
// the first quarter of the exponentials); then the P.V MFMAs of tile j and,
// between them, the rest of tile j's exponentials and its row sum.  Each MFMA
// (32 cycles on the matrix core) thus has independent VALU work behind it,
// and the matrix core is never idle while the softmax runs.  The copies of
// K(j+2) and V(j+1) are in flight during iteration j; one barrier per
// iteration hands the stages over.
//
// Only tiles that intersect the key range of the workgroup's rows are visited
// (causal and window bounds), tiles whose key-mask word is zero are skipped
// without loading K or V, and per-element masking runs only on tiles that are
// not fully visible to every row of the wave.
//
// Scheduling.  Blocks are ordered so that the Hq/Hkv heads sharing a kv head
// and q tile are adjacent (they read the same K/V tiles together) and, over
// the up to 4 kv heads that one XCD serves at a time, the heaviest causal
// tiles go first; the block id is remapped so that each of the 8 XCDs
// (round-robin dispatch, one L2 each) receives a contiguous range of that
// order.
#include "mfa_device.h"
#include "mfa_internal.h"

#include <math.h>

#include <type_traits>

namespace mfa {
namespace {

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile

// LDS layout: two K stages then two V stages, each [BN rows][D] of 16-bit
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

// source of one K or V tile: first row and byte range up to key Lk - 1
struct TileSrc {
    const void* p;
    int n;
};

__device__ inline int remap_xcd(int p, int n) {
    const int per = n / 8;
    if (p < per * 8) return (p % 8) * per + p / 8;
    return p;
}

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int QK_LA = 4;  // K fragment reads in flight ahead of the MFMA

// K fragment f = (key block f & 1, k-step f >> 1): consecutive MFMAs alternate
// between the two score accumulators.  f is a compile-time constant after
// unrolling.
template <int RS, int BASE>
__device__ inline void mfa_qk_issue(u32x4_t* kf, const uint32_t* rd_k, int f) {
    if ((f & 1) == 0) lds_read_b128_asm<BASE>(kf[f], rd_k[f >> 1]);
    else lds_read_b128_asm<BASE + 32 * RS>(kf[f], rd_k[f >> 1]);
}
// Wait for K fragment f.  Reads issued after it may stay in flight: the K
// reads up to f + LA and, once f > XF, the XN reads issued behind K read
// XF + LA (LDS reads of a wave complete in order).
template <int LA, int NF, int XF, int XN>
__device__ inline void mfa_qk_wait(u32x4_t* kf, int f) {
    const int after = (f + LA < NF ? f + LA : NF) - f - 1 + (f > XF ? XN : 0);
    switch (after) {
        case 0: lds_wait_b128<0>(kf[f]); break;
        case 1: lds_wait_b128<1>(kf[f]); break;
        case 2: lds_wait_b128<2>(kf[f]); break;
        case 3: lds_wait_b128<3>(kf[f]); break;
        case 4: lds_wait_b128<4>(kf[f]); break;
        case 5: lds_wait_b128<5>(kf[f]); break;
        case 6: lds_wait_b128<6>(kf[f]); break;
        case 7: lds_wait_b128<7>(kf[f]); break;
        case 8: lds_wait_b128<8>(kf[f]); break;
        case 9: lds_wait_b128<9>(kf[f]); break;
        case 10: lds_wait_b128<10>(kf[f]); break;
        default: lds_wait_b128<11>(kf[f]); break;
    }
}

// Bits lo..hi (clipped to 0..63) set; zero when the range is empty.
__device__ inline uint64_t range_bits64(int lo, int hi) {
    lo = lo < 0 ? 0 : lo;
    hi = hi > 63 ? 63 : hi;
    if (lo > hi) return 0ull;
    return (~0ull << lo) & (~0ull >> (63 - hi));
}

// ---- bf16 inputs: fp16 operands for P.V.  Rounding a weight to bf16 keeps 8
// significant bits, which on std-2 data costs up to about 0.03 in O (V up to
// ~9, two comparable weights); fp16 keeps 11.  The MFMA needs both operands
// in one type, so V is converted to fp16 once per call by v16_prepass_kernel
// (exact below 65504 in magnitude: bf16 has fewer significant bits), and the
// prefill reads that copy.  A (batch, kv head) whose V holds a magnitude of
// 65504 or more (or an infinity) is flagged and its blocks run on bf16
// operands from the original V.  Converting in the prefill instead, once per
// workgroup and tile, measured 14 % slower on the causal GQA prefill: every V
// tile is read by ~32 workgroups there.

// One dword of two bf16 values as two fp16 values (round to nearest even,
// exact below 65504 in magnitude); their magnitudes are folded into mx.
__device__ inline uint32_t cvt_bf16x2_f16x2(uint32_t x, float& mx) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xffff0000u);
    mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(__builtin_fabsf(lo), __builtin_fabsf(hi)));
    const h2 r = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(uint32_t, r);
}

// The work of one workgroup: its 128 query rows of one query head, from
// the first copies to the stores.  With CV (bf16 inputs, a.v16 holding V
// converted to fp16) P.V runs on fp16 operands; it returns false, having
// written nothing to global memory, when the block's (batch, kv head) is
// flagged, and the caller then runs it with CV off.  smem: the kernel's LDS
// (L::BYTES bytes, 1024-byte aligned).
template <typename T, int D, bool CAP, bool MASK, bool SEQ, bool BIAS, bool DROP, bool CV>
__device__ __attribute__((always_inline)) inline bool prefill_block(const FwdArgs& a, int nqt, char* smem) {
    typedef PfLds<D> L;
    constexpr int CPR = L::CPR;
    constexpr int NKS = D / 16;             // k-steps of Q.K^T
    constexpr int NQK = 2 * NKS;            // Q.K^T MFMAs per tile
    constexpr int NDB = D / 32;             // 32-wide d blocks of O
    constexpr int RPI = 64 / CPR;           // tile rows per DMA instruction
    constexpr int IPW = BN / RPI / 4;       // DMA instructions per wave per tile
    constexpr bool LOGIT = CAP || BIAS;     // scores turned into base-2 logits before the max
    // With a cap and no additive mask the logit cap*log2e - 2 cap*log2e * r,
    // r = 1 / (2^(2 log2e s scale / cap) + 1), falls as r grows: the scores
    // are kept as r (a hidden one as +inf), the row's largest logit comes from
    // its smallest r, and the last fma of the cap joins the exponential's
    // argument, 2^(fma(r, -2 cap log2e, cap log2e - m)): one instruction per
    // score fewer.
    constexpr bool RDOM = CAP && !BIAS;
    constexpr int NSA = LOGIT ? 13 : 9;     // softmax steps run beside Q.K^T
    // K fragment reads in flight: two with an additive mask (its next tile's
    // values take 32 registers) or dropout, so that those kernels, at two
    // workgroups per CU, spill little: a spill's reload in the loop waits for
    // every copy in flight (vector memory completes in order)
    constexpr int QKLA = (BIAS || DROP) ? 2 : QK_LA;
    constexpr int TRS = NQK - QKLA;         // slot issuing the first V reads
    static_assert(TRS > 0 && TRS + QKLA == NQK, "V reads follow the last K read");
    typedef typename Mfma<T>::v8 v8;
    constexpr float LOG2E = 1.4426950408889634f;
    // CV: P.V on fp16 operands (see cvt_bf16x2_f16x2)
    typedef typename std::conditional<CV, _Float16, T>::type PT;   // P.V operand type
    typedef typename Mfma<PT>::v8 pv8;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lq = lane & 31;               // query row within the wave
    const int h2 = lane >> 5;               // lane half
    const int grp16 = lane >> 4, j16 = lane & 15;

    // ---- block -> (batch, kv head, q tile, q head)
    // Blocks come in chunks of KG kv heads (all of one XCD's share when it
    // holds up to 4); within a chunk the latest q tile (largest causal key
    // range) of every head comes first.
    const int n = remap_xcd(blockIdx.x, gridDim.x);
    const int g = a.group;
    const int per_group = g * nqt;
    const int nbk = a.B * a.Hkv;
    const int per_xcd = (nbk & 7) == 0 ? nbk >> 3 : 1;
    const int KG = (per_xcd & 3) == 0 ? 4 : ((per_xcd & 1) == 0 ? 2 : 1);
    const int chunk = n / (KG * per_group);
    const int rem = n - chunk * KG * per_group;
    const int lvl = rem / (KG * g);
    const int rest = rem - lvl * KG * g;
    const int bk = chunk * KG + rest / g;   // b * Hkv + kvh
    const int qt = nqt - 1 - lvl;
    const int b = bk / a.Hkv;
    const int kvh = bk - b * a.Hkv;
    const int hq = kvh * g + (rest % g);

    const int i0 = qt * BM;
    const int i_last = min(i0 + BM, a.Lq) - 1;
    const int w_first = i0 + wave * 32;
    const int w_last = min(w_first + 31, i_last);
    const int qrow = w_first + lq;

    // key ranges: workgroup (tiles to visit), wave (interior test), lane (mask)
    int lo_blk, hi_tmp, lo_tmp, hi_blk;
    row_key_range<SEQ>(a, i0, lo_blk, hi_tmp);
    row_key_range<SEQ>(a, i_last, lo_tmp, hi_blk);
    int wlo_last = a.Lk, whi_first = -1;
    if (w_first <= i_last) {
        int t0, t1;
        row_key_range<SEQ>(a, w_first, t0, whi_first);
        row_key_range<SEQ>(a, w_last, wlo_last, t1);
    }
    int rlo = 1, rhi = 0;
    if (qrow <= i_last) row_key_range<SEQ>(a, qrow, rlo, rhi);

    const int64_t q_stride = a.q_stride;
    const int64_t kv_stride = a.kv_stride;
    const T* __restrict__ qbase = static_cast<const T*>(a.q) + (int64_t)b * a.Lq * q_stride + (int64_t)hq * D;
    const T* __restrict__ kbase = static_cast<const T*>(a.k) + (int64_t)b * a.Lk * kv_stride + (int64_t)kvh * D;
    // CV: V from the fp16 copy (same element offsets as V)
    const PT* __restrict__ vbase = static_cast<const PT*>(CV ? a.v16 : a.v) + (int64_t)b * a.Lk * kv_stride +
                                   (int64_t)kvh * D;
    // CV: a (batch, kv head) whose V could not all be converted runs on bf16
    // operands, and so does a call without the copy.  The first 64 flag
    // words (16384 keys) are loaded here and arrive under the prologue's
    // first barrier; any further ones are read after the loop, where all are
    // tested: a flagged block drops what it computed and is redone (rare: a
    // magnitude of 65504 or more in V).  No loop or branch on the flags comes
    // before the first copies, so their latency overlaps the copies'.
    const uint32_t* v16_fl = nullptr;
    uint32_t v16_any = 0u;
    bool v16_flagged = false;
    if constexpr (CV) {
        if (!a.v16) return false;
        v16_fl = reinterpret_cast<const uint32_t*>(a.v16_flags + (int64_t)bk * a.v16_fwords * 4);
        // unconditional (index clamped, value masked): a branch here would
        // pull the test, and its wait, ahead of the copies
        v16_any = v16_fl[lane < a.v16_fwords ? lane : a.v16_fwords - 1] & (lane < a.v16_fwords ? ~0u : 0u);
    }
    (void)v16_fl; (void)v16_any; (void)v16_flagged;
    // The mask words are read-only while the kernel runs (written by the
    // launch before it): reading them through the constant address space
    // lets the compiler use scalar loads, which the scalar cache serves,
    // instead of vector loads whose latency the next copy would wait on.
    typedef const __attribute__((address_space(4))) uint64_t cword_t;
    cword_t* words = MASK ? (cword_t*)(a.mask_words + (int64_t)b * a.words_per_batch) : nullptr;

    // ---- Q^T operand: lane holds Q[qrow][16 ks + 8 h2 .. +7]
    v8 qop[NKS];
    {
        const int r = qrow <= i_last ? qrow : i_last;
        const T* qp = qbase + (int64_t)r * q_stride + h2 * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4_t raw = *reinterpret_cast<const u32x4_t*>(qp + ks * 16);
            if constexpr (!LOGIT) raw = (raw ^ a.q_xor) & ~a.q_clear;   // scale <= 0: see the launcher
            qop[ks] = bitcast<v8>(raw);
        }
    }

    // ---- DMA: instruction i of this wave fills tile rows R..R+RPI-1,
    // R = (wave * IPW + i) * RPI; lane -> physical (row, chunk), fetching the
    // logical chunk that the swizzle stores there.  Source offsets are byte
    // offsets within the tile, read through a buffer descriptor whose base is
    // the tile's first row and whose range ends at key Lk - 1: rows of a
    // partial last tile past it read as zero (and are masked anyway).
    const int dma_r0 = wave * IPW * RPI + lane / CPR;   // tile row of copy 0
    uint32_t dma_koff[IPW], dma_voff[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int r = dma_r0 + i * RPI;
        const int pc = lane % CPR;
        dma_koff[i] = (uint32_t)(r * (int)kv_stride + (pc ^ L::swz_k(r)) * 8) * 2u;
        dma_voff[i] = (uint32_t)(r * (int)kv_stride + (pc ^ L::swz_v(r)) * 8) * 2u;
    }
    // per-lane LDS read addresses (bytes; stage offsets go in the immediate)
    const uint32_t lds_base = lds_offset(smem);
    //  K (A operand): row 32 kb + lq, logical chunk 2 ks + h2
    uint32_t rd_k[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) rd_k[ks] = lds_base + lq * L::RS + (((2 * ks + h2) ^ L::swz_k(lq)) * 16);
    //  V (transposing read): rows 32 kb + 16 hh + 4 h2 + j/4 (and +8),
    //  d columns 32 db + 16 (group & 1) + 4 (j & 3) .. +3
    uint32_t rd_v[NDB];
    {
        const int r0 = h2 * 4 + (j16 >> 2);  // row within the 16-row step (low bits fix the swizzle)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int chunk = db * 4 + (grp16 & 1) * 2 + ((j16 & 3) >> 1);
            rd_v[db] = lds_base + r0 * L::RS + ((chunk ^ L::swz_v(r0)) * 16) + (j16 & 1) * 8;
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

    // additive mask of this lane's row (rows past the end read the last row);
    // bnx[g] holds the bias of scores 4 g .. 4 g + 3 of the next tile to finish
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    f32x4v bnx[8];
    const float* brow = nullptr;
    if constexpr (BIAS)
        brow = a.bias + b * a.bias_stride[0] + hq * a.bias_stride[1] +
               (int64_t)(qrow <= i_last ? qrow : i_last) * a.bias_stride[2];
    (void)bnx; (void)brow;
// bias of tile TT: group g covers keys TT*BN + 32 (g/4) + 8 (g%4) + 4 h2 .. +3;
// groups at or past key Lk (which the mask clears) read nothing
#define MFA_BIAS_LOAD(TT)                                                                    \
    do {                                                                                     \
        if constexpr (BIAS) {                                                                \
            const int _kb0 = (TT) * BN + 4 * h2;                                             \
            _Pragma("unroll") for (int _g = 0; _g < 8; ++_g) {                               \
                const int _key = _kb0 + 32 * (_g >> 2) + 8 * (_g & 3);                       \
                bnx[_g] = _key < a.Lk ? *reinterpret_cast<const f32x4v*>(brow + _key)         \
                                      : f32x4v{0.0f, 0.0f, 0.0f, 0.0f};                      \
            }                                                                                \
        }                                                                                    \
    } while (0)

// next tile at or after x that has a visible key
#define MFA_NEXT_TILE(x) ({ int _t = (x); if (MASK) while (_t <= kt_hi && words[_t] == 0ull) ++_t; _t; })

// source of tile TT of K or V (BASE): first row of the tile and the byte range
// up to the end of key Lk - 1
#define MFA_RSRC(BASE, TT)                                                                   \
    ({                                                                                       \
        const int _t = (TT);                                                                 \
        const int _rows = min(BN, a.Lk - _t * BN);                                           \
        TileSrc{(const void*)((BASE) + (int64_t)_t * BN * kv_stride),                        \
                (_rows - 1) * (int)kv_stride * 2 + D * 2};                                   \
    })
// copy I (0 .. IPW-1) of a K or V tile (source RS, lane offsets OFF) into the
// LDS tile at byte offset DST
#define MFA_DMA1(RS, OFF, I, DST)                                                            \
    buffer_copy16_to_lds((RS).p, (RS).n, smem + (wave * IPW + (I)) * 1024 + (DST), OFF[I])
// copy I of a V tile; M = MFA_VMASKED(key-mask word of the tile).  With a key
// mask the row of a masked key is read out of range (bit 31 set in its
// offset), so the copy writes zeros there and fetches nothing: its weight is
// zero, and whatever the row holds (never-written memory, NaN) cannot reach O
// through a product with it.  Bit RPI * I of M: this lane's row of copy I is
// masked.  (CV: the fp16 copy of V already holds zeros in those rows.)
#define MFA_VMASKED(W) ((MASK && !CV) ? ~(uint32_t)((W) >> dma_r0) : 0u)
#define MFA_DMAV(RS, I, DST, M)                                                              \
    buffer_copy16_to_lds((RS).p, (RS).n, smem + (wave * IPW + (I)) * 1024 + (DST),           \
                         dma_voff[I] | (((M) >> (RPI * (I))) << 31))
// copy K (and/or V) of tile TT into stage STG
#define MFA_DMA(TT, STG, DO_K, DO_V)                                                         \
    do {                                                                                     \
        if (DO_K) {                                                                          \
            const auto _r = MFA_RSRC(kbase, TT);                                             \
            _Pragma("unroll") for (int i = 0; i < IPW; ++i)                                  \
                MFA_DMA1(_r, dma_koff, i, L::KST + (STG) * L::TILE);                         \
        }                                                                                    \
        if (DO_V) {                                                                          \
            const auto _r = MFA_RSRC(vbase, TT);                                             \
            const uint32_t _m = MFA_VMASKED(MASK ? words[TT] : ~0ull);                       \
            _Pragma("unroll") for (int i = 0; i < IPW; ++i)                                  \
                MFA_DMAV(_r, i, L::VST + (STG) * L::TILE, _m);                               \
        }                                                                                    \
    } while (0)

// transposing reads of V for 16-key step S (rows 16 S .. 16 S + 15 of the V
// tile at LDS byte offset _vb)
#define MFA_TR_ISSUE(S, LO, HI)                                                              \
    do {                                                                                     \
        if constexpr (NDB == 4)                                                              \
            lds_read_tr16_pair4<_vb + (S) * 16 * L::RS, _vb + (S) * 16 * L::RS + 8 * L::RS>(rd_v, LO, HI); \
        else                                                                                 \
            lds_read_tr16_pair2<_vb + (S) * 16 * L::RS, _vb + (S) * 16 * L::RS + 8 * L::RS>(rd_v, LO, HI); \
    } while (0)

// Score i (0..31) of this lane: key k0 + 32 (i / 16) + 8 ((i % 16) / 4) + 4 h2 + i % 4.
#define MFA_X(SC, I) SC[(I) >> 4][(I) & 15]

// Keep bits of this lane's 32 weights of the tile at key K0 (bit i: score i,
// key K0 + 32 (i / 16) + 8 ((i % 16) / 4) + 4 h2 + i % 4).  The tile's 64 keys
// are four 16-key Philox blocks of this lane's row, which lanes l and l ^ 32
// share: each evaluates two (blocks h2 and h2 + 2) and they swap them.
#define MFA_KEEP(K0)                                                                         \
    ({                                                                                       \
        const uint32_t _own = dropout_keep16(a, b, hq, qrow, ((K0) >> 4) + h2) |             \
                              (dropout_keep16(a, b, hq, qrow, ((K0) >> 4) + 2 + h2) << 16);   \
        const uint32_t _oth = (uint32_t)__shfl_xor((int)_own, 32);                           \
        const uint32_t _b02 = h2 ? _oth : _own, _b13 = h2 ? _own : _oth;                     \
        const uint32_t _lo = (_b02 & 0xffffu) | (_b13 << 16);          /* keys 0 .. 31 */    \
        const uint32_t _hi = (_b02 >> 16) | (_b13 & 0xffff0000u);      /* keys 32 .. 63 */   \
        pack_even_nibbles(_lo >> (4 * h2)) | (pack_even_nibbles(_hi >> (4 * h2)) << 16);     \
    })
// zero the dropped weights among scores E0 .. E0 + 7 (after the row sum has them)
#define MFA_DROP8(SC, E0)                                                                    \
    do {                                                                                     \
        if constexpr (DROP) {                                                                \
            _Pragma("unroll") for (int _e = 0; _e < 8; ++_e)                                 \
                MFA_X(SC, (E0) + _e) = (keepw >> ((E0) + _e)) & 1u ? MFA_X(SC, (E0) + _e) : 0.0f; \
        }                                                                                    \
    } while (0)

// the row's extreme over scores (RDOM: the smallest r) and a score's weight
#define MFA_EXT(X, Y) (RDOM ? fmin_fast((X), (Y)) : fmax_fast((X), (Y)))
#define MFA_EXP(X) (RDOM ? fast_exp2(fmaf((X), -two_cap_l2, neg_m))                          \
                         : LOGIT ? fast_exp2((X) + neg_m) : fast_exp2(fmaf((X), c_log2, neg_m)))

// Softmax step U (a constant, 0 .. NSA-1) of the tile whose raw scores are in
// SC.  With a cap the base-2 logit is
// cap*log2e - 2 cap*log2e / (2^(2 log2e s scale / cap) + 1); without one it is
// s * c_log2, folded into the exponent.  Steps: [cap x 4], mask, max x 3,
// max finish + rescale, exponentials of scores 0..7 (two per step).  The other
// 24 exponentials run beside the P.V MFMAs, which leave the VALU idle.
#define MFA_SA(U, SC)                                                                        \
    do {                                                                                     \
        constexpr int _u = (U) - (LOGIT ? 4 : 0);                                            \
        if constexpr (LOGIT && (U) < 4) {                                                    \
            _Pragma("unroll") for (int _e = 0; _e < 8; ++_e) {                               \
                const float _s = MFA_X(SC, 8 * (U) + _e);                                    \
                float _x;                                                                    \
                if constexpr (RDOM) _x = fast_rcp(fast_exp2(_s * cap_arg) + 1.0f);             \
                else if constexpr (CAP) _x = cap_l2 - two_cap_l2 * fast_rcp(fast_exp2(_s * cap_arg) + 1.0f); \
                else _x = _s * c_log2;                                                       \
                /* score i = 8 U + e has its bias in group i / 4, component i % 4 */        \
                if constexpr (BIAS) _x = fmaf(bnx[(8 * (U) + _e) >> 2][(8 * (U) + _e) & 3], LOG2E, _x); \
                MFA_X(SC, 8 * (U) + _e) = _x;                                                \
            }                                                                                \
        } else if constexpr (_u == 0) {                                                      \
            if (!interior) {                                                                 \
                /* bit c of _vis: key k0 + 4 h2 + c visible to this lane's row */           \
                uint64_t _vis = range_bits64(rlo - k0 - 4 * h2, rhi - k0 - 4 * h2);          \
                if (MASK) _vis &= word >> (4 * h2);                                          \
                const int _vlo = (int)(uint32_t)_vis, _vhi = (int)(uint32_t)(_vis >> 32);     \
                _Pragma("unroll") for (int _i = 0; _i < 32; ++_i) {                          \
                    /* all ones when visible (sign-extended bit), then a bit select */      \
                    const int _c = (_i >> 4) * 32 + ((_i & 15) >> 2) * 8 + (_i & 3);          \
                    const uint32_t _mw = (uint32_t)__builtin_amdgcn_sbfe(_c < 32 ? _vlo : _vhi, _c & 31, 1); \
                    MFA_X(SC, _i) = __uint_as_float((__float_as_uint(MFA_X(SC, _i)) & _mw) |  \
                                                    ((RDOM ? 0x7f800000u : 0xff800000u) & ~_mw)); \
                }                                                                            \
            }                                                                                \
        } else if constexpr (_u >= 1 && _u <= 3) {                                           \
            _Pragma("unroll") for (int _d = 0; _d < 4; ++_d) {                               \
                const int _p = 4 * (_u - 1) + _d;                                            \
                if (_p < 10)                                                                 \
                    pm[_p] = MFA_EXT(MFA_EXT(MFA_X(SC, 3 * _p), MFA_X(SC, 3 * _p + 1)), MFA_X(SC, 3 * _p + 2)); \
            }                                                                                \
            if (_u == 3) pm[10] = MFA_EXT(MFA_X(SC, 30), MFA_X(SC, 31));                    \
        } else if constexpr (_u == 4) {                                                      \
            float _t = MFA_EXT(MFA_EXT(MFA_EXT(pm[0], pm[1]), pm[2]),                        \
                               MFA_EXT(MFA_EXT(pm[3], pm[4]), pm[5]));                       \
            _t = MFA_EXT(_t, MFA_EXT(MFA_EXT(pm[6], pm[7]), pm[8]));                         \
            _t = MFA_EXT(MFA_EXT(_t, pm[9]), pm[10]);                                        \
            _t = RDOM ? xor32_min(_t) : xor32_max(_t);                                       \
            /* base-2 logit units (RDOM: the smallest r gives the largest logit) */         \
            const float _tl2 = RDOM ? fmaf(_t, -two_cap_l2, cap_l2) : (LOGIT ? _t : _t * c_log2); \
            /* Lazy rescale: the running max only moves when a tile's max     */            \
            /* exceeds it by more than 8 (base 2), so every weight 2^(x - m)  */            \
            /* stays <= 256 and the accumulator is rescaled rarely.  Exact    */            \
            /* after O = acc / l.  Rows that do not grow keep alpha = 1.      */            \
            const bool _grow = _tl2 > m + 8.0f;                                              \
            if (__any(_grow)) {                                                              \
                const float _alpha = _grow ? fast_exp2(m - _tl2) : 1.0f;  /* 0 when m = -inf */ \
                m = _grow ? _tl2 : m;                                                        \
                l *= _alpha;                                                                 \
                _Pragma("unroll") for (int _db = 0; _db < NDB; ++_db)                        \
                    _Pragma("unroll") for (int _e = 0; _e < 16; ++_e) oacc[_db][_e] *= _alpha; \
            }                                                                                \
            neg_m = m == -INFINITY ? 0.0f : -m;                                              \
            if constexpr (RDOM) neg_m += cap_l2;   /* the exponent's constant: cap log2e - m */ \
        } else {                                                                             \
            _Pragma("unroll") for (int _d = 0; _d < 2; ++_d) {                               \
                const int _e = 2 * (_u - 5) + _d;                                            \
                MFA_X(SC, _e) = MFA_EXP(MFA_X(SC, _e));                                      \
            }                                                                                \
            psum0 += MFA_X(SC, 2 * (_u - 5));                                                \
            psum1 += MFA_X(SC, 2 * (_u - 5) + 1);                                            \
            if constexpr (_u == 8) {                                                         \
                MFA_DROP8(SC, 0);                                                            \
                pop[0] = pack8_at<PT>(SC[0], 0);                                             \
            }                                                                                \
        }                                                                                    \
    } while (0)

// Softmax work beside the P.V MFMAs: quarter U of P.V step S4 (constants).
// S4 = 0, 1, 2: exponentials of scores 8 (S4 + 1) .. +7 and the operand of step
// S4 + 1; the row sum is complete after step 2.
#define MFA_SB(S4, U, SC)                                                                    \
    do {                                                                                     \
        if constexpr ((S4) < 3) {                                                            \
            _Pragma("unroll") for (int _d = 0; _d < 2; ++_d) {                               \
                const int _e = 8 + 8 * (S4) + 2 * (U) + _d;                                  \
                MFA_X(SC, _e) = MFA_EXP(MFA_X(SC, _e));                                      \
            }                                                                                \
            psum0 += MFA_X(SC, 8 + 8 * (S4) + 2 * (U));                                      \
            psum1 += MFA_X(SC, 8 + 8 * (S4) + 2 * (U) + 1);                                  \
            if constexpr ((U) == 3) {                                                        \
                MFA_DROP8(SC, 8 * (1 + (S4)));                                               \
                pop[1 + (S4)] = pack8_at<PT>(SC[(1 + (S4)) >> 1], 8 * ((1 + (S4)) & 1));      \
            }                                                                                \
            if constexpr ((S4) == 2 && (U) == 3) l += psum0 + psum1;                         \
        }                                                                                    \
    } while (0)

// Slot F of the Q.K^T pass (a constant): wait for K fragment F, issue the read
// QK_LA ahead, issue the MFMA, then the softmax steps of SC assigned to this
// slot (SM).  Slot TRS, the first after the last K read is issued, also issues
// the transposing V reads of the first P.V step (SM).
#define MFA_SA_IF(U, F, SC) if constexpr ((U) < ((F) + 1) * NSA / NQK) MFA_SA(U, SC);
// copy J of the iteration (V copies, then K copies) goes in slot J * NQK / (2 IPW)
#define MFA_DMA_IF(F, J)                                                                     \
    if constexpr ((J) < 2 * IPW && (F) == (J) * NQK / (2 * IPW)) {                           \
        if constexpr ((J) < IPW) MFA_DMAV(_rv, (J), _dv_dst, _wv);                           \
        else MFA_DMA1(_rk, dma_koff, (J) - IPW, _dk_dst);                                    \
    }
#define MFA_QK_SLOT(F, SC, SN, SM)                                                           \
    if constexpr ((F) < NQK) {                                                               \
        mfa_qk_wait<QKLA, NQK, (SM) ? TRS : NQK, 2 * NDB>(_kf, (F));                         \
        if constexpr ((F) + QKLA < NQK) mfa_qk_issue<L::RS, _kb>(_kf, rd_k, (F) + QKLA);    \
        if constexpr ((SM) && (F) == TRS) MFA_TR_ISSUE(0, vlo[0], vhi[0]);                  \
        if constexpr (SM) {                                                                  \
            MFA_DMA_IF(F, 0) MFA_DMA_IF(F, 1) MFA_DMA_IF(F, 2) MFA_DMA_IF(F, 3)              \
            MFA_DMA_IF(F, 4) MFA_DMA_IF(F, 5) MFA_DMA_IF(F, 6) MFA_DMA_IF(F, 7)              \
        }                                                                                    \
        SN[(F) & 1] = Mfma<T>::mma32(bitcast<v8>(_kf[F]), qop[(F) >> 1], SN[(F) & 1]);       \
        if constexpr (SM) {                                                                  \
            MFA_SA_IF((F) * NSA / NQK + 0, F, SC)                                            \
            MFA_SA_IF((F) * NSA / NQK + 1, F, SC)                                            \
            MFA_SA_IF((F) * NSA / NQK + 2, F, SC)                                            \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
    }

// Q.K^T of the K tile in stage KSTG into SN, with the softmax steps of SC
// spread over its MFMAs when SM.
#define MFA_PART1(SC, SN, KSTG, SM)                                                          \
    do {                                                                                     \
        constexpr int _kb = L::KST + (KSTG) * L::TILE;                                       \
        u32x4_t _kf[NQK];                                                                    \
        _Pragma("unroll") for (int f = 0; f < QKLA; ++f) mfa_qk_issue<L::RS, _kb>(_kf, rd_k, f); \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                     \
            _Pragma("unroll") for (int e = 0; e < 16; ++e) SN[kb][e] = 0.0f;                \
        MFA_QK_SLOT(0, SC, SN, SM) MFA_QK_SLOT(1, SC, SN, SM)                                \
        MFA_QK_SLOT(2, SC, SN, SM) MFA_QK_SLOT(3, SC, SN, SM)                                \
        MFA_QK_SLOT(4, SC, SN, SM) MFA_QK_SLOT(5, SC, SN, SM)                                \
        MFA_QK_SLOT(6, SC, SN, SM) MFA_QK_SLOT(7, SC, SN, SM)                                \
        MFA_QK_SLOT(8, SC, SN, SM) MFA_QK_SLOT(9, SC, SN, SM)                                \
        MFA_QK_SLOT(10, SC, SN, SM) MFA_QK_SLOT(11, SC, SN, SM)                              \
        MFA_QK_SLOT(12, SC, SN, SM) MFA_QK_SLOT(13, SC, SN, SM)                              \
        MFA_QK_SLOT(14, SC, SN, SM) MFA_QK_SLOT(15, SC, SN, SM)                              \
    } while (0)

// Slot (S4, DB) of the P.V pass (constants): at DB = 0 wait for the V
// fragments of step S4 (step 0's wait comes before the pass) and issue those
// of S4 + 1; then the MFMA and the softmax work assigned to the slot.
#define MFA_SB_IF(S4, U, DB, SC) if constexpr ((U) < ((DB) + 1) * 4 / NDB) MFA_SB(S4, U, SC);
#define MFA_PV_SLOT(S4, DB, SC)                                                          \
    if constexpr ((DB) < NDB) {                                                              \
        if constexpr ((DB) == 0) {                                                           \
            if constexpr ((S4) > 0) lds_wait<NDB>(vlo[(S4) & 1], vhi[(S4) & 1]);             \
            if constexpr ((S4) < 3) MFA_TR_ISSUE((S4) + 1, vlo[((S4) + 1) & 1], vhi[((S4) + 1) & 1]); \
        }                                                                                    \
        {                                                                                    \
            const i16x4_t _lo4 = vlo[(S4) & 1][DB], _hi4 = vhi[(S4) & 1][DB];                \
            const i16x8_t _vv = {_lo4[0], _lo4[1], _lo4[2], _lo4[3], _hi4[0], _hi4[1], _hi4[2], _hi4[3]}; \
            oacc[DB] = Mfma<PT>::mma32(bitcast<pv8>(_vv), pop[S4], oacc[DB]);                \
        }                                                                                    \
        MFA_SB_IF(S4, (DB) * 4 / NDB + 0, DB, SC)                                            \
        MFA_SB_IF(S4, (DB) * 4 / NDB + 1, DB, SC)                                            \
        MFA_SB_IF(S4, (DB) * 4 / NDB + 2, DB, SC)                                            \
        MFA_SB_IF(S4, (DB) * 4 / NDB + 3, DB, SC)                                            \
        __builtin_amdgcn_sched_barrier(0);                                                   \
    }
#define MFA_PV_STEP(S4, SC) MFA_PV_SLOT(S4, 0, SC) MFA_PV_SLOT(S4, 1, SC) MFA_PV_SLOT(S4, 2, SC) MFA_PV_SLOT(S4, 3, SC)

// One pipeline iteration: tile tcur (scores in SC, V in stage ST) is finished
// and the scores of tile tnxt (K in stage ST ^ 1) are computed into SN.
#define MFA_ITER(SC, SN, ST)                                                                 \
    do {                                                                                     \
        has_nxt = tnxt <= kt_hi;                                                             \
        tnx2 = has_nxt ? MFA_NEXT_TILE(tnxt + 1) : kt_hi + 1;                                \
        /* copies spread over the Q.K^T slots: K(tnx2) into K(tcur)'s stage, V(tnxt)  */    \
        /* into V(tcur-1)'s stage; near the end of the range tile tcur is re-copied   */    \
        /* instead (harmless: those stages are not read again)                        */    \
        const auto _rk = MFA_RSRC(kbase, tnx2 <= kt_hi ? tnx2 : tcur);                       \
        const auto _rv = MFA_RSRC(vbase, has_nxt ? tnxt : tcur);                             \
        const uint32_t _wv = MFA_VMASKED(MASK ? words[has_nxt ? tnxt : tcur] : ~0ull);       \
        constexpr int _dk_dst = L::KST + (ST) * L::TILE;                                     \
        constexpr int _dv_dst = L::VST + ((ST) ^ 1) * L::TILE;                               \
        const int k0 = tcur * BN;                                                            \
        const uint64_t word = MASK ? words[tcur] : ~0ull;                                    \
        const bool interior = __builtin_amdgcn_readfirstlane(                                \
            (k0 >= wlo_last && k0 + BN - 1 <= whi_first && (!MASK || word == ~0ull)) ? 1 : 0); \
        uint32_t keepw = ~0u;                                                                \
        if constexpr (DROP) keepw = MFA_KEEP(k0);                                            \
        (void)keepw;                                                                         \
        constexpr int _vb = L::VST + (ST) * L::TILE;                                         \
        i16x4_t vlo[2][NDB], vhi[2][NDB];                                                    \
        float pm[11];                                                                        \
        float neg_m = 0.0f, psum0 = 0.0f, psum1 = 0.0f;                                      \
        pv8 pop[4];                                                                          \
        /* stage ST ^ 1 holds K(tnxt); on the last tile its scores are discarded */         \
        MFA_PART1(SC, SN, (ST) ^ 1, true);                                                   \
        if (has_nxt) MFA_BIAS_LOAD(tnxt);   /* this tile's bias is consumed: fetch the next */ \
        lds_wait<NDB>(vlo[0], vhi[0]);      /* V fragments of P.V step 0 */                  \
        MFA_PV_STEP(0, SC) MFA_PV_STEP(1, SC) MFA_PV_STEP(2, SC) MFA_PV_STEP(3, SC)          \
        __syncthreads();  /* copies of this iteration landed; stages handed over */         \
    } while (0)

    // ---- the prologue and the pipelined loop over the block's key tiles
    int tcur = MFA_NEXT_TILE(kt_lo);
    if (tcur <= kt_hi) {
        int tnxt = MFA_NEXT_TILE(tcur + 1), tnx2;
        bool has_nxt;
        // prologue: K,V of the first tile into stage 0, K of the second into
        // stage 1 (K of the first again when there is no second: never read).
        // The same copies in every case, so that the first scores wait only
        // for K of the first tile (copies complete in order; the additive
        // mask's loads come later still, and with them this waits for more);
        // the other two land while the scores run.
        MFA_DMA(tcur, 0, true, true);
        MFA_DMA(tnxt <= kt_hi ? tnxt : tcur, 1, true, false);
        MFA_BIAS_LOAD(tcur);
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(2 * IPW));
        if constexpr (CV) {
            asm volatile("" : "+v"(v16_any));   // first use here, past the barrier
            v16_flagged = __any(v16_any != 0u);
        }
        f32x16_t sa[2], sb[2];
        {
            // scores of the first tile; no softmax and no V reads (names unused)
            i16x4_t vlo[2][NDB], vhi[2][NDB];
            float pm[11], neg_m, psum0, psum1;
            pv8 pop[4];
            const int k0 = 0;
            const uint64_t word = 0;
            const bool interior = true;
            const uint32_t keepw = ~0u;
            (void)keepw;
            constexpr int _vb = 0, _dk_dst = 0, _dv_dst = 0;
            const auto _rk = MFA_RSRC(kbase, tcur);
            const auto _rv = _rk;
            const uint32_t _wv = 0u;
            (void)_wv;
            (void)vlo; (void)vhi; (void)pm; (void)neg_m; (void)psum0; (void)psum1; (void)pop;
            (void)k0; (void)word; (void)interior; (void)_vb; (void)_dk_dst; (void)_dv_dst;
            (void)_rk; (void)_rv;
            MFA_PART1(sa, sa, 0, false);
        }
        // The first iteration copies K of the tile after next into stage 0,
        // which the scores above just read: every wave must be past them; it
        // also reads V(tcur) and K(tnxt), which must have landed.
        __syncthreads();
        while (true) {
            MFA_ITER(sa, sb, 0);
            if (!has_nxt) break;
            tcur = tnxt; tnxt = tnx2;
            MFA_ITER(sb, sa, 1);
            if (!has_nxt) break;
            tcur = tnxt; tnxt = tnx2;
        }
    }
#undef MFA_NEXT_TILE
#undef MFA_BIAS_LOAD
#undef MFA_DMA
#undef MFA_DMA1
#undef MFA_DMAV
#undef MFA_VMASKED
#undef MFA_DMA_IF
#undef MFA_RSRC
#undef MFA_TR_ISSUE
#undef MFA_X
#undef MFA_KEEP
#undef MFA_DROP8
#undef MFA_SA
#undef MFA_EXT
#undef MFA_EXP
#undef MFA_SB
#undef MFA_SA_IF
#undef MFA_SB_IF
#undef MFA_QK_SLOT
#undef MFA_PV_SLOT
#undef MFA_PV_STEP
#undef MFA_PART1
#undef MFA_ITER

    if constexpr (CV) {
        uint32_t more = 0u;
        for (int w = lane + 64; w < a.v16_fwords; w += 64) more |= v16_fl[w];
        if (v16_flagged || __any(more != 0u)) return false;
    }

    // ---- epilogue: normalise, round, store; LSE in natural log.  O is staged
    // through LDS (this wave's 32 rows, chunk-swizzled; every stage is free
    // after the loop's last barrier) so that each store writes whole rows.
    l = xor32_sum(l);
    {
        // with dropout every kept weight carries the factor 1 / (1 - p)
        const float inv = l > 0.0f ? (DROP ? a.drop_scale : 1.0f) / l : 0.0f;
        char* stg = smem + wave * 32 * L::RS;
        char* wrow = stg + lq * L::RS;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // oacc[db][4 j + i] is column d = 32 db + 8 j + 4 h2 + i
                T o4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = static_cast<T>(oacc[db][4 * j + i] * inv);
                const int c = 4 * db + j;
                *reinterpret_cast<uint2*>(wrow + ((c ^ (lq & (CPR - 1))) * 16) + h2 * 8) =
                    *reinterpret_cast<const uint2*>(o4);
            }
        }
        T* obase = static_cast<T*>(a.out) + ((int64_t)b * a.Lq + w_first) * a.o_stride + (int64_t)hq * D;
#pragma unroll
        for (int s = 0; s < 32 * CPR / 64; ++s) {
            const int r = s * (64 / CPR) + lane / CPR, c = lane % CPR;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + r * L::RS + ((c ^ (r & (CPR - 1))) * 16));
            if (w_first + r <= i_last) *reinterpret_cast<u32x4_t*>(obase + (int64_t)r * a.o_stride + c * 8) = v;
        }
    }
    if (a.lse && h2 == 0 && qrow <= i_last)
        a.lse[((int64_t)b * a.Hq + hq) * a.Lq + qrow] = l > 0.0f ? (m + log2f(l)) * 0.6931471805599453f : -INFINITY;
    return true;
}

// The block on bf16 operands, out of line so that its registers and code
// stay apart from the kernel's hot loop (it runs only for a (batch, kv head)
// whose V holds a magnitude that fp16 cannot carry).
// It reads the kernel's arguments straight from the kernel-argument segment
// (kargs: the kernel's first argument), so the kernel keeps no copy of them.
template <typename T, int D, bool CAP, bool MASK, bool SEQ, bool BIAS, bool DROP>
__device__ __attribute__((noinline)) void prefill_block_bf16_operands(const void* kargs, int nqt, char* smem) {
    const FwdArgs& a = *static_cast<const FwdArgs*>(kargs);
    prefill_block<T, D, CAP, MASK, SEQ, BIAS, DROP, false>(a, nqt, smem);
}

// BIAS adds an additive score mask read from global memory into registers one
// tile ahead (32 more VGPRs).  DROP applies attention dropout: the keep bits
// of a tile's 32 weights per lane come from two Philox blocks (and the two
// the lane ^ 32 partner evaluates) before its softmax, dropped weights are
// zeroed after they enter the row sum and before they become the P.V operand,
// and the 1 / (1 - p) factor is folded into the final normalisation.  Either
// one runs two workgroups per CU: at D = 128 the compiler then spills a few
// values (fewer with two K reads in flight), and both still run faster than
// with one workgroup per CU and no spills.  With both, D = 64 still fits two
// workgroups per CU without spills; D = 128 takes one (at two it spills ~80).
// bf16 inputs run P.V on fp16 operands.
template <typename T, int D, bool CAP, bool MASK, bool SEQ, bool BIAS, bool DROP>
__global__ __launch_bounds__(256, (BIAS && DROP) ? (D == 64 ? 2 : 1) : (BIAS || DROP) ? 2 : (D == 64 ? 3 : 2))
void prefill_kernel(FwdArgs a, int nqt) {
    constexpr bool CVT = std::is_same<T, __bf16>::value;
    __shared__ __attribute__((aligned(1024))) char smem[PfLds<D>::BYTES];
    if constexpr (CVT) {
        // every wave sees the same flags, so a flagged block leaves with all
        // its waves past the loop's last barrier (no copy or LDS read left)
        if (!prefill_block<T, D, CAP, MASK, SEQ, BIAS, DROP, true>(a, nqt, smem))
            prefill_block_bf16_operands<T, D, CAP, MASK, SEQ, BIAS, DROP>(
                (const void*)__builtin_amdgcn_kernarg_segment_ptr(), nqt, smem);
    } else {
        prefill_block<T, D, CAP, MASK, SEQ, BIAS, DROP, false>(a, nqt, smem);
    }
}

// V of a bf16 call to fp16, one 64-row tile of one (batch, kv head) per
// workgroup, with the same element offsets as V (so also for the packed QKV
// layout); flag byte (b, kv head, tile) = 1 when a magnitude reached 65504
// (or is infinite).  Rows past Lk are not touched.
template <int D>
__global__ __launch_bounds__(256) void v16_prepass_kernel(const __bf16* __restrict__ v, _Float16* __restrict__ v16,
                                                         uint8_t* __restrict__ flags,
                                                         const uint64_t* __restrict__ words, int words_per_batch,
                                                         int Lk, int Hkv, int64_t kv_stride, int ntiles, int fwords) {
    constexpr int CPR = D / 8;                     // 16-byte chunks per row
    constexpr int NCH = 64 * CPR / 256;            // chunks per thread
    const int t = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int64_t base = ((int64_t)b * Lk) * kv_stride + (int64_t)kvh * D;
    // key-mask bits of the tile's 64 keys: a masked key's row is not read
    // and its copy holds zeros (so never-written memory cannot reach O)
    const uint64_t keep = words ? words[(int64_t)b * words_per_batch + t] : ~0ull;
    float mx = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int chunk = threadIdx.x + 256 * c;
        const int row = t * 64 + chunk / CPR;
        if (row < Lk) {
            const int64_t off = base + (int64_t)row * kv_stride + (chunk % CPR) * 8;
            u32x4_t x = u32x4_t{0u, 0u, 0u, 0u};
            if ((keep >> (chunk / CPR)) & 1ull) {
                x = *reinterpret_cast<const u32x4_t*>(v + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = cvt_bf16x2_f16x2(x[e], mx);
            }
            *reinterpret_cast<u32x4_t*>(v16 + off) = x;
        }
    }
    const int over = __syncthreads_or(!(mx < 65504.0f) && mx == mx);   // NaN is no reason
    if (threadIdx.x == 0) flags[((int64_t)b * Hkv + kvh) * fwords * 4 + t] = over ? 1 : 0;
    // the padding bytes of the last word are cleared by its own tiles' threads
    if (t == ntiles - 1 && threadIdx.x > 0 && threadIdx.x < fwords * 4 - t)
        flags[((int64_t)b * Hkv + kvh) * fwords * 4 + t + threadIdx.x] = 0;
}


template <typename T, int D, bool CAP, bool MASK, bool SEQ, bool BIAS = false, bool DROP = false>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    const int nqt = (a.Lq + BM - 1) / BM;
    const int64_t blocks = (int64_t)a.B * a.Hq * nqt;
    // instrumentation: a bf16 call's start event went on its V conversion
    hipExtLaunchKernelGGL((prefill_kernel<T, D, CAP, MASK, SEQ, BIAS, DROP>), dim3((unsigned)blocks), dim3(256), 0, s,
                          a.v16 ? nullptr : instr_event_begin(), instr_event_end(), 0,
                       a, nqt);
    return hipGetLastError();
}

// the additive-mask and dropout kernels of plain batches
template <typename T, int D, bool BIAS, bool DROP>
hipError_t launch_extras(const FwdArgs& a, bool cap, bool mask, hipStream_t s) {
    if (cap) return mask ? launch_t<T, D, true, true, false, BIAS, DROP>(a, s) : launch_t<T, D, true, false, false, BIAS, DROP>(a, s);
    return mask ? launch_t<T, D, false, true, false, BIAS, DROP>(a, s) : launch_t<T, D, false, false, false, BIAS, DROP>(a, s);
}

// Packed inputs (per-row positions or sequence bounds) have their own
// instantiations without the key mask, so plain batches keep the leaner code.
template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
    const bool cap = a.softcap > 0.0f, mask = a.key_mask != nullptr;
    const bool drop = a.drop_scale > 0.0f;
    if (a.bias || drop) {
        if (a.seq_bounds || a.row_pos || (a.bias && !mfma_bias_supported(a))) return hipErrorInvalidValue;
        if (a.bias) return drop ? launch_extras<T, D, true, true>(a, cap, mask, s) : launch_extras<T, D, true, false>(a, cap, mask, s);
        return launch_extras<T, D, false, true>(a, cap, mask, s);
    }
    if (a.seq_bounds || a.row_pos) {
        if (mask) return hipErrorInvalidValue;
        return cap ? launch_t<T, D, true, false, true>(a, s) : launch_t<T, D, false, false, true>(a, s);
    }
    if (cap) return mask ? launch_t<T, D, true, true, false>(a, s) : launch_t<T, D, true, false, false>(a, s);
    return mask ? launch_t<T, D, false, true, false>(a, s) : launch_t<T, D, false, false, false>(a, s);
}

}  // namespace

size_t v16_workspace_bytes(const FwdArgs& a) {
    const int ntiles = (a.Lk + 63) / 64, fwords = (ntiles + 3) / 4;
    const size_t v16 = ((size_t)a.B * a.Lk * a.kv_stride * 2 + 255) & ~size_t(255);
    return v16 + (((size_t)a.B * a.Hkv * fwords * 4 + 255) & ~size_t(255));
}

hipError_t launch_v16_prepass(FwdArgs& a, void* ws, hipStream_t s) {
    const int ntiles = (a.Lk + 63) / 64, fwords = (ntiles + 3) / 4;
    const size_t v16 = ((size_t)a.B * a.Lk * a.kv_stride * 2 + 255) & ~size_t(255);
    a.v16 = ws;
    a.v16_flags = static_cast<const uint8_t*>(ws) + v16;
    a.v16_fwords = fwords;
    uint8_t* flags = static_cast<uint8_t*>(ws) + v16;
    const dim3 grid(ntiles, a.Hkv, a.B);
    // instrumentation: the conversion belongs to the bf16 prefill it feeds,
    // so the start event goes here and the stop event on the prefill kernel
    if (a.D == 64)
        hipExtLaunchKernelGGL(v16_prepass_kernel<64>, grid, dim3(256), 0, s, instr_event_begin(), nullptr, 0,
                              static_cast<const __bf16*>(a.v), static_cast<_Float16*>(ws), flags,
                              a.key_mask ? a.mask_words : nullptr, a.words_per_batch, a.Lk, a.Hkv,
                              a.kv_stride, ntiles, fwords);
    else
        hipExtLaunchKernelGGL(v16_prepass_kernel<128>, grid, dim3(256), 0, s, instr_event_begin(), nullptr, 0,
                              static_cast<const __bf16*>(a.v), static_cast<_Float16*>(ws), flags,
                              a.key_mask ? a.mask_words : nullptr, a.words_per_batch, a.Lk, a.Hkv,
                              a.kv_stride, ntiles, fwords);
    return hipGetLastError();
}

bool mfma_bias_supported(const FwdArgs& a) {
    // 16-byte loads of four keys: keys contiguous, every row start 16-byte aligned
    return a.bias && a.bias_stride[3] == 1 && a.Lk % 4 == 0 && (reinterpret_cast<uintptr_t>(a.bias) & 15) == 0 &&
           a.bias_stride[0] % 4 == 0 && a.bias_stride[1] % 4 == 0 && a.bias_stride[2] % 4 == 0;
}

bool mfma_prefill_supported(int dtype, int D) {
    return (dtype == kBF16 || dtype == kF16) && (D == 64 || D == 128);
}

hipError_t launch_mfma_prefill(const FwdArgs& a0, int dtype, hipStream_t s) {
    if ((int64_t)a0.B * a0.Hq * ((a0.Lq + BM - 1) / BM) > 0x7fffffff) return hipErrorInvalidValue;
    FwdArgs a = a0;
    a.q_xor = 0u;
    a.q_clear = 0u;
    // Without a soft-cap or an additive mask the kernel masks raw scores and
    // takes their max before applying scale * log2(e), which needs a positive
    // factor.  A negative scale moves onto Q instead (its elements change
    // sign, the factor becomes |scale| log2(e)); a zero scale zeroes Q, so
    // every score is 0 whatever factor is used.
    if (!(a.softcap > 0.0f) && !a.bias && !(a.scale > 0.0f)) {
        const float log2e = 1.4426950408889634f;
        if (a.scale < 0.0f) {
            a.q_xor = 0x80008000u;
            a.score_to_log2 = -a.scale * log2e;
        } else {
            a.q_clear = 0xffffffffu;
            a.score_to_log2 = log2e;
        }
    }
    if (dtype == kBF16) return a.D == 64 ? launch_d<__bf16, 64>(a, s) : launch_d<__bf16, 128>(a, s);
    if (dtype == kF16) return a.D == 64 ? launch_d<_Float16, 64>(a, s) : launch_d<_Float16, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace mfa
