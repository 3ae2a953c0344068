// mfa_internal.h -- kernel arguments, key-range arithmetic and launchers
// shared by the libmfa host code and its HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfa {

enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Everything a forward kernel needs, passed by value as one kernel argument.
struct FwdArgs {
    const void* q;            // [B, Lq, Hq, D]
    const void* k;            // [B, Lk, Hkv, D]
    const void* v;            // [B, Lk, Hkv, D]
    void* out;                // [B, Lq, Hq, D]
    float* lse;               // [B, Hq, Lq] or null
    const float* key_mask;    // [B, Lk] or null
    const uint64_t* mask_words;  // [B, words_per_batch]: bit t of word w = key 64w+t kept
    int B, Lq, Lk, Hq, Hkv, D;
    int group;                // Hq / Hkv
    int causal, window, q_offset;
    int words_per_batch;      // ceil(Lk / 64)
    float scale;              // applied to Q.K
    float softcap;            // <= 0: off
    float score_to_log2;      // log2(e) * scale when the cap is off, log2(e) otherwise
    // elements from one row to the next: q, k/v and out (Hq*D, Hkv*D, Hq*D
    // for separate tensors; 3*H*D, 3*H*D, H*D for a packed QKV tensor)
    int64_t q_stride, kv_stride, o_stride;
    const int* seq_bounds;    // [Lq, 2]: row i only sees keys in [s0, s1) of its own sequence, or null
    const int* row_pos;       // [Lq]: absolute key-axis position of row i, or null (i + q_offset)
    // additive score mask: element (b, hq, i, j) at the dot product of
    // (b, hq, i, j) with bias_stride (0 for a broadcast dimension), or null
    const float* bias;
    int64_t bias_stride[4];
    // attention dropout: weight (b, hq, i, j) is kept iff 16-bit field
    // f = j % 16 (bits 16 (f % 4) .. +15 of word f / 4) of
    // Philox4x64-10(counter (j / 16, i, hq, b), key (drop_seed, 0)) is at
    // least drop_threshold (round(p * 2^16)); drop_seed holds the low 32 bits
    // of the caller's seed; a kept weight is multiplied by drop_scale (> 0
    // turns dropout on)
    uint32_t drop_threshold;
    float drop_scale;
    uint64_t drop_seed;
    // backward with dropout: the keep bits of every 16-key block, uint16
    // [B, Hq, ceil(Lk / 16), Lq] (bit f: key 16 jb + f of row i), written by the
    // dK/dV kernel and read by the dQ kernel that runs after it; null: each
    // kernel evaluates the blocks it needs
    uint16_t* keep_bits;
    // MFMA prefill only: each 32-bit word of the Q operand is replaced by
    // (word ^ q_xor) & ~q_clear when it is loaded (sign flip or zeroing of
    // the 16-bit elements), set by its launcher for a scale <= 0
    uint32_t q_xor, q_clear;
    // MFMA prefill of bf16 inputs: V converted to fp16 (same element offsets
    // as v) and one flag byte per (batch, kv head, 64-key tile), v16_fwords
    // 32-bit words per (batch, kv head); set by launch_v16_prepass
    const void* v16;
    const uint8_t* v16_flags;
    int v16_fwords;
};

// Keys [lo, hi] (inclusive) in range for a query at absolute position aq,
// before the key mask.  Causal: keys up to aq and, with a window, no earlier
// than aq - window + 1.  Bidirectional with a window: window/2 keys on either
// side.  window <= 0: no window.  Both bounds are nondecreasing in aq, so the
// range of a block of consecutive queries is [lo(first), hi(last)].
__host__ __device__ inline void key_range(int aq, int Lk, int causal, int window,
                                          int& lo, int& hi) {
    if (causal) {
        hi = aq;
        lo = window > 0 ? aq - window + 1 : 0;
    } else if (window > 0) {
        lo = aq - window / 2;
        hi = aq + window / 2;
    } else {
        lo = 0;
        hi = Lk - 1;
    }
    if (lo < 0) lo = 0;
    if (hi > Lk - 1) hi = Lk - 1;
}

// Keys [lo, hi] of query row i: key_range at its position aq (row_pos[i], or
// i + q_offset), cut to the row's own sequence [s0, s1) when per-row bounds
// are given.  A row left with no key gets the empty range [s1, s1 - 1], so
// that for sequences packed back to back both bounds stay nondecreasing in i
// (rows past a window's reach lie at the end of their sequence).
// SEQ = false ignores row_pos and seq_bounds (kernels instantiated for
// plain batches); SEQ = true reads whichever of them is given.
// Whatever the bounds hold, the sequence ends are first clamped to [0, Lk],
// so a nonempty range always lies inside [0, Lk - 1] and an empty one is
// [s1, s1 - 1] with s1 in [0, Lk].
template <bool SEQ = true>
__host__ __device__ inline void row_key_range(const FwdArgs& a, int i, int& lo, int& hi) {
    key_range(SEQ && a.row_pos ? a.row_pos[i] : i + a.q_offset, a.Lk, a.causal, a.window, lo, hi);
    if (SEQ && a.seq_bounds) {
        int s0 = a.seq_bounds[2 * i], s1 = a.seq_bounds[2 * i + 1];
        s0 = s0 < 0 ? 0 : (s0 > a.Lk ? a.Lk : s0);
        s1 = s1 < 0 ? 0 : (s1 > a.Lk ? a.Lk : s1);
        lo = lo > s0 ? lo : s0;
        hi = hi < s1 - 1 ? hi : s1 - 1;
        if (lo > hi) { lo = s1; hi = s1 - 1; }
    }
}

// Philox4x64-10 (Salmon et al., SC 2011): ten rounds of two 64x64 -> 128-bit
// products with the round constants, the halves mixed with the other counter
// words and the key, the key bumped by the Weyl constants.  c0..c3 in: the
// counter; out: the block.
// The 128-bit product of the 64-bit words m and c as four 32 x 32 + 64-bit
// multiply-adds (each partial sum fits 64 bits) and one 64-bit add.
__device__ inline void mul64_wide(uint64_t m, uint64_t c, uint64_t& hi, uint64_t& lo) {
    const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32), cl = (uint32_t)c, ch = (uint32_t)(c >> 32);
    const uint64_t t0 = (uint64_t)ml * cl;
    const uint64_t t1 = (uint64_t)ml * ch + (t0 >> 32);
    const uint64_t t2 = (uint64_t)mh * cl + (uint32_t)t1;
    hi = (uint64_t)mh * ch + (t1 >> 32) + (t2 >> 32);
    lo = (t2 << 32) | (uint32_t)t0;
}

__device__ inline void philox4x64(uint64_t& c0, uint64_t& c1, uint64_t& c2, uint64_t& c3, uint64_t k0,
                                  uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t hi0, lo0, hi1, lo1;
        mul64_wide(M0, c0, hi0, lo0);
        mul64_wide(M1, c2, hi1, lo1);
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B97F4A7C15ull;
        k1 += 0xBB67AE8584CAA73Bull;
    }
}

// Dropout decisions of weights (b, hq, i, 16 jb .. 16 jb + 15): bit f set
// iff 16-bit field f (bits 16 (f % 4) .. +15 of word f / 4) of
// Philox4x64-10 with counter (jb, i, hq, b) and key (drop_seed, 0) reaches
// the threshold round(p * 2^16).
__device__ inline uint32_t dropout_keep16(const FwdArgs& a, int b, int hq, int i, int jb) {
    uint64_t c0 = (uint64_t)jb, c1 = (uint64_t)i, c2 = (uint64_t)hq, c3 = (uint64_t)b;
    philox4x64(c0, c1, c2, c3, a.drop_seed, 0);
    const uint32_t t = a.drop_threshold;
    const uint32_t w[8] = {(uint32_t)c0, (uint32_t)(c0 >> 32), (uint32_t)c1, (uint32_t)(c1 >> 32),
                           (uint32_t)c2, (uint32_t)(c2 >> 32), (uint32_t)c3, (uint32_t)(c3 >> 32)};
    uint32_t m = 0u;
#pragma unroll
    for (int f = 0; f < 16; ++f) m |= ((((w[f >> 1] >> (16 * (f & 1))) & 0xffffu) >= t) ? 1u : 0u) << f;
    return m;
}

// Dropout decision of weight (b, hq, i, j).
__device__ inline bool dropout_keep(const FwdArgs& a, int b, int hq, int i, int j) {
    return (dropout_keep16(a, b, hq, i, j >> 4) >> (j & 15)) & 1u;
}

// The nibbles at bits 0, 8, 16 and 24 of x (every other nibble) packed into
// bits 0 .. 15.
__device__ inline uint32_t pack_even_nibbles(uint32_t x) {
    x &= 0x0f0f0f0fu;
    x = (x | (x >> 4)) & 0x00ff00ffu;
    return (x | (x >> 8)) & 0x0000ffffu;
}

// Instrumentation events of the calling host thread (mfa_set_kernel_events,
// null when unset): the main kernel launch of a call takes them as the start
// and stop events of hipExtLaunchKernelGGL, whose timestamps come from the
// dispatch itself (a separate event record would add a marker packet and a
// gap of its own between kernels).
hipEvent_t instr_event_begin();
hipEvent_t instr_event_end();

// Launchers (each returns the hipError_t of its launch).
hipError_t launch_mask_words(const FwdArgs& a, uint64_t* words, hipStream_t s);
// Per-row position and key bounds of a varlen packing: row i of sequence b
// (cu_q[b] <= i < cu_q[b+1]) gets row_pos[i] = cu_k[b] + i - cu_q[b] and
// bounds [cu_k[b], cu_k[b+1]); rows of no sequence get the empty [Tk, Tk).
// Prefix sums are clamped to [0, Tq] and [0, Tk].
hipError_t launch_varlen_rows(const int* cu_q, const int* cu_k, int batch, int Tq, int Tk, int* row_pos,
                              int* seq_bounds, hipStream_t s);
hipError_t launch_generic(const FwdArgs& a, int dtype, hipStream_t s);
// Backward on the generic path: a.out is the forward output O, a.lse its LSE;
// dout [B, Lq, Hq, D] the upstream gradient; delta [B, Hq, Lq] fp32 scratch.
// dq, dk, dv are written in the input dtype (every element overwritten).
hipError_t launch_backward(const FwdArgs& a, const void* dout, float* delta, void* dq, void* dk, void* dv,
                           int dtype, hipStream_t s);
// The matrix-core backward (fp16/bf16, D 64/128, plain batches, any additive
// mask and dropout); delta must already hold <dO, O> per row.
bool bwd_mfma_supported(const FwdArgs& a, int dtype);
// Bytes of a.keep_bits for this call (0 when its kernels do not share them:
// no dropout, or not the matrix-core backward, whose 16-key dK/dV kernel
// evaluates the pattern that its dQ kernel then reads).
size_t bwd_keep_bits_bytes(const FwdArgs& a, int dtype);
hipError_t launch_backward_mfma(const FwdArgs& a, const void* dout, const float* delta, void* dq, void* dk, void* dv,
                                int dtype, hipStream_t s);
hipError_t launch_mfma_prefill(const FwdArgs& a, int dtype, hipStream_t s);
// bf16 MFMA prefill: bytes of the fp16 copy of V and its flags, and the
// launch that fills them from a.v into ws (256-byte aligned) and points
// a.v16 / a.v16_flags / a.v16_fwords there.  Must precede launch_mfma_prefill
// on the same stream.
size_t v16_workspace_bytes(const FwdArgs& a);
hipError_t launch_v16_prepass(FwdArgs& a, void* ws, hipStream_t s);
bool mfma_prefill_supported(int dtype, int D);
// Whether the MFMA prefill kernel can read a's additive mask (keys contiguous,
// Lk and every row start a multiple of four floats).
bool mfma_bias_supported(const FwdArgs& a);
// Split decode: a.Lq query rows per batch (1 unless d_len is given).  With
// d_len (device [B]) the key range of batch b is its first d_len[b] keys.
// With pos_from_mask (one query row, a key mask and its packed words in
// a.mask_words) the query sits at the batch's last valid key and a window
// counts back from there.
hipError_t launch_split_decode(const FwdArgs& a, const int* d_len, int dtype, int splits,
                               float* partials, hipStream_t s, bool pos_from_mask = false);
bool split_decode_supported(int dtype, int D, int Lq, int group);
bool decode_len_supported(int dtype, int D, int R, int group);
int split_decode_default_splits(int B, int Hkv, int Lk, int group);
size_t split_decode_workspace_bytes(int B, int R, int Hq, int D, int splits);

}  // namespace mfa
