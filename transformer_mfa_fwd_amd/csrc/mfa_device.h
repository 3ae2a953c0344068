// mfa_device.h -- device-side helpers shared by the MFMA kernels: vector
// types, MFMA wrappers, conversions, LDS swizzles and the soft-cap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;
// 16 raw bytes as a native vector (kept in registers; HIP's uint4 struct is not)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Element-type traits: storage type, 8-wide MFMA operand type and the MFMAs.
template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
    typedef bf16x8_t v8;
    static __device__ inline f32x4_t mma16(v8 a, v8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ inline f32x16_t mma32(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<_Float16> {
    typedef f16x8_t v8;
    static __device__ inline f32x4_t mma16(v8 a, v8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ inline f32x16_t mma32(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <typename V, typename S>
__device__ inline V bitcast(S s) {
    static_assert(sizeof(V) == sizeof(S), "size mismatch");
    V v;
    __builtin_memcpy(&v, &s, sizeof(V));
    return v;
}

// Eight fp32 values rounded to nearest-even into one MFMA operand.
template <typename T>
__device__ inline typename Mfma<T>::v8 pack8(const float* x) {
    typename Mfma<T>::v8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = static_cast<T>(x[e]);
    return r;
}

// Elements OFF .. OFF+7 of a 16-float accumulator, rounded into one operand.
template <typename T>
__device__ inline typename Mfma<T>::v8 pack8_at(const f32x16_t& x, int off) {
    typename Mfma<T>::v8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = static_cast<T>(x[off + e]);
    return r;
}

// Transposing LDS read: within each group of 16 lanes, source lane j supplies
// the address of 4 consecutive 16-bit elements; result lane i element e is
// element (i % 4) of source lane 4e + i/4.  With source lane j pointing at
// row (j / 4), columns 4 (j % 4) .. +3 of a row-major block, lane i receives
// column i of the 4 rows.
__device__ inline i16x4_t lds_read_tr16(const void* lds_ptr) {
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
}

// The same transposing read issued through inline assembly, for code that
// keeps direct global->LDS copies in flight: the compiler waits for every
// outstanding copy before the intrinsic form, since it cannot tell which LDS
// bytes the intrinsic reads.  The caller must wait (lds_wait) before using
// the result; lds_wait ties the registers so no consumer is hoisted above it.
// Issues N reads at immediate byte offsets OFF0/OFF1 from addr[k].
template <int OFF0, int OFF1>
__device__ inline void lds_read_tr16_pair4(const uint32_t (&addr)[4], i16x4_t (&lo)[4], i16x4_t (&hi)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]),
          "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(OFF0), "i"(OFF1));
}
template <int OFF0, int OFF1>
__device__ inline void lds_read_tr16_pair2(const uint32_t (&addr)[2], i16x4_t (&lo)[2], i16x4_t (&hi)[2]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
        "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%7"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
        : "v"(addr[0]), "v"(addr[1]), "i"(OFF0), "i"(OFF1));
}
template <int N>
__device__ inline void lds_wait(i16x4_t (&lo)[N], i16x4_t (&hi)[N]) {
    if constexpr (N == 4)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(lo[0]), "+v"(hi[0]), "+v"(lo[1]), "+v"(hi[1]),
                       "+v"(lo[2]), "+v"(hi[2]), "+v"(lo[3]), "+v"(hi[3]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(lo[0]), "+v"(hi[0]), "+v"(lo[1]), "+v"(hi[1]));
}
// 16-byte LDS read at an immediate offset, and a wait until at most N LDS
// reads are outstanding that ties the result register (LDS reads of one wave
// complete in order, so N counts the reads issued after the one awaited).
template <int OFF>
__device__ inline void lds_read_b128_asm(u32x4_t& dst, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF));
}
template <int N>
__device__ inline void lds_wait_b128(u32x4_t& r) {
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}

// Direct copy of 16 bytes per lane from global memory into LDS through a raw
// buffer descriptor (base, range nbytes): lane l writes LDS bytes
// lds + 16 l .. + 15 with the bytes at base + voffset, or zeros when voffset is
// at or past nbytes.  lds must be wave-uniform.  The load carries the sc0
// cache-policy bit (measured faster for K/V tiles than the default policy
// and than the non-temporal ones).
__device__ inline void buffer_copy16_to_lds(const void* base, int nbytes, void* lds, uint32_t voffset) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 1);
}

// LDS byte offset of a pointer into __shared__ memory
__device__ inline uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// IEEE maximum (gfx950 v_maximum3_f32 for chains); unlike fmaxf it needs no
// canonicalisation of its operands.  Scores are finite or -inf.
__device__ inline float fmax_fast(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ inline float fmin_fast(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ inline float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Max / min / sum of a value over lanes l and l ^ 32.  v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second, so
// with both operands equal each lane ends up holding {v[l], v[l ^ 32]}; this
// stays on the VALU (no LDS permute).
__device__ inline float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmax_fast(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_min(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmin_fast(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// c * tanh(s / c) through tanh(y) = 1 - 2 / (exp(2y) + 1), with the hardware
// base-2 exponential.  Saturates correctly at both ends (exp2 -> inf or 0).
__device__ inline float softcap_apply(float s, float cap, float two_log2e_over_cap) {
    const float e = fast_exp2(s * two_log2e_over_cap);
    return cap - 2.0f * cap * fast_rcp(e + 1.0f);
}

// LDS swizzles for a [rows][D] tile of 16-bit elements stored as 16-byte
// chunks (D/8 chunks per row).  The chunk index is XOR-ed with a function of
// the row so that the access patterns of the kernels hit distinct banks.
//  - K-style (16 consecutive rows, same chunk): chunk ^ row-bits.
//  - V-style (transposing reads of 2 adjacent chunks from 8 rows): chunk pairs
//    permuted by row-bits.
template <int D>
__device__ inline int swz_k(int row, int chunk) {
    return D == 128 ? (chunk ^ (row & 15)) : (chunk ^ ((row >> 1) & 7));
}
template <int D>
__device__ inline int swz_v(int row, int chunk) {
    return D == 128 ? (chunk ^ ((row & 7) << 1)) : (chunk ^ (((row >> 1) & 3) << 1));
}

}  // namespace mfa
