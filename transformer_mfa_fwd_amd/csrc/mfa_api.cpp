// mfa_api.cpp -- the C ABI of libmfa: argument checks, kernel choice,
// workspace handling and launches.  Declarations and semantics: include/mfa.h.
#include "mfa.h"
#include "mfa_internal.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_last_error;

// Instrumentation events (mfa_set_kernel_events), per host thread.
thread_local hipEvent_t g_ev_begin = nullptr, g_ev_end = nullptr;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

struct Call {
    const void *q, *k, *v;
    void* out;
    float* lse;
    int B, Lq, Lk, Hq, Hkv, D;
    float scale;
    int causal, window, q_offset;
    float softcap;
    const float* key_mask;
    int dtype;
    const float* bias = nullptr;     // additive score mask [bias_dims] or null
    int bias_dims[4] = {1, 1, 1, 1};
    float dropout_p = 0.0f;
    uint64_t seed = 0;
};

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Host-side checks; no HIP call happens here.
// A pointer to a tensor that holds no element may be null: nothing is read
// from or written to it (torch hands out null for empty tensors).
int validate(const Call& c) {
    if (c.B < 0 || c.Lq < 0 || c.Lk <= 0 || c.Hq <= 0 || c.Hkv <= 0 || c.D <= 0)
        return fail(MFA_ERROR_INVALID_VALUE,
                    "bad dimensions B=%d Lq=%d Lk=%d Hq=%d Hkv=%d D=%d (B, Lq >= 0; others > 0)",
                    c.B, c.Lq, c.Lk, c.Hq, c.Hkv, c.D);
    const bool q_empty = c.B == 0 || c.Lq == 0, kv_empty = c.B == 0;
    if ((!q_empty && (!c.q || !c.out)) || (!kv_empty && (!c.k || !c.v)))
        return fail(MFA_ERROR_INVALID_VALUE, "q, k, v and out must be non-null");
    if (c.Hq % c.Hkv != 0)
        return fail(MFA_ERROR_INVALID_VALUE, "Hkv=%d does not divide Hq=%d", c.Hkv, c.Hq);
    if (c.q_offset < 0 || (int64_t)c.q_offset + c.Lq > c.Lk)
        return fail(MFA_ERROR_INVALID_VALUE, "need 0 <= q_offset and q_offset + Lq <= Lk (q_offset=%d Lq=%d Lk=%d)",
                    c.q_offset, c.Lq, c.Lk);
    if (!std::isfinite(c.scale) || !std::isfinite(c.softcap))
        return fail(MFA_ERROR_INVALID_VALUE, "scale and softcap must be finite");
    if (c.dtype != MFA_F32 && c.dtype != MFA_F16 && c.dtype != MFA_BF16)
        return fail(MFA_ERROR_NOT_SUPPORTED, "unknown dtype %d", c.dtype);
    if (c.D != 64 && c.D != 128)
        return fail(MFA_ERROR_NOT_SUPPORTED, "head dim %d not supported (64 or 128)", c.D);
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.out, 16))
        return fail(MFA_ERROR_INVALID_VALUE, "q, k, v and out must be 16-byte aligned");
    if (!aligned(c.lse, 4) || !aligned(c.key_mask, 4))
        return fail(MFA_ERROR_INVALID_VALUE, "lse and key_mask must be 4-byte aligned");
    if (c.bias) {
        const int full[4] = {c.B, c.Hq, c.Lq, c.Lk};
        for (int e = 0; e < 4; ++e)
            if (c.bias_dims[e] != 1 && c.bias_dims[e] != full[e])
                return fail(MFA_ERROR_INVALID_VALUE, "bias dimension %d is %d: must be 1 or %d", e,
                            c.bias_dims[e], full[e]);
        if (!aligned(c.bias, 4)) return fail(MFA_ERROR_INVALID_VALUE, "bias must be 4-byte aligned");
    }
    if (!(c.dropout_p >= 0.0f && c.dropout_p < 1.0f))
        return fail(MFA_ERROR_INVALID_VALUE, "dropout probability %g not in [0, 1)", (double)c.dropout_p);
    // sizes must fit the kernels' 64-bit element offsets and 32-bit row indices
    const int64_t q_elems = (int64_t)c.B * c.Lq * c.Hq * c.D;
    const int64_t kv_elems = (int64_t)c.B * c.Lk * c.Hkv * c.D;
    if (q_elems < 0 || kv_elems < 0 || (int64_t)c.B * c.Hq > (int64_t)1 << 30)
        return fail(MFA_ERROR_INVALID_VALUE, "problem too large");
    return MFA_SUCCESS;
}

int auto_path(int B, int Lq, int Lk, int Hq, int Hkv, int D, int dtype) {
    (void)B; (void)Lk;
    const int group = Hq / Hkv;
    if (Lq == 1 && mfa::split_decode_supported(dtype, D, Lq, group)) return MFA_PATH_SPLIT_DECODE;
    if (mfa::mfma_prefill_supported(dtype, D)) return MFA_PATH_MFMA;
    return MFA_PATH_GENERIC;
}

int words_per_batch(int Lk) { return (Lk + 63) / 64; }

size_t mask_words_bytes(int B, int Lk) { return align256((size_t)B * words_per_batch(Lk) * 8); }

// Bytes of the fp16 copy of V (and its flags) that a bf16 call on the MFMA
// prefill kernel needs; kv_stride elements from one key row to the next.
size_t v16_bytes(int B, int Lk, int Hkv, int D, int64_t kv_stride) {
    mfa::FwdArgs t{};
    t.B = B; t.Lk = Lk; t.Hkv = Hkv; t.D = D; t.kv_stride = kv_stride;
    return align256(mfa::v16_workspace_bytes(t));
}

size_t workspace_bytes(int B, int Lq, int Lk, int Hq, int Hkv, int D, int dtype, int path, int splits) {
    size_t ws = mask_words_bytes(B, Lk);
    if (path == MFA_PATH_SPLIT_DECODE) {
        (void)Lq;
        ws += align256(mfa::split_decode_workspace_bytes(B, 1, Hq, D, splits));
    }
    if (path == MFA_PATH_MFMA && dtype == MFA_BF16) ws += v16_bytes(B, Lk, Hkv, D, (int64_t)Hkv * D);
    return ws;
}

constexpr int kMaxDevices = 64;
std::once_flag g_pool_once[kMaxDevices];
hipMemPool_t g_pool[kMaxDevices] = {};

// The library's own stream-ordered pool on device dev, created on first use
// and kept until the process ends: freed workspace stays in it instead of
// going back to the driver after every call.  The device's default pool is
// left as it is.  Null if it could not be created (then the default pool
// serves).
hipMemPool_t library_pool(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_pool_once[dev], [dev]() {
        hipMemPoolProps props{};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        uint64_t thr = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
        g_pool[dev] = pool;
    });
    return g_pool[dev];
}

// Stream-ordered workspace of n bytes on the current device (released with
// hipFreeAsync on the same stream); an MFA status.
int pool_alloc(void** p, size_t n, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_ERROR_HIP, "hipGetDevice failed");
    }
    hipMemPool_t pool = library_pool(dev);
    hipError_t e = pool ? hipMallocFromPoolAsync(p, n, pool, stream) : hipMallocAsync(p, n, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(e == hipErrorOutOfMemory ? MFA_ERROR_OUT_OF_MEMORY : MFA_ERROR_HIP,
                    "workspace allocation of %zu bytes failed: %s", n, hipGetErrorString(e));
    }
    return MFA_SUCCESS;
}

mfa::FwdArgs make_args(const Call& c) {
    mfa::FwdArgs a{};
    a.q = c.q; a.k = c.k; a.v = c.v; a.out = c.out; a.lse = c.lse;
    a.key_mask = c.key_mask;
    a.B = c.B; a.Lq = c.Lq; a.Lk = c.Lk; a.Hq = c.Hq; a.Hkv = c.Hkv; a.D = c.D;
    a.group = c.Hq / c.Hkv;
    a.causal = c.causal ? 1 : 0;
    a.window = c.window > 0 ? c.window : 0;
    a.q_offset = c.q_offset;
    a.words_per_batch = words_per_batch(c.Lk);
    a.q_stride = (int64_t)c.Hq * c.D;
    a.kv_stride = (int64_t)c.Hkv * c.D;
    a.o_stride = (int64_t)c.Hq * c.D;
    a.seq_bounds = nullptr;
    if (c.bias) {
        a.bias = c.bias;
        const int64_t n3 = c.bias_dims[3], n2 = c.bias_dims[2] * n3, n1 = c.bias_dims[1] * n2;
        a.bias_stride[0] = c.bias_dims[0] > 1 ? n1 : 0;
        a.bias_stride[1] = c.bias_dims[1] > 1 ? n2 : 0;
        a.bias_stride[2] = c.bias_dims[2] > 1 ? n3 : 0;
        a.bias_stride[3] = c.bias_dims[3] > 1 ? 1 : 0;
    }
    if (c.dropout_p > 0.0f) {
        a.drop_threshold = (uint32_t)std::llround((double)c.dropout_p * 65536.0);
        a.drop_scale = 1.0f / (1.0f - c.dropout_p);
        a.drop_seed = c.seed & 0xffffffffull;   // only the seed's low 32 bits drive the pattern
    }
    a.scale = c.scale;
    a.softcap = c.softcap > 0.0f ? c.softcap : 0.0f;
    const float log2e = 1.4426950408889634f;
    a.score_to_log2 = a.softcap > 0.0f ? log2e : log2e * c.scale;
    return a;
}

int run(const Call& c, int path, int splits, void* workspace, size_t ws_bytes, hipStream_t stream) {
    int st = validate(c);
    if (st != MFA_SUCCESS) return st;
    if (c.B == 0 || c.Lq == 0) return MFA_SUCCESS;

    const int group = c.Hq / c.Hkv;
    // an additive mask and dropout run on the MFMA prefill kernel (fp16/bf16,
    // D 64 or 128) when the mask's rows can be read four keys at a time, and
    // on the generic kernel otherwise
    const bool extras = c.bias != nullptr || c.dropout_p > 0.0f;
    bool extras_mfma = false;
    if (extras && mfa::mfma_prefill_supported(c.dtype, c.D)) {
        const mfa::FwdArgs t = make_args(c);
        extras_mfma = !c.bias || mfa::mfma_bias_supported(t);
    }
    if (path == MFA_PATH_AUTO)
        path = extras ? (extras_mfma ? MFA_PATH_MFMA : MFA_PATH_GENERIC)
                      : auto_path(c.B, c.Lq, c.Lk, c.Hq, c.Hkv, c.D, c.dtype);
    if (extras && path != MFA_PATH_GENERIC && !(extras_mfma && path == MFA_PATH_MFMA))
        return fail(MFA_ERROR_NOT_SUPPORTED,
                    "this additive mask or dropout call needs the generic path (MFMA: fp16/bf16, D 64/128, "
                    "mask rows of Lk %% 4 == 0 floats, 16-byte aligned)");
    switch (path) {
        case MFA_PATH_GENERIC: break;
        case MFA_PATH_MFMA:
            if (!mfa::mfma_prefill_supported(c.dtype, c.D))
                return fail(MFA_ERROR_NOT_SUPPORTED, "MFMA path needs fp16/bf16 and D in {64,128}");
            break;
        case MFA_PATH_SPLIT_DECODE:
            if (!mfa::split_decode_supported(c.dtype, c.D, c.Lq, group))
                return fail(MFA_ERROR_NOT_SUPPORTED,
                            "split decode needs Lq = 1, fp16/bf16, D in {64,128} and Hq/Hkv <= 16");
            if (splits <= 0) splits = mfa::split_decode_default_splits(c.B, c.Hkv, c.Lk, group);
            if (splits > c.Lk) splits = c.Lk;
            break;
        default: return fail(MFA_ERROR_NOT_SUPPORTED, "unknown path %d", path);
    }

    const size_t need = workspace_bytes(c.B, c.Lq, c.Lk, c.Hq, c.Hkv, c.D, c.dtype, path, splits);
    const bool use_pool = workspace == nullptr && ws_bytes == 0;
    if (!use_pool) {
        if (!workspace) return fail(MFA_ERROR_INVALID_VALUE, "workspace is null but ws_bytes > 0");
        if (!aligned(workspace, 256)) return fail(MFA_ERROR_INVALID_VALUE, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(MFA_ERROR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    }

    mfa::FwdArgs a = make_args(c);

    const bool v16 = path == MFA_PATH_MFMA && c.dtype == MFA_BF16;
    const bool needs_ws = c.key_mask != nullptr || path == MFA_PATH_SPLIT_DECODE || v16;
    void* ws = workspace;
    if (needs_ws && use_pool) {
        const int pst = pool_alloc(&ws, need, stream);
        if (pst != MFA_SUCCESS) return pst;
    }
    char* wsb = static_cast<char*>(ws);
    hipError_t e = hipSuccess;
    if (c.key_mask) {
        a.mask_words = reinterpret_cast<const uint64_t*>(wsb);
        e = mfa::launch_mask_words(a, reinterpret_cast<uint64_t*>(wsb), stream);
    }
    if (e == hipSuccess && v16) e = mfa::launch_v16_prepass(a, wsb + mask_words_bytes(c.B, c.Lk), stream);
    if (e == hipSuccess) {
        switch (path) {
            case MFA_PATH_GENERIC: e = mfa::launch_generic(a, c.dtype, stream); break;
            case MFA_PATH_MFMA: e = mfa::launch_mfma_prefill(a, c.dtype, stream); break;
            case MFA_PATH_SPLIT_DECODE:
                e = mfa::launch_split_decode(a, nullptr, c.dtype, splits,
                                             reinterpret_cast<float*>(wsb + mask_words_bytes(c.B, c.Lk)),
                                             stream);
                break;
        }
    }
    if (needs_ws && use_pool) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_ERROR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return MFA_SUCCESS;
}

struct LenCall {
    const void *q, *k, *v;
    void* out;
    float* lse;
    const int* d_len;
    int B, R, Lmax, Hq, Hkv, D;
    float scale, softcap;
    int dtype;
};

int validate_len(const LenCall& c) {
    if (c.B != 0 && (!c.q || !c.k || !c.v || !c.out || !c.d_len))
        return fail(MFA_ERROR_INVALID_VALUE, "q, k_cache, v_cache, out and d_len must be non-null");
    if (c.B < 0 || c.R <= 0 || c.Lmax <= 0 || c.Hq <= 0 || c.Hkv <= 0 || c.D <= 0)
        return fail(MFA_ERROR_INVALID_VALUE,
                    "bad dimensions B=%d R=%d Lmax=%d Hq=%d Hkv=%d D=%d (B >= 0; others > 0)",
                    c.B, c.R, c.Lmax, c.Hq, c.Hkv, c.D);
    if (c.Hq % c.Hkv != 0)
        return fail(MFA_ERROR_INVALID_VALUE, "Hkv=%d does not divide Hq=%d", c.Hkv, c.Hq);
    if (!std::isfinite(c.scale) || !std::isfinite(c.softcap))
        return fail(MFA_ERROR_INVALID_VALUE, "scale and softcap must be finite");
    if (c.dtype != MFA_F32 && c.dtype != MFA_F16 && c.dtype != MFA_BF16)
        return fail(MFA_ERROR_NOT_SUPPORTED, "unknown dtype %d", c.dtype);
    if (!mfa::decode_len_supported(c.dtype, c.D, c.R, c.Hq / c.Hkv))
        return fail(MFA_ERROR_NOT_SUPPORTED,
                    "decode over a device length needs fp16/bf16, D in {64,128} and R * Hq/Hkv <= 16 "
                    "(dtype=%d D=%d R=%d Hq/Hkv=%d)", c.dtype, c.D, c.R, c.Hq / c.Hkv);
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.out, 16))
        return fail(MFA_ERROR_INVALID_VALUE, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (!aligned(c.lse, 4) || !aligned(c.d_len, 4))
        return fail(MFA_ERROR_INVALID_VALUE, "lse and d_len must be 4-byte aligned");
    const int64_t q_elems = (int64_t)c.B * c.R * c.Hq * c.D;
    const int64_t kv_elems = (int64_t)c.B * c.Lmax * c.Hkv * c.D;
    if (q_elems < 0 || kv_elems < 0 || (int64_t)c.B * c.R * c.Hq > (int64_t)1 << 30)
        return fail(MFA_ERROR_INVALID_VALUE, "problem too large");
    return MFA_SUCCESS;
}

int len_splits(int B, int Hkv, int Lmax, int group, int splits) {
    if (splits <= 0) splits = mfa::split_decode_default_splits(B, Hkv, Lmax, group);
    return splits > Lmax ? Lmax : splits;
}

int run_len(const LenCall& c, int splits, void* workspace, size_t ws_bytes, hipStream_t stream) {
    int st = validate_len(c);
    if (st != MFA_SUCCESS) return st;
    if (c.B == 0) return MFA_SUCCESS;
    const int group = c.Hq / c.Hkv;
    splits = len_splits(c.B, c.Hkv, c.Lmax, group, splits);
    const size_t need = align256(mfa::split_decode_workspace_bytes(c.B, c.R, c.Hq, c.D, splits));
    const bool use_pool = workspace == nullptr && ws_bytes == 0;
    if (!use_pool) {
        if (!workspace) return fail(MFA_ERROR_INVALID_VALUE, "workspace is null but ws_bytes > 0");
        if (!aligned(workspace, 256)) return fail(MFA_ERROR_INVALID_VALUE, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(MFA_ERROR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    }

    mfa::FwdArgs a{};
    a.q = c.q; a.k = c.k; a.v = c.v; a.out = c.out; a.lse = c.lse;
    a.B = c.B; a.Lq = c.R; a.Lk = c.Lmax; a.Hq = c.Hq; a.Hkv = c.Hkv; a.D = c.D;
    a.group = group;
    a.causal = 1;
    a.q_stride = (int64_t)c.Hq * c.D;
    a.kv_stride = (int64_t)c.Hkv * c.D;
    a.o_stride = (int64_t)c.Hq * c.D;
    a.scale = c.scale;
    a.softcap = c.softcap > 0.0f ? c.softcap : 0.0f;
    const float log2e = 1.4426950408889634f;
    a.score_to_log2 = a.softcap > 0.0f ? log2e : log2e * c.scale;

    void* ws = workspace;
    if (use_pool) {
        const int pst = pool_alloc(&ws, need, stream);
        if (pst != MFA_SUCCESS) return pst;
    }
    hipError_t e = mfa::launch_split_decode(a, c.d_len, c.dtype, splits, static_cast<float*>(ws), stream);
    if (use_pool) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_ERROR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return MFA_SUCCESS;
}

// Per-device addresses of the static scratch of mfa_decode_len_noalloc
// (defined after this namespace), looked up once per device.
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};

int noalloc_scratch(void** p);

struct MaskedCall {
    const void *q, *k, *v;
    void* out;
    float* lse;
    const float* d_mask;
    int B, Lmax, Hq, Hkv, D;
    float scale;
    int window;
    float softcap;
    int dtype;
};

int validate_masked(const MaskedCall& c) {
    if (c.B != 0 && (!c.q || !c.k || !c.v || !c.out || !c.d_mask))
        return fail(MFA_ERROR_INVALID_VALUE, "q, k_cache, v_cache, out and d_mask must be non-null");
    if (c.B < 0 || c.Lmax <= 0 || c.Hq <= 0 || c.Hkv <= 0 || c.D <= 0)
        return fail(MFA_ERROR_INVALID_VALUE,
                    "bad dimensions B=%d Lmax=%d Hq=%d Hkv=%d D=%d (B >= 0; others > 0)",
                    c.B, c.Lmax, c.Hq, c.Hkv, c.D);
    if (c.Hq % c.Hkv != 0)
        return fail(MFA_ERROR_INVALID_VALUE, "Hkv=%d does not divide Hq=%d", c.Hkv, c.Hq);
    if (!std::isfinite(c.scale) || !std::isfinite(c.softcap))
        return fail(MFA_ERROR_INVALID_VALUE, "scale and softcap must be finite");
    if (c.dtype != MFA_F32 && c.dtype != MFA_F16 && c.dtype != MFA_BF16)
        return fail(MFA_ERROR_NOT_SUPPORTED, "unknown dtype %d", c.dtype);
    if (!mfa::split_decode_supported(c.dtype, c.D, 1, c.Hq / c.Hkv))
        return fail(MFA_ERROR_NOT_SUPPORTED,
                    "masked decode needs fp16/bf16, D in {64,128} and Hq/Hkv <= 16 (dtype=%d D=%d Hq/Hkv=%d)",
                    c.dtype, c.D, c.Hq / c.Hkv);
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.out, 16))
        return fail(MFA_ERROR_INVALID_VALUE, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (!aligned(c.lse, 4) || !aligned(c.d_mask, 4))
        return fail(MFA_ERROR_INVALID_VALUE, "lse and d_mask must be 4-byte aligned");
    const int64_t q_elems = (int64_t)c.B * c.Hq * c.D;
    const int64_t kv_elems = (int64_t)c.B * c.Lmax * c.Hkv * c.D;
    if (q_elems < 0 || kv_elems < 0 || (int64_t)c.B * c.Hq > (int64_t)1 << 30)
        return fail(MFA_ERROR_INVALID_VALUE, "problem too large");
    return MFA_SUCCESS;
}

size_t masked_ws_bytes(int B, int Lmax, int Hq, int D, int splits) {
    return mask_words_bytes(B, Lmax) + align256(mfa::split_decode_workspace_bytes(B, 1, Hq, D, splits));
}

int run_masked(const MaskedCall& c, int splits, void* workspace, size_t ws_bytes, hipStream_t stream) {
    int st = validate_masked(c);
    if (st != MFA_SUCCESS) return st;
    if (c.B == 0) return MFA_SUCCESS;
    const int group = c.Hq / c.Hkv;
    splits = len_splits(c.B, c.Hkv, c.Lmax, group, splits);
    const size_t need = masked_ws_bytes(c.B, c.Lmax, c.Hq, c.D, splits);
    const bool use_pool = workspace == nullptr && ws_bytes == 0;
    if (!use_pool) {
        if (!workspace) return fail(MFA_ERROR_INVALID_VALUE, "workspace is null but ws_bytes > 0");
        if (!aligned(workspace, 256)) return fail(MFA_ERROR_INVALID_VALUE, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(MFA_ERROR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    }

    mfa::FwdArgs a{};
    a.q = c.q; a.k = c.k; a.v = c.v; a.out = c.out; a.lse = c.lse;
    a.key_mask = c.d_mask;
    a.B = c.B; a.Lq = 1; a.Lk = c.Lmax; a.Hq = c.Hq; a.Hkv = c.Hkv; a.D = c.D;
    a.group = group;
    a.causal = 1;
    a.window = c.window > 0 ? c.window : 0;
    a.words_per_batch = words_per_batch(c.Lmax);
    a.q_stride = (int64_t)c.Hq * c.D;
    a.kv_stride = (int64_t)c.Hkv * c.D;
    a.o_stride = (int64_t)c.Hq * c.D;
    a.scale = c.scale;
    a.softcap = c.softcap > 0.0f ? c.softcap : 0.0f;
    const float log2e = 1.4426950408889634f;
    a.score_to_log2 = a.softcap > 0.0f ? log2e : log2e * c.scale;

    void* ws = workspace;
    if (use_pool) {
        const int pst = pool_alloc(&ws, need, stream);
        if (pst != MFA_SUCCESS) return pst;
    }
    char* wsb = static_cast<char*>(ws);
    a.mask_words = reinterpret_cast<const uint64_t*>(wsb);
    hipError_t e = mfa::launch_mask_words(a, reinterpret_cast<uint64_t*>(wsb), stream);
    if (e == hipSuccess)
        e = mfa::launch_split_decode(a, nullptr, c.dtype, splits,
                                     reinterpret_cast<float*>(wsb + mask_words_bytes(c.B, c.Lmax)), stream,
                                     /*pos_from_mask=*/true);
    if (use_pool) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_ERROR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return MFA_SUCCESS;
}

int run_packed(const void* qkv, const int* seq_bounds, void* out, float* lse, int L, int H, int D,
               float scale, int window, float softcap, int dtype, hipStream_t stream) {
    if (L != 0 && (!qkv || !seq_bounds || !out))
        return fail(MFA_ERROR_INVALID_VALUE, "qkv, seq_bounds and out must be non-null");
    if (L < 0 || H <= 0 || D <= 0)
        return fail(MFA_ERROR_INVALID_VALUE, "bad dimensions L=%d H=%d D=%d (L >= 0; others > 0)", L, H, D);
    if (!std::isfinite(scale) || !std::isfinite(softcap))
        return fail(MFA_ERROR_INVALID_VALUE, "scale and softcap must be finite");
    if (dtype != MFA_F32 && dtype != MFA_F16 && dtype != MFA_BF16)
        return fail(MFA_ERROR_NOT_SUPPORTED, "unknown dtype %d", dtype);
    if (D != 64 && D != 128)
        return fail(MFA_ERROR_NOT_SUPPORTED, "head dim %d not supported (64 or 128)", D);
    if (!aligned(qkv, 16) || !aligned(out, 16))
        return fail(MFA_ERROR_INVALID_VALUE, "qkv and out must be 16-byte aligned");
    if (!aligned(lse, 4) || !aligned(seq_bounds, 4))
        return fail(MFA_ERROR_INVALID_VALUE, "lse and seq_bounds must be 4-byte aligned");
    if ((int64_t)L * 3 * H * D < 0 || H > (1 << 20))
        return fail(MFA_ERROR_INVALID_VALUE, "problem too large");
    if (L == 0) return MFA_SUCCESS;

    const size_t el = dtype == MFA_F32 ? 4 : 2;
    const char* base = static_cast<const char*>(qkv);
    mfa::FwdArgs a{};
    a.q = base;
    a.k = base + (size_t)H * D * el;
    a.v = base + (size_t)2 * H * D * el;
    a.out = out; a.lse = lse;
    a.B = 1; a.Lq = L; a.Lk = L; a.Hq = H; a.Hkv = H; a.D = D;
    a.group = 1;
    a.causal = 0;
    a.window = window > 0 ? window : 0;
    a.q_offset = 0;
    a.q_stride = (int64_t)3 * H * D;
    a.kv_stride = (int64_t)3 * H * D;
    a.o_stride = (int64_t)H * D;
    a.seq_bounds = seq_bounds;
    a.scale = scale;
    a.softcap = softcap > 0.0f ? softcap : 0.0f;
    const float log2e = 1.4426950408889634f;
    a.score_to_log2 = a.softcap > 0.0f ? log2e : log2e * scale;
    const bool mfma = mfa::mfma_prefill_supported(dtype, D);
    // bf16 on the MFMA kernel: the fp16 copy of V comes from the pool
    const bool v16 = mfma && dtype == MFA_BF16;
    void* ws = nullptr;
    if (v16) {
        const int pst = pool_alloc(&ws, v16_bytes(1, L, H, D, a.kv_stride), stream);
        if (pst != MFA_SUCCESS) return pst;
    }
    hipError_t e = v16 ? mfa::launch_v16_prepass(a, ws, stream) : hipSuccess;
    if (e == hipSuccess) e = mfma ? mfa::launch_mfma_prefill(a, dtype, stream) : mfa::launch_generic(a, dtype, stream);
    if (v16) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_ERROR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return MFA_SUCCESS;
}

// Per-row positions and bounds, then (bf16 on the MFMA kernel) the fp16 copy
// of V.
size_t varlen_ws_bytes(int Tq, int Tk, int Hkv, int D, int dtype) {
    size_t ws = align256((size_t)Tq * 3 * sizeof(int));
    if (dtype == MFA_BF16 && mfa::mfma_prefill_supported(dtype, D) && Tk > 0)
        ws += v16_bytes(1, Tk, Hkv, D, (int64_t)Hkv * D);
    return ws;
}

int run_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int* cu_q,
               const int* cu_k, int batch, int Tq, int Tk, int Hq, int Hkv, int D, float scale, int causal,
               int window, float softcap, int dtype, void* workspace, size_t ws_bytes, hipStream_t stream) {
    if ((Tq != 0 && (!q || !out)) || (Tk != 0 && (!k || !v)) || !cu_q || !cu_k)
        return fail(MFA_ERROR_INVALID_VALUE, "q, k, v, out, cu_seqlens_q and cu_seqlens_k must be non-null");
    if (batch < 0 || Tq < 0 || Tk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || (batch == 0 && Tq > 0))
        return fail(MFA_ERROR_INVALID_VALUE,
                    "bad dimensions batch=%d Tq=%d Tk=%d Hq=%d Hkv=%d D=%d (batch >= 1 when Tq > 0)",
                    batch, Tq, Tk, Hq, Hkv, D);
    if (Hq % Hkv != 0) return fail(MFA_ERROR_INVALID_VALUE, "Hkv=%d does not divide Hq=%d", Hkv, Hq);
    if (!std::isfinite(scale) || !std::isfinite(softcap))
        return fail(MFA_ERROR_INVALID_VALUE, "scale and softcap must be finite");
    if (dtype != MFA_F32 && dtype != MFA_F16 && dtype != MFA_BF16)
        return fail(MFA_ERROR_NOT_SUPPORTED, "unknown dtype %d", dtype);
    if (D != 64 && D != 128)
        return fail(MFA_ERROR_NOT_SUPPORTED, "head dim %d not supported (64 or 128)", D);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(MFA_ERROR_INVALID_VALUE, "q, k, v and out must be 16-byte aligned");
    if (!aligned(lse, 4) || !aligned(cu_q, 4) || !aligned(cu_k, 4))
        return fail(MFA_ERROR_INVALID_VALUE, "lse and the prefix sums must be 4-byte aligned");
    if ((int64_t)Tq * Hq * D < 0 || (int64_t)Tk * Hkv * D < 0 || Hq > (1 << 20))
        return fail(MFA_ERROR_INVALID_VALUE, "problem too large");
    if (Tq == 0) return MFA_SUCCESS;
    const size_t need = varlen_ws_bytes(Tq, Tk, Hkv, D, dtype);
    const bool use_pool = workspace == nullptr && ws_bytes == 0;
    if (!use_pool) {
        if (!workspace) return fail(MFA_ERROR_INVALID_VALUE, "workspace is null but ws_bytes > 0");
        if (!aligned(workspace, 256)) return fail(MFA_ERROR_INVALID_VALUE, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(MFA_ERROR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    }
    void* ws = workspace;
    if (use_pool) {
        const int pst = pool_alloc(&ws, need, stream);
        if (pst != MFA_SUCCESS) return pst;
    }
    int* row_pos = static_cast<int*>(ws);
    int* bounds = row_pos + Tq;

    mfa::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.B = 1; a.Lq = Tq; a.Lk = Tk > 0 ? Tk : 1; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
    a.group = Hq / Hkv;
    a.causal = causal ? 1 : 0;
    a.window = window > 0 ? window : 0;
    a.q_offset = 0;
    a.q_stride = (int64_t)Hq * D;
    a.kv_stride = (int64_t)Hkv * D;
    a.o_stride = (int64_t)Hq * D;
    a.seq_bounds = bounds;
    a.row_pos = row_pos;
    a.scale = scale;
    a.softcap = softcap > 0.0f ? softcap : 0.0f;
    const float log2e = 1.4426950408889634f;
    a.score_to_log2 = a.softcap > 0.0f ? log2e : log2e * scale;
    hipError_t e = mfa::launch_varlen_rows(cu_q, cu_k, batch, Tq, Tk, row_pos, bounds, stream);
    const bool mfma = mfa::mfma_prefill_supported(dtype, D);
    if (e == hipSuccess && mfma && dtype == MFA_BF16 && Tk > 0)
        e = mfa::launch_v16_prepass(a, static_cast<char*>(ws) + align256((size_t)Tq * 3 * sizeof(int)), stream);
    if (e == hipSuccess) e = mfma ? mfa::launch_mfma_prefill(a, dtype, stream) : mfa::launch_generic(a, dtype, stream);
    if (use_pool) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_ERROR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return MFA_SUCCESS;
}

}  // namespace

// Scratch of mfa_decode_len_noalloc: the split partials of that call live
// here rather than in caller or pool memory.  Every device that runs the call
// holds its own copy of the array until the process ends.  On the host the
// name only stands in for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device, never the name itself.
static __device__ __align__(256) unsigned char scratch[MFA_NOALLOC_SCRATCH_BYTES];

namespace {

// This device's address of `scratch`, found with hipGetSymbolAddress on the
// first call made with the device current and kept for later calls (a failed
// lookup is kept too and reported by every later call on that device).
int noalloc_scratch(void** p) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_ERROR_HIP, "hipGetDevice failed");
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MFA_ERROR_NOT_SUPPORTED, "device %d is beyond the %d the library serves", dev, kMaxDevices);
    std::call_once(g_scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) (void)hipGetLastError();
        g_scratch_err[dev] = e != hipSuccess ? e : (ptr ? hipSuccess : hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess)
        return fail(MFA_ERROR_HIP, "no address for the static scratch on device %d: %s", dev,
                    hipGetErrorString(g_scratch_err[dev]));
    *p = g_scratch_ptr[dev];
    return MFA_SUCCESS;
}

}  // namespace

namespace mfa {
hipEvent_t instr_event_begin() { return g_ev_begin; }
hipEvent_t instr_event_end() { return g_ev_end; }
}  // namespace mfa

extern "C" {

int mfa_varlen_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                   const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q, int total_k,
                   int Hq, int Hkv, int D, float scale, int causal, int window, float softcap, int dtype,
                   void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    return run_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, Hq, Hkv, D,
                      scale, causal, window, softcap, dtype, workspace, ws_bytes,
                      static_cast<hipStream_t>(stream));
}

size_t mfa_varlen_workspace_size(int total_q, int total_k, int Hkv, int D, int dtype) {
    if (total_q <= 0 || total_k < 0 || Hkv <= 0 || D <= 0) return 0;
    return varlen_ws_bytes(total_q, total_k, Hkv, D, dtype);
}

int mfa_packed_qkv_fwd(const void* qkv, const int* seq_bounds, void* out, float* lse,
                       int L, int H, int D, float scale, int window, float softcap, int dtype,
                       void* stream) {
    g_last_error.clear();
    return run_packed(qkv, seq_bounds, out, lse, L, H, D, scale, window, softcap, dtype,
                      static_cast<hipStream_t>(stream));
}

int mfa_decode_len(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                   const int* d_len, int B, int R, int Lmax, int Hq, int Hkv, int D,
                   float scale, float softcap, int dtype, int splits,
                   void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    LenCall c{q, k_cache, v_cache, out, lse, d_len, B, R, Lmax, Hq, Hkv, D, scale, softcap, dtype};
    return run_len(c, splits, workspace, ws_bytes, static_cast<hipStream_t>(stream));
}

int mfa_decode_len_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                           const int* d_len, int B, int R, int Lmax, int Hq, int Hkv, int D,
                           float scale, float softcap, int dtype, int splits, void* stream) {
    g_last_error.clear();
    LenCall c{q, k_cache, v_cache, out, lse, d_len, B, R, Lmax, Hq, Hkv, D, scale, softcap, dtype};
    int st = validate_len(c);
    if (st != MFA_SUCCESS || B == 0) return st;
    splits = len_splits(B, Hkv, Lmax, Hq / Hkv, splits);
    const size_t need = align256(mfa::split_decode_workspace_bytes(B, R, Hq, D, splits));
    if (need > MFA_NOALLOC_SCRATCH_BYTES)
        return fail(MFA_ERROR_INVALID_VALUE,
                    "these sizes need %zu bytes of scratch (B=%d R=%d Hq=%d D=%d, %d splits) but the static "
                    "scratch holds %zu: pass fewer splits, or call mfa_decode_len with a workspace",
                    need, B, R, Hq, D, splits, (size_t)MFA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st != MFA_SUCCESS) return st;
    // every partial slot the combine reads is written by the split kernel of
    // the same call first, so nothing in the scratch needs clearing
    return run_len(c, splits, ws, MFA_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream));
}

size_t mfa_decode_len_workspace_size(int B, int R, int Lmax, int Hq, int Hkv, int D, int dtype, int splits) {
    if (B <= 0 || R <= 0 || Lmax <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return 0;
    if (!mfa::decode_len_supported(dtype, D, R, Hq / Hkv)) return 0;
    splits = len_splits(B, Hkv, Lmax, Hq / Hkv, splits);
    return align256(mfa::split_decode_workspace_bytes(B, R, Hq, D, splits));
}

int mfa_decode_masked(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                      const float* d_mask, int B, int Lmax, int Hq, int Hkv, int D,
                      float scale, int window, float softcap, int dtype, int splits,
                      void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    MaskedCall c{q, k_cache, v_cache, out, lse, d_mask, B, Lmax, Hq, Hkv, D, scale, window, softcap, dtype};
    return run_masked(c, splits, workspace, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t mfa_decode_masked_workspace_size(int B, int Lmax, int Hq, int Hkv, int D, int dtype, int splits) {
    if (B <= 0 || Lmax <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return 0;
    if (!mfa::split_decode_supported(dtype, D, 1, Hq / Hkv)) return 0;
    splits = len_splits(B, Hkv, Lmax, Hq / Hkv, splits);
    return masked_ws_bytes(B, Lmax, Hq, D, splits);
}

int mfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
            int B, int Lq, int Lk, int Hq, int Hkv, int D,
            float scale, int causal, int window, int q_offset, float softcap,
            const float* key_mask, int dtype, void* stream) {
    g_last_error.clear();
    Call c{q, k, v, out, lse, B, Lq, Lk, Hq, Hkv, D, scale, causal, window, q_offset, softcap, key_mask, dtype};
    return run(c, MFA_PATH_AUTO, 0, nullptr, 0, static_cast<hipStream_t>(stream));
}

int mfa_fwd_bias_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int Lq, int Lk, int Hq, int Hkv, int D,
                         float scale, int causal, int window, int q_offset, float softcap,
                         const float* key_mask, const float* bias, int bias_B, int bias_H, int bias_Lq,
                         int bias_Lk, float dropout_p, unsigned long long seed, int dtype, void* stream) {
    g_last_error.clear();
    Call c{q, k, v, out, lse, B, Lq, Lk, Hq, Hkv, D, scale, causal, window, q_offset, softcap, key_mask, dtype};
    c.bias = bias;
    c.bias_dims[0] = bias_B; c.bias_dims[1] = bias_H; c.bias_dims[2] = bias_Lq; c.bias_dims[3] = bias_Lk;
    c.dropout_p = dropout_p;
    c.seed = seed;
    return run(c, MFA_PATH_AUTO, 0, nullptr, 0, static_cast<hipStream_t>(stream));
}

size_t mfa_bwd_workspace_size(int B, int Lq, int Hq) {
    if (B <= 0 || Lq <= 0 || Hq <= 0) return 0;
    return align256((size_t)B * Hq * Lq * sizeof(float));
}

int mfa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
            void* dq, void* dk, void* dv, int B, int Lq, int Lk, int Hq, int Hkv, int D,
            float scale, int causal, int window, int q_offset, float softcap,
            const float* key_mask, const float* bias, int bias_B, int bias_H, int bias_Lq, int bias_Lk,
            float dropout_p, unsigned long long seed, int dtype, void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    Call c{q, k, v, const_cast<void*>(out), const_cast<float*>(lse), B, Lq, Lk, Hq, Hkv, D, scale, causal, window,
           q_offset, softcap, key_mask, dtype};
    c.bias = bias;
    c.bias_dims[0] = bias_B; c.bias_dims[1] = bias_H; c.bias_dims[2] = bias_Lq; c.bias_dims[3] = bias_Lk;
    c.dropout_p = dropout_p;
    c.seed = seed;
    int st = validate(c);
    if (st != MFA_SUCCESS) return st;
    const bool q_empty = B == 0 || Lq == 0;
    if ((!q_empty && (!dout || !lse || !dq)) || (B != 0 && (!dk || !dv)))
        return fail(MFA_ERROR_INVALID_VALUE, "dout, lse, dq, dk and dv must be non-null");
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return fail(MFA_ERROR_INVALID_VALUE, "dout, dq, dk and dv must be 16-byte aligned");
    if (B == 0) return MFA_SUCCESS;   // (Lq = 0 still writes the zero dK and dV)
    const size_t need = mfa_bwd_workspace_size(B, Lq, Hq);
    const bool use_pool = workspace == nullptr && ws_bytes == 0;
    if (!use_pool) {
        if (!workspace) return fail(MFA_ERROR_INVALID_VALUE, "workspace is null but ws_bytes > 0");
        if (!aligned(workspace, 256)) return fail(MFA_ERROR_INVALID_VALUE, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(MFA_ERROR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    }
    mfa::FwdArgs a = make_args(c);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // With dropout the dK/dV kernel can store the keep bits for the dQ kernel,
    // behind Delta in the workspace: in the pool's, or in a caller's that has
    // room for them (up to 4 GiB; otherwise each kernel evaluates its own).
    size_t keep = mfa::bwd_keep_bits_bytes(a, dtype);
    if (keep > ((size_t)4 << 30) || (!use_pool && ws_bytes < need + keep)) keep = 0;
    void* ws = workspace;
    if (use_pool && need + keep > 0) {
        int pst = pool_alloc(&ws, need + keep, s);
        if (pst == MFA_ERROR_OUT_OF_MEMORY && keep > 0) {   // without room for the pattern
            g_last_error.clear();
            keep = 0;
            pst = pool_alloc(&ws, need, s);
        }
        if (pst != MFA_SUCCESS) return pst;
    }
    const size_t total = need + keep;
    if (keep > 0) a.keep_bits = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + need);
    hipError_t e = mfa::launch_backward(a, dout, static_cast<float*>(ws), dq, dk, dv, dtype, s);
    if (use_pool && total > 0) {
        hipError_t e2 = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_ERROR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return MFA_SUCCESS;
}

size_t mfa_fwd_workspace_size(int B, int Lq, int Lk, int Hq, int Hkv, int D, int dtype) {
    if (B <= 0 || Lq <= 0 || Lk <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return 0;
    const int path = auto_path(B, Lq, Lk, Hq, Hkv, D, dtype);
    const int splits = path == MFA_PATH_SPLIT_DECODE
                           ? mfa::split_decode_default_splits(B, Hkv, Lk, Hq / Hkv) : 0;
    return workspace_bytes(B, Lq, Lk, Hq, Hkv, D, dtype, path, splits > Lk ? Lk : splits);
}

int mfa_fwd_ws(const void* q, const void* k, const void* v, void* out, float* lse,
               int B, int Lq, int Lk, int Hq, int Hkv, int D,
               float scale, int causal, int window, int q_offset, float softcap,
               const float* key_mask, int dtype, void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    Call c{q, k, v, out, lse, B, Lq, Lk, Hq, Hkv, D, scale, causal, window, q_offset, softcap, key_mask, dtype};
    if (!workspace && ws_bytes == 0) {
        // nothing given: valid only when the plan needs no workspace
        const int p = auto_path(B, Lq, Lk, Hq, Hkv, D, dtype);
        if (mfa_fwd_workspace_size(B, Lq, Lk, Hq, Hkv, D, dtype) > 0 &&
            (key_mask || p == MFA_PATH_SPLIT_DECODE || (p == MFA_PATH_MFMA && dtype == MFA_BF16)))
            return fail(MFA_ERROR_INVALID_VALUE, "this call needs a workspace");
    }
    return run(c, MFA_PATH_AUTO, 0, workspace, ws_bytes, static_cast<hipStream_t>(stream));
}

int mfa_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
               int B, int Lq, int Lk, int Hq, int Hkv, int D,
               float scale, int causal, int window, int q_offset, float softcap,
               const float* key_mask, int dtype, int path, int splits,
               void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    Call c{q, k, v, out, lse, B, Lq, Lk, Hq, Hkv, D, scale, causal, window, q_offset, softcap, key_mask, dtype};
    return run(c, path, splits, workspace, ws_bytes, static_cast<hipStream_t>(stream));
}

int mfa_fwd_plan(int B, int Lq, int Lk, int Hq, int Hkv, int D, int dtype, int* splits) {
    int s = 0;
    int path = MFA_PATH_GENERIC;
    if (Hkv > 0 && Hq > 0 && Hq % Hkv == 0) {
        path = auto_path(B, Lq, Lk, Hq, Hkv, D, dtype);
        if (path == MFA_PATH_SPLIT_DECODE) {
            s = mfa::split_decode_default_splits(B, Hkv, Lk, Hq / Hkv);
            if (s > Lk) s = Lk;
        }
    }
    if (splits) *splits = s;
    return path;
}

const char* mfa_status_string(int status) {
    switch (status) {
        case MFA_SUCCESS: return "success";
        case MFA_ERROR_INVALID_VALUE: return "invalid value";
        case MFA_ERROR_NOT_SUPPORTED: return "not supported";
        case MFA_ERROR_HIP: return "HIP error";
        case MFA_ERROR_OUT_OF_MEMORY: return "out of memory";
    }
    return "unknown status";
}

const char* mfa_last_error(void) { return g_last_error.c_str(); }

void mfa_set_kernel_events(void* begin, void* end) {
    g_ev_begin = static_cast<hipEvent_t>(begin);
    g_ev_end = static_cast<hipEvent_t>(end);
}

int mfa_version(void) { return 300; }

}  // extern "C"
