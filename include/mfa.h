/*
 * mfa.h -- C ABI of libmfa, a fused attention forward for AMD Instinct MI355X
 * (gfx950).
 *
 * One operation:  O = softmax(scale * Q K^T + masks) V,  with the per-row
 * natural-log log-sum-exp LSE saved alongside.  It is computed tile by tile
 * with an online softmax, so the Lq x Lk score matrix never exists in memory
 * (vision_rs flash_attn2.rs, module doc and forward kernel; brotensor
 * flash_attention.h, flash_attention_forward: tiled online softmax with fp32
 * accumulation).
 *
 * Feature set (brotensor flash_attention.h; ferrotensor attention.rs):
 *   - grouped-query heads: Hkv divides Hq and q head h reads kv head
 *     h / (Hq / Hkv) (flash_attention_gqa_forward, flash_attention_decode);
 *   - queries sit at absolute positions aq = i + q_offset of the key axis
 *     (flash_attention_windowed_forward; AttentionOptions::causal_offset);
 *   - causal: key j visible only when j <= aq; with window > 0 also
 *     j >= aq - window + 1 (flash_attention_windowed_forward, causal form);
 *   - bidirectional (causal = 0) with window > 0: keys aq - window/2 through
 *     aq + window/2, integer halving, clipped to [0, Lk) (same function,
 *     bidirectional form); window <= 0 means no window in either form;
 *   - key mask: key j of batch b is dropped unless key_mask[b*Lk + j] > 0.5
 *     (flash_attention_forward mask description; flash_attention_backward
 *     threshold);
 *   - soft-cap > 0: each scaled score s becomes softcap * tanh(s / softcap)
 *     before masking and the softmax (flash_attention_decode);
 *   - Lq = 1 decode over a long cache runs as a split over the keys plus a
 *     combine pass (flash_attention_decode_len: the work divides the valid
 *     keys and split points only change rounding).
 *
 * Layouts (row-major, contiguous, all in device memory):
 *   q, out     [B, Lq, Hq, D]   element type `dtype`
 *   k, v       [B, Lk, Hkv, D]  element type `dtype`
 *   lse        [B, Hq, Lq]      float32, may be NULL (then not written)
 *   key_mask   [B, Lk]          float32, may be NULL (no mask)
 * q, k, v and out must be 16-byte aligned; lse and key_mask 4-byte aligned.
 *
 * A row with no visible key gets O = 0 and LSE = -inf.
 *
 * Rows nobody uses: the K and V rows of masked keys may hold anything (NaN
 * in unwritten cache slots, say).  They never reach O: their V rows are not
 * fetched, and a score from their K rows is replaced, never used in
 * arithmetic.  The split decode kernels (mfa_fwd at Lq = 1 on that path,
 * mfa_decode_len, mfa_decode_masked) also never fetch rows outside every
 * query's window or past the length.  The prefill kernels read every
 * unmasked row of each key tile they visit, including rows that the causal
 * or window bounds hide from some queries, so unmasked rows must hold finite
 * values.  Rows at or past Lk are never read.  The backward (mfa_bwd) treats
 * masked rows the same way: they never reach a gradient, and the gradients
 * of masked keys are zero.
 *
 * Ownership: every pointer is caller-owned device memory.  The library keeps
 * no reference after a call returns and writes only out, lse and (for the
 * _ws / _ex forms) the workspace.  In every entry point, a pointer to a tensor
 * that holds no element (for instance q and out when B = 0 or Lq = 0, k and v
 * when B = 0, or the key packing of mfa_varlen_fwd when total_k = 0) may be
 * NULL: nothing is read from or written to it.
 *
 * Streams: every call is asynchronous on `stream` (a hipStream_t; NULL is the
 * null stream) and never synchronises the device.  A fault in a kernel shows
 * at the caller's next synchronisation.
 *
 * Errors: arguments are checked on the host before any device work; on a
 * non-zero return nothing has been launched and nothing written.
 * mfa_last_error() then holds a description (per host thread).
 */
#ifndef MFA_H
#define MFA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out. */
typedef enum { MFA_F32 = 0, MFA_F16 = 1, MFA_BF16 = 2 } mfa_dtype;

typedef enum {
    MFA_SUCCESS = 0,
    /* a null pointer, a misaligned pointer, a dimension < 0 (or Hq, Hkv, D,
     * Lk = 0), Hq % Hkv != 0, q_offset < 0, q_offset + Lq > Lk, a non-finite
     * scale or softcap, or a workspace that is too small */
    MFA_ERROR_INVALID_VALUE = 1,
    /* D not in {64, 128}, an unknown dtype, or a forced path that cannot
     * serve the arguments */
    MFA_ERROR_NOT_SUPPORTED = 2,
    /* a HIP runtime call or kernel launch failed */
    MFA_ERROR_HIP = 3,
    /* the workspace pool could not provide device memory */
    MFA_ERROR_OUT_OF_MEMORY = 4
} mfa_status;

/* Kernel path selection for mfa_fwd_ex. */
typedef enum {
    MFA_PATH_AUTO = 0,        /* what mfa_fwd chooses */
    MFA_PATH_GENERIC = 1,     /* fp32-arithmetic tiled kernel, every dtype */
    MFA_PATH_MFMA = 2,        /* bf16/fp16 MFMA prefill kernel */
    MFA_PATH_SPLIT_DECODE = 3 /* Lq = 1 split-over-keys kernel + combine */
} mfa_path;

/*
 * Attention forward.  B = 0 or Lq = 0 is an empty call that succeeds without
 * launching anything.  `scale` is used as given (the conventional value is
 * 1/sqrt(D)).  Any workspace the chosen kernels need comes from a
 * stream-ordered memory pool that the library creates on each device on first
 * use (it keeps freed memory for later calls and never changes the device's
 * default pool) and is released in stream order.
 *
 * Precision: fp16/bf16 inputs multiply in their own type with fp32
 * accumulation; the softmax weights enter P.V as fp16 (11 significant bits)
 * for both, so a bf16 call on the MFMA prefill first converts V to an fp16
 * copy in the workspace (B * Lk * Hkv * D * 2 bytes, plus a flag byte per
 * 64 keys).  A (batch, kv head) whose V holds a magnitude of 65504 or more
 * runs on bf16 operands (8-bit weights) instead.
 */
int mfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
            int B, int Lq, int Lk, int Hq, int Hkv, int D,
            float scale, int causal, int window, int q_offset, float softcap,
            const float* key_mask, int dtype, void* stream);

/*
 * mfa_fwd with two more of the pages' forward features (ferrotensor
 * attention.rs, flash_attention_v2: an additive mask whose size-1 dimensions
 * broadcast, and attention dropout driven by a seed).
 *
 *   bias        float32, contiguous [bias_B, bias_H, bias_Lq, bias_Lk], each
 *               dimension 1 (broadcast) or B, Hq, Lq, Lk; added to the
 *               scaled (and soft-capped) score before the causal, window and
 *               key masks; may be NULL; finite values or -inf
 *   dropout_p   in [0, 1): each normalised weight is dropped with this
 *               probability and a kept one divided by 1 - p; the saved LSE
 *               is the undropped one.  Weight (b, hq, i, j) is kept iff
 *               16-bit field f = j mod 16 (bits 16 (f mod 4) .. +15 of word
 *               floor(f / 4)) of the Philox4x64-10 block with counter
 *               (floor(j / 16), i, hq, b) and key (seed mod 2^32, 0) is at
 *               least round(p * 2^16), so a pattern is reproducible from the
 *               seed alone; only the seed's low 32 bits count
 *               (ferrotensor attention.rs, AttentionOptions).
 *
 * A row whose every visible key has a bias of -inf gets O = 0, LSE = -inf.
 * An fp16/bf16 call with D 64 or 128 runs on the MFMA prefill kernel unless
 * it has a bias that kernel cannot read four keys at a time (it needs
 * bias_Lk = Lk, Lk a multiple of 4 and a 16-byte aligned bias); every other
 * call runs on the fp32-arithmetic kernel (MFA_PATH_GENERIC).  Other
 * arguments, errors and streams as for mfa_fwd; a bias dimension other than
 * 1 or full size, or p outside [0, 1), is MFA_ERROR_INVALID_VALUE.
 */
int mfa_fwd_bias_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int Lq, int Lk, int Hq, int Hkv, int D,
                         float scale, int causal, int window, int q_offset, float softcap,
                         const float* key_mask, const float* bias, int bias_B, int bias_H, int bias_Lq,
                         int bias_Lk, float dropout_p, unsigned long long seed, int dtype, void* stream);

/*
 * Backward of mfa_fwd / mfa_fwd_bias_dropout: the gradients dQ, dK, dV of a
 * loss for its gradient dout with respect to the output (vision_rs
 * flash_attn2.rs, backward kernels; ferrotensor attention.rs,
 * flash_attention_v2_backward_with: the same options and mask as the forward,
 * dropout regenerated from the seed, no gradient for the additive mask).
 *
 *   out, dout     [B, Lq, Hq, D]   the forward's output and its gradient
 *   lse           [B, Hq, Lq]      float32, the forward's saved LSE
 *   dq            [B, Lq, Hq, D]   written, element type `dtype`
 *   dk, dv        [B, Lk, Hkv, D]  written (summed over the Hq/Hkv query
 *                                  heads that share each kv head)
 * Every other argument must repeat the forward call's.  The weights are
 * recomputed from q, k and lse (P = exp(s - LSE)); with Delta = <dO, O> per
 * row, dS = P (Z <dO, V> - Delta) and the chain rule through the scale and
 * soft-cap.  Each gradient element is written by one workgroup, with no
 * atomics, so a call is deterministic.  fp16/bf16 calls with D 64 or 128 run
 * on the matrix cores (P and dS rounded to the input type as operands, fp32
 * accumulation); the others in fp32 arithmetic.  The
 * workspace holds Delta: caller-owned (256-byte
 * aligned, at least mfa_bwd_workspace_size bytes) or NULL with ws_bytes = 0
 * for the stream-ordered pool.  With dropout on the matrix cores (fp16 and
 * bf16, D = 64 or 128),
 * a workspace with room for another
 * 2 * B * Hq * ceil(Lk / 16) * Lq bytes after those (up to 4 GiB; the pool
 * always gives it) also holds the dropout pattern, evaluated once by the
 * dK/dV kernel and read by the dQ kernel; with a smaller one each kernel
 * evaluates the pattern itself.  The gradients are the same either way.  B = 0 does nothing; Lq = 0 writes zero dK,
 * dV.  Errors as for mfa_fwd_bias_dropout, plus null or misaligned
 * out/dout/lse/dq/dk/dv.
 */
int mfa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
            void* dq, void* dk, void* dv, int B, int Lq, int Lk, int Hq, int Hkv, int D,
            float scale, int causal, int window, int q_offset, float softcap,
            const float* key_mask, const float* bias, int bias_B, int bias_H, int bias_Lq, int bias_Lk,
            float dropout_p, unsigned long long seed, int dtype, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes mfa_bwd needs (0 when B, Lq or Hq is 0). */
size_t mfa_bwd_workspace_size(int B, int Lq, int Hq);

/* Workspace bytes that mfa_fwd_ws needs for these sizes (0 if none); the
 * figure covers every flag combination. */
size_t mfa_fwd_workspace_size(int B, int Lq, int Lk, int Hq, int Hkv, int D, int dtype);

/* mfa_fwd with a caller-owned device workspace of ws_bytes bytes (256-byte
 * aligned, at least mfa_fwd_workspace_size).  The workspace must not be used
 * by other work until this call's kernels finish on `stream`. */
int mfa_fwd_ws(const void* q, const void* k, const void* v, void* out, float* lse,
               int B, int Lq, int Lk, int Hq, int Hkv, int D,
               float scale, int causal, int window, int q_offset, float softcap,
               const float* key_mask, int dtype,
               void* workspace, size_t ws_bytes, void* stream);

/*
 * mfa_fwd_ws with the kernel path forced (`path`, an mfa_path) and, for the
 * split decode, the number of key splits (`splits` <= 0 chooses).  Returns
 * MFA_ERROR_NOT_SUPPORTED when the forced path cannot serve the arguments.
 * Paths differ only in rounding; the test suite uses this to compare them.
 * workspace may be NULL when ws_bytes is 0, in which case the pool is used.
 */
int mfa_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
               int B, int Lq, int Lk, int Hq, int Hkv, int D,
               float scale, int causal, int window, int q_offset, float softcap,
               const float* key_mask, int dtype, int path, int splits,
               void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode over a fixed-capacity KV cache whose valid length is read on the
 * device (brotensor flash_attention.h, flash_attention_decode_len).  Batch b
 * holds R query rows, the last R positions of its first len_b = d_len[b] cache
 * rows: row r attends causally to keys 0 .. len_b - R + r (the first
 * len_b - R + 1 + r keys), with GQA and the optional soft-cap as in mfa_fwd.
 * The launch shape depends only on the capacity Lmax, never on the lengths,
 * so the call can be captured once in a HIP graph and replayed while the
 * caller rewrites d_len between replays; the key splits divide each batch's
 * valid keys, so rows past the length are neither read nor computed.
 *
 *   q, out             [B, R, Hq, D]     element type `dtype` (fp16 or bf16)
 *   k_cache, v_cache   [B, Lmax, Hkv, D] element type `dtype`
 *   lse                [B, Hq, R]        float32, may be NULL
 *   d_len              [B]               int32 in device memory, read by the
 *                                        kernels when they run; values are
 *                                        clamped to [0, Lmax]
 *
 * A row that sees no key (len_b = 0, or len_b < R for the first rows) gets
 * O = 0 and LSE = -inf.  Requires D in {64, 128} and R * Hq/Hkv <= 16
 * (otherwise MFA_ERROR_NOT_SUPPORTED).  `splits` <= 0 chooses the split count
 * from B, Hkv and Lmax.  The workspace is caller-owned (256-byte aligned, at
 * least mfa_decode_len_workspace_size bytes, not used by other work until
 * this call's kernels finish); workspace = NULL with ws_bytes = 0 takes it
 * from the stream-ordered pool instead (not for graph capture).  q, k_cache,
 * v_cache and out must be 16-byte aligned, lse and d_len 4-byte aligned.
 * Errors, ownership and streams as for mfa_fwd.
 */
int mfa_decode_len(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                   const int* d_len, int B, int R, int Lmax, int Hq, int Hkv, int D,
                   float scale, float softcap, int dtype, int splits,
                   void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes mfa_decode_len needs for these sizes and split count
 * (`splits` <= 0: the count it would choose); 0 for unsupported arguments. */
size_t mfa_decode_len_workspace_size(int B, int R, int Lmax, int Hq, int Hkv, int D, int dtype,
                                     int splits);

/* Bytes of device scratch that mfa_decode_len_noalloc holds on each device. */
#define MFA_NOALLOC_SCRATCH_BYTES ((size_t)16 * 1024 * 1024)

/*
 * mfa_decode_len for callers that cannot allocate device memory or hand in a
 * workspace: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.  Same arguments (minus the workspace), checks,
 * kernels and results as mfa_decode_len with the same split count; the split
 * partials go to a static device array of MFA_NOALLOC_SCRATCH_BYTES that each
 * device holds from its first such call until the process ends.  The call
 * itself allocates nothing: its first call on a device only looks up that
 * array's address there.  Sizes whose workspace
 * (mfa_decode_len_workspace_size) exceeds MFA_NOALLOC_SCRATCH_BYTES are
 * rejected with MFA_ERROR_INVALID_VALUE before any device work (a smaller
 * `splits` shrinks it).  Every call on one device shares its array, so calls
 * whose kernels overlap on one device (other streams, or other host threads)
 * race and give undefined results; calls in order on one stream are safe.
 */
int mfa_decode_len_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                           const int* d_len, int B, int R, int Lmax, int Hq, int Hkv, int D,
                           float scale, float softcap, int dtype, int splits, void* stream);

/*
 * Single-query decode over a fixed-capacity KV cache whose valid rows are
 * marked by a key mask in device memory (brotensor flash_attention.h,
 * flash_attention_decode_masked: the graph-capturable twin of the plain
 * decode, validity kept in the mask, fully masked key tiles skipped without
 * touching K/V).  For batch b, key j is valid when d_mask[b*Lmax + j] > 0.5.
 * The query's position p_b is the highest valid key index; key j is used
 * when it is valid and, with window > 0, also j > p_b - window, i.e. j in
 * [max(0, p_b - window + 1), p_b]; window <= 0 uses every valid key.  GQA,
 * scale and soft-cap as in mfa_fwd.
 *
 *   q, out             [B, 1, Hq, D]     element type `dtype` (fp16 or bf16)
 *   k_cache, v_cache   [B, Lmax, Hkv, D] element type `dtype`
 *   lse                [B, Hq, 1]        float32, may be NULL
 *   d_mask             [B, Lmax]         float32 in device memory, read by the
 *                                        kernels when they run
 *
 * p_b is found on the device, so the launch shape depends only on B, Lmax,
 * Hq, Hkv and D: the call can be captured once in a HIP graph and replayed
 * while the caller rewrites d_mask between replays.  The key splits divide
 * the tiles of [max(0, p_b - window + 1), p_b] (or [0, p_b]); tiles holding
 * no valid key are skipped before any K/V read.  With the prefix mask of n
 * valid keys the result is bit-identical to mfa_decode_len with R = 1,
 * d_len[b] = n and the same split count (the same tiles and arithmetic).  A
 * batch with no valid key gets O = 0 and LSE = -inf.  Requires D in
 * {64, 128} and Hq/Hkv <= 16 (otherwise MFA_ERROR_NOT_SUPPORTED).  `splits`
 * <= 0 chooses the split count from B, Hkv and Lmax.  The workspace holds the
 * packed mask bits and the split partials: caller-owned (256-byte aligned, at
 * least mfa_decode_masked_workspace_size bytes, not used by other work until
 * this call's kernels finish), or NULL with ws_bytes = 0 for the
 * stream-ordered pool (not for graph capture).  q, k_cache, v_cache and out
 * 16-byte aligned, lse and d_mask 4-byte aligned.  Errors, ownership and
 * streams as for mfa_fwd.
 */
int mfa_decode_masked(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                      const float* d_mask, int B, int Lmax, int Hq, int Hkv, int D,
                      float scale, int window, float softcap, int dtype, int splits,
                      void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes mfa_decode_masked needs for these sizes and split count
 * (`splits` <= 0: the count it would choose); 0 for unsupported arguments. */
size_t mfa_decode_masked_workspace_size(int B, int Lmax, int Hq, int Hkv, int D, int dtype, int splits);

/*
 * Bidirectional self-attention over many independent sequences packed back to
 * back in one fused QKV tensor, with no padding (brotensor flash_attention.h,
 * flash_attention_packed_qkv_forward: the encoder-batching entry point).
 *
 *   qkv         [L, 3, H, D]  each row holds its H query heads, then its H key
 *                             heads, then its H value heads (the output of one
 *                             fused QKV projection); fp32, fp16 or bf16
 *   seq_bounds  [L, 2] int32  row r belongs to the sequence of rows
 *                             [seq_bounds[r][0], seq_bounds[r][1]), which must
 *                             contain r; sequences lie back to back
 *   out         [L, H, D]     element type `dtype`
 *   lse         [H, L]        float32, natural log, may be NULL
 *
 * Row r attends to the keys j of its own sequence, and with window > 0 only
 * to those with |r - j| <= window / 2 (integer halving; same header,
 * flash_attention_windowed_forward, bidirectional form).  Scale and soft-cap
 * as in mfa_fwd.  Which row belongs to which sequence is data read by the
 * kernels: the launch shape depends on L only, so a graph captured for one L
 * replays for any packing of it.  Bounds that do not describe back-to-back
 * sequences containing their rows give unspecified results, but every access
 * stays inside the L rows.  D in {64, 128}; qkv and out 16-byte aligned, lse
 * and seq_bounds 4-byte aligned.  L = 0 succeeds without work.  Errors,
 * ownership and streams as for mfa_fwd.  fp16 and fp32 calls need no
 * workspace; a bf16 call takes the fp16 copy of V that its P.V operands
 * need (see mfa_fwd) from the stream-ordered pool, so capture bf16 calls in
 * a graph only where stream-ordered allocation may be captured.
 */
int mfa_packed_qkv_fwd(const void* qkv, const int* seq_bounds, void* out, float* lse,
                       int L, int H, int D, float scale, int window, float softcap, int dtype,
                       void* stream);

/*
 * Attention over sequences packed back to back with separate query and key
 * packings and no padding (brotensor flash_attention.h,
 * flash_attention_varlen_forward).  Sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key/value rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]); nothing attends across sequences.
 * Positions count from each sequence's start: causal keeps key j for query i
 * when j - cu_seqlens_k[b] <= i - cu_seqlens_q[b], and the window (causal or
 * bidirectional, as in mfa_fwd) applies to those positions.  GQA, scale and
 * soft-cap as in mfa_fwd.
 *
 *   q, out        [total_q, Hq, D]   element type `dtype`
 *   k, v          [total_k, Hkv, D]  element type `dtype`
 *   lse           [Hq, total_q]      float32, may be NULL
 *   cu_seqlens_*  [batch + 1] int32 in device memory: prefix sums starting at
 *                 0, nondecreasing, ending at total_q / total_k
 *
 * The prefix sums are read on the device, so the launch shape depends only on
 * total_q: a graph captured once replays for any lengths with those totals.
 * A row of a sequence without keys (or of no sequence) gets O = 0 and
 * LSE = -inf.  Prefix sums that break the rules above give unspecified
 * results, but every access stays inside the given tensors.  A first kernel
 * turns the prefix sums into per-row positions and key bounds in the
 * workspace: caller-owned (256-byte aligned, at least
 * mfa_varlen_workspace_size(total_q, total_k, Hkv, D, dtype) bytes), or NULL
 * with ws_bytes = 0 for the
 * stream-ordered pool.  batch >= 1 unless total_q = 0 (then nothing is done).
 * D in {64, 128}; alignment, errors, ownership and streams as for mfa_fwd.
 */
int mfa_varlen_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                   const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q, int total_k,
                   int Hq, int Hkv, int D, float scale, int causal, int window, float softcap, int dtype,
                   void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes mfa_varlen_fwd needs (0 when total_q <= 0): the per-row
 * positions and bounds, plus for bf16 the fp16 copy of V (see mfa_fwd). */
size_t mfa_varlen_workspace_size(int total_q, int total_k, int Hkv, int D, int dtype);

/* The path mfa_fwd would take for these arguments (an mfa_path value), and
 * the split count it would use (through *splits, may be NULL). */
int mfa_fwd_plan(int B, int Lq, int Lk, int Hq, int Hkv, int D, int dtype, int* splits);

/* Static text for a status code. */
const char* mfa_status_string(int status);

/* Detail of the last failed call on this host thread ("" if none). */
const char* mfa_last_error(void);

/*
 * Instrumentation.  begin and end are hipEvent_t handles (or NULL, the
 * default, for none; created by the caller before use) that every later
 * forward or decode call made on this host thread attaches to the launch of
 * its main kernel as start and stop events (hipExtLaunchKernel), so that
 * hipEventElapsedTime between them gives that dispatch's own duration: the
 * prefill kernel (MFMA or fp32), for bf16 the conversion of V through the
 * prefill kernel, or the split decode kernel through its combine kernel; not
 * the key-mask packing or the varlen row prepass.  The caller keeps the
 * events alive while they are set.  The backward uses neither.
 */
void mfa_set_kernel_events(void* begin, void* end);

/* Library version as major*10000 + minor*100 + patch. */
int mfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MFA_H */
