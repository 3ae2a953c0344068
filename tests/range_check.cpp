// Host check of the key-range helpers in mfa_internal.h under hostile
// per-row sequence bounds (any int32 pair, as a caller of the packed-QKV
// entry point may pass): every nonempty range must lie inside [0, Lk - 1],
// every empty one must be [s, s - 1] with s in [0, Lk], and the 64-key tile
// range a 128-row block derives from its first and last rows (as the MFMA
// prefill kernel does) must stay inside the key axis.  Built and run by
// tests/test_range_host.py; prints "ok" and exits 0 on success.
#include "mfa_internal.h"

#include <climits>
#include <cstdio>
#include <random>
#include <vector>

int main() {
    std::mt19937 rng(12345);
    const int hostile[] = {INT_MIN, INT_MIN + 1, -1000000, -65, -64, -1, 0, 1, 2, 63, 64, 65, 127, 128,
                           1000, INT_MAX - 1, INT_MAX};
    const int nh = sizeof(hostile) / sizeof(hostile[0]);
    long checked = 0;
    for (int Lk : {1, 2, 63, 64, 65, 200, 1000}) {
        for (int causal = 0; causal < 2; ++causal) {
            for (int window : {0, 1, 3, 64, 129, 5000}) {
                for (int use_pos = 0; use_pos < 2; ++use_pos) {
                    const int L = Lk;
                    std::vector<int> bounds(2 * L), pos(L);
                    for (int trial = 0; trial < 40; ++trial) {
                        for (int i = 0; i < L; ++i) {
                            const bool h = rng() % 2;
                            bounds[2 * i] = h ? hostile[rng() % nh] : (int)(rng() % (2 * Lk + 3)) - Lk;
                            bounds[2 * i + 1] = h ? hostile[rng() % nh] : (int)(rng() % (2 * Lk + 3)) - 1;
                            pos[i] = (int)(rng() % (Lk + 1));   // the varlen prepass clamps to [0, Lk]
                        }
                        mfa::FwdArgs a{};
                        a.Lq = L; a.Lk = Lk; a.causal = causal; a.window = window; a.q_offset = 0;
                        a.seq_bounds = bounds.data();
                        a.row_pos = use_pos ? pos.data() : nullptr;
                        for (int i = 0; i < L; ++i) {
                            int lo, hi;
                            mfa::row_key_range<true>(a, i, lo, hi);
                            ++checked;
                            if (lo <= hi) {
                                if (lo < 0 || hi > Lk - 1) {
                                    std::printf("FAIL row %d: nonempty [%d, %d] outside [0, %d]\n", i, lo, hi, Lk - 1);
                                    return 1;
                                }
                            } else if (!(hi == lo - 1 && lo >= 0 && lo <= Lk)) {
                                std::printf("FAIL row %d: empty range [%d, %d] not [s, s - 1], s in [0, %d]\n", i, lo,
                                            hi, Lk);
                                return 1;
                            }
                        }
                        for (int i0 = 0; i0 < L; i0 += 128) {
                            const int il = (i0 + 128 < L ? i0 + 128 : L) - 1;
                            int lo_blk, t, hi_blk;
                            mfa::row_key_range<true>(a, i0, lo_blk, t);
                            mfa::row_key_range<true>(a, il, t, hi_blk);
                            if (lo_blk <= hi_blk) {
                                const int kt_lo = lo_blk / 64, kt_hi = hi_blk / 64;
                                if (kt_lo < 0 || kt_hi > (Lk - 1) / 64) {
                                    std::printf("FAIL block %d: tiles [%d, %d] outside [0, %d]\n", i0, kt_lo, kt_hi,
                                                (Lk - 1) / 64);
                                    return 1;
                                }
                            }
                        }
                    }
                }
            }
        }
    }
    std::printf("ok %ld rows\n", checked);
    return 0;
}
