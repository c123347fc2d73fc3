// kda_gate_exact.h -- exact in-chunk gate products for chunks whose decay is too strong
// for the factored form.
//
// Inside a 16-token chunk every pair of tokens i <= r is weighted per key channel by
// exp(G_r - G_i), G the running log-gate. The fast path factors this as
// exp(G_r - G_ref) * exp(G_ref - G_i) around the chunk's 8th token, so that one MFMA
// forms all pairs at once. That is exact while both factors stay inside fp32's normal
// range. Beyond that, a factor would overflow while its partner underflowed, and
// their product would be inf * 0 = NaN, although the true weight is at most 1 for a
// decay (g <= 0). A chunk whose running gate moves more than kGateSpan away from the
// reference, in any channel, therefore takes the per-pair form below, which never
// factors. Decays of any strength then give exact results. The pages state only that
// the gate range at 16-token chunks suits bf16 (augursoft.site "Kimi K3 的三個系統設計",
// section "為什麼 FlashKDA 選擇 16-token chunks"); strong decays are legal inputs of
// the recurrence all the same.
#pragma once

#include "kda_device.h"

namespace kda {

// Largest |G_r - G_ref| the factored form takes. exp(72) = 1.9e31, and the low bf16
// term of exp(-72) (about 2^-9 of it) is still a normal number, so both factors keep
// their full two-term precision.
constexpr float kGateSpan = 72.f;

// Wave-uniform: true when the predicate holds in any lane.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Per-pair sums of one chunk for the row token of this lane: for lane (c, grp) and each
// column token i <= c,
//   a[i] = sum_ch k[c,ch] k[i,ch] exp(G[c,ch] - G[i,ch]),
//   p[i] = sum_ch q[c,ch] k[i,ch] exp(G[c,ch] - G[i,ch])
// over all 128 channels (this lane's 32 channels, then summed over the four lane
// groups). Lane (c, 0) writes them to rows c of `a_rows` and `p_rows` (row-major
// 16 x 16 in LDS). Columns i > c are written as 0. The lane holds token c, channels
// chan_of(e, grp) (element e) of k, q and the running gate; the sums do not depend on
// which channels a lane holds.
__device__ __forceinline__ void exact_pair_rows(const float (&kr)[32], const float (&qr)[32], const float (&G)[32],
                                                int lane, float *a_rows, float *p_rows) {
    const int c = lane & 15, grp = lane >> 4, base = lane & 48;
#pragma unroll 1
    for (int i = 0; i < 16; ++i) {
        const int src = base | i;
        float sa = 0.f, sp = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const float ki = __shfl(kr[e], src, 64);
            const float gi = __shfl(G[e], src, 64);
            // column tokens after the row token are never used; their exponent may be
            // positive and large, so they are not evaluated
            const float w = i <= c ? ki * __expf(G[e] - gi) : 0.f;
            sa += kr[e] * w;
            sp += qr[e] * w;
        }
        sa += __shfl_xor(sa, 16, 64);
        sa += __shfl_xor(sa, 32, 64);
        sp += __shfl_xor(sp, 16, 64);
        sp += __shfl_xor(sp, 32, 64);
        if (grp == 0) {
            a_rows[c * 16 + i] = sa;
            p_rows[c * 16 + i] = sp;
        }
    }
}

}  // namespace kda
