// kda_intra_wave.h -- one wave's intra-chunk work for one (16-token chunk, head),
// bf16 io, K = V = 128: from q, k, g, beta to the chunk's record (W, Q~, K^d, T',
// M, gamma) in the layout the recurrent kernels read. Used by the intra-chunk
// kernel (records to HBM) and by the fused prefill (records into the recurrent
// workgroup's LDS ring).
//
// Per chunk, with S0 the state at the chunk start and G_r = g_1 + ... + g_r the
// running log-gate, the recurrence becomes (I + A) Delta = diag(beta)(V - K+ S0) with
//   A[r,i] = beta_r sum_c k[r,c] k[i,c] exp(G[r,c] - G[i,c])  (i < r),
//   P[r,i] =        sum_c q[r,c] k[i,c] exp(G[r,c] - G[i,c])  (i <= r),
// K+ = k * exp(G), Q+ = q * exp(G), K^d = k * exp(G_C - G), gamma = exp(G_C).
// With T = (I + A)^-1 and T' = T diag(beta): Delta = T' V - W S0 with W = T' K+,
// and the chunk output O = Q+ S0 + P Delta = Q~ S0 + M V with M = P T' and
// Q~ = Q+ - M K+ (augursoft.site "Kimi K3 的三個系統設計", section
// "為什麼 FlashKDA 選擇 16-token chunks": 16-token chunks and a 16 x 16 inversion).
//
// Numerics: gates enter A and P through exp(G - G_ref) and exp(G_ref - G) with
// G_ref the running gate at the chunk's 8th token. Both factors stay in fp32's normal
// range while |G - G_ref| <= kGateSpan in every channel; a chunk with a stronger decay
// recomputes A, P and K^d pair by pair without factoring (kda_gate_exact.h), so every
// decay gives finite, exact results. A and P, W and M K+ use two-term bf16 splits
// (x = x_hi + x_lo) of their factors for ~16-bit accuracy; W, Q~ and K^d are rounded
// to bf16 once, at the end.
#pragma once

#include "kda_device.h"
#include "kda_gate_exact.h"
#include "kda_internal.h"
#include "kda_ring.h"

namespace kda {
namespace intra {

constexpr int KD = 128;
constexpr int kChStride = 20;  // LDS elements per channel in channel-major tiles (16 tokens + 4 pad)

// One wave's LDS. The q and k tiles, K^d, A and K+ have disjoint lifetimes and share
// one area: q and k (the loads, 8 KiB), K^d (A/P products -> its record store), A
// (forward substitution), K+ (W and M K+ products). At 12.9 KiB per wave, three 4-wave workgroups fit in a CU.
struct alignas(16) IntraLds {
    union {
        float kp[KD * kChStride];   // K+ channel-major [channel][token]
        __bf16 kd[KD * kChStride];  // K^d channel-major, bf16
        float a[256];               // A row-major [r][i]
    };
    float p[256];   // P row-major
    float tb[256];  // T' row-major
    float gam[KD];  // gamma = exp(G_C) per channel
    float beta[16];
};
static_assert(sizeof(float) * KD * kChStride >= 2 * 16 * KD * sizeof(__bf16), "q and k tiles fit the K+ area");

// Every wave works in its own LDS area, so ordering among the lanes of one wave is
// all that is needed: LDS accesses of a wave execute in program order, and this
// keeps the compiler from moving them across the point.
__device__ __forceinline__ void wave_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// A 16-byte record store. Records are written once and read back by the recurrent
// kernel, never by this one, so they are stored non-temporal (streamed past the
// caches' retention policy).
template <typename T>
__device__ __forceinline__ void rec_store(char *p, const T &v) {
    static_assert(sizeof(T) == 16, "16-byte stores");
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}

// Eight consecutive bf16 values (one 16-byte load, global or LDS) as fp32.
__device__ __forceinline__ void load_bf16x8(const __bf16 *p, float *dst) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(p);
    const unsigned int w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dst[2 * i] = __uint_as_float(w[i] << 16);
        dst[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// The record of chunk [start, start + len) of head h (len in 1..16), written to
// `rec` (global or LDS memory) unless !head_ok (then the wave only computes, as a
// stand-in that keeps its workgroup's waves in step). SCALAR_GATE: g is [T, H],
// one decay per token and head for all channels (the scalar-gated delta rule); the
// per-channel gate arithmetic then works on one value per lane, which the
// compiler shares across the channels. Lane l holds token l % 16 of the chunk.
// BWD: also the backward record (same factors in the operand layouts of the reverse
// pass) to `brec` in global memory.
template <bool SCALAR_GATE, bool BWD = false>
__device__ __forceinline__ void chunk_record(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                                             const float *__restrict__ g, const float *__restrict__ beta,
                                             int64_t start, int len, int h, int H, bool head_ok, IntraLds &L,
                                             char *rec, int lane, char *brec = nullptr) {
    const int c = lane & 15;
    const int grp = lane >> 4;

    // ---- load: lane holds token c, channels chan_of(e, grp) = 32s + 8grp + u (element
    // e = 8s + u). q and k come by DMA (buffer_load ... lds) into the K+ area, free until
    // the A / P products: whole 256-byte rows, four per wave-wide load, 16-byte chunk j of
    // row r at slot j ^ r so that the per-lane reads below do not conflict; rows past the
    // chunk read as zero. g is read directly, 16 bytes per load. ----
    const bool row_ok = c < len;
    const int64_t t = start + c;
    float kr[32], qr[32], gr[32];
    const size_t rowoff = ((size_t)(row_ok ? t : start) * H + h) * KD + 8 * grp;
    const float gs = (SCALAR_GATE && row_ok) ? g[(size_t)t * H + h] : 0.f;
    char *tq = reinterpret_cast<char *>(L.kp), *tk = tq + 16 * KD * 2;
    {
        const unsigned int rowb = (unsigned int)H * KD * 2;  // one token row of q or k, bytes
        const size_t row0 = ((size_t)start * H + h) * KD;
        const int bytes = (int)((len - 1) * rowb + KD * 2);  // H <= 2^16: below 2^28
        const __amdgpu_buffer_rsrc_t rq = rsrc(q + row0, bytes), rk = rsrc(k + row0, bytes);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = 4 * s + (lane >> 4), j = (lane & 15) ^ r;
            const unsigned int off = (unsigned int)r * rowb + 16u * j;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void *)(tq + 1024 * s), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(tk + 1024 * s), 16, off, 0, 0, 0);
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if (row_ok) {
            if (SCALAR_GATE) {
#pragma unroll
                for (int u = 0; u < 8; ++u) gr[8 * s + u] = gs;
            } else {
                const float4 g0 = *reinterpret_cast<const float4 *>(g + rowoff + 32 * s);
                const float4 g1 = *reinterpret_cast<const float4 *>(g + rowoff + 32 * s + 4);
                gr[8 * s] = g0.x; gr[8 * s + 1] = g0.y; gr[8 * s + 2] = g0.z; gr[8 * s + 3] = g0.w;
                gr[8 * s + 4] = g1.x; gr[8 * s + 5] = g1.y; gr[8 * s + 6] = g1.z; gr[8 * s + 7] = g1.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) gr[8 * s + u] = 0.f;
        }
    }
    wait_vmcnt<0>();  // the DMA has landed (this wave's own loads)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int slot = c * KD * 2 + ((((4 * s + grp) ^ c) & 15) << 4);  // chunk 4s + grp of row c
        load_bf16x8(reinterpret_cast<const __bf16 *>(tq + slot), qr + 8 * s);
        load_bf16x8(reinterpret_cast<const __bf16 *>(tk + slot), kr + 8 * s);
    }
    wave_sync();  // read before the K^d writes below reuse the area
    const float b = row_ok ? beta[(size_t)t * H + h] : 0.f;

    // ---- running log-gate over the chunk's tokens (16-lane DPP scan), in place ----
#pragma unroll
    for (int e = 0; e < 32; ++e) gr[e] = row_inclusive_sum(gr[e]);
    float *G = gr;

    // ---- A and P on the MFMA: two-term bf16 splits of both factors. Gate factors
    // up = exp(G - G_ref), dn = exp(G_ref - G) with G_ref the running gate at token 7;
    // K^d = k exp(G_C - G) = k dn exp(G_C - G_ref) goes to LDS right away. ----
    f32x4 acc_a = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc_p = {0.f, 0.f, 0.f, 0.f};
    float span = 0.f;  // largest |G - G_ref| of this lane
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        unsigned int khh[4], khl[4], kbh[4], kbl[4], qhh[4], qhl[4], kdr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = 8 * s + 2 * u;
            const float d0 = G[e] - row_bcast<7>(G[e]), d1 = G[e + 1] - row_bcast<7>(G[e + 1]);
            span = fmaxf(span, fmaxf(fabsf(d0), fabsf(d1)));
            const float up0 = __expf(d0), up1 = __expf(d1);
            const float dn0 = __expf(-d0), dn1 = __expf(-d1);
            const int ch = chan_of(e, grp);  // channel of e; e + 1 is ch + 1
            const __bf16 kd0 = to_bf16(kr[e] * (dn0 * row_bcast<15>(up0)));
            const __bf16 kd1 = to_bf16(kr[e + 1] * (dn1 * row_bcast<15>(up1)));
            L.kd[ch * kChStride + c] = kd0;
            L.kd[(ch + 1) * kChStride + c] = kd1;
            if (BWD) {
                bf16x2 pr;
                pr[0] = kd0;
                pr[1] = kd1;
                kdr[u] = __builtin_bit_cast(unsigned int, pr);  // elements 2u, 2u + 1 of slab s
            }
            split_pair(kr[e] * up0, kr[e + 1] * up1, khh[u], khl[u]);
            split_pair(qr[e] * up0, qr[e + 1] * up1, qhh[u], qhl[u]);
            split_pair(kr[e] * dn0, kr[e + 1] * dn1, kbh[u], kbl[u]);
        }
        const bf16x8 vkhh = __builtin_bit_cast(bf16x8, make_uint4(khh[0], khh[1], khh[2], khh[3]));
        const bf16x8 vkhl = __builtin_bit_cast(bf16x8, make_uint4(khl[0], khl[1], khl[2], khl[3]));
        const bf16x8 vkbh = __builtin_bit_cast(bf16x8, make_uint4(kbh[0], kbh[1], kbh[2], kbh[3]));
        const bf16x8 vkbl = __builtin_bit_cast(bf16x8, make_uint4(kbl[0], kbl[1], kbl[2], kbl[3]));
        const bf16x8 vqhh = __builtin_bit_cast(bf16x8, make_uint4(qhh[0], qhh[1], qhh[2], qhh[3]));
        const bf16x8 vqhl = __builtin_bit_cast(bf16x8, make_uint4(qhl[0], qhl[1], qhl[2], qhl[3]));
        acc_a = mfma_16x16x32(vkhh, vkbh, acc_a);
        acc_a = mfma_16x16x32(vkhl, vkbh, acc_a);
        acc_a = mfma_16x16x32(vkhh, vkbl, acc_a);
        acc_p = mfma_16x16x32(vqhh, vkbh, acc_p);
        acc_p = mfma_16x16x32(vqhl, vkbh, acc_p);
        acc_p = mfma_16x16x32(vqhh, vkbl, acc_p);
        if (BWD && head_ok)  // K^d in the W layout: token c, channels chan_of(8s + u, grp)
            *reinterpret_cast<uint4 *>(brec + kBRecKD + (s * 64 + lane) * 16) =
                make_uint4(kdr[0], kdr[1], kdr[2], kdr[3]);
    }

    if (wave_any(span > kGateSpan)) {
        // Decay too strong for the factored form: A~ and P pair by pair, through the
        // (still unused) T' and P areas as row-major scratch, and K^d = k exp(G_C - G)
        // in one exponential, replacing what the factored loop left.
        exact_pair_rows(kr, qr, gr, lane, L.tb, L.p);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            unsigned int kdr[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = 8 * s + 2 * u;
                const int ch = chan_of(e, grp);
                const __bf16 kd0 = to_bf16(kr[e] * __expf(row_bcast<15>(G[e]) - G[e]));
                const __bf16 kd1 = to_bf16(kr[e + 1] * __expf(row_bcast<15>(G[e + 1]) - G[e + 1]));
                L.kd[ch * kChStride + c] = kd0;
                L.kd[(ch + 1) * kChStride + c] = kd1;
                bf16x2 pr;
                pr[0] = kd0;
                pr[1] = kd1;
                kdr[u] = __builtin_bit_cast(unsigned int, pr);
            }
            if (BWD && head_ok)
                *reinterpret_cast<uint4 *>(brec + kBRecKD + (s * 64 + lane) * 16) =
                    make_uint4(kdr[0], kdr[1], kdr[2], kdr[3]);
        }
        wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // into the accumulator layout: row 4grp + i, column c
            acc_a[i] = L.tb[(4 * grp + i) * 16 + c];
            acc_p[i] = L.p[(4 * grp + i) * 16 + c];
        }
    }

    wave_sync();
    // K^d to the record now, so that its LDS area is free for A and K+: tile pair mp,
    // lane (c, grp) holds keys key_of(2mp, c) (low 8 bytes) and key_of(2mp + 1, c),
    // tokens 4grp .. + 3
    if (head_ok) {
#pragma unroll
        for (int mp = 0; mp < 4; ++mp) {
            const uint2 lo = *reinterpret_cast<const uint2 *>(&L.kd[key_of(2 * mp, c) * kChStride + 4 * grp]);
            const uint2 hi = *reinterpret_cast<const uint2 *>(&L.kd[key_of(2 * mp + 1, c) * kChStride + 4 * grp]);
            rec_store(rec + kRecKD + (mp * 64 + lane) * 16, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
    }
    if (grp == 0) L.beta[c] = b;
    wave_sync();
    const f32x4 brow = *reinterpret_cast<const f32x4 *>(&L.beta[4 * grp]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        L.a[r * 16 + c] = (c < r) ? brow[i] * acc_a[i] : 0.f;
        L.p[r * 16 + c] = (c <= r) ? acc_p[i] : 0.f;
    }
    wave_sync();

    // ---- T = (I + A)^-1 by forward substitution; every lane solves column c ----
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc -= L.a[r * 16 + i] * x[i];
        x[r] = acc;
    }
    // T'[r][c] = T[r][c] * beta_c (this lane's own token is c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float xi = grp == 0 ? x[i] : (grp == 1 ? x[4 + i] : (grp == 2 ? x[8 + i] : x[12 + i]));
        L.tb[(4 * grp + i) * 16 + c] = xi * b;
    }

    // ---- K+ channel-major in LDS for the transposed operand; Q+ in place; gamma =
    // exp(G_C) is token 15's exp(G), broadcast ----
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const int ch = chan_of(e, grp);
        const float ep = __expf(G[e]);
        L.kp[ch * kChStride + c] = kr[e] * ep;
        qr[e] *= ep;
        const float gam = row_bcast<15>(ep);
        if (c == 0) L.gam[ch] = gam;
    }
    const float *qp = qr;
    wave_sync();

    // ---- M = P T' (row c, columns 4grp..4grp+3) ----
    const f32x4 tbrow = *reinterpret_cast<const f32x4 *>(&L.tb[c * 16 + 4 * grp]);
    f32x4 mrow = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
        const float pck = L.p[c * 16 + kk];
        const f32x4 trow = *reinterpret_cast<const f32x4 *>(&L.tb[kk * 16 + 4 * grp]);
        mrow += pck * trow;
    }
    bf16x4 tbh, tbl, mmh, mml;
    split_bf16x4(tbrow, tbh, tbl);
    split_bf16x4(mrow, mmh, mml);
    // B operands [X; X] over the 32-long reduction, for X = T'_hi, T'_lo, M_hi, M_lo
    bf16x8 tbh2, tbl2, mmh2, mml2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tbh2[i] = tbh2[4 + i] = tbh[i];
        tbl2[i] = tbl2[4 + i] = tbl[i];
        mmh2[i] = mmh2[4 + i] = mmh[i];
        mml2[i] = mml2[4 + i] = mml[i];
    }

    // ---- W^T = K+^T T'^T and (M K+)^T = K+^T M^T, tile by tile of 16 channels: tile jt
    // holds keys key_of(jt, 0 .. 15), so its outputs land on elements 4jt .. + 3 of the
    // row layout.
    // A operand [K+_hi | K+_lo]: ([K+_hi | K+_lo] . [X; X]) = (K+_hi + K+_lo) X. ----
    bf16x8 wv[4], qv[4];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
        const f32x4 kpt = *reinterpret_cast<const f32x4 *>(&L.kp[key_of(jt, c) * kChStride + 4 * grp]);
        bf16x4 kph, kpl;
        split_bf16x4(kpt, kph, kpl);
        bf16x8 kp2;
#pragma unroll
        for (int i = 0; i < 4; ++i) { kp2[i] = kph[i]; kp2[4 + i] = kpl[i]; }
        f32x4 wt = {0.f, 0.f, 0.f, 0.f};
        wt = mfma_16x16x32(kp2, tbh2, wt);
        wt = mfma_16x16x32(kp2, tbl2, wt);
        f32x4 pt = {0.f, 0.f, 0.f, 0.f};
        pt = mfma_16x16x32(kp2, mmh2, pt);
        pt = mfma_16x16x32(kp2, mml2, pt);
        // element e = 4 jt + i: slab jt >> 1, position 4 (jt & 1) + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wv[jt >> 1][4 * (jt & 1) + i] = to_bf16(wt[i]);
            qv[jt >> 1][4 * (jt & 1) + i] = to_bf16(qp[4 * jt + i] - pt[i]);
        }
    }

    if (!head_ok) return;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        rec_store(rec + kRecW + (s * 64 + lane) * 16, wv[s]);
        rec_store(rec + kRecQT + (s * 64 + lane) * 16, qv[s]);
    }
    bf16x8 tbv, mmv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tbv[i] = tbh[i]; tbv[4 + i] = tbl[i];
        mmv[i] = mmh[i]; mmv[4 + i] = mml[i];
    }
    *reinterpret_cast<bf16x8 *>(rec + kRecTB + lane * 16) = tbv;
    *reinterpret_cast<bf16x8 *>(rec + kRecMM + lane * 16) = mmv;
    if (c < 8) {
        // gamma_perm[grp][4c + i] = gamma[key_of(c, 4grp + i)]: accumulator tile c, row 4grp + i
        const float4 gv = *reinterpret_cast<const float4 *>(&L.gam[key_of(c, 4 * grp)]);
        *reinterpret_cast<float4 *>(rec + kRecGAM + (grp * 32 + 4 * c) * 4) = gv;
        if (BWD) *reinterpret_cast<float4 *>(brec + kBRecGAM + (grp * 32 + 4 * c) * 4) = gv;
    }
    if (BWD) {
        // W and Q~ channel-major through the K+ area (its last reads were above),
        // then read back in the K^d layout: lane (c, grp), pair mp holds key
        // key_of(2mp, c) (low 8 bytes) and key_of(2mp + 1, c) (high 8 bytes), tokens 4grp .. + 3
        wave_sync();
        __bf16 *tw = reinterpret_cast<__bf16 *>(L.kp);
        __bf16 *tq = tw + KD * kChStride;
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = key_of(jt, 4 * grp + i);
                tw[ch * kChStride + c] = wv[jt >> 1][4 * (jt & 1) + i];
                tq[ch * kChStride + c] = qv[jt >> 1][4 * (jt & 1) + i];
            }
        }
        wave_sync();
#pragma unroll
        for (int mp = 0; mp < 4; ++mp) {
            const int lo = key_of(2 * mp, c) * kChStride + 4 * grp, hi = key_of(2 * mp + 1, c) * kChStride + 4 * grp;
            const uint2 wl = *reinterpret_cast<const uint2 *>(&tw[lo]), wh = *reinterpret_cast<const uint2 *>(&tw[hi]);
            const uint2 ql = *reinterpret_cast<const uint2 *>(&tq[lo]), qh = *reinterpret_cast<const uint2 *>(&tq[hi]);
            *reinterpret_cast<uint4 *>(brec + kBRecWT + (mp * 64 + lane) * 16) = make_uint4(wl.x, wl.y, wh.x, wh.y);
            *reinterpret_cast<uint4 *>(brec + kBRecQT + (mp * 64 + lane) * 16) = make_uint4(ql.x, ql.y, qh.x, qh.y);
        }
    }
}

}  // namespace intra
}  // namespace kda
