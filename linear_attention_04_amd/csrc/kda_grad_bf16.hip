// kda_grad_bf16.hip -- token-parallel gradient kernel of the backward pass, bf16 io,
// K = V = 128.
//
// One wave per (16-token chunk, head), independent of every other wave. Inputs: the
// chunk's q, k, v, g, beta, d_out, its start state S0 (from the recomputed forward)
// and the gradient R reaching its end state (from the reverse pass), both bf16
// fragments. With the chunk factors recomputed as in the intra-chunk kernel
// (G, A~ = K^ K~^T, A = diag(beta) A~, P, T = (I + A)^-1, T' = T diag(beta), K+, Q+, K^d,
// gamma; K^ = k exp(G - G_ref), Q^ = q exp(G - G_ref), K~ = k exp(G_ref - G)):
//   U = V - K+ S0,  Delta = T' U,  dDelta = P^T dO + K^d R,  dU = T'^T dDelta = dv,
//   dQ+ = dO S0^T,  dK+ = -dU S0^T,  dK^d = Delta R^T,  dgamma = rowsum(R * S0),
//   dP = tril(dO Delta^T),  dT' = dDelta U^T,
//   dbeta = colsum(dT' * T) + rowsum(dA * A~),  dT = dT' diag(beta),
//   dA = -tril(T^T dT T^T, -1),  dA~ = diag(beta) dA,
//   dK^ = dA~ K~,  dK~ = dA~^T K^ + dP^T Q^,  dQ^ = dP K~,
// and then dq, dk and the running-gate gradient dG from the products that formed
// each factor; dg is the suffix sum of dG over the chunk, with the chunk-end gate
// G_C's gradient (through K^d and gamma) added at the last token.
//
// Layouts. "Row layout": lane (c, grp) = (lane % 16, lane / 16) holds token c and
// channels chan_of(e, grp) = 32s + 8grp + u (element e = 8s + u, kda_device.h); "slab" s
// of it is elements 8s .. 8s + 7 (eight bf16, the 16x16x32 operand that matches the
// state fragments' key order), and "key tile" kt is elements 4kt .. 4kt + 3, keys
// key_of(kt, 4grp + i) = rows 4grp + i of accumulator tile kt. Products
// over the 128 keys take the state fragments as stored. Products over the 128 value
// columns need the state with keys across lanes: half of a fragment (16 keys x 16
// columns) taken as a 16x16x16 operand and multiplied by the identity comes out with
// the keys across lanes, exactly (the values are bf16 and the accumulator fp32), and the
// same identity product turns a token-per-lane tile into a column-per-lane tile. Every
// layout change in this kernel is such an exact MFMA. Each state fragment is loaded
// once; LDS holds the 16 x 16 matrices and the K+ and K^d operands. q, k and g are
// read twice, for the chunk factors and again for the per-channel gradients: at two
// waves per SIMD neither the registers nor LDS can keep them in between. The second
// read is issued before the 16 x 16 backward, so that its latency is hidden.
#include <type_traits>

#include "kda_chunks.h"
#include "kda_device.h"
#include "kda_gate_exact.h"
#include "kda_internal.h"
#include "kda_ring.h"  // buffer descriptors and counter waits for the loads into LDS

namespace kda {
namespace {

constexpr int KD = 128;
constexpr int VD = 128;
constexpr int kWaves = 4;

// One wave's 16 x 16 matrices, row-major. The matrices and the K+/K^d area are also
// reused to gather each output tile before it is written out in whole rows
// (dv in dt..dp during the value tiles; dg in a..dp and dq, dk in kps/kds at the end).
struct alignas(16) GradLds {
    float a[256];    // A = diag(beta) A~, strictly lower (the forward substitution)
    float at[256];   // A~ (strictly lower)
    float t[256];    // T = (I + A)^-1
    float tb[256];   // T' = T diag(beta)
    float dt[256];   // dT = dT' diag(beta)
    float y[256];    // Y = dT T^T
    float dat[256];  // dA~
    float dp[256];   // dP (i <= r)
    float xdat[256]; // copies of dA~ and dP for the per-pair path of strongly decaying
    float xdp[256];  // chunks (the originals' area gathers dg there)
    float beta[16];
    bf16x8 kps[4][64];  // K+ slabs (row layout, bf16), one per 32 keys
    bf16x8 kds[4][64];  // K^d slabs
};

// A 16-token tile of row bytes `row` (256 or 512) in LDS, 16-byte chunks swizzled by
// the row (chunk ^ r) so that neither the per-token writes nor the per-row reads
// conflict in the banks.
template <int ROW>
__device__ __forceinline__ int tile_off(int r, int byte) {
    return r * ROW + ((((byte >> 4) ^ r) << 4) | (byte & 15));
}

// Write the 16 x ROW-byte tile at `lds` to global rows (row r at `g0 + r * gstride`),
// rows r < len only: each wave-wide store moves 1 KiB of whole rows.
template <int ROW>
__device__ __forceinline__ void store_tile(const char *lds, char *g0, size_t gstride, int len, int lane) {
    constexpr int kLanesPerRow = ROW / 16;
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
#pragma unroll
    for (int s = 0; s < 16 / kRowsPerStore; ++s) {
        const int r = s * kRowsPerStore + lane / kLanesPerRow, j = lane % kLanesPerRow;
        const uint4 x = *reinterpret_cast<const uint4 *>(lds + tile_off<ROW>(r, 16 * j));
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        // non-temporal: the gradients are final outputs, not read again here
        if (r < len)
            __builtin_nontemporal_store(u32x4{x.x, x.y, x.z, x.w},
                                        reinterpret_cast<u32x4 *>(g0 + (size_t)r * gstride + 16 * j));
    }
}

__device__ __forceinline__ void wave_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ __forceinline__ bf16x8 dup8(bf16x4 a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3); }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 bf16x4_to_f32(bf16x4 x) {
    return f32x4{from_bf16(x[0]), from_bf16(x[1]), from_bf16(x[2]), from_bf16(x[3])};
}

// 16 x 16 fp32 matrix entries (four per lane) split into two bf16 terms, each
// duplicated over both halves of the 32-long reduction: [M_hi; M_hi] and [M_lo; M_lo].
struct SplitDup {
    bf16x8 hi, lo;
};
__device__ __forceinline__ SplitDup split_dup(f32x4 m) {
    bf16x4 h, l;
    split_bf16x4(m, h, l);
    return SplitDup{dup8(h), dup8(l)};
}
// Elements 4h .. 4h + 3 of an 8-element operand, as a 16x16x16 operand.
__device__ __forceinline__ s16x4 half4(bf16x8 x, int h) {
    const bf16x4 r = h ? __builtin_shufflevector(x, x, 4, 5, 6, 7) : __builtin_shufflevector(x, x, 0, 1, 2, 3);
    return as_s16x4(r);
}
// [M_hi | M_lo] over the two halves of the reduction.
__device__ __forceinline__ bf16x8 split_cat(f32x4 m) {
    bf16x4 h, l;
    split_bf16x4(m, h, l);
    return cat8(h, l);
}

template <bool SCALAR_GATE>
__global__ __launch_bounds__(64 * kWaves) void kda_grad_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const __bf16 *__restrict__ dout,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ chunk_seq,
    int64_t T, int H, int N, int64_t max_chunks, const char *__restrict__ states, const char *__restrict__ dstates,
    __bf16 *__restrict__ dq, __bf16 *__restrict__ dk, __bf16 *__restrict__ dv, float *__restrict__ dg,
    float *__restrict__ dbeta) {
    __shared__ GradLds lds_all[kWaves];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, grp = lane >> 4;
    const int head_groups = (H + kWaves - 1) / kWaves;
    const int64_t chunk = blockIdx.x / head_groups;
    const int h = (int)(blockIdx.x - chunk * head_groups) * kWaves + wave;
    if (h >= H) return;  // waves are independent
    int64_t start;
    int len;
    chunk_span(cu, chunk_off, chunk_seq, chunk, T, N, max_chunks, start, len);
    if (len == 0) return;
    GradLds &L = lds_all[wave];
    const bool row_ok = c < len;
    const int64_t tok = start + c;
    const size_t krow = ((size_t)(row_ok ? tok : start) * H + h) * KD;  // q, k, g, dq, dk, dg row of token c
    const size_t vrow = ((size_t)(row_ok ? tok : start) * H + h) * VD;  // v, d_out, dv row
    const size_t hc = (size_t)chunk * H + h;  // chunk-major, like the records
    const char *S0 = states + hc * kStateBytesBf16 + lane * 16;
    const char *Rs = dstates + hc * kStateBytesBf16 + lane * 16;
    const float b = row_ok ? beta[(size_t)tok * H + h] : 0.f;

    // the 16 x 16 identity as a 16x16x16 B operand (exact 0/1 entries)
    s16x4 I4;
#pragma unroll
    for (int j = 0; j < 4; ++j) I4[j] = (4 * grp + j == c) ? (short)0x3F80 : (short)0;

    // q and k of the chunk as whole 256-byte rows by DMA into the K+ / K^d area, in the
    // tile layout of tile_off<256> (16-byte chunk j of row r at slot j ^ r); rows past the
    // chunk read as zero. Used for the chunk factors here and again before the key tiles.
    char *tq = reinterpret_cast<char *>(L.kps);
    char *tk = reinterpret_cast<char *>(L.kds);
    auto dma_qk = [&]() {
        // The offsets are recomputed at each call, not held in registers between the two
        // calls: the opaque copy of the lane id keeps the compiler from sharing them, which
        // would take the kernel past the register budget of two waves per SIMD.
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const unsigned int rowb = (unsigned int)H * KD * 2;  // one token row of q or k, bytes
        const size_t row0 = ((size_t)start * H + h) * KD;
        const int bytes = (int)((len - 1) * rowb + KD * 2);  // H <= 2^16: below 2^28
        const __amdgpu_buffer_rsrc_t rq = rsrc(q + row0, bytes), rk = rsrc(k + row0, bytes);
#pragma unroll
        for (int s = 0; s < 4; ++s) {  // rows 4s .. 4s + 3, 1 KiB per wave-wide load
            const int r = 4 * s + (lane >> 4), j = (lane & 15) ^ r;  // LDS chunk lane & 15 holds chunk j
            const unsigned int off = (unsigned int)r * rowb + 16u * j;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void *)(tq + 1024 * s), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(tk + 1024 * s), 16, off, 0, 0, 0);
        }
    };

    // ================= 1. chunk factors (as the intra-chunk kernel) =================
    f32x4 pcol;  // P[4grp + i][c] (i <= r kept)
    bool exact;  // wave-uniform: this chunk takes the per-pair gate path (kda_gate_exact.h)
    {
        float kr[32], qr[32], G[32];
        dma_qk();
        float4 gl[8];  // g of token c, channels 32s + 8grp .. + 3 (gl[2s]) and + 4 .. + 7 (gl[2s + 1])
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            gl[2 * s] = gl[2 * s + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row_ok && !SCALAR_GATE) {
                gl[2 * s] = *reinterpret_cast<const float4 *>(g + krow + 32 * s + 8 * grp);
                gl[2 * s + 1] = *reinterpret_cast<const float4 *>(g + krow + 32 * s + 8 * grp + 4);
            }
        }
        wait_vmcnt<0>();  // q and k have landed in LDS
        asm volatile("" ::: "memory");
#pragma unroll
        for (int s = 0; s < 4; ++s) {  // channels 32s + 8grp .. + 7 of q and of k
            const int cb = 2 * (32 * s + 8 * grp);
            const uint4 qw = *reinterpret_cast<const uint4 *>(tq + tile_off<256>(c, cb));
            const uint4 kw = *reinterpret_cast<const uint4 *>(tk + tile_off<256>(c, cb));
            const float4 g0 = gl[2 * s], g1 = gl[2 * s + 1];
            const unsigned int qa[4] = {qw.x, qw.y, qw.z, qw.w}, ka[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qr[8 * s + 2 * i] = __uint_as_float(qa[i] << 16);
                qr[8 * s + 2 * i + 1] = __uint_as_float(qa[i] & 0xffff0000u);
                kr[8 * s + 2 * i] = __uint_as_float(ka[i] << 16);
                kr[8 * s + 2 * i + 1] = __uint_as_float(ka[i] & 0xffff0000u);
            }
            G[8 * s] = g0.x;
            G[8 * s + 1] = g0.y;
            G[8 * s + 2] = g0.z;
            G[8 * s + 3] = g0.w;
            G[8 * s + 4] = g1.x;
            G[8 * s + 5] = g1.y;
            G[8 * s + 6] = g1.z;
            G[8 * s + 7] = g1.w;
        }
        wave_sync();  // read before the K+ / K^d slabs below overwrite the area
        if (SCALAR_GATE) {
            const float gs = row_inclusive_sum(row_ok ? g[(size_t)tok * H + h] : 0.f);
#pragma unroll
            for (int e = 0; e < 32; ++e) G[e] = gs;
        } else {
#pragma unroll
            for (int e = 0; e < 32; ++e) G[e] = row_inclusive_sum(G[e]);
        }

        // A~ and P (two-term bf16 splits of both factors); K^d and K+ slabs
        f32x4 acc_a = zero4(), acc_p = zero4();
        float span = 0.f;  // largest |G - G_ref| of this lane
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            unsigned int khh[4], khl[4], kbh[4], kbl[4], qhh[4], qhl[4], kdw[4], kpw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = 8 * s + 2 * u;
                const float d0 = G[e] - row_bcast<7>(G[e]), d1 = G[e + 1] - row_bcast<7>(G[e + 1]);
                span = fmaxf(span, fmaxf(fabsf(d0), fabsf(d1)));
                const float up0 = __expf(d0), up1 = __expf(d1);
                const float dn0 = __expf(-d0), dn1 = __expf(-d1);
                kdw[u] = pack_bf16x2(kr[e] * (dn0 * row_bcast<15>(up0)), kr[e + 1] * (dn1 * row_bcast<15>(up1)));
                kpw[u] = pack_bf16x2(kr[e] * __expf(G[e]), kr[e + 1] * __expf(G[e + 1]));
                split_pair(kr[e] * up0, kr[e + 1] * up1, khh[u], khl[u]);
                split_pair(qr[e] * up0, qr[e + 1] * up1, qhh[u], qhl[u]);
                split_pair(kr[e] * dn0, kr[e + 1] * dn1, kbh[u], kbl[u]);
            }
            L.kds[s][lane] = __builtin_bit_cast(bf16x8, make_uint4(kdw[0], kdw[1], kdw[2], kdw[3]));
            L.kps[s][lane] = __builtin_bit_cast(bf16x8, make_uint4(kpw[0], kpw[1], kpw[2], kpw[3]));
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
        }
        exact = wave_any(span > kGateSpan);
        if (exact) {
            // Decay too strong for the factored form: A~ and P pair by pair, through
            // the (not yet used) Y and dA~ areas as row-major scratch, and the K^d
            // slabs from one exponential each.
            exact_pair_rows(kr, qr, G, lane, L.y, L.dat);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                unsigned int kdw[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = 8 * s + 2 * u;
                    kdw[u] = pack_bf16x2(kr[e] * __expf(row_bcast<15>(G[e]) - G[e]),
                                         kr[e + 1] * __expf(row_bcast<15>(G[e + 1]) - G[e + 1]));
                }
                L.kds[s][lane] = __builtin_bit_cast(bf16x8, make_uint4(kdw[0], kdw[1], kdw[2], kdw[3]));
            }
            wave_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc_a[i] = L.y[(4 * grp + i) * 16 + c];
                acc_p[i] = L.dat[(4 * grp + i) * 16 + c];
            }
        }
        // acc_a[i] = A~[4grp + i][c], acc_p[i] = P[4grp + i][c]
        if (grp == 0) L.beta[c] = b;
        wave_sync();
        const f32x4 brow = *reinterpret_cast<const f32x4 *>(&L.beta[4 * grp]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * grp + i;
            // strictly lower only: the factored products above the diagonal are
            // never used and overflow under strong decays (dA is 0 there, and 0 * inf
            // would be NaN in dbeta's row sums)
            L.at[r * 16 + c] = (c < r) ? acc_a[i] : 0.f;
            L.a[r * 16 + c] = (c < r) ? brow[i] * acc_a[i] : 0.f;
            pcol[i] = (c <= r) ? acc_p[i] : 0.f;
        }
        wave_sync();
    }
    // T = (I + A)^-1 by forward substitution, lane column c; T' = T diag(beta)
    {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= L.a[r * 16 + i] * x[i];
            x[r] = acc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float xi = grp == 0 ? x[i] : (grp == 1 ? x[4 + i] : (grp == 2 ? x[8 + i] : x[12 + i]));
            L.t[(4 * grp + i) * 16 + c] = xi;
            L.tb[(4 * grp + i) * 16 + c] = xi * b;
        }
    }
    wave_sync();
    // T' row c and column c, [hi | lo]; P column c, [hi | lo]
    const bf16x8 tbr = split_cat(*reinterpret_cast<const f32x4 *>(&L.tb[c * 16 + 4 * grp]));
    f32x4 tcol;
#pragma unroll
    for (int i = 0; i < 4; ++i) tcol[i] = L.tb[(4 * grp + i) * 16 + c];
    const bf16x8 tbc = split_cat(tcol);
    const bf16x8 pc = split_cat(pcol);

    // ================= 2. per 16-column value tile: products over the keys, then over the values ====
    // Each state fragment is loaded once: the tile's eight fragments (S0 and R, four key
    // slabs) serve the products over the keys as stored and, moved across lanes by the
    // selection MFMAs, this tile's share of the products over the values.
    f32x4 dpa = zero4(), dtpa = zero4();  // dP[4grp + i][c], dT'[4grp + i][c]
    f32x4 dqp[8], dkp[8], dkd[8];         // (dO S0^T)^T, (dU S0^T)^T, (Delta R^T)^T: token c, keys key_of(kt, 4grp + i)
    float dgam[8];                        // key key_of(kt, c), summed over this lane group's columns
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
        dqp[kt] = dkp[kt] = dkd[kt] = zero4();
        dgam[kt] = 0.f;
    }
#pragma unroll 1
    for (int vt = 0; vt < 8; ++vt) {
        bf16x8 s0f[4], rf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            s0f[ks] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(S0 + (vt * 4 + ks) * 1024));
            rf[ks] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(Rs + (vt * 4 + ks) * 1024));
        }
        const int col = 16 * vt + 4 * grp;
        bf16x4 vt4 = {}, dt4 = {};
        if (row_ok) {
            vt4 = *reinterpret_cast<const bf16x4 *>(v + vrow + col);
            dt4 = *reinterpret_cast<const bf16x4 *>(dout + vrow + col);
        }
        f32x4 ksv = zero4(), kst = zero4(), xv = zero4(), xt = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kp = L.kps[ks][lane], kd = L.kds[ks][lane];
            ksv = mfma_16x16x32(kp, s0f[ks], ksv);  // K+ S0, column per lane
            kst = mfma_16x16x32(s0f[ks], kp, kst);  // the same, token per lane
            xv = mfma_16x16x32(kd, rf[ks], xv);     // K^d R
            xt = mfma_16x16x32(rf[ks], kd, xt);
        }
        // column per lane: V[4grp + i][16vt + c], dO likewise (identity MFMA, exact)
        const f32x4 vcol = mfma_16x16x16(as_s16x4(vt4), I4, zero4());
        const f32x4 dcol = mfma_16x16x16(as_s16x4(dt4), I4, zero4());
        const f32x4 ucol = vcol - ksv;               // U, column per lane
        const f32x4 utk = bf16x4_to_f32(vt4) - kst;  // U, token per lane
        bf16x4 uh, ul;
        split_bf16x4(ucol, uh, ul);
        // Delta^T = U^T T'^T: token per lane
        f32x4 del = mfma_16x16x32(dup8(uh), tbr, zero4());
        del = mfma_16x16x32(dup8(ul), tbr, del);
        const bf16x8 dcd = dup8(to_bf16x4(dcol));  // dO column tile (exact)
        // dDelta = P^T dO + K^d R, column per lane and token per lane
        const f32x4 ddc = mfma_16x16x32(pc, dcd, xv);
        const f32x4 ddt = mfma_16x16x32(dcd, pc, xt);
        // dU^T = dDelta^T T': token per lane
        bf16x4 dh, dl;
        split_bf16x4(ddc, dh, dl);
        f32x4 du = mfma_16x16x32(dup8(dh), tbc, zero4());
        du = mfma_16x16x32(dup8(dl), tbc, du);
        const bf16x4 utok = to_bf16x4(utk), deltok = to_bf16x4(del), ddtok = to_bf16x4(ddt);
        const bf16x4 dutok = to_bf16x4(du);
        *reinterpret_cast<bf16x4 *>(reinterpret_cast<char *>(L.dt) + tile_off<256>(c, 2 * col)) = dutok;
        dpa = mfma_16x16x16(as_s16x4(dt4), as_s16x4(deltok), dpa);     // dO Delta^T
        dtpa = mfma_16x16x16(as_s16x4(ddtok), as_s16x4(utok), dtpa);   // dDelta U^T
        // products over this tile's 16 columns, for all 128 keys
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            // key key_of(kt, c) across lanes, columns 16vt + 4grp + i: the fragment's half
            // (kt & 1) as a 16x16x16 operand (rows: columns of S), times the identity
            const f32x4 st = mfma_16x16x16(half4(s0f[kt >> 1], kt & 1), I4, zero4());
            const f32x4 rt = mfma_16x16x16(half4(rf[kt >> 1], kt & 1), I4, zero4());
            dgam[kt] += st[0] * rt[0] + st[1] * rt[1] + st[2] * rt[2] + st[3] * rt[3];
            const s16x4 stb = as_s16x4(to_bf16x4(st)), rtb = as_s16x4(to_bf16x4(rt));
            dqp[kt] = mfma_16x16x16(stb, as_s16x4(dt4), dqp[kt]);
            dkp[kt] = mfma_16x16x16(stb, as_s16x4(dutok), dkp[kt]);
            dkd[kt] = mfma_16x16x16(rtb, as_s16x4(deltok), dkd[kt]);
        }
    }

    wave_sync();
    store_tile<256>(reinterpret_cast<const char *>(L.dt), reinterpret_cast<char *>(dv + ((size_t)start * H + h) * VD),
                    (size_t)H * VD * 2, len, lane);
    wave_sync();
    // The key tiles need q, k and g again. q and k go straight to the K+ / K^d area,
    // free from here on, in the swizzled tile layout that later gathers dq and dk (each
    // lane reads its inputs there before writing its outputs in the same place). g goes
    // to registers, which the 16 x 16 backward leaves free. Both are in flight during
    // that backward.
    dma_qk();
    float4 gk[8];  // g of token c, channels key_of(kt, 4grp) .. + 3
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
        gk[kt] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (!SCALAR_GATE && row_ok)
            gk[kt] = *reinterpret_cast<const float4 *>(g + krow + key_of(kt, 4 * grp));
    }

    // ================= 3. the 16 x 16 backward =================
    float dbeta_c;
    {
        f32x4 dpm, tcolT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * grp + i;
            dpm[i] = (c <= r) ? dpa[i] : 0.f;
            tcolT[i] = L.t[r * 16 + c];
            L.dt[r * 16 + c] = dtpa[i] * b;  // dT[r][c] = dT'[r][c] beta_c
            L.dp[r * 16 + c] = dpm[i];
            if (exact) L.xdp[r * 16 + c] = dpm[i];
        }
        float db1 = dtpa[0] * tcolT[0] + dtpa[1] * tcolT[1] + dtpa[2] * tcolT[2] + dtpa[3] * tcolT[3];
        db1 += __shfl_xor(db1, 16, 64);
        db1 += __shfl_xor(db1, 32, 64);
        wave_sync();
        // Y[c][4grp + j] = sum_m dT[c][m] T[4grp + j][m]
        f32x4 yv = zero4();
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const f32x4 dtr = *reinterpret_cast<const f32x4 *>(&L.dt[c * 16 + 4 * m4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 trow = *reinterpret_cast<const f32x4 *>(&L.t[(4 * grp + j) * 16 + 4 * m4]);
                yv[j] += dtr[0] * trow[0] + dtr[1] * trow[1] + dtr[2] * trow[2] + dtr[3] * trow[3];
            }
        }
        *reinterpret_cast<f32x4 *>(&L.y[c * 16 + 4 * grp]) = yv;
        wave_sync();
        // dA[c][4grp + j] = -sum_m T[m][c] Y[m][4grp + j], strictly lower
        f32x4 da = zero4();
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float tmc = L.t[m * 16 + c];
            da -= tmc * *reinterpret_cast<const f32x4 *>(&L.y[m * 16 + 4 * grp]);
        }
        const f32x4 atr = *reinterpret_cast<const f32x4 *>(&L.at[c * 16 + 4 * grp]);
        float db2 = 0.f;
        f32x4 dat;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            da[j] = (4 * grp + j < c) ? da[j] : 0.f;
            db2 += da[j] * atr[j];
            dat[j] = b * da[j];
        }
        db2 += __shfl_xor(db2, 16, 64);
        db2 += __shfl_xor(db2, 32, 64);
        dbeta_c = db1 + db2;
        *reinterpret_cast<f32x4 *>(&L.dat[c * 16 + 4 * grp]) = dat;
        if (exact) *reinterpret_cast<f32x4 *>(&L.xdat[c * 16 + 4 * grp]) = dat;
        wave_sync();
    }
    if (grp == 0 && row_ok) dbeta[(size_t)tok * H + h] = dbeta_c;

    // ================= 4. per 16-channel key tile: dq, dk, dg =================
    float dgs = 0.f;  // scalar gate: sum of dg over this lane's channels
    f32x4 dacol, dpcol;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dacol[j] = L.dat[(4 * grp + j) * 16 + c];
        dpcol[j] = L.dp[(4 * grp + j) * 16 + c];
    }
    // dA~ and dP rows and columns, two bf16 terms each
    const SplitDup m_darow = split_dup(*reinterpret_cast<const f32x4 *>(&L.dat[c * 16 + 4 * grp]));
    const SplitDup m_dacol = split_dup(dacol);
    const SplitDup m_dprow = split_dup(*reinterpret_cast<const f32x4 *>(&L.dp[c * 16 + 4 * grp]));
    const SplitDup m_dpcol = split_dup(dpcol);
    wait_vmcnt<0>();  // q and k have landed in LDS
    wave_sync();  // the matrices' area now gathers dg, the K+/K^d area dq and dk
    char *tg = reinterpret_cast<char *>(L.a);
    // One key tile; EXACT: the chunk's decay is too strong for the factored gate form,
    // so the products of A~ and P with the gates are differentiated pair by pair.
    auto key_tile = [&](int kt, auto exact_tag) {
        constexpr bool EXACT = decltype(exact_tag)::value;
        const int cb = 2 * key_of(kt, 4 * grp);  // byte of channel key_of(kt, 4grp) in a bf16 row
        // channels key_of(kt, 4grp) + i of token c
        const f32x4 kk = bf16x4_to_f32(*reinterpret_cast<const bf16x4 *>(tk + tile_off<256>(c, cb)));
        const f32x4 qq = bf16x4_to_f32(*reinterpret_cast<const bf16x4 *>(tq + tile_off<256>(c, cb)));
        f32x4 G;
        if (SCALAR_GATE) {
            const float gs = row_ok ? g[(size_t)tok * H + h] : 0.f;
            G = f32x4{gs, gs, gs, gs};
        } else {
            G = f32x4{gk[kt].x, gk[kt].y, gk[kt].z, gk[kt].w};
        }
        // ga: the gradient reaching k through A~ and P (dK^ exp(G - G_ref) + dK~ exp(G_ref - G)),
        // gq: reaching q through P (dQ^ exp(G - G_ref)), gg: reaching G through them
        f32x4 eg, ed, gam, ga, gq, gg;
#pragma unroll
        for (int i = 0; i < 4; ++i) G[i] = row_inclusive_sum(G[i]);
        if (!EXACT) {
            f32x4 up, dn, khat, qhat, krev;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float d = G[i] - row_bcast<7>(G[i]);
                up[i] = __expf(d);
                dn[i] = __expf(-d);
                eg[i] = __expf(G[i]);
                ed[i] = dn[i] * row_bcast<15>(up[i]);
                gam[i] = row_bcast<15>(eg[i]);
                khat[i] = kk[i] * up[i];
                qhat[i] = qq[i] * up[i];
                krev[i] = kk[i] * dn[i];
            }
            // channel per lane, [hi | lo] over tokens 4grp .. + 3 (identity MFMAs, exact)
            auto chan_major = [&](f32x4 x) {
                bf16x4 xh, xl;
                split_bf16x4(x, xh, xl);
                const f32x4 th = mfma_16x16x16(as_s16x4(xh), I4, zero4());
                const f32x4 tl = mfma_16x16x16(as_s16x4(xl), I4, zero4());
                return cat8(to_bf16x4(th), to_bf16x4(tl));
            };
            const bf16x8 krev_c = chan_major(krev), khat_c = chan_major(khat), qhat_c = chan_major(qhat);
            f32x4 dkhat = mfma_16x16x32(krev_c, m_darow.hi, zero4());
            dkhat = mfma_16x16x32(krev_c, m_darow.lo, dkhat);
            f32x4 dkrev = mfma_16x16x32(khat_c, m_dacol.hi, zero4());
            dkrev = mfma_16x16x32(khat_c, m_dacol.lo, dkrev);
            dkrev = mfma_16x16x32(qhat_c, m_dpcol.hi, dkrev);
            dkrev = mfma_16x16x32(qhat_c, m_dpcol.lo, dkrev);
            f32x4 dqhat = mfma_16x16x32(krev_c, m_dprow.hi, zero4());
            dqhat = mfma_16x16x32(krev_c, m_dprow.lo, dqhat);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ga[i] = dkhat[i] * up[i] + dkrev[i] * dn[i];
                gq[i] = dqhat[i] * up[i];
                gg[i] = dkhat[i] * khat[i] - dkrev[i] * krev[i] + dqhat[i] * qhat[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                eg[i] = __expf(G[i]);
                ed[i] = __expf(row_bcast<15>(G[i]) - G[i]);
                gam[i] = row_bcast<15>(eg[i]);
                ga[i] = gq[i] = gg[i] = 0.f;
            }
            // A~[r][j] = sum k_r k_j w and P[r][j] = sum q_r k_j w with w = exp(G_r - G_j):
            // this token as row r (columns j <= c) and as column j (rows r >= c)
#pragma unroll 1
            for (int j = 0; j < 16; ++j) {
                const int src = (lane & 48) | j;
                const float ar = L.xdat[c * 16 + j], pr = L.xdp[c * 16 + j];  // row c
                const float ac = L.xdat[j * 16 + c], pc = L.xdp[j * 16 + c];  // column c
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float kj = __shfl(kk[i], src, 64), qj = __shfl(qq[i], src, 64);
                    const float gj = __shfl(G[i], src, 64);
                    // the weights of pairs outside the triangle are never used (their
                    // coefficients are 0) and may overflow, so they are not evaluated
                    const float wr = j <= c ? kj * __expf(G[i] - gj) : 0.f;
                    const float wc = j >= c ? (ac * kj + pc * qj) * __expf(gj - G[i]) : 0.f;
                    ga[i] += ar * wr + wc;
                    gq[i] += pr * wr;
                    gg[i] += (ar * kk[i] + pr * qq[i]) * wr - kk[i] * wc;
                }
            }
        }

        // dgamma for this lane's four channels: sum over the lane groups, then
        // channel key_of(kt, 4grp + i) sits in lane 4grp + i
        float dgt = dgam[kt];
        dgt += __shfl_xor(dgt, 16, 64);
        dgt += __shfl_xor(dgt, 32, 64);
        f32x4 dkq, dqq, dgv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float dkplus = -dkp[kt][i];
            const float kd = kk[i] * ed[i];
            dkq[i] = ga[i] + dkplus * eg[i] + dkd[kt][i] * ed[i];
            dqq[i] = gq[i] + dqp[kt][i] * eg[i];
            float dG = gg[i] + dkplus * (kk[i] * eg[i]) + dqp[kt][i] * (qq[i] * eg[i]) - dkd[kt][i] * kd;
            const float dgc =
                row_bcast<15>(row_inclusive_sum(dkd[kt][i] * kd)) + __shfl(dgt, 4 * grp + i, 64) * gam[i];
            if (c == len - 1) dG += dgc;
            dgv[i] = row_suffix_sum(dG);
        }
        *reinterpret_cast<bf16x4 *>(tk + tile_off<256>(c, cb)) = to_bf16x4(dkq);
        *reinterpret_cast<bf16x4 *>(tq + tile_off<256>(c, cb)) = to_bf16x4(dqq);
        if (SCALAR_GATE) {
            if (row_ok) dgs += dgv[0] + dgv[1] + dgv[2] + dgv[3];
        } else {
            *reinterpret_cast<f32x4 *>(tg + tile_off<512>(c, 2 * cb)) = dgv;
        }
    };
    if (!exact) {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) key_tile(kt, std::false_type{});
    } else {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) key_tile(kt, std::true_type{});
    }
    wave_sync();
    const size_t row0 = ((size_t)start * H + h) * KD;
    store_tile<256>(tk, reinterpret_cast<char *>(dk + row0), (size_t)H * KD * 2, len, lane);
    store_tile<256>(tq, reinterpret_cast<char *>(dq + row0), (size_t)H * KD * 2, len, lane);
    if (!SCALAR_GATE) store_tile<512>(tg, reinterpret_cast<char *>(dg + row0), (size_t)H * KD * 4, len, lane);
    if (SCALAR_GATE) {
        dgs += __shfl_xor(dgs, 16, 64);
        dgs += __shfl_xor(dgs, 32, 64);
        if (grp == 0 && row_ok) dg[(size_t)tok * H + h] = dgs;
    }
}

}  // namespace

hipError_t launch_grad_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                            const void *d_out, const int32_t *cu_seqlens, void *dq, void *dk, void *dv, float *dg,
                            float *dbeta, const Geometry &geo, const void *ws, hipStream_t stream) {
    if (geo.max_chunks == 0) return hipSuccess;
    const char *base = static_cast<const char *>(ws);
    const int32_t *chunk_off = reinterpret_cast<const int32_t *>(base + geo.off_chunk_off);
    const int32_t *chunk_seq = reinterpret_cast<const int32_t *>(base + geo.off_chunk_seq);
    const int64_t blocks = geo.max_chunks * ((geo.H + kWaves - 1) / kWaves);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    auto kern = geo.scalar_gate ? kda_grad_bf16_kernel<true> : kda_grad_bf16_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kWaves), 0, stream, static_cast<const __bf16 *>(q),
                       static_cast<const __bf16 *>(k), static_cast<const __bf16 *>(v), g, beta,
                       static_cast<const __bf16 *>(d_out), cu_seqlens, chunk_off, chunk_seq, geo.T, geo.H, geo.N,
                       geo.max_chunks, base + geo.off_states, base + geo.off_dstates, static_cast<__bf16 *>(dq),
                       static_cast<__bf16 *>(dk), static_cast<__bf16 *>(dv), dg, dbeta);
    return hipGetLastError();
}

}  // namespace kda
