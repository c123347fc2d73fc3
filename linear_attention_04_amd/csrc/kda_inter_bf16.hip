// kda_inter_bf16.hip -- recurrent inter-chunk kernel, bf16 io, K = V = 128.
//
// Carries each (sequence, head) state S (128 x 128 fp32) from chunk to chunk: the
// low-parallelism half of the two-kernel split (augursoft.site
// "Kimi K3 的三個系統設計", section "為什麼 FlashKDA 選擇 16-token chunks"). The
// state's value columns are independent (column j of S and of the output depends
// only on column j of v and of the initial state), so one 64-lane wave owns 16
// columns of one head: its 128 x 16 slice of S lives in MFMA accumulator registers
// for the whole sequence and no wave ever waits for another.
//
// Per chunk, with S the state at the chunk start and V the chunk's 16 x 16 value
// tile (T', M, W, Q~, K^d and gamma from the intra-chunk kernel):
//   U     = T' V                      (two-term bf16 split of T'; V is exact)
//   Delta = U - W S                   (S rounded to bf16 as the MFMA operand)
//   O     = Q~ S + M V                -> out (bf16)
//   S     = Diag(gamma) S + K^d^T Delta   (two-term bf16 split of Delta)
// The accumulator layout of S (lane: rows 4grp + i of column c) is, after rounding
// to bf16, directly the B operand of W S and Q~ S, because the intra-chunk kernel
// stores W and Q~ with matching channel order; Delta's accumulator layout is the B
// operand of K^d^T Delta. Nothing moves across lanes except gamma, which is
// broadcast inside 16-lane rows with DPP.
#include "kda_chunks.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int KD = 128;
constexpr int VD = 128;
constexpr int kTiles = VD / 16;  // value-column tiles per head, one wave each

struct ChunkOps {
    bf16x8 w[4];
    bf16x8 qt[4];
    bf16x8 kd[4];
    bf16x8 tb;
    bf16x8 mm;
    float2 gam;
    uint2 v;  // V[4grp + i][16vt + c] for i = 0..3, bf16 bit patterns, two per word
};

__device__ __forceinline__ void load_ops(ChunkOps &o, const char *__restrict__ rec,
                                         const unsigned short *__restrict__ v, int64_t tok0, int len,
                                         int H, int h, int vt, int lane) {
    const int c = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        o.w[s] = *reinterpret_cast<const bf16x8 *>(rec + kRecW + (s * 64 + lane) * 16);
        o.qt[s] = *reinterpret_cast<const bf16x8 *>(rec + kRecQT + (s * 64 + lane) * 16);
        o.kd[s] = *reinterpret_cast<const bf16x8 *>(rec + kRecKD + (s * 64 + lane) * 16);
    }
    o.tb = *reinterpret_cast<const bf16x8 *>(rec + kRecTB + lane * 16);
    o.mm = *reinterpret_cast<const bf16x8 *>(rec + kRecMM + lane * 16);
    o.gam = *reinterpret_cast<const float2 *>(rec + kRecGAM + (grp * 32 + 2 * c) * 4);
    unsigned int bits[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        bits[i] = r < len ? (unsigned int)v[((size_t)(tok0 + r) * H + h) * VD + 16 * vt + c] : 0u;
    }
    o.v.x = bits[0] | (bits[1] << 16);
    o.v.y = bits[2] | (bits[3] << 16);
}

// {x[0..3], x[0..3]} and {x[4..7], x[4..7]}: a 4-element operand repeated over both
// halves of the 32-long reduction of v_mfma_f32_16x16x32_bf16.
__device__ __forceinline__ bf16x8 dup_lo(bf16x8 x) {
    bf16x8 r;
    r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
    r[4] = x[0]; r[5] = x[1]; r[6] = x[2]; r[7] = x[3];
    return r;
}
__device__ __forceinline__ bf16x8 dup_hi(bf16x8 x) {
    bf16x8 r;
    r[0] = x[4]; r[1] = x[5]; r[2] = x[6]; r[3] = x[7];
    r[4] = x[4]; r[5] = x[5]; r[6] = x[6]; r[7] = x[7];
    return r;
}

template <int M, int I>
__device__ __forceinline__ float gamma_of(const float2 gam) {
    // element e = 4M + I of this lane group's permuted gamma sits in lane e >> 1, slot e & 1
    return row_bcast<((4 * M + I) >> 1)>((I & 1) ? gam.y : gam.x);
}

template <int M>
__device__ __forceinline__ void decay_tile(f32x4 &s, const float2 gam) {
    s[0] *= gamma_of<M, 0>(gam);
    s[1] *= gamma_of<M, 1>(gam);
    s[2] *= gamma_of<M, 2>(gam);
    s[3] *= gamma_of<M, 3>(gam);
}

// One chunk. Two-term products use the 32-long reduction of the MFMA as two
// concatenated 16-long ones: [X_hi | X_lo] . [Y ; Y] = (X_hi + X_lo) Y.
__device__ __forceinline__ void chunk_step(const ChunkOps &o, f32x4 (&S)[8], unsigned short *__restrict__ out,
                                           int64_t tok0, int len, int H, int h, int vt, int lane) {
    const int c = lane & 15, grp = lane >> 4;
    bf16x8 sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sb[s][i] = to_bf16(S[2 * s][i]);
            sb[s][4 + i] = to_bf16(S[2 * s + 1][i]);
        }
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 x = zero, y = zero;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        x = mfma_16x16x32(o.w[s], sb[s], x);
        y = mfma_16x16x32(o.qt[s], sb[s], y);
    }
    // [V; V] over the 32-long reduction (whole-vector bit cast of the packed words)
    const bf16x8 vv = __builtin_bit_cast(bf16x8, make_uint4(o.v.x, o.v.y, o.v.x, o.v.y));
    const f32x4 u = mfma_16x16x32(o.tb, vv, zero);  // T' V
    y = mfma_16x16x32(o.mm, vv, y);                 // + M V

    // Delta = U - W S, split into bf16 hi + lo for the state update
    const f32x4 d = u - x;
    bf16x8 db;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        db[i] = to_bf16(d[i]);
        db[4 + i] = to_bf16(d[i] - from_bf16(db[i]));
    }

    decay_tile<0>(S[0], o.gam);
    decay_tile<1>(S[1], o.gam);
    decay_tile<2>(S[2], o.gam);
    decay_tile<3>(S[3], o.gam);
    decay_tile<4>(S[4], o.gam);
    decay_tile<5>(S[5], o.gam);
    decay_tile<6>(S[6], o.gam);
    decay_tile<7>(S[7], o.gam);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const bf16x8 a = (m & 1) ? dup_hi(o.kd[m >> 1]) : dup_lo(o.kd[m >> 1]);
        S[m] = mfma_16x16x32(a, db, S[m]);  // K^d^T (Delta_hi + Delta_lo)
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        if (r < len) {
            const __bf16 ov = to_bf16(y[i]);
            out[((size_t)(tok0 + r) * H + h) * VD + 16 * vt + c] = __builtin_bit_cast(unsigned short, ov);
        }
    }
}

__global__ __launch_bounds__(64) void kda_inter_bf16_kernel(
    const unsigned short *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const float *__restrict__ s0, unsigned short *__restrict__ out,
    float *__restrict__ sT, int64_t T, int H, int N, int64_t max_chunks,
    const char *__restrict__ records) {
    int pair, vt;
    xcd_unit_split(blockIdx.x, kTiles, pair, vt);
    if (pair >= N * H) return;
    const int n = pair / H, h = pair % H;
    const int lane = threadIdx.x;
    const int c = lane & 15, grp = lane >> 4;
    const SeqChunks sc = seq_chunks(cu, chunk_off, n, T, max_chunks);

    f32x4 S[8];
    const size_t sbase = (size_t)pair * KD * VD + 16 * vt + c;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[m][i] = s0 ? s0[sbase + (size_t)(16 * m + 4 * grp + i) * VD] : 0.f;

    auto span = [&](int64_t ci, int64_t &tok0, int &len) {
        tok0 = sc.tok_begin + 16 * (ci - sc.chunk_begin);
        const int64_t rem = sc.tok_end - tok0;
        len = rem <= 0 ? 0 : (rem >= 16 ? 16 : (int)rem);
    };
    auto rec_of = [&](int64_t ci) { return records + ((size_t)ci * H + h) * kRecBytesBf16; };

    ChunkOps opa, opb;
    int64_t ci = sc.chunk_begin;
    int64_t tok_a = 0, tok_b = 0;
    int len_a = 0, len_b = 0;
    if (ci < sc.chunk_end) {
        span(ci, tok_a, len_a);
        load_ops(opa, rec_of(ci), v, tok_a, len_a, H, h, vt, lane);
    }
    while (ci < sc.chunk_end) {
        if (ci + 1 < sc.chunk_end) {
            span(ci + 1, tok_b, len_b);
            load_ops(opb, rec_of(ci + 1), v, tok_b, len_b, H, h, vt, lane);
        }
        chunk_step(opa, S, out, tok_a, len_a, H, h, vt, lane);
        if (++ci >= sc.chunk_end) break;
        if (ci + 1 < sc.chunk_end) {
            span(ci + 1, tok_a, len_a);
            load_ops(opa, rec_of(ci + 1), v, tok_a, len_a, H, h, vt, lane);
        }
        chunk_step(opb, S, out, tok_b, len_b, H, h, vt, lane);
        ++ci;
    }

    if (sT) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sT[sbase + (size_t)(16 * m + 4 * grp + i) * VD] = S[m][i];
    }
}

}  // namespace

hipError_t launch_inter_bf16(const void *v, const int32_t *cu_seqlens, const float *s0, void *out,
                             float *sT, const Geometry &geo, const void *ws, hipStream_t stream) {
    const int pairs = geo.N * geo.H;
    const int blocks = ((pairs + 7) / 8) * 8 * kTiles;
    const char *base = static_cast<const char *>(ws);
    const int32_t *chunk_off = reinterpret_cast<const int32_t *>(base + geo.off_chunk_off);
    hipLaunchKernelGGL(kda_inter_bf16_kernel, dim3(blocks), dim3(64), 0, stream,
                       static_cast<const unsigned short *>(v), cu_seqlens, chunk_off, s0,
                       static_cast<unsigned short *>(out), sT, geo.T, geo.H, geo.N, geo.max_chunks,
                       base + geo.off_records);
    return hipGetLastError();
}

}  // namespace kda
