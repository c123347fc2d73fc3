// kda_inter_bf16.hip -- recurrent inter-chunk kernel, bf16 io, K = V = 128.
//
// Carries each (sequence, head) state S (128 x 128 fp32) from chunk to chunk: the
// low-parallelism half of the two-kernel split (augursoft.site
// "Kimi K3 的三個系統設計", section "為什麼 FlashKDA 選擇 16-token chunks"). The
// state's value columns are independent (column j of S and of the output depends
// only on column j of v and of the initial state), so one 64-lane wave owns 16
// columns of one head: its 128 x 16 slice of S lives in MFMA accumulator registers
// for the whole sequence. A workgroup of 2 waves covers 32 columns of one head and
// shares one copy of each chunk's operands.
//
// Per chunk, with S the state at the chunk start and V the chunk's value tile
// (T', M, W, Q~, K^d and gamma from the intra-chunk kernel):
//   U     = T' V                      (two-term bf16 split of T'; V is exact)
//   Delta = U - W S                   (S rounded to bf16 as the MFMA operand)
//   O     = Q~ S + M V                -> out (bf16)
//   S     = Diag(gamma) S + K^d^T Delta   (two-term bf16 split of Delta)
// The accumulator layout of S (lane: rows 4grp + i of column c) is, after rounding
// to bf16, directly the B operand of W S and Q~ S, because the intra-chunk kernel
// stores W and Q~ with matching channel order; Delta's accumulator layout is the B
// operand of K^d^T Delta. Nothing moves across lanes except gamma, which is
// broadcast inside 16-lane rows with DPP.
//
// Memory pipeline: a chunk step takes a few hundred cycles while an HBM load takes
// on the order of a microsecond, so each workgroup keeps a ring of DEPTH chunk
// slots in LDS that two producer waves fill with direct buffer->LDS loads
// (buffer_load_dwordx4 ... lds) several chunks ahead; the loads hold no registers.
// A producer waits (s_waitcnt vmcnt) for its own part of a chunk, then one
// s_barrier per chunk publishes the slot to the compute waves.
#include "kda_chunks.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int KD = 128;
constexpr int VD = 128;
constexpr int kTiles = VD / 16;  // 16-column value tiles per head

typedef __attribute__((address_space(3))) void lds_void;

// A workgroup has kNW compute waves (16 value columns each) and kNW producer waves.
// Producers stream each chunk into a ring slot of 16 KiB with 16 wave-wide 1 KiB
// loads (64 lanes x 16 B), eight per producer:
//   pieces 0..13  record bytes [0, 14336)          (W, Q~, K^d, T', M)
//   piece 14      record bytes [14336, 14848) = gamma, lanes 32..63 load it again into [14848, 15360)
//   piece 15      value tile [16 tokens][32 columns] bf16 at kVOff
// Producer p issues record pieces 7p .. 7p + 6 and then piece 14 + p, so every load
// of a producer has one role and each producer issues exactly kPerWave per chunk.
// Only producers wait on the vector-memory counter, and they never store, so the
// count they wait on covers their own loads alone; compute waves only read LDS,
// compute and store.
constexpr int kNW = 2;
constexpr int kPerWave = 8;
constexpr int kSlotBytes = 16384;
constexpr int kVOff = 15360;
static_assert(kRecGAM == 14336 && kRecBytesBf16 == 14848, "record layout");

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

// s_waitcnt vmcnt(N) without waiting on the LDS / export counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this (producer) wave's loads for one chunk have landed: at most
// `later` chunks' loads, issued after that chunk's, may stay outstanding. Vector
// memory loads complete in issue order and producers issue nothing else, so the
// count is exact. `later` is wave-uniform and in [0, DEPTH - 2].
template <int PER_WAVE, int DEPTH>
__device__ __forceinline__ void wait_for_chunk(int later) {
    static_assert(DEPTH >= 2 && DEPTH <= 8, "extend the switch");
    switch (later) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<(DEPTH > 2 ? 1 : 0) * PER_WAVE>(); break;
    case 2: wait_vmcnt<(DEPTH > 3 ? 2 : 0) * PER_WAVE>(); break;
    case 3: wait_vmcnt<(DEPTH > 4 ? 3 : 0) * PER_WAVE>(); break;
    case 4: wait_vmcnt<(DEPTH > 5 ? 4 : 0) * PER_WAVE>(); break;
    case 5: wait_vmcnt<(DEPTH > 6 ? 5 : 0) * PER_WAVE>(); break;
    default: wait_vmcnt<(DEPTH > 7 ? 6 : 0) * PER_WAVE>(); break;
    }
}

// Per-lane byte offsets that stay fixed for the whole sequence.
struct LaneOffsets {
    unsigned int rec;    // lane * 16: record pieces
    unsigned int gam;    // (lane & 31) * 16: gamma (lanes 32..63 load it twice)
    unsigned int v;      // value tile load of this lane: token row lane / 4, 8 columns
    unsigned int out;    // output: token c, columns col + 4grp .. + 3, within the chunk
    unsigned int vrow;   // one token row of v / out in bytes (H * VD * 2)
};

// Buffer descriptor over `bytes` bytes at `base` (wave-uniform). Buffer accesses
// are range-checked by the hardware: loads past the end return zero and stores
// past the end are dropped, which is how rows past a short chunk are handled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Bytes of a chunk's rows [0, len) restricted to the workgroup's 32 columns.
__device__ __forceinline__ int tile_bytes(int len, unsigned int vrow) {
    return len > 0 ? (len - 1) * (int)vrow + kNW * 32 : 0;
}

// Issue producer `producer`'s share of one chunk's loads into the ring slot at LDS byte
// offset `slot`. `rec` (the chunk's record) and `vchunk` (the chunk's first token
// row of v at column col0) are wave-uniform; every address is a scalar base plus a
// per-lane offset fixed for the whole sequence.
__device__ __forceinline__ void issue_chunk(char *ring, unsigned int slot, const char *rec, const char *vchunk,
                                            int len, int producer, const LaneOffsets &lo) {
    const __amdgpu_buffer_rsrc_t rr = rsrc(rec, kRecBytesBf16);
#pragma unroll
    for (int k = 0; k < kPerWave - 1; ++k) {
        const int piece = 7 * producer + k;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(ring + slot + piece * 1024), 16, lo.rec,
                                                 piece * 1024, 0, 0);
    }
    if (producer == 0) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(ring + slot + kRecGAM), 16, lo.gam, kRecGAM, 0,
                                                 0);
    } else {
        const __amdgpu_buffer_rsrc_t rv = rsrc(vchunk, tile_bytes(len, lo.vrow));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(ring + slot + kVOff), 16, lo.v, 0, 0, 0);
    }
}

// One chunk's operands in registers (read from its ring slot ahead of use).
struct ChunkOps {
    bf16x8 w[4], qt[4];
    bf16x8 kd[8];  // K^d^T tile m repeated over both halves of the 32-long reduction
    bf16x8 tb, mm;
    float2 gam;
    bf16x8 vv;     // [V; V] over the 32-long reduction
};

__device__ __forceinline__ void read_ops(ChunkOps &o, const char *slot, int wave, int lane) {
    const int c = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        o.w[s] = *reinterpret_cast<const bf16x8 *>(slot + kRecW + (s * 64 + lane) * 16);
        o.qt[s] = *reinterpret_cast<const bf16x8 *>(slot + kRecQT + (s * 64 + lane) * 16);
    }
    // the same 8 bytes read twice from LDS (an opaque offset keeps the two reads
    // apart) instead of duplicating registers
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        int off = kRecKD + ((m >> 1) * 64 + lane) * 16 + (m & 1) * 8;
        const uint2 a = *reinterpret_cast<const uint2 *>(slot + off);
        asm volatile("" : "+v"(off));
        const uint2 b = *reinterpret_cast<const uint2 *>(slot + off);
        o.kd[m] = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
    }
    o.tb = *reinterpret_cast<const bf16x8 *>(slot + kRecTB + lane * 16);
    o.mm = *reinterpret_cast<const bf16x8 *>(slot + kRecMM + lane * 16);
    o.gam = *reinterpret_cast<const float2 *>(slot + kRecGAM + (grp * 32 + 2 * c) * 4);
    // rows past the end of a short chunk were loaded as zeros (range-checked loads)
    const unsigned short *vt = reinterpret_cast<const unsigned short *>(slot + kVOff);
    unsigned int vb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vb[i] = vt[(4 * grp + i) * (kNW * 16) + wave * 16 + c];
    const unsigned int v01 = vb[0] | (vb[1] << 16), v23 = vb[2] | (vb[3] << 16);
    o.vv = __builtin_bit_cast(bf16x8, make_uint4(v01, v23, v01, v23));
}

__device__ __forceinline__ void compute_chunk(const ChunkOps &o, f32x4 (&S)[8], char *ochunk, int len,
                                              const LaneOffsets &lo) {
    bf16x8 sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sb[s][i] = to_bf16(S[2 * s][i]);
            sb[s][4 + i] = to_bf16(S[2 * s + 1][i]);
        }
    }
    // The output is formed transposed, O^T = S^T Q~^T + V^T M^T, by swapping the
    // operands: 16x16x32 operand layouts are symmetric (lane l: row / column l % 16,
    // eight reduction elements), so the same registers serve. Each lane then holds
    // four consecutive value columns of one token and stores them at once.
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 x = zero, y = zero;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        x = mfma_16x16x32(o.w[s], sb[s], x);
        y = mfma_16x16x32(sb[s], o.qt[s], y);
    }
    const f32x4 u = mfma_16x16x32(o.tb, o.vv, zero);  // T' V
    y = mfma_16x16x32(o.vv, o.mm, y);                 // + (M V)^T

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
    for (int m = 0; m < 8; ++m) S[m] = mfma_16x16x32(o.kd[m], db, S[m]);  // K^d^T (Delta_hi + Delta_lo)

    // y[i] = O[token c][column 4grp + i]: one 8-byte store per lane; rows past the
    // end of a short chunk fall outside the descriptor and are dropped
    const __amdgpu_buffer_rsrc_t ro = rsrc(ochunk, tile_bytes(len, lo.vrow));
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 packed = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    __builtin_amdgcn_raw_buffer_store_b64(packed, ro, lo.out, 0, 0);
}

template <int DEPTH>
__global__ __launch_bounds__(128 * kNW) void kda_inter_bf16_kernel(
    const unsigned short *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const float *__restrict__ s0, unsigned short *__restrict__ out,
    float *__restrict__ sT, int64_t T, int H, int N, int64_t max_chunks,
    const char *__restrict__ records) {
    static_assert(DEPTH >= 3, "a slot is refilled two chunks after it was read");
    static_assert((DEPTH - 1) * kPerWave < 64, "a producer's loads in flight must fit the 6-bit counter");
    extern __shared__ __attribute__((aligned(1024))) char ring[];
    int pair, vg;
    xcd_unit_split(blockIdx.x, kTiles / kNW, pair, vg);
    if (pair >= N * H) return;  // whole workgroup
    const int n = pair / H, h = pair % H;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, grp = lane >> 4;
    const int col0 = vg * kNW * 16;  // first value column of the workgroup
    const SeqChunks sc = seq_chunks(cu, chunk_off, n, T, max_chunks);
    const int64_t nchunks = sc.chunk_end - sc.chunk_begin;

    LaneOffsets lo;
    lo.vrow = (unsigned int)H * VD * 2;
    lo.rec = lane * 16;
    lo.gam = (lane & 31) * 16;
    lo.v = (lane >> 2) * lo.vrow + (lane & 3) * 16;
    lo.out = c * lo.vrow + (wid * 16 + 4 * grp) * 2;  // compute waves: token c, columns 4grp..+3 (from col0)
    const size_t tok_bytes = ((size_t)sc.tok_begin * H + h) * VD * 2 + (size_t)col0 * 2;
    const size_t chunk_rows = (size_t)16 * lo.vrow;  // bytes of 16 token rows
    auto len_of = [&](int64_t j) {
        const int64_t rem = sc.tok_end - (sc.tok_begin + 16 * j);
        return rem <= 0 ? 0 : (rem >= 16 ? 16 : (int)rem);
    };
    auto slot_off = [&](int64_t j) { return (unsigned int)__builtin_amdgcn_readfirstlane((int)(j % DEPTH) * kSlotBytes); };
    auto barrier = [&]() {
        asm volatile("" ::: "memory");  // no LDS or global access moves across the barrier
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // Barrier B_j (j = 0 .. nchunks - 1) publishes chunk j's slot. Every wave of the
    // workgroup passes each B_j exactly once.
    if (wid >= kNW) {
        // ---- producer ----
        const int p = wid - kNW;
        const char *rec0 = records + ((size_t)h * max_chunks + sc.chunk_begin) * kRecBytesBf16;  // head-major
        const char *v0 = reinterpret_cast<const char *>(v) + tok_bytes;
        auto issue = [&](int64_t j) {
            issue_chunk(ring, slot_off(j), rec0 + (size_t)j * kRecBytesBf16, v0 + (size_t)j * chunk_rows,
                        len_of(j), p, lo);
        };
        for (int64_t j = 0; j < DEPTH - 1 && j < nchunks; ++j) issue(j);
        for (int64_t j = 0; j < nchunks; ++j) {
            // chunks issued so far: 0 .. last
            const int64_t lim = j == 0 ? DEPTH - 2 : j + DEPTH - 3;
            const int64_t last = lim < nchunks - 1 ? lim : nchunks - 1;
            asm volatile("" ::: "memory");
            wait_for_chunk<kPerWave, DEPTH>((int)(last - j));
            barrier();
            // The slot of chunk j - 2 is free: compute waves read it before B_{j-1} and
            // finished using it before B_j.
            if (j >= 1 && j + DEPTH - 2 < nchunks) issue(j + DEPTH - 2);
        }
        return;
    }

    // ---- compute wave: 16 value columns col0 + 16 wid .. + 15 ----
    f32x4 S[8];
    const size_t sbase = (size_t)pair * KD * VD + col0 + wid * 16 + c;
    if (s0) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[m][i] = s0[sbase + (size_t)(16 * m + 4 * grp + i) * VD];
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    char *o0 = reinterpret_cast<char *>(out) + tok_bytes;

    // Software pipeline: chunk j + 1's operands are read from LDS while chunk j is computed.
    auto step = [&](int64_t j, const ChunkOps &cur, ChunkOps &next) {
        if (j + 1 < nchunks) {
            barrier();  // B_{j+1}
            read_ops(next, ring + slot_off(j + 1), wid, lane);
        }
        compute_chunk(cur, S, o0 + (size_t)j * chunk_rows, len_of(j), lo);
    };
    ChunkOps opa, opb;
    if (nchunks > 0) {
        barrier();  // B_0
        read_ops(opa, ring + slot_off(0), wid, lane);
    }
    for (int64_t j = 0; j < nchunks; j += 2) {
        step(j, opa, opb);
        if (j + 1 < nchunks) step(j + 1, opb, opa);
    }

    if (sT) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sT[sbase + (size_t)(16 * m + 4 * grp + i) * VD] = S[m][i];
    }
}

template <int DEPTH>
hipError_t launch(const void *v, const int32_t *cu_seqlens, const float *s0, void *out, float *sT,
                  const Geometry &geo, const void *ws, hipStream_t stream) {
    const int pairs = geo.N * geo.H;
    const int blocks = ((pairs + 7) / 8) * 8 * (kTiles / kNW);
    const char *base = static_cast<const char *>(ws);
    const int32_t *chunk_off = reinterpret_cast<const int32_t *>(base + geo.off_chunk_off);
    const size_t lds = (size_t)DEPTH * kSlotBytes;
    auto kern = kda_inter_bf16_kernel<DEPTH>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(128 * kNW), lds, stream, static_cast<const unsigned short *>(v),
                       cu_seqlens, chunk_off, s0, static_cast<unsigned short *>(out), sT, geo.T, geo.H, geo.N,
                       geo.max_chunks, base + geo.off_records);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_inter_bf16(const void *v, const int32_t *cu_seqlens, const float *s0, void *out,
                             float *sT, const Geometry &geo, const void *ws, hipStream_t stream) {
    // One workgroup (2 compute + 2 producer waves) per 32 value columns of a
    // (sequence, head). With at most one workgroup per CU the ring is 8 chunks deep
    // (128 KiB of LDS); beyond that it is 4 deep so that two workgroups fit on a CU.
    constexpr int kCUs = 256;
    const int blocks = ((geo.N * geo.H + 7) / 8) * 8 * (kTiles / kNW);
    if (blocks <= kCUs) return launch<8>(v, cu_seqlens, s0, out, sT, geo, ws, stream);
    return launch<4>(v, cu_seqlens, s0, out, sT, geo, ws, stream);
}

}  // namespace kda
