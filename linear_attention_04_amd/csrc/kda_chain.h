// kda_chain.h -- the compute side of the recurrent inter-chunk step, bf16 io, K = V = 128:
// the waves that carry a (sequence, head) state slice from chunk to chunk over an LDS
// ring of chunk records. Shared by the two-kernel prefill's recurrent kernel and the
// single-kernel ablation, which differ only in how the ring is filled; the Sync
// argument is the barrier the chain's waves pass once per chunk (the hardware
// workgroup barrier for both).
//
// Per chunk, with S the state at the chunk start and V the chunk's value tile
// (T', M, W, Q~, K^d and gamma from the chunk's record):
//   U     = T' V                      (two-term bf16 split of T'; V is exact)
//   Delta = U - W S                   (S rounded to bf16 as the MFMA operand)
//   O     = Q~ S + M V                -> out (bf16)
//   S     = Diag(gamma) S + K^d^T Delta   (two-term bf16 split of Delta)
// (augursoft.site "Kimi K3 的三個系統設計", section "為什麼 FlashKDA 選擇 16-token chunks":
// the recurrent half of the two-kernel split.)
#pragma once

#include "kda_chunks.h"
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_ring.h"

namespace kda {
namespace {

constexpr int KD = 128;
constexpr int VD = 128;
constexpr int kTiles = VD / 16;  // 16-column value tiles per head


// A workgroup covers NW tiles of 16 value columns (NW = 2, or 4 when 2-tile
// workgroups would outnumber the CUs) with its compute waves, two per tile in the
// two-wave form or one in the whole-tile form, and two producer waves. Producers
// stream each chunk into a ring slot of 15 KiB + NW / 2 KiB with wave-wide 1 KiB
// loads (64 lanes x 16 B):
//   pieces 0..13  record bytes [0, 14336)          (W, Q~, K^d, T', M)
//   piece 14      record bytes [14336, 14848) = gamma, lanes 32..63 load it again into [14848, 15360)
//   then          value tile [16 tokens][16 NW columns] bf16 at kVOff, NW / 2 pieces
// Producer 0 issues record pieces 0 .. 6 and gamma (kPerWave0 loads per chunk),
// producer 1 record pieces 7 .. 13 and the value tile (per_wave1<NW>()), so every
// load of a producer has one role and each producer issues a fixed number per chunk.
// Only producers wait on the vector-memory counter, and they never store, so the
// count they wait on covers their own loads alone; compute waves only read LDS,
// compute and store (or stage their stores in LDS for a store wave, below).
constexpr int kNW = 2;  // the default tile count (and the single-kernel ablation's)
constexpr int kPerWave0 = 8;
template <int NW>
constexpr int per_wave1() { return 7 + NW / 2; }
constexpr int kVOff = 15360;
template <int NW>
constexpr int slot_bytes() { return kVOff + 512 * NW; }
constexpr int kSlotBytes = slot_bytes<kNW>();  // 16 KiB
static_assert(kRecGAM == 14336 && kRecBytesBf16 == 14848, "record layout");


// Per-lane byte offsets that stay fixed for the whole sequence.
struct LaneOffsets {
    unsigned int rec;    // lane * 16: record pieces
    unsigned int gam;    // (lane & 31) * 16: gamma (lanes 32..63 load it twice)
    unsigned int v;      // value tile load of this lane (NW = 2: token row lane / 4, 8 columns;
                         // NW = 4: token row lane / 8, 8 columns)
    unsigned int v2;     // NW = 4: the second value tile load (token rows 8 .. 15)
    unsigned int out;    // output: token c, columns col + 4grp .. + 3, within the chunk
    unsigned int vrow;   // one token row of v / out in bytes (H * VD * 2)
    unsigned int stage;  // staged output (4-tile whole-tile form): byte in a staging buffer
};


// Bytes of a chunk's rows [0, len) restricted to the workgroup's 16 NW columns.
template <int NW>
__device__ __forceinline__ int tile_bytes(int len, unsigned int vrow) {
    return len > 0 ? (len - 1) * (int)vrow + NW * 32 : 0;
}

// Issue producer `producer`'s share of one chunk's loads into the ring slot at LDS byte
// offset `slot`. `rec` (the chunk's record) and `vchunk` (the chunk's first token
// row of v at column col0) are wave-uniform; every address is a scalar base plus a
// per-lane offset fixed for the whole sequence.
template <int NW>
__device__ __forceinline__ void issue_chunk(char *ring, unsigned int slot, const char *rec, const char *vchunk,
                                            int len, int producer, const LaneOffsets &lo) {
    const __amdgpu_buffer_rsrc_t rr = rsrc(rec, kRecBytesBf16);
#pragma unroll
    for (int k = 0; k < 7; ++k) {
        const int piece = 7 * producer + k;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(ring + slot + piece * 1024), 16, lo.rec,
                                                 piece * 1024, 0, 0);
    }
    if (producer == 0) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(ring + slot + kRecGAM), 16, lo.gam, kRecGAM, 0,
                                                 0);
    } else {
        const __amdgpu_buffer_rsrc_t rv = rsrc(vchunk, tile_bytes<NW>(len, lo.vrow));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(ring + slot + kVOff), 16, lo.v, 0, 0, 0);
        if (NW == 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(ring + slot + kVOff + 1024), 16, lo.v2, 0, 0,
                                                     0);
    }
}

// Compute waves of the two-wave form: NW value tiles x 2 halves of the key
// dimension. Compute wave (vt, kh) holds rows 64 kh .. 64 kh + 63 of tile vt's
// 128 x 16 state slice, i.e. the four 16 x 16 accumulator tiles M = 4 kh .. 4 kh + 3.
// W S, Q~ S and K^d^T Delta all split along those rows, so each chunk costs a wave
// half the MFMA and VALU work of the whole slice; the two halves of a tile swap their
// partial W S through LDS at the chunk barrier, and half 1 hands half 0 its partial
// Q~ S for the output.
constexpr int kHalves = 2;
constexpr int kProducers = 2;
template <int NW>
constexpr int compute_waves() { return NW * kHalves; }
template <int NW>
constexpr int waves() { return compute_waves<NW>() + kProducers; }  // compute waves, then producers
constexpr int kComputeWaves = compute_waves<kNW>();

// Exchange area after the ring: [chunk parity][tile][slot][64 lanes] f32x4 with
// slot 0 = half 0's W S part, slot 1 = half 1's W S part minus T' V, slot 2 = half
// 1's Q~ S part (transposed output layout).
constexpr int kXchgSlots = 3;
template <int NW>
constexpr int xchg_bytes() { return 2 * NW * kXchgSlots * 1024; }
constexpr int kXchgBytes = xchg_bytes<kNW>();

// Output staging of the 4-tile forms (both the one-wave and the two-wave form). The
// compute waves that form the output write each chunk's output tile (16 token rows x 64
// columns, bf16) to LDS, and a store wave writes it to HBM as whole 128-byte rows, so
// the compute waves issue no global stores. Two chunk buffers after the ring (and the
// exchange area of the two-wave form); rows padded to 144 bytes so that the compute
// waves' 8-byte writes spread over the banks. Every wave of the workgroup passes one
// extra barrier at the end, after which the store wave takes the last chunk's output.
constexpr int kStageRow = 144;
constexpr int kStageBytes = 16 * kStageRow;
constexpr int kStageBufs = 2;
template <int NW, bool OUT>
constexpr bool staged_out() { return OUT && NW == 4; }
template <int NW, bool OUT>
constexpr int stage_bytes() { return staged_out<NW, OUT>() ? kStageBufs * kStageBytes : 0; }

// Saved-state staging of the training forward (the 2-tile two-wave form with SAVE and
// OUT). Its compute waves write each chunk's start state, the workgroup's eight 1 KiB
// bf16 fragments, to LDS, and a store wave writes them to HBM after the chunk's
// barrier, so the chain's waves issue none of the 1 GiB of state stores (at H=64,
// T=8192) themselves. Two chunk buffers after the exchange area. The backward's
// recomputed forward (SAVE without OUT) stores its states directly: staged, it was
// slower.
constexpr int kSaveStageBytes = 2 * 4096;
template <int NW, bool SAVE, bool OUT>
constexpr bool staged_save() { return SAVE && OUT && NW == 2; }
template <int NW, bool SAVE, bool OUT>
constexpr int save_stage_bytes() { return staged_save<NW, SAVE, OUT>() ? 2 * kSaveStageBytes : 0; }

// One chunk's operands for one half, in registers (read from the ring slot ahead of use).
struct HalfOps {
    bf16x8 w[2], qt[2];  // slabs 2 kh, 2 kh + 1 of W and Q~
    bf16x8 kd[4];        // K^d^T tiles 4 kh .. 4 kh + 3, each over both halves of the 32-long reduction
    bf16x8 tv;           // half 0: M (hi | lo), for M V; half 1: T' (hi | lo), for T' V
    float2 gam;
    bf16x8 vv;           // [V; V] over the 32-long reduction
};

template <int KH, int NW>
__device__ __forceinline__ void read_ops(HalfOps &o, const char *slot, int vt, int lane) {
    const int c = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        o.w[s] = *reinterpret_cast<const bf16x8 *>(slot + kRecW + ((2 * KH + s) * 64 + lane) * 16);
        o.qt[s] = *reinterpret_cast<const bf16x8 *>(slot + kRecQT + ((2 * KH + s) * 64 + lane) * 16);
    }
    // the same 8 bytes read twice from LDS (volatile LDS reads are not merged into
    // one) instead of duplicating registers
    typedef const volatile __attribute__((address_space(3))) unsigned long long lds_u64;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
        const int m = 4 * KH + mm;
        lds_u64 *pk = (lds_u64 *)(slot + kRecKD + ((m >> 1) * 64 + lane) * 16 + (m & 1) * 8);
        const unsigned long long a = *pk;
        const unsigned long long b = *pk;
        o.kd[mm] = __builtin_bit_cast(bf16x8, make_uint4((unsigned)a, (unsigned)(a >> 32), (unsigned)b,
                                                         (unsigned)(b >> 32)));
    }
    o.tv = *reinterpret_cast<const bf16x8 *>(slot + (KH ? kRecTB : kRecMM) + lane * 16);
    o.gam = *reinterpret_cast<const float2 *>(slot + kRecGAM + (grp * 32 + 2 * c) * 4);
    // rows past the end of a short chunk were loaded as zeros (range-checked loads)
    const unsigned short *vt16 = reinterpret_cast<const unsigned short *>(slot + kVOff);
    unsigned int vb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vb[i] = vt16[(4 * grp + i) * (NW * 16) + vt * 16 + c];
    const unsigned int v01 = vb[0] | (vb[1] << 16), v23 = vb[2] | (vb[3] << 16);
    o.vv = __builtin_bit_cast(bf16x8, make_uint4(v01, v23, v01, v23));
}


// First half of a chunk step, before the barrier: partial W S and Q~ S over this
// wave's rows, published to the partner; then the decay of this wave's rows.
// SAVE (the forward for a backward pass): the chunk's start state goes to `sdst` as
// bf16 fragments (ct, 2 KH) and (ct, 2 KH + 1), in HBM, or with SST in the LDS staging
// buffer. OUT: the output's partial products are formed (a recomputed forward that
// only saves states skips them).
template <int KH, bool SAVE = false, bool OUT = true, bool SST = false>
__device__ __forceinline__ void chunk_part_a(const HalfOps &o, f32x4 (&S)[4], f32x4 &x, f32x4 &y,
                                             char *xchg, int lane, char *sdst = nullptr) {
    bf16x8 sb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sb[s][i] = to_bf16(S[2 * s][i]);
            sb[s][4 + i] = to_bf16(S[2 * s + 1][i]);
        }
    }
    // The output is formed transposed, O^T = S^T Q~^T + V^T M^T, by swapping the
    // operands: 16x16x32 operand layouts are symmetric (lane l: row / column l % 16,
    // eight reduction elements), so the same registers serve. Each lane then holds
    // four consecutive value columns of one token.
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if (SAVE) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        if (SST) {
            *reinterpret_cast<u32x4 *>(sdst) = __builtin_bit_cast(u32x4, sb[0]);
            *reinterpret_cast<u32x4 *>(sdst + 1024) = __builtin_bit_cast(u32x4, sb[1]);
        } else {
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sb[0]), reinterpret_cast<u32x4 *>(sdst));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sb[1]), reinterpret_cast<u32x4 *>(sdst + 1024));
        }
    }
    x = mfma_16x16x32(o.w[0], sb[0], zero);
    if (OUT) y = mfma_16x16x32(sb[0], o.qt[0], zero);
    x = mfma_16x16x32(o.w[1], sb[1], x);
    if (OUT) y = mfma_16x16x32(sb[1], o.qt[1], y);
    if (KH == 0) {
        *reinterpret_cast<f32x4 *>(xchg + lane * 16) = x;
        if (OUT) y = mfma_16x16x32(o.vv, o.tv, y);  // + (M V)^T
    } else {
        x -= mfma_16x16x32(o.tv, o.vv, zero);  // - T' V
        *reinterpret_cast<f32x4 *>(xchg + 1024 + lane * 16) = x;
        if (OUT) *reinterpret_cast<f32x4 *>(xchg + 2048 + lane * 16) = y;
    }
    decay_tile<4 * KH + 0>(S[0], o.gam);
    decay_tile<4 * KH + 1>(S[1], o.gam);
    decay_tile<4 * KH + 2>(S[2], o.gam);
    decay_tile<4 * KH + 3>(S[3], o.gam);
}

// The partner half's contribution for chunk parity buffer `xchg`: half 0 takes
// half 1's W S part (minus T' V) and output part; half 1 takes half 0's W S part.
template <int KH, bool OUT = true>
__device__ __forceinline__ void read_partner(const char *xchg, int lane, f32x4 &px, f32x4 &py) {
    if (KH == 0) {
        px = *reinterpret_cast<const f32x4 *>(xchg + 1024 + lane * 16);
        if (OUT) py = *reinterpret_cast<const f32x4 *>(xchg + 2048 + lane * 16);
    } else {
        px = *reinterpret_cast<const f32x4 *>(xchg + lane * 16);
    }
}

// Second half, after the barrier: Delta = T' V - W S from both parts (the two
// halves form the same sum, so they hold bitwise equal Delta), the state update of
// this wave's rows and, on half 0, the output.
// STO: the output goes to the LDS staging buffer `stage`, not to `ochunk`.
template <int KH, bool OUT, int NW, bool STO = false>
__device__ __forceinline__ void chunk_part_b(const HalfOps &o, f32x4 (&S)[4], const f32x4 &x, const f32x4 &y,
                                             const f32x4 &px, const f32x4 &py, char *ochunk, int len,
                                             const LaneOffsets &lo, char *stage = nullptr) {
    const f32x4 x0 = KH == 0 ? x : px;
    const f32x4 z1 = KH == 0 ? px : x;
    const f32x4 d = -(x0 + z1);
    unsigned int h01, h23, l01, l23;  // Delta = hi + lo, packed pairs
    split_pair(d[0], d[1], h01, l01);
    split_pair(d[2], d[3], h23, l23);
    const bf16x8 db = __builtin_bit_cast(bf16x8, make_uint4(h01, h23, l01, l23));
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) S[mm] = mfma_16x16x32(o.kd[mm], db, S[mm]);  // K^d^T (Delta_hi + Delta_lo)
    if (KH == 0 && OUT) {
        const f32x4 yt = y + py;
        // yt[i] = O[token c][column 4grp + i]: one 8-byte store (or staging write) per
        // lane; rows past the end of a short chunk fall outside the descriptor and are dropped
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 packed = {pack_bf16x2(yt[0], yt[1]), pack_bf16x2(yt[2], yt[3])};
        if (STO) {
            *reinterpret_cast<u32x2 *>(stage + lo.stage) = packed;
            // kept here, a chunk step ahead of the wait on it (left to the scheduler it
            // sinks to just before that wait)
            __builtin_amdgcn_sched_barrier(0);
        } else {
            const __amdgpu_buffer_rsrc_t ro = rsrc(ochunk, tile_bytes<NW>(len, lo.vrow));
            __builtin_amdgcn_raw_buffer_store_b64(packed, ro, lo.out, 0, 0);
        }
    }
}


// The chunk loop of compute wave (vt, KH). Barrier B_j (j = 0 .. nchunks) is passed
// once by every wave of the workgroup: B_j (j < nchunks) publishes chunk j's ring
// slot, and B_{j+1} also publishes the partial products of chunk j (and with SST, the
// chunk's start state in staging buffer j % 2, `sdst0` being this wave's place in
// buffer 0).
template <int KH, int DEPTH, bool SAVE, bool OUT, int NW, bool SST, bool STO, class Sync>
__device__ __forceinline__ void compute_wave(f32x4 (&S)[4], char *ring, int64_t nchunks, int64_t tok_rows,
                                             char *o0, size_t chunk_rows, int vt, int lane, const LaneOffsets &lo,
                                             Sync &sync, char *sdst0 = nullptr, size_t sstride = 0) {
    auto slot_of = [&](int64_t j) {
        return ring + (unsigned int)__builtin_amdgcn_readfirstlane((int)(j % DEPTH) * slot_bytes<NW>());
    };
    auto xchg_of = [&](int64_t j) {
        return ring + DEPTH * slot_bytes<NW>() + (((int)(j & 1) * NW + vt) * kXchgSlots) * 1024;
    };
    auto len_of = [&](int64_t j) {
        const int64_t rem = tok_rows - 16 * j;
        return rem <= 0 ? 0 : (rem >= 16 ? 16 : (int)rem);
    };
    // Every step reads the next slot, also after the last chunk: that read lands in
    // LDS the workgroup owns and its values are never used, and it keeps the loop
    // body free of branches.
    // STO: chunk j's output goes to staging buffer `buf` = j % 2 (the loop's steps start
    // at even j), waited for before B_{j+2} like the partial products
    char *const ostage0 = ring + DEPTH * slot_bytes<NW>() + xchg_bytes<NW>();
    auto step = [&](int64_t j, const HalfOps &cur, HalfOps &next, int buf) {
        f32x4 x, y, px, py;
        char *xc = xchg_of(j);
        char *sdst = !SAVE ? nullptr : SST ? sdst0 + (int)(j & 1) * kSaveStageBytes : sdst0 + (size_t)j * sstride;
        chunk_part_a<KH, SAVE, OUT, SST>(cur, S, x, y, xc, lane, sdst);
        if (SST) asm volatile("" ::: "memory");  // the staged state is written before the wait
        wait_lgkm0();  // the partial products (and a staged state) are in LDS before the barrier
        sync.barrier(j + 1);  // B_{j+1}
        read_partner<KH, OUT>(xc, lane, px, py);
        read_ops<KH, NW>(next, slot_of(j + 1), vt, lane);
        chunk_part_b<KH, OUT, NW, STO>(cur, S, x, y, px, py, OUT ? o0 + (size_t)j * chunk_rows : nullptr,
                                        len_of(j), lo, ostage0 + buf * kStageBytes);
    };
    HalfOps opa, opb;
    sync.barrier(0);  // B_0
    read_ops<KH, NW>(opa, slot_of(0), vt, lane);
    int64_t j = 0;
    for (; j + 2 <= nchunks; j += 2) {
        step(j, opa, opb, 0);
        step(j + 1, opb, opa, 1);
    }
    if (j < nchunks) step(j, opa, opb, 0);
    if (STO) {
        wait_lgkm0();
        sync.barrier(nchunks + 1);  // B_{nchunks+1}: the last chunk's staged output is in LDS
    }
}

// The compute waves' part of a recurrent workgroup: the state slice in, the chunk
// loop over the LDS ring, the state slice out. Compute wave (vt, kh) owns value
// columns col0 + 16 vt .. + 15 and key rows 64 kh .. + 63. SAVE: `states` points at
// the sequence's first chunk in the [max_chunks][H] array of chunk start states, and
// `sstride` is the distance between a pair's consecutive chunks there.
// OUT: the chunk outputs go to `out`. The final state goes to `sT` unless it is NULL.
template <int DEPTH, bool SAVE, bool OUT, int NW, bool SST, bool STO, class Sync>
__device__ __forceinline__ void compute_role(char *ring, int wid, int lane, int pair, int col0, const SeqChunks &sc,
                                             size_t tok_bytes, size_t chunk_rows, LaneOffsets lo,
                                             const float *__restrict__ s0, unsigned short *__restrict__ out,
                                             float *__restrict__ sT, Sync &sync, char *states = nullptr,
                                             size_t sstride = 0) {
    const int c = lane & 15, grp = lane >> 4;
    const int vt = wid >> 1, kh = wid & 1;
    lo.out = c * lo.vrow + (vt * 16 + 4 * grp) * 2;  // token c, columns 4grp .. + 3 of the tile
    lo.stage = c * kStageRow + (vt * 16 + 4 * grp) * 2;
    f32x4 S[4];
    const size_t sbase = (size_t)pair * KD * VD + (size_t)(64 * kh) * VD + col0 + vt * 16 + c;
    if (s0) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[m][i] = s0[sbase + (size_t)key_of(m, 4 * grp + i) * VD];
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Settle the state loads here: otherwise the counter wait that guards S's first
    // use sits inside the chunk loop and, since stores count on the same counter,
    // makes every chunk wait for the previous chunk's output store to complete.
    wait_vmcnt<0>();
    char *o0 = OUT ? reinterpret_cast<char *>(out) + tok_bytes : nullptr;
    const int64_t nchunks = sc.chunk_end - sc.chunk_begin;
    const int64_t tok_rows = sc.tok_end - sc.tok_begin;
    // fragment (ct, 2 kh) of each chunk start state, ct = this wave's value tile; with
    // SST its place in the staging buffer, which holds the workgroup's fragments in order
    char *sdst0 = !SAVE ? nullptr
                  : SST ? ring + DEPTH * slot_bytes<NW>() + xchg_bytes<NW>() + ((vt * 4 + 2 * kh) * 64 + lane) * 16
                        : states + ((size_t)(((col0 >> 4) + vt) * 4 + 2 * kh) * 64 + lane) * 16;
    if (kh == 0)
        compute_wave<0, DEPTH, SAVE, OUT, NW, SST, STO>(S, ring, nchunks, tok_rows, o0, chunk_rows, vt, lane, lo,
                                                        sync, sdst0, sstride);
    else
        compute_wave<1, DEPTH, SAVE, OUT, NW, SST, STO>(S, ring, nchunks, tok_rows, o0, chunk_rows, vt, lane, lo,
                                                        sync, sdst0, sstride);

    if (sT) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[sbase + (size_t)key_of(m, 4 * grp + i) * VD] = S[m][i];
    }
}


// ---------------------------------------------------------------------------
// Whole-tile form: one compute wave per tile holds all 128 key rows of the tile's
// 128 x 16 slice (the eight accumulator tiles M = 0 .. 7). There is no partner and
// no exchange: the barrier a chunk step passes only hands ring slots over from the
// producers, and nothing on the chain waits for another wave. A step does the two
// halves' work of the split form in one wave with the same operations in the same
// order (x0, x1 and y0, y1 below are the halves' partial products), so both forms
// give bitwise equal outputs and states.
struct TileOps {
    bf16x8 w[4], qt[4];  // the four slabs of W and Q~
    bf16x8 kd[8];        // K^d^T tiles 0 .. 7, each over both halves of the 32-long reduction
    bf16x8 tb, mm;       // T' (hi | lo) and M (hi | lo)
    float2 gam;
    unsigned int vb[4];  // value tile column c, token rows 4 grp .. + 3 (as read; see tile_vv)
};

// [V; V] over the 32-long reduction from the four values read. Kept out of
// read_tile_ops: formed there, right after the reads are issued, it makes the wave
// wait for every read of the step in the middle of the state update.
__device__ __forceinline__ bf16x8 tile_vv(const TileOps &o) {
    const unsigned int v01 = o.vb[0] | (o.vb[1] << 16), v23 = o.vb[2] | (o.vb[3] << 16);
    return __builtin_bit_cast(bf16x8, make_uint4(v01, v23, v01, v23));
}

template <int NW>
__device__ __forceinline__ void read_tile_ops(TileOps &o, const char *slot, int vt, int lane) {
    const int c = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        o.w[s] = *reinterpret_cast<const bf16x8 *>(slot + kRecW + (s * 64 + lane) * 16);
        o.qt[s] = *reinterpret_cast<const bf16x8 *>(slot + kRecQT + (s * 64 + lane) * 16);
    }
    // [K^d; K^d]: with two tiles per workgroup, two reads of the same 8 bytes (the
    // volatile keeps them apart), which costs the chain less than two register copies;
    // with four, whose compute waves share the CU's LDS bandwidth, one read copied.
    typedef const volatile __attribute__((address_space(3))) unsigned long long lds_u64;
    if (NW == 4) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const unsigned long long a = *reinterpret_cast<const unsigned long long *>(
                slot + kRecKD + ((m >> 1) * 64 + lane) * 16 + (m & 1) * 8);
            o.kd[m] = __builtin_bit_cast(bf16x8, make_uint4((unsigned)a, (unsigned)(a >> 32), (unsigned)a,
                                                            (unsigned)(a >> 32)));
        }
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            lds_u64 *pk = (lds_u64 *)(slot + kRecKD + ((m >> 1) * 64 + lane) * 16 + (m & 1) * 8);
            const unsigned long long a = *pk;
            const unsigned long long b = *pk;
            o.kd[m] = __builtin_bit_cast(bf16x8, make_uint4((unsigned)a, (unsigned)(a >> 32), (unsigned)b,
                                                            (unsigned)(b >> 32)));
        }
    }
    o.tb = *reinterpret_cast<const bf16x8 *>(slot + kRecTB + lane * 16);
    o.mm = *reinterpret_cast<const bf16x8 *>(slot + kRecMM + lane * 16);
    o.gam = *reinterpret_cast<const float2 *>(slot + kRecGAM + (grp * 32 + 2 * c) * 4);
    const unsigned short *vt16 = reinterpret_cast<const unsigned short *>(slot + kVOff);
#pragma unroll
    for (int i = 0; i < 4; ++i) o.vb[i] = vt16[(4 * grp + i) * (NW * 16) + vt * 16 + c];
}

// Before the barrier: W S in two partial sums over key rows 0 .. 63 (x0) and
// 64 .. 127 (x1, then minus T' V), the output's two partial sums (M V joins y0),
// then the decay of all eight accumulator tiles.
template <bool OUT>
__device__ __forceinline__ void tile_part_a(const TileOps &o, f32x4 (&S)[8], f32x4 &x0, f32x4 &x1, f32x4 &y) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    bf16x8 sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sb[s][i] = to_bf16(S[2 * s][i]);
            sb[s][4 + i] = to_bf16(S[2 * s + 1][i]);
        }
    }
    f32x4 y0, y1;
    x0 = mfma_16x16x32(o.w[0], sb[0], zero);
    x1 = mfma_16x16x32(o.w[2], sb[2], zero);
    if (OUT) y0 = mfma_16x16x32(sb[0], o.qt[0], zero);
    if (OUT) y1 = mfma_16x16x32(sb[2], o.qt[2], zero);
    x0 = mfma_16x16x32(o.w[1], sb[1], x0);
    x1 = mfma_16x16x32(o.w[3], sb[3], x1);
    if (OUT) y0 = mfma_16x16x32(sb[1], o.qt[1], y0);
    if (OUT) y1 = mfma_16x16x32(sb[3], o.qt[3], y1);
    const bf16x8 vv = tile_vv(o);
    x1 -= mfma_16x16x32(o.tb, vv, zero);  // - T' V
    if (OUT) {
        y0 = mfma_16x16x32(vv, o.mm, y0);  // + (M V)^T
        y = y0 + y1;
    }
    decay_tile<0>(S[0], o.gam);
    decay_tile<1>(S[1], o.gam);
    decay_tile<2>(S[2], o.gam);
    decay_tile<3>(S[3], o.gam);
    decay_tile<4>(S[4], o.gam);
    decay_tile<5>(S[5], o.gam);
    decay_tile<6>(S[6], o.gam);
    decay_tile<7>(S[7], o.gam);
}

// After the barrier: Delta = T' V - W S, the state update of all eight tiles and
// the output store.
// ST: the output goes to the LDS staging buffer `stage`, not to `ochunk`.
template <bool OUT, int NW, bool ST = false>
__device__ __forceinline__ void tile_part_b(const TileOps &o, f32x4 (&S)[8], const f32x4 &x0, const f32x4 &x1,
                                            const f32x4 &y, char *ochunk, int len, const LaneOffsets &lo,
                                            char *stage = nullptr) {
    const f32x4 d = -(x0 + x1);
    unsigned int h01, h23, l01, l23;
    split_pair(d[0], d[1], h01, l01);
    split_pair(d[2], d[3], h23, l23);
    const bf16x8 db = __builtin_bit_cast(bf16x8, make_uint4(h01, h23, l01, l23));
#pragma unroll
    for (int m = 0; m < 8; ++m) S[m] = mfma_16x16x32(o.kd[m], db, S[m]);
    if (OUT) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 packed = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        if (ST) {
            *reinterpret_cast<u32x2 *>(stage + lo.stage) = packed;
            // Issued here, a chunk step before the wait on it: left to the scheduler, the
            // write sinks to just before that wait and its latency lands on the chain.
            __builtin_amdgcn_sched_barrier(0);
        } else {
            const __amdgpu_buffer_rsrc_t ro = rsrc(ochunk, tile_bytes<NW>(len, lo.vrow));
            __builtin_amdgcn_raw_buffer_store_b64(packed, ro, lo.out, 0, 0);
        }
    }
}

// The chunk loop of the whole-tile compute wave of tile vt; barriers as in
// compute_wave (B_j publishes chunk j's ring slot).
// STAGE: chunk j's output goes to staging buffer j % 2 after the ring, for the store
// wave (store_wave). A compute wave writes it after B_{j+1} and waits for its LDS
// accesses before B_{j+2}; after the last chunk it passes the extra barrier B_{nchunks+1}.
template <int DEPTH, bool OUT, int NW, bool STAGE, class Sync>
__device__ __forceinline__ void compute_wave_full(f32x4 (&S)[8], char *ring, int64_t nchunks, int64_t tok_rows,
                                                  char *o0, size_t chunk_rows, int vt, int lane,
                                                  const LaneOffsets &lo, Sync &sync) {
    auto slot_of = [&](int64_t j) {
        return ring + (unsigned int)__builtin_amdgcn_readfirstlane((int)(j % DEPTH) * slot_bytes<NW>());
    };
    auto len_of = [&](int64_t j) {
        const int64_t rem = tok_rows - 16 * j;
        return rem <= 0 ? 0 : (rem >= 16 ? 16 : (int)rem);
    };
    char *const stage0 = ring + DEPTH * slot_bytes<NW>();
    // buf: chunk j's staging buffer, j % 2 (the loop's steps start at even j)
    auto step = [&](int64_t j, const TileOps &cur, TileOps &next, int buf) {
        f32x4 x0, x1, y;
        tile_part_a<OUT>(cur, S, x0, x1, y);
        if (STAGE) wait_lgkm0();  // the previous chunk's staged output is in LDS
        sync.barrier(j + 1);      // B_{j+1}
        read_tile_ops<NW>(next, slot_of(j + 1), vt, lane);
        tile_part_b<OUT, NW, STAGE>(cur, S, x0, x1, y, OUT ? o0 + (size_t)j * chunk_rows : nullptr, len_of(j), lo,
                                    stage0 + buf * kStageBytes);
    };
    TileOps opa, opb;
    sync.barrier(0);  // B_0
    read_tile_ops<NW>(opa, slot_of(0), vt, lane);
    int64_t j = 0;
    for (; j + 2 <= nchunks; j += 2) {
        step(j, opa, opb, 0);
        step(j + 1, opb, opa, 1);
    }
    if (j < nchunks) step(j, opa, opb, 0);
    if (STAGE) {
        wait_lgkm0();
        sync.barrier(nchunks + 1);  // B_{nchunks+1}: the last chunk's staged output is in LDS
    }
}

// compute_role for the whole-tile form: compute wave vt owns value columns
// col0 + 16 vt .. + 15 and all 128 key rows.
template <int DEPTH, bool OUT, int NW, bool STAGE, class Sync>
__device__ __forceinline__ void compute_role_full(char *ring, int vt, int lane, int pair, int col0,
                                                  const SeqChunks &sc, size_t tok_bytes, size_t chunk_rows,
                                                  LaneOffsets lo, const float *__restrict__ s0,
                                                  unsigned short *__restrict__ out, float *__restrict__ sT,
                                                  Sync &sync) {
    const int c = lane & 15, grp = lane >> 4;
    lo.out = c * lo.vrow + (vt * 16 + 4 * grp) * 2;
    lo.stage = c * kStageRow + (vt * 16 + 4 * grp) * 2;
    f32x4 S[8];
    const size_t sbase = (size_t)pair * KD * VD + col0 + vt * 16 + c;
    if (s0) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[m][i] = s0[sbase + (size_t)key_of(m, 4 * grp + i) * VD];
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    wait_vmcnt<0>();  // as in compute_role: no state load left for the loop's counter waits
    char *o0 = OUT ? reinterpret_cast<char *>(out) + tok_bytes : nullptr;
    compute_wave_full<DEPTH, OUT, NW, STAGE>(S, ring, sc.chunk_end - sc.chunk_begin, sc.tok_end - sc.tok_begin,
                                             o0, chunk_rows, vt, lane, lo, sync);
    if (sT) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[sbase + (size_t)key_of(m, 4 * grp + i) * VD] = S[m][i];
    }
}


// The store wave of the staged form: chunk j's output tile leaves staging buffer j % 2
// after barrier B_{j+2}, by which the compute waves have written it (after B_{j+1},
// waiting for the writes before B_{j+2}), and before B_{j+3}, after which they write
// the buffer again. Rows past a short last chunk are dropped by the buffer range. It
// passes the same nchunks + 2 barriers as the other waves. Lane l stores bytes
// 16 (l % 8) .. + 15 of rows l / 8 and l / 8 + 8.
template <int NW, class Sync>
__device__ __forceinline__ void store_wave(const char *stage0, int64_t nchunks, int64_t tok_rows, char *o0,
                                           size_t chunk_rows, int lane, unsigned int vrow, Sync &sync) {
    static_assert(NW == 4, "a staged row is 128 bytes");
    const int r = lane >> 3, p = lane & 7;
    const unsigned int off = (unsigned int)r * vrow + 16u * p;
    sync.barrier(0);  // B_0
    sync.barrier(1);  // B_1
    for (int64_t j = 0; j < nchunks; ++j) {
        sync.barrier(j + 2);  // B_{j+2}
        const int64_t rem = tok_rows - 16 * j;
        const int len = rem >= 16 ? 16 : (int)rem;  // >= 1
        const char *st = stage0 + (int)(j & 1) * kStageBytes;
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 a = *reinterpret_cast<const u32x4 *>(st + r * kStageRow + 16 * p);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(st + (r + 8) * kStageRow + 16 * p);
        const __amdgpu_buffer_rsrc_t ro = rsrc(o0 + (size_t)j * chunk_rows, tile_bytes<NW>(len, vrow));
        __builtin_amdgcn_raw_buffer_store_b128(a, ro, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(b, ro, off + 8 * vrow, 0, 0);
    }
}

// The store wave of the staged two-wave form with SAVE: chunk j's start state (the
// workgroup's 8 KiB of fragments, in HBM order) leaves staging buffer j % 2 after
// B_{j+1}, by which the compute waves have written it, and before B_{j+2}, after which
// they write the buffer again. `block0`: the workgroup's first fragment of the
// sequence's first chunk; chunk j's is `sstride` bytes further per chunk. It passes
// the same nchunks + 1 barriers as the other waves.
template <int DEPTH, int NW, class Sync>
__device__ __forceinline__ void save_store_wave(char *ring, int64_t nchunks, char *block0, size_t sstride,
                                                int lane, Sync &sync) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int kFrags = kSaveStageBytes / 1024;
    const char *stage0 = ring + DEPTH * slot_bytes<NW>() + xchg_bytes<NW>() + lane * 16;
    sync.barrier(0);  // B_0
    for (int64_t j = 0; j < nchunks; ++j) {
        sync.barrier(j + 1);  // B_{j+1}
        const char *st = stage0 + (int)(j & 1) * kSaveStageBytes;
        char *dst = block0 + (size_t)j * sstride + lane * 16;
        u32x4 f[kFrags];
#pragma unroll
        for (int k = 0; k < kFrags; ++k) f[k] = *reinterpret_cast<const u32x4 *>(st + k * 1024);
#pragma unroll
        for (int k = 0; k < kFrags; ++k) __builtin_nontemporal_store(f[k], reinterpret_cast<u32x4 *>(dst + k * 1024));
    }
}

// The hardware workgroup barrier: every wave of the workgroup takes part.
struct HwSync {
    __device__ __forceinline__ void barrier(int64_t) { kda::barrier(); }
};

}  // namespace
}  // namespace kda
