// kda_inter_bf16.hip -- recurrent inter-chunk kernel, bf16 io, K = V = 128.
//
// Carries each (sequence, head) state S (128 x 128 fp32) from chunk to chunk: the
// low-parallelism half of the two-kernel split (augursoft.site
// "Kimi K3 的三個系統設計", section "為什麼 FlashKDA 選擇 16-token chunks"). The
// state's value columns are independent (column j of S and of the output depends
// only on column j of v and of the initial state), so a workgroup owns 16 NW columns
// of one head as NW 16-column tiles, and shares one copy of each chunk's operands
// between them. NW = 2 while each 2-tile workgroup can have a CU of its own, else 4.
// Each tile's 128 x 16 slice of S lives in MFMA accumulator registers for the whole
// sequence: in the prefill, in one compute wave per tile (compute_role_full); in the
// training forward, which also saves every chunk's start state, split by rows over two
// waves that swap partial products through LDS (compute_role). Both forms give bitwise
// equal results (kda_chain.h).
//
// Per chunk, with S the state at the chunk start and V the chunk's value tile
// (T', M, W, Q~, K^d and gamma from the intra-chunk kernel):
//   U     = T' V                      (two-term bf16 split of T'; V is exact)
//   Delta = U - W S                   (S rounded to bf16 as the MFMA operand)
//   O     = Q~ S + M V                -> out (bf16)
//   S     = Diag(gamma) S + K^d^T Delta   (two-term bf16 split of Delta)
// The accumulator layout of S (lane: rows 4grp + i of column c, row r of tile m being key
// key_of(m, r)) is, after rounding
// to bf16, directly the B operand of W S and Q~ S, because the intra-chunk kernel
// stores W and Q~ with matching channel order; Delta's accumulator layout is the B
// operand of K^d^T Delta. Across lanes, only gamma moves (DPP broadcasts inside
// 16-lane rows); across waves, nothing in the one-wave form, and the partial W S and
// Q~ S (through LDS) in the two-wave form.
//
// Memory pipeline: a chunk step takes a few hundred cycles while an HBM load takes
// on the order of a microsecond, so each workgroup keeps a ring of DEPTH chunk
// slots in LDS that two producer waves fill with direct buffer->LDS loads
// (buffer_load_dwordx4 ... lds) several chunks ahead; the loads hold no registers.
// A producer waits (s_waitcnt vmcnt) for its own part of a chunk, then one
// s_barrier per chunk publishes the slot to the compute waves (and, in the two-wave
// form, the previous chunk's partial products between the two halves of a tile).
// The same barrier hands a store wave what the compute waves staged in LDS: the
// output tiles of the 4-tile forms and the saved chunk states of the 2-tile training
// forward, which the chain's own stores would otherwise slow down (kda_chain.h).
#include "kda_chain.h"
#include "kda_intra_wave.h"

namespace kda {
namespace {

// SAVE: every chunk's start state goes to `states` ([max_chunks][H] x 32 KiB
// fragments), for a backward pass. OUT: the output is written (a recomputed forward
// that only saves states writes neither output nor final state). FULL: one compute
// wave per tile (compute_role_full) instead of two (compute_role); the prefill's form.
template <int NW, bool FULL>
constexpr int inter_compute_waves() { return FULL ? NW : compute_waves<NW>(); }
// a store wave when outputs (staged_out) or saved states (staged_save) go through LDS
template <int NW, bool FULL, bool SAVE, bool OUT>
constexpr int inter_waves() {
    return inter_compute_waves<NW, FULL>() + kProducers +
           ((staged_out<NW, OUT>() || staged_save<NW, SAVE, OUT>()) ? 1 : 0);
}
template <int NW, bool FULL>
constexpr int inter_xchg_bytes() { return FULL ? 0 : xchg_bytes<NW>(); }

template <int DEPTH, bool SAVE, bool OUT, int NW, bool FULL>
__global__ __launch_bounds__((64 * inter_waves<NW, FULL, SAVE, OUT>())) void kda_inter_bf16_kernel(
    const unsigned short *__restrict__ v, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const float *__restrict__ s0, unsigned short *__restrict__ out,
    float *__restrict__ sT, int64_t T, int H, int N, int64_t max_chunks,
    const char *__restrict__ records, char *__restrict__ states, int xccs) {
    static_assert(NW == 2 || NW == 4, "two or four value tiles per workgroup");
    static_assert(!(FULL && SAVE), "the whole-tile form does not save chunk states");
    static_assert(DEPTH >= 3, "a slot is refilled two chunks after it was read");
    static_assert((DEPTH - 1) * per_wave1<NW>() < 64, "a producer's loads in flight must fit the 6-bit counter");
    extern __shared__ __attribute__((aligned(1024))) char ring[];
    int pair, vg;
    xcd_unit_split(blockIdx.x, kTiles / NW, xccs, pair, vg);
    if (pair >= N * H) return;  // whole workgroup
    const int n = pair / H, h = pair % H;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int col0 = vg * NW * 16;  // first value column of the workgroup
    const SeqChunks sc = seq_chunks(cu, chunk_off, n, T, max_chunks);
    const int64_t nchunks = sc.chunk_end - sc.chunk_begin;

    LaneOffsets lo;
    lo.vrow = (unsigned int)H * VD * 2;
    lo.rec = lane * 16;
    lo.gam = (lane & 31) * 16;
    // a value tile row is 2 NW 16-byte pieces; one wave-wide load covers 32 / NW rows
    lo.v = (lane / (2 * NW)) * lo.vrow + (lane % (2 * NW)) * 16;
    lo.v2 = lo.v + 8 * lo.vrow;
    const size_t tok_bytes = ((size_t)sc.tok_begin * H + h) * VD * 2 + (size_t)col0 * 2;
    const size_t chunk_rows = (size_t)16 * lo.vrow;  // bytes of 16 token rows

    if constexpr (staged_save<NW, SAVE, OUT>()) {
        if (wid == inter_waves<NW, FULL, SAVE, OUT>() - 1) {
            // ---- saved-state store wave ----
            HwSync ssync;
            char *block0 = states + ((size_t)sc.chunk_begin * H + h) * kStateBytesBf16 + (size_t)(col0 >> 4) * 4096;
            save_store_wave<DEPTH, NW>(ring, nchunks, block0, (size_t)H * kStateBytesBf16, lane, ssync);
            return;
        }
    }
    if constexpr (staged_out<NW, OUT>()) {
        if (wid == inter_waves<NW, FULL, SAVE, OUT>() - 1) {
            // ---- output store wave ----
            HwSync ssync;
            store_wave<NW>(ring + DEPTH * slot_bytes<NW>() + inter_xchg_bytes<NW, FULL>(), nchunks,
                           sc.tok_end - sc.tok_begin, reinterpret_cast<char *>(out) + tok_bytes, chunk_rows, lane,
                           lo.vrow, ssync);
            return;
        }
    }
    if (wid >= inter_compute_waves<NW, FULL>()) {
        // ---- producer ----
        const int p = wid - inter_compute_waves<NW, FULL>();
        // records are chunk-major: a chunk's records for all heads are contiguous, so the
        // workgroups in flight, which move through the chunks at about the same pace, read
        // one region of HBM (and K1's workgroups in flight write one)
        const char *rec0 = records + ((size_t)sc.chunk_begin * H + h) * kRecBytesBf16;
        const size_t rec_stride = (size_t)H * kRecBytesBf16;
        const char *v0 = reinterpret_cast<const char *>(v) + tok_bytes;
        auto len_of = [&](int64_t j) {
            const int64_t rem = sc.tok_end - (sc.tok_begin + 16 * j);
            return rem <= 0 ? 0 : (rem >= 16 ? 16 : (int)rem);
        };
        auto issue = [&](int64_t j) {
            const unsigned int slot =
                (unsigned int)__builtin_amdgcn_readfirstlane((int)(j % DEPTH) * slot_bytes<NW>());
            issue_chunk<NW>(ring, slot, rec0 + (size_t)j * rec_stride, v0 + (size_t)j * chunk_rows, len_of(j), p,
                            lo);
        };
        for (int64_t j = 0; j < DEPTH - 1 && j < nchunks; ++j) issue(j);
        for (int64_t j = 0; j < nchunks; ++j) {
            // chunks issued so far: 0 .. last
            const int64_t lim = j == 0 ? DEPTH - 2 : j + DEPTH - 3;
            const int64_t last = lim < nchunks - 1 ? lim : nchunks - 1;
            asm volatile("" ::: "memory");
            if (p == 0)
                wait_for_chunk<kPerWave0, DEPTH>((int)(last - j));
            else
                wait_for_chunk<per_wave1<NW>(), DEPTH>((int)(last - j));
            barrier();  // B_j
            // The slot of chunk j - 2 is free: compute waves read it after B_{j-2}
            // and consumed what they read before B_{j-1}.
            if (j >= 1 && j + DEPTH - 2 < nchunks) issue(j + DEPTH - 2);
        }
        barrier();  // B_nchunks
        if (staged_out<NW, OUT>()) barrier();  // B_{nchunks+1}, for the output store wave
        return;
    }

    HwSync sync;
    if (FULL) {
        compute_role_full<DEPTH, OUT, NW, staged_out<NW, OUT>()>(ring, wid, lane, pair, col0, sc, tok_bytes,
                                                                  chunk_rows, lo, s0, out, OUT ? sT : nullptr, sync);
        return;
    }
    // chunk start states, chunk-major like the records: chunk j of this pair is H states on
    char *st = SAVE ? states + ((size_t)sc.chunk_begin * H + h) * kStateBytesBf16 : nullptr;
    const size_t sstride = (size_t)H * kStateBytesBf16;
    compute_role<DEPTH, SAVE, OUT, NW, staged_save<NW, SAVE, OUT>(), staged_out<NW, OUT>()>(
        ring, wid, lane, pair, col0, sc, tok_bytes, chunk_rows, lo, s0, out, OUT ? sT : nullptr, sync, st, sstride);
}

template <int DEPTH, bool SAVE, bool OUT, int NW, bool FULL>
hipError_t launch(const void *v, const int32_t *cu_seqlens, const float *s0, void *out, float *sT,
                  const Geometry &geo, const void *ws, const DeviceShape &dev, hipStream_t stream) {
    const int64_t blocks = (int64_t)round_to_xccs(geo.N * geo.H, dev.xccs) * (kTiles / NW);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const char *base = static_cast<const char *>(ws);
    const int32_t *chunk_off = reinterpret_cast<const int32_t *>(base + geo.off_chunk_off);
    constexpr size_t lds = (size_t)DEPTH * slot_bytes<NW>() + inter_xchg_bytes<NW, FULL>() + stage_bytes<NW, OUT>() +
                           save_stage_bytes<NW, SAVE, OUT>();
    static_assert(lds <= 160 * 1024, "LDS of one CU");
    auto kern = kda_inter_bf16_kernel<DEPTH, SAVE, OUT, NW, FULL>;
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * inter_waves<NW, FULL, SAVE, OUT>()), lds, stream,
                       static_cast<const unsigned short *>(v), cu_seqlens, chunk_off, s0,
                       static_cast<unsigned short *>(out), sT, geo.T, geo.H, geo.N, geo.max_chunks,
                       base + geo.off_records, SAVE ? const_cast<char *>(base) + geo.off_states : nullptr,
                       dev.xccs);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Single-kernel ablation: the same recurrent workgroup, with the intra-chunk work
// done inside it. The pages report that FlashKDA's split into a token-parallel
// and a recurrent kernel beat one fused kernel, in which the token-parallel work
// ran at the recurrence's low parallelism (augursoft.site "Kimi K3 的三個系統設計",
// section "為什麼 FlashKDA 選擇 16-token chunks"). Here the two producer waves are
// replaced by kIntraWaves waves that build each chunk's record (intra::chunk_record,
// the intra-chunk kernel's own per-wave code) straight into the LDS ring and load
// its value tile; nothing goes through HBM but q, k, v, g, beta, out and the states.
// Each column group of a head builds the head's records itself.
//
// Intra wave i builds chunks i, i + kIntraWaves, ...: chunk m right after passing
// B_{m - kIntraWaves} (chunks below kIntraWaves before B_0). Its slot last held chunk
// m - kFusedDepth, which the compute waves finished reading before they reached
// B_{m - kFusedDepth + 1} = B_{m - kIntraWaves}; they read chunk m after B_m. An
// intra wave busy with a chunk holds every barrier until it is done, so the intra
// waves work in step, kIntraWaves chunks at a time, alternating with the chain.
constexpr int kIntraWaves = 4;
constexpr int kFusedDepth = kIntraWaves + 1;
constexpr int kFusedWaves = kComputeWaves + kIntraWaves;
constexpr size_t kFusedLds = (size_t)kFusedDepth * kSlotBytes + kXchgBytes + kIntraWaves * sizeof(intra::IntraLds);
static_assert(kFusedLds <= 160 * 1024, "LDS of one CU");

template <bool SCALAR_GATE>
__global__ __launch_bounds__(64 * kFusedWaves) void kda_fused_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const unsigned short *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, const float *__restrict__ s0, unsigned short *__restrict__ out,
    float *__restrict__ sT, int64_t T, int H, int N, int64_t max_chunks, int xccs) {
    extern __shared__ __attribute__((aligned(1024))) char ring[];  // slots, exchange, intra scratch
    int pair, vg;
    xcd_unit_split(blockIdx.x, kTiles / kNW, xccs, pair, vg);
    if (pair >= N * H) return;  // whole workgroup
    const int n = pair / H, h = pair % H;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int col0 = vg * kNW * 16;
    const SeqChunks sc = seq_chunks(cu, chunk_off, n, T, max_chunks);
    const int64_t nchunks = sc.chunk_end - sc.chunk_begin;

    LaneOffsets lo;
    lo.vrow = (unsigned int)H * VD * 2;
    const size_t tok_bytes = ((size_t)sc.tok_begin * H + h) * VD * 2 + (size_t)col0 * 2;
    const size_t chunk_rows = (size_t)16 * lo.vrow;

    if (wid >= kComputeWaves) {
        // ---- intra wave ----
        const int i = wid - kComputeWaves;
        intra::IntraLds &L = *reinterpret_cast<intra::IntraLds *>(
            ring + kFusedDepth * kSlotBytes + kXchgBytes + i * sizeof(intra::IntraLds));
        const char *v0 = reinterpret_cast<const char *>(v) + tok_bytes;
        auto produce = [&](int64_t m) {
            const int64_t start = sc.tok_begin + 16 * m;
            const int64_t rem = sc.tok_end - start;
            const int len = rem >= 16 ? 16 : (int)rem;
            char *slot = ring + (unsigned int)__builtin_amdgcn_readfirstlane((int)(m % kFusedDepth) * kSlotBytes);
            intra::chunk_record<SCALAR_GATE>(q, k, g, beta, start, len, h, H, true, L, slot, lane);
            // value tile [16 tokens][32 columns] bf16, lane: token lane / 4, 8 columns;
            // rows past the end of the chunk are zero
            const int row = lane >> 2;
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (row < len)
                val = *reinterpret_cast<const uint4 *>(v0 + (size_t)m * chunk_rows + (size_t)row * lo.vrow +
                                                       (lane & 3) * 16);
            *reinterpret_cast<uint4 *>(slot + kVOff + lane * 16) = val;
            wait_lgkm0();  // the slot is complete in LDS before this wave's next barrier
        };
        if (i < nchunks) produce(i);
        for (int64_t b = 0; b <= nchunks; ++b) {
            barrier();  // B_b
            if (b % kIntraWaves == i && b + kIntraWaves < nchunks) produce(b + kIntraWaves);
        }
        return;
    }
    HwSync sync;
    compute_role<kFusedDepth, false, true, kNW, false, false>(ring, wid, lane, pair, col0, sc, tok_bytes, chunk_rows, lo, s0, out, sT,
                                                sync);
}

}  // namespace

namespace {

// One workgroup per 16 NW value columns of a (sequence, head). While 2-tile
// workgroups fit one per CU: 2 tiles with an 8-chunk ring (128 KiB, plus a 12 KiB
// exchange in the two-wave form). Beyond that: 4 tiles sharing one record stream, one
// workgroup per CU at a time: in the one-wave form, four compute waves (one per SIMD)
// and an 8-chunk ring (136 KiB); in the two-wave form, eight compute waves (two per
// SIMD), a 7-chunk ring (119 KiB) and a 24 KiB exchange. Two 2-tile workgroups per CU
// (4-chunk rings) were slower: each streams its own copy of the records.
template <bool SAVE, bool OUT>
hipError_t launch_by_size(const void *v, const int32_t *cu_seqlens, const float *s0, void *out, float *sT,
                          const Geometry &geo, const void *ws, hipStream_t stream) {
    DeviceShape dev;
    const hipError_t e = device_shape(&dev);
    if (e != hipSuccess) return e;
    constexpr bool FULL = OUT && !SAVE;
    if ((int64_t)round_to_xccs(geo.N * geo.H, dev.xccs) * (kTiles / 2) <= dev.cus)
        return launch<8, SAVE, OUT, 2, FULL>(v, cu_seqlens, s0, out, sT, geo, ws, dev, stream);
    return launch<FULL ? 8 : 7, SAVE, OUT, 4, FULL>(v, cu_seqlens, s0, out, sT, geo, ws, dev, stream);
}

}  // namespace

hipError_t launch_inter_bf16(const void *v, const int32_t *cu_seqlens, const float *s0, void *out,
                             float *sT, const Geometry &geo, const void *ws, hipStream_t stream) {
    return launch_by_size<false, true>(v, cu_seqlens, s0, out, sT, geo, ws, stream);
}

hipError_t launch_inter_bf16_states(const void *v, const int32_t *cu_seqlens, const float *s0,
                                    const Geometry &geo, void *ws, hipStream_t stream) {
    return launch_by_size<true, false>(v, cu_seqlens, s0, nullptr, nullptr, geo, ws, stream);
}

hipError_t launch_inter_bf16_states_out(const void *v, const int32_t *cu_seqlens, const float *s0, void *out,
                                        float *sT, const Geometry &geo, void *ws, hipStream_t stream) {
    return launch_by_size<true, true>(v, cu_seqlens, s0, out, sT, geo, ws, stream);
}

}  // namespace kda

namespace kda {

hipError_t launch_fused_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                             const int32_t *cu_seqlens, const float *s0, void *out, float *sT,
                             const Geometry &geo, const void *ws, hipStream_t stream) {
    DeviceShape dev;
    hipError_t e = device_shape(&dev);
    if (e != hipSuccess) return e;
    const int64_t blocks = (int64_t)round_to_xccs(geo.N * geo.H, dev.xccs) * (kTiles / kNW);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const char *base = static_cast<const char *>(ws);
    const int32_t *chunk_off = reinterpret_cast<const int32_t *>(base + geo.off_chunk_off);
    auto kern = geo.scalar_gate ? kda_fused_bf16_kernel<true> : kda_fused_bf16_kernel<false>;
    e = set_dynamic_lds(reinterpret_cast<const void *>(kern), (int)kFusedLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kFusedWaves), kFusedLds, stream,
                       static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k),
                       static_cast<const unsigned short *>(v), g, beta, cu_seqlens, chunk_off, s0,
                       static_cast<unsigned short *>(out), sT, geo.T, geo.H, geo.N, geo.max_chunks, dev.xccs);
    return hipGetLastError();
}

}  // namespace kda
