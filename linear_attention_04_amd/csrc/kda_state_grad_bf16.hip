// kda_state_grad_bf16.hip -- reverse recurrent kernel of the backward pass, bf16 io,
// K = V = 128.
//
// Over one sequence, with R the gradient reaching a chunk's end state, each chunk
// (taken last to first) maps R to the gradient reaching its start state:
//     X = K^d R,   R <- Diag(gamma) R + Q~^T dO - W^T X,
// the transpose of the forward's state map S_C = Diag(gamma) S_0 + K^d^T (T' V - W S_0)
// plus the output's Q~ S_0 term (W, Q~, K^d, gamma as in the intra-chunk kernel). R
// at each chunk end is stored for the token-parallel gradient kernel (bf16 fragments,
// the layout the forward recomputation stores the start states in), and R after the
// first chunk is the initial state's gradient.
//
// The workgroup mirrors the forward recurrent kernel: 16 NW value columns of one
// (sequence, head) as NW 16-column tiles (NW = 2 while each 2-tile workgroup can have a
// CU of its own, else 4), each tile's 128 x 16 slice of R held in MFMA
// accumulators by two waves (64 key rows each), two producer waves streaming each
// chunk's backward record and d_out tile into an LDS ring with direct buffer->LDS
// loads, one barrier per chunk. X is a sum over all 128 keys, so the two halves of a
// tile swap their partial X through LDS at the barrier and both form the same sum.
#include "kda_chunks.h"
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_ring.h"

namespace kda {
namespace {

constexpr int KD = 128;
constexpr int VD = 128;
constexpr int kTiles = VD / 16;

// Ring slot: backward record bytes [0, 12288) as 12 wave-wide 1 KiB loads, gamma
// (512 B) loaded twice into [12288, 13312), the d_out tile [16 tokens][16 NW columns]
// bf16 at kDOff (NW / 2 loads). Producer 0 issues record pieces 0 .. 5 and gamma
// (kPerWave0 loads per chunk), producer 1 record pieces 6 .. 11 and the d_out tile
// (per_wave1<NW>()).
constexpr int kPerWave0 = 7;
template <int NW>
constexpr int per_wave1() { return 6 + NW / 2; }
constexpr int kGamOff = kBRecGAM;
constexpr int kDOff = kBRecGAM + 1024;
template <int NW>
constexpr int slot_bytes() { return NW == 2 ? 16384 : kDOff + 512 * NW; }
static_assert(kBRecGAM == 12288 && kBRecBytes == 12800 && kDOff + 1024 <= slot_bytes<2>(), "backward record layout");

constexpr int kHalves = 2;
constexpr int kProducers = 2;
template <int NW>
constexpr int compute_waves() { return NW * kHalves; }
template <int NW>
constexpr int waves() { return compute_waves<NW>() + kProducers; }

// Exchange area after the ring: [chunk parity][tile][half][64 lanes] f32x4, each half's
// partial X.
template <int NW>
constexpr int xchg_bytes() { return 2 * NW * kHalves * 1024; }

struct LaneOffsets {
    unsigned int rec;   // lane * 16
    unsigned int gam;   // (lane & 31) * 16
    unsigned int d;     // d_out tile load of this lane (a row is 2 NW 16-byte pieces)
    unsigned int d2;    // NW = 4: the second d_out tile load (token rows 8 .. 15)
    unsigned int vrow;  // one token row of d_out in bytes (H * VD * 2)
};

template <int NW>
__device__ __forceinline__ int tile_bytes(int len, unsigned int vrow) {
    return len > 0 ? (len - 1) * (int)vrow + NW * 32 : 0;
}

template <int NW>
__device__ __forceinline__ void issue_chunk(char *ring, unsigned int slot, const char *brec, const char *dchunk,
                                            int len, int producer, const LaneOffsets &lo) {
    const __amdgpu_buffer_rsrc_t rr = rsrc(brec, kBRecBytes);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        const int piece = 6 * producer + k;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(ring + slot + piece * 1024), 16, lo.rec,
                                                 piece * 1024, 0, 0);
    }
    if (producer == 0) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(ring + slot + kGamOff), 16, lo.gam, kBRecGAM, 0,
                                                 0);
    } else {
        const __amdgpu_buffer_rsrc_t rd = rsrc(dchunk, tile_bytes<NW>(len, lo.vrow));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void *)(ring + slot + kDOff), 16, lo.d, 0, 0, 0);
        if (NW == 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void *)(ring + slot + kDOff + 1024), 16, lo.d2, 0, 0,
                                                     0);
    }
}

// One chunk's operands for one half (rows 64 KH .. 64 KH + 63 of a tile).
struct HalfOps {
    bf16x8 kd[2];  // K^d slabs 2 KH, 2 KH + 1 (token c, keys chan_of(8s + u, grp))
    bf16x8 wt[4];  // W^T tiles 4 KH .. + 3, tokens 4grp .. + 3 twice (both halves of the reduction)
    s16x4 qt[4];   // Q~^T tiles 4 KH .. + 3, tokens 4grp .. + 3
    float2 gam;
    s16x4 dd;      // d_out: tokens 4grp .. + 3 of column c
};

template <int KH, int NW>
__device__ __forceinline__ void read_ops(HalfOps &o, const char *slot, int vt, int lane) {
    const int c = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s)
        o.kd[s] = *reinterpret_cast<const bf16x8 *>(slot + kBRecKD + ((2 * KH + s) * 64 + lane) * 16);
    // W^T: the same 8 bytes read twice from LDS (volatile LDS reads are not merged into
    // one) instead of duplicating registers
    typedef const volatile __attribute__((address_space(3))) unsigned long long lds_u64;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
        const int m = 4 * KH + mm;
        const int base = ((m >> 1) * 64 + lane) * 16 + (m & 1) * 8;
        lds_u64 *pw = (lds_u64 *)(slot + kBRecWT + base);
        const unsigned long long a = *pw;
        const unsigned long long b = *pw;
        o.wt[mm] = __builtin_bit_cast(bf16x8, make_uint4((unsigned)a, (unsigned)(a >> 32), (unsigned)b,
                                                         (unsigned)(b >> 32)));
        o.qt[mm] = *reinterpret_cast<const s16x4 *>(slot + kBRecQT + base);
    }
    o.gam = *reinterpret_cast<const float2 *>(slot + kGamOff + (grp * 32 + 2 * c) * 4);
    // rows past the end of a short chunk were loaded as zeros (range-checked loads)
    const unsigned short *d16 = reinterpret_cast<const unsigned short *>(slot + kDOff);
    s16x4 dd;
#pragma unroll
    for (int i = 0; i < 4; ++i) dd[i] = (short)d16[(4 * grp + i) * (NW * 16) + vt * 16 + c];
    o.dd = dd;
}

// Before the barrier: R (the gradient at the chunk end) to the store, this half's
// partial X = K^d R over its 64 keys to the partner, then Diag(gamma) R + Q~^T dO.
template <int KH>
__device__ __forceinline__ void chunk_part_a(const HalfOps &o, f32x4 (&R)[4], f32x4 &x, char *xchg, int lane,
                                             char *rdst) {
    bf16x8 rb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rb[s][i] = to_bf16(R[2 * s][i]);
            rb[s][4 + i] = to_bf16(R[2 * s + 1][i]);
        }
    }
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, rb[0]), reinterpret_cast<u32x4 *>(rdst));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, rb[1]), reinterpret_cast<u32x4 *>(rdst + 1024));
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    x = mfma_16x16x32(o.kd[0], rb[0], zero);
    x = mfma_16x16x32(o.kd[1], rb[1], x);
    *reinterpret_cast<f32x4 *>(xchg + KH * 1024 + lane * 16) = x;
    decay_tile<4 * KH + 0>(R[0], o.gam);
    decay_tile<4 * KH + 1>(R[1], o.gam);
    decay_tile<4 * KH + 2>(R[2], o.gam);
    decay_tile<4 * KH + 3>(R[3], o.gam);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) R[mm] = mfma_16x16x16(o.qt[mm], o.dd, R[mm]);
}

// After the barrier: X from both halves (half 0's part first on both, so they hold
// bitwise equal X), then R -= W^T X with X split into two bf16 terms.
template <int KH>
__device__ __forceinline__ void chunk_part_b(const HalfOps &o, f32x4 (&R)[4], const f32x4 &x, const f32x4 &px) {
    const f32x4 x0 = KH == 0 ? x : px;
    const f32x4 x1 = KH == 0 ? px : x;
    const f32x4 d = -(x0 + x1);
    unsigned int h01, h23, l01, l23;  // -X = hi + lo, packed pairs
    split_pair(d[0], d[1], h01, l01);
    split_pair(d[2], d[3], h23, l23);
    const bf16x8 db = __builtin_bit_cast(bf16x8, make_uint4(h01, h23, l01, l23));
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) R[mm] = mfma_16x16x32(o.wt[mm], db, R[mm]);
}

// The chunk loop of compute wave (vt, KH): barrier B_j (j = 0 .. nchunks) as in the
// forward recurrent kernel, with the chunks taken last to first (step j works on
// chunk nchunks - 1 - j). rdst0 points at this lane's fragment of the sequence's first
// chunk in the end-state gradient array, and consecutive chunks are rstride bytes apart.
template <int KH, int DEPTH, int NW>
__device__ __forceinline__ void compute_wave(f32x4 (&R)[4], char *ring, int64_t nchunks, int vt, int lane,
                                             char *rdst0, size_t rstride) {
    auto slot_of = [&](int64_t j) {
        return ring + (unsigned int)__builtin_amdgcn_readfirstlane((int)(j % DEPTH) * slot_bytes<NW>());
    };
    auto xchg_of = [&](int64_t j) {
        return ring + DEPTH * slot_bytes<NW>() + ((int)(j & 1) * NW + vt) * kHalves * 1024;
    };
    auto step = [&](int64_t j, const HalfOps &cur, HalfOps &next) {
        f32x4 x, px;
        char *xc = xchg_of(j);
        chunk_part_a<KH>(cur, R, x, xc, lane, rdst0 + (size_t)(nchunks - 1 - j) * rstride);
        wait_lgkm0();  // the partial X is in LDS before the barrier
        barrier();     // B_{j+1}
        px = *reinterpret_cast<const f32x4 *>(xc + (1 - KH) * 1024 + lane * 16);
        read_ops<KH, NW>(next, slot_of(j + 1), vt, lane);
        chunk_part_b<KH>(cur, R, x, px);
    };
    HalfOps opa, opb;
    barrier();  // B_0
    read_ops<KH, NW>(opa, slot_of(0), vt, lane);
    int64_t j = 0;
    for (; j + 2 <= nchunks; j += 2) {
        step(j, opa, opb);
        step(j + 1, opb, opa);
    }
    if (j < nchunks) step(j, opa, opb);
}

template <int DEPTH, int NW>
__global__ __launch_bounds__(64 * waves<NW>()) void kda_state_grad_bf16_kernel(
    const unsigned short *__restrict__ d_out, const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off,
    const float *__restrict__ dsT, float *__restrict__ ds0, int64_t T, int H, int N, int64_t max_chunks,
    const char *__restrict__ brecords, char *__restrict__ dstates, int xccs) {
    static_assert(NW == 2 || NW == 4, "two or four value tiles per workgroup");
    static_assert(DEPTH >= 3, "a slot is refilled two chunks after it was read");
    static_assert((DEPTH - 1) * per_wave1<NW>() < 64, "a producer's loads in flight must fit the 6-bit counter");
    extern __shared__ __attribute__((aligned(1024))) char ring[];
    int pair, vg;
    xcd_unit_split(blockIdx.x, kTiles / NW, xccs, pair, vg);
    if (pair >= N * H) return;  // whole workgroup
    const int n = pair / H, h = pair % H;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int col0 = vg * NW * 16;
    const SeqChunks sc = seq_chunks(cu, chunk_off, n, T, max_chunks);
    const int64_t nchunks = sc.chunk_end - sc.chunk_begin;
    // backward records and end-state gradients are chunk-major ([max_chunks][H]): this
    // pair's chunk c sits H entries after its chunk c - 1
    const size_t head_chunk0 = (size_t)sc.chunk_begin * H + h;  // index of chunk 0

    if (wid >= compute_waves<NW>()) {
        // ---- producer: chunk nchunks - 1 - j into slot j % DEPTH ----
        const int p = wid - compute_waves<NW>();
        LaneOffsets lo;
        lo.vrow = (unsigned int)H * VD * 2;
        lo.rec = lane * 16;
        lo.gam = (lane & 31) * 16;
        lo.d = (lane / (2 * NW)) * lo.vrow + (lane % (2 * NW)) * 16;
        lo.d2 = lo.d + 8 * lo.vrow;
        const char *rec0 = brecords + head_chunk0 * kBRecBytes;
        const char *d0 = reinterpret_cast<const char *>(d_out) + ((size_t)sc.tok_begin * H + h) * VD * 2 +
                         (size_t)col0 * 2;
        const size_t chunk_rows = (size_t)16 * lo.vrow;
        auto issue = [&](int64_t j) {
            const int64_t c = nchunks - 1 - j;
            const int64_t rem = sc.tok_end - (sc.tok_begin + 16 * c);
            const int len = rem <= 0 ? 0 : (rem >= 16 ? 16 : (int)rem);
            const unsigned int slot =
                (unsigned int)__builtin_amdgcn_readfirstlane((int)(j % DEPTH) * slot_bytes<NW>());
            issue_chunk<NW>(ring, slot, rec0 + (size_t)c * H * kBRecBytes, d0 + (size_t)c * chunk_rows, len, p, lo);
        };
        for (int64_t j = 0; j < DEPTH - 1 && j < nchunks; ++j) issue(j);
        for (int64_t j = 0; j < nchunks; ++j) {
            const int64_t lim = j == 0 ? DEPTH - 2 : j + DEPTH - 3;
            const int64_t last = lim < nchunks - 1 ? lim : nchunks - 1;
            asm volatile("" ::: "memory");
            if (p == 0)
                wait_for_chunk<kPerWave0, DEPTH>((int)(last - j));
            else
                wait_for_chunk<per_wave1<NW>(), DEPTH>((int)(last - j));
            barrier();  // B_j
            // the slot of step j - 2 is free (read after B_{j-2}, consumed before B_{j-1})
            if (j >= 1 && j + DEPTH - 2 < nchunks) issue(j + DEPTH - 2);
        }
        barrier();  // B_nchunks
        return;
    }

    // ---- compute wave (vt, kh): value columns col0 + 16 vt .. + 15, key rows 64 kh .. + 63 ----
    const int c = lane & 15, grp = lane >> 4;
    const int vt = wid >> 1, kh = wid & 1;
    f32x4 R[4];
    const size_t sbase = (size_t)pair * KD * VD + (size_t)(64 * kh) * VD + col0 + vt * 16 + c;
    if (dsT) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) R[m][i] = dsT[sbase + (size_t)key_of(m, 4 * grp + i) * VD];
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) R[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    wait_vmcnt<0>();  // settle the loads before the loop (stores share the counter)
    char *rdst0 = dstates + head_chunk0 * kStateBytesBf16 +
                  ((size_t)(((col0 >> 4) + vt) * 4 + 2 * kh) * 64 + lane) * 16;
    if (kh == 0)
        compute_wave<0, DEPTH, NW>(R, ring, nchunks, vt, lane, rdst0, (size_t)H * kStateBytesBf16);
    else
        compute_wave<1, DEPTH, NW>(R, ring, nchunks, vt, lane, rdst0, (size_t)H * kStateBytesBf16);
    if (ds0) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) ds0[sbase + (size_t)key_of(m, 4 * grp + i) * VD] = R[m][i];
    }
}

template <int DEPTH, int NW>
hipError_t launch(const void *d_out, const int32_t *cu_seqlens, const float *dsT, float *ds0, const Geometry &geo,
                  void *ws, const DeviceShape &dev, hipStream_t stream) {
    const int64_t blocks = (int64_t)round_to_xccs(geo.N * geo.H, dev.xccs) * (kTiles / NW);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    char *base = static_cast<char *>(ws);
    const int32_t *chunk_off = reinterpret_cast<const int32_t *>(base + geo.off_chunk_off);
    constexpr size_t lds = (size_t)DEPTH * slot_bytes<NW>() + xchg_bytes<NW>();
    static_assert(lds <= 160 * 1024, "LDS of one CU");
    auto kern = kda_state_grad_bf16_kernel<DEPTH, NW>;
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * waves<NW>()), lds, stream,
                       static_cast<const unsigned short *>(d_out),
                       cu_seqlens, chunk_off, dsT, ds0, geo.T, geo.H, geo.N, geo.max_chunks,
                       base + geo.off_brecords, base + geo.off_dstates, dev.xccs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_grad_bf16(const void *d_out, const int32_t *cu_seqlens, const float *dsT, float *ds0,
                                  const Geometry &geo, void *ws, hipStream_t stream) {
    // as the forward recurrent kernel: 2-tile workgroups while each can have a CU of
    // its own, else 4-tile ones sharing one record stream (8-deep rings: 128 KiB + 8 KiB,
    // 120 KiB + 16 KiB)
    DeviceShape dev;
    const hipError_t e = device_shape(&dev);
    if (e != hipSuccess) return e;
    if ((int64_t)round_to_xccs(geo.N * geo.H, dev.xccs) * (kTiles / 2) <= dev.cus)
        return launch<8, 2>(d_out, cu_seqlens, dsT, ds0, geo, ws, dev, stream);
    return launch<8, 4>(d_out, cu_seqlens, dsT, ds0, geo, ws, dev, stream);
}

}  // namespace kda
