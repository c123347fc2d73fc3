// kda_noalloc.hip -- kda_chunk_prefill for callers that cannot allocate device memory
// (code under stream capture, serving loops, harnesses that forbid it): the same
// kernels, with their workspace in a fixed array this library holds on every device
// it runs on, instead of a caller-provided buffer.
//
// The array `scratch` below is a device symbol. In host code its name is only a
// host-side stand-in, so every use goes through the device address obtained once
// per device with hipGetSymbolAddress (kept in g_scratch).
//
// What runs: a problem whose workspace fits runs as one kda_chunk_prefill. A single
// sequence that does not fit runs in segments of whole chunks, each one
// kda_intra_chunk + kda_inter_chunk over the segment's tokens. The fp32 state passes
// from one segment to the next through two carrier areas at the end of the array
// (alternating, so no launch reads and writes the same one). Results are bitwise
// those of kda_chunk_prefill: the records are per chunk, and the carried state is
// the fp32 state the recurrent kernel holds. Packed batches (num_seqs > 1) must fit
// whole.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace kda {

static_assert(KDA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device (nullptr: not looked up yet)

// The current device's address of `scratch`: looked up on the device's first call.
int scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return KDA_ERR_LAUNCH;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KDA_OK;
}

size_t align_down(size_t x) { return x / 256 * 256; }

}  // namespace
}  // namespace kda

extern "C" int kda_chunk_prefill_noalloc(const void *q, const void *k, const void *v, const float *g,
                                         const float *beta, const int32_t *cu_seqlens, const float *initial_state,
                                         void *out, float *final_state, const kda_dims_t *dims, void *stream) {
    kda::Geometry geo;
    int st = kda::make_geometry(dims, &geo);
    if (st != KDA_OK) return st;
    // the argument checks of kda_chunk_prefill, before the device is touched
    if (cu_seqlens == nullptr && dims->num_seqs != 1) return KDA_ERR_ARG;
    if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_ALIGN;
    if (geo.T > 0) {
        for (const void *p : {q, k, v, static_cast<const void *>(g), static_cast<const void *>(beta),
                              static_cast<const void *>(out)}) {
            if (p == nullptr) return KDA_ERR_ARG;
        }
    }
    for (const void *p : {q, k, v, static_cast<const void *>(g), static_cast<const void *>(beta),
                          static_cast<const void *>(out), static_cast<const void *>(initial_state),
                          static_cast<const void *>(final_state)}) {
        if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return KDA_ERR_ALIGN;
    }
    void *ws = nullptr;
    constexpr size_t cap = KDA_NOALLOC_SCRATCH_BYTES;
    if (geo.total_bytes <= cap) {
        st = kda::scratch_address(&ws);
        if (st != KDA_OK) return st;
        return kda_chunk_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, dims, ws, cap,
                                 stream);
    }
    if (dims->num_seqs != 1) return KDA_ERR_CAPACITY;

    // One sequence in segments: the two state carriers at the end of the array, the
    // segment workspace (chunk table and records) before them.
    const size_t state_bytes = (size_t)geo.H * geo.K * geo.V * sizeof(float);
    const size_t carrier = (state_bytes + 255) / 256 * 256;
    if (2 * carrier >= cap) return KDA_ERR_CAPACITY;
    const size_t seg_ws = kda::align_down(cap - 2 * carrier);
    // chunks per segment: the largest count whose workspace fits seg_ws
    int64_t seg_chunks = (int64_t)(seg_ws / ((size_t)geo.H * geo.record_bytes));
    kda_dims_t sd = *dims;
    for (; seg_chunks > 0; --seg_chunks) {
        sd.total_tokens = 16 * seg_chunks;
        if (kda_workspace_bytes(&sd) <= seg_ws) break;
    }
    if (seg_chunks < 1) return KDA_ERR_CAPACITY;
    st = kda::scratch_address(&ws);
    if (st != KDA_OK) return st;
    char *base = static_cast<char *>(ws);
    float *carriers[2] = {reinterpret_cast<float *>(base + cap - 2 * carrier),
                          reinterpret_cast<float *>(base + cap - carrier)};

    // Byte strides of one token row. The segments start at multiples of 16 tokens, so
    // every offset pointer keeps the 16-byte alignment of its base.
    const size_t es = geo.io == KDA_IO_BF16 ? 2 : 4;
    const size_t qk_row = (size_t)geo.H * geo.K * es, v_row = (size_t)geo.H * geo.V * es;
    const size_t g_row = (size_t)geo.H * (geo.scalar_gate ? 1 : geo.K) * sizeof(float);
    const size_t b_row = (size_t)geo.H * sizeof(float);
    const int64_t seg_tokens = 16 * seg_chunks;
    int s = 0;
    for (int64_t t0 = 0; t0 < geo.T; t0 += seg_tokens, ++s) {
        const int64_t n = geo.T - t0 < seg_tokens ? geo.T - t0 : seg_tokens;
        const bool last = t0 + n >= geo.T;
        sd.total_tokens = n;
        const float *s0 = s == 0 ? initial_state : carriers[(s - 1) & 1];
        float *sT = last ? final_state : carriers[s & 1];
        const char *qb = static_cast<const char *>(q) + t0 * qk_row;
        const char *kb = static_cast<const char *>(k) + t0 * qk_row;
        const char *vb = static_cast<const char *>(v) + t0 * v_row;
        char *ob = static_cast<char *>(out) + t0 * v_row;
        const float *gb = reinterpret_cast<const float *>(reinterpret_cast<const char *>(g) + t0 * g_row);
        const float *bb = reinterpret_cast<const float *>(reinterpret_cast<const char *>(beta) + t0 * b_row);
        // one sequence: its boundaries are [0, T) by the contract, so the segments
        // need no table
        st = kda_intra_chunk(qb, kb, gb, bb, nullptr, &sd, ws, seg_ws, stream);
        if (st != KDA_OK) return st;
        st = kda_inter_chunk(vb, nullptr, s0, ob, sT, &sd, ws, seg_ws, stream);
        if (st != KDA_OK) return st;
    }
    return KDA_OK;
}
