// kda_intra_bf16.hip -- token-parallel intra-chunk kernel, bf16 io, K = V = 128.
//
// One wave per (chunk, head); a workgroup holds the 4 heads h..h+3 of one chunk.
// The pages describe this half of FlashKDA as the work with token-level
// parallelism, split from the recurrent propagation (augursoft.site
// "Kimi K3 的三個系統設計", section "為什麼 FlashKDA 選擇 16-token chunks").
// The per-wave work is intra::chunk_record (kda_intra_wave.h); this kernel maps
// workgroups to chunks and heads and writes each record to the workspace.
#include "kda_chunks.h"
#include "kda_intra_wave.h"

namespace kda {
namespace {

constexpr int kWaves = 4;

// BWD: also each chunk's backward record, to `brecords` ([max_chunks][H] like the records).
template <bool SCALAR_GATE, bool BWD>
__global__ __launch_bounds__(64 * kWaves) void kda_intra_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off,
    const int32_t *__restrict__ chunk_seq, int64_t T, int H, int N, int64_t max_chunks,
    char *__restrict__ records, char *__restrict__ brecords) {
    __shared__ intra::IntraLds lds[kWaves];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int lane = threadIdx.x & 63;
    // Head groups vary fastest over the linear workgroup id, so the workgroups in
    // flight together read all heads of a contiguous token range (one sequential
    // stream per input tensor) instead of a narrow strided column of it.
    const int head_groups = (H + kWaves - 1) / kWaves;
    const int64_t chunk = blockIdx.x / head_groups;
    const int h_raw = (int)(blockIdx.x - chunk * head_groups) * kWaves + wave;
    const bool head_ok = h_raw < H;
    const int h = head_ok ? h_raw : H - 1;

    int64_t start;
    int len;
    chunk_span(cu, chunk_off, chunk_seq, chunk, T, N, max_chunks, start, len);
    if (len == 0) return;  // same chunk for the whole workgroup
    char *rec = records + ((size_t)chunk * H + h) * kRecBytesBf16;  // chunk-major
    char *brec = BWD ? brecords + ((size_t)chunk * H + h) * kBRecBytes : nullptr;  // chunk-major
    intra::chunk_record<SCALAR_GATE, BWD>(q, k, g, beta, start, len, h, H, head_ok, lds[wave], rec, lane, brec);
}

template <bool BWD>
hipError_t launch_intra(const void *q, const void *k, const float *g, const float *beta, const int32_t *cu_seqlens,
                        const Geometry &geo, void *ws, hipStream_t stream) {
    if (geo.max_chunks == 0) return hipSuccess;
    char *base = static_cast<char *>(ws);
    const int32_t *chunk_off = reinterpret_cast<const int32_t *>(base + geo.off_chunk_off);
    const int32_t *chunk_seq = reinterpret_cast<const int32_t *>(base + geo.off_chunk_seq);
    const int64_t blocks = geo.max_chunks * ((geo.H + kWaves - 1) / kWaves);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    auto kern = geo.scalar_gate ? kda_intra_bf16_kernel<true, BWD> : kda_intra_bf16_kernel<false, BWD>;
    hipLaunchKernelGGL(kern, grid, dim3(64 * kWaves), 0, stream,
                       static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k), g, beta,
                       cu_seqlens, chunk_off, chunk_seq, geo.T, geo.H, geo.N, geo.max_chunks,
                       base + geo.off_records, BWD ? base + geo.off_brecords : nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_intra_bf16(const void *q, const void *k, const float *g, const float *beta,
                             const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                             hipStream_t stream) {
    return launch_intra<false>(q, k, g, beta, cu_seqlens, geo, ws, stream);
}

hipError_t launch_intra_bf16_bwd(const void *q, const void *k, const float *g, const float *beta,
                                 const int32_t *cu_seqlens, const Geometry &geo, void *ws, hipStream_t stream) {
    return launch_intra<true>(q, k, g, beta, cu_seqlens, geo, ws, stream);
}

}  // namespace kda
