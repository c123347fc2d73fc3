// kda_internal.h -- host-side geometry and kernel launchers of libkda (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

constexpr int kChunk = 16;

// bf16 K = V = 128 record of one (chunk, head), written by the intra-chunk kernel and
// read by the inter-chunk kernel. Byte offsets:
//   W    0      [4 slabs][64 lanes][8 bf16]  W = T' K+ in 16x16x32 A-operand layout
//   QT   4096   [4 slabs][64 lanes][8 bf16]  Q~ = Q+ - M K+, same layout
//   KD   8192   [4 pairs][64 lanes][8 bf16]  K^d, 16x16x16 A-operand layout of K^d^T tiles
//   TB   12288  [64 lanes][4 hi, 4 lo bf16]  T' = T diag(beta), 16x16x16 A-operand layout
//   MM   13312  [64 lanes][4 hi, 4 lo bf16]  M = P T', same layout
//   GAM  14336  [4 groups][32 fp32]          gamma = exp(G_C), permuted per lane group
constexpr int kRecW = 0;
constexpr int kRecQT = 4096;
constexpr int kRecKD = 8192;
constexpr int kRecTB = 12288;
constexpr int kRecMM = 13312;
constexpr int kRecGAM = 14336;
constexpr int kRecBytesBf16 = 14848;

// fp32 record for head dimension K: W, QT, KD [16][K]; TB, MM [16][16]; GAM [K] (all fp32).
constexpr size_t rec_bytes_f32(int K) { return 4u * (3u * 16u * (size_t)K + 2u * 256u + (size_t)K); }

struct Geometry {
    int64_t T;
    int H, K, V, N, io;
    bool scalar_gate;        // g is [T, H] (one decay per token and head) instead of [T, H, K]
    int64_t max_chunks;      // upper bound on chunks over all sequences
    size_t off_chunk_off;    // int32 [N + 1]
    size_t off_chunk_seq;    // int32 [max_chunks]
    size_t off_records;      // records [H][max_chunks] (head-major: a head's chunks are contiguous)
    size_t record_bytes;
    size_t total_bytes;
};

// Fills g from d; returns KDA_OK or a negative status (no device access).
int make_geometry(const kda_dims_t *d, Geometry *g);

hipError_t launch_chunk_table(const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                              hipStream_t stream);
hipError_t launch_intra_bf16(const void *q, const void *k, const float *g, const float *beta,
                             const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                             hipStream_t stream);
hipError_t launch_inter_bf16(const void *v, const int32_t *cu_seqlens, const float *s0, void *out,
                             float *sT, const Geometry &geo, const void *ws, hipStream_t stream);
hipError_t launch_fused_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                             const int32_t *cu_seqlens, const float *s0, void *out, float *sT,
                             const Geometry &geo, const void *ws, hipStream_t stream);
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         float *state, void *out, int64_t B, int H, int io, bool scalar_gate, hipStream_t stream);
hipError_t launch_intra_f32(const float *q, const float *k, const float *g, const float *beta,
                            const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                            hipStream_t stream);
hipError_t launch_inter_f32(const float *v, const int32_t *cu_seqlens, const float *s0, float *out,
                            float *sT, const Geometry &geo, const void *ws, hipStream_t stream);

// Token range of chunk `c` of a packed batch, resolved on the device from the table.
struct ChunkSpan {
    int64_t start;
    int len;
};

}  // namespace kda
