// kda_internal.h -- host-side geometry and kernel launchers of libkda (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

constexpr int kChunk = 16;
constexpr int kMaxSeqs = 1 << 20;  // packed sequences per call

// bf16 K = V = 128 record of one (chunk, head), written by the intra-chunk kernel and
// read by the inter-chunk kernel. Keys follow chan_of / key_of (kda_device.h). Byte offsets:
//   W    0      [4 slabs][64 lanes][8 bf16]  W = T' K+ in 16x16x32 A-operand layout: slab s,
//                                            lane (c, grp), element u = token c, key 32s + 8grp + u
//   QT   4096   [4 slabs][64 lanes][8 bf16]  Q~ = Q+ - M K+, same layout
//   KD   8192   [4 pairs][64 lanes][8 bf16]  K^d, A-operand layout of K^d^T tiles: pair mp,
//                                            lane (c, grp) = keys key_of(2mp, c), key_of(2mp + 1, c),
//                                            tokens 4grp .. + 3
//   TB   12288  [64 lanes][4 hi, 4 lo bf16]  T' = T diag(beta), 16x16x16 A-operand layout
//   MM   13312  [64 lanes][4 hi, 4 lo bf16]  M = P T', same layout
//   GAM  14336  [4 groups][32 fp32]          gamma = exp(G_C): group grp, entry 4m + i is the
//                                            key of accumulator tile m, row 4grp + i
constexpr int kRecW = 0;
constexpr int kRecQT = 4096;
constexpr int kRecKD = 8192;
constexpr int kRecTB = 12288;
constexpr int kRecMM = 13312;
constexpr int kRecGAM = 14336;
constexpr int kRecBytesBf16 = 14848;

// bf16 backward record of one (chunk, head), written by the intra-chunk kernel next to
// the forward record when a backward pass needs it, and read by the reverse
// state-gradient kernel. The reverse pass multiplies by K^d where the forward
// multiplies by W and by W^T, Q~^T where the forward multiplies by K^d^T, so the
// same factors are stored in the other operand layouts:
//   KD   0      [4 slabs][64 lanes][8 bf16]  K^d in the layout of W above
//   WT   4096   [4 pairs][64 lanes][8 bf16]  W in the layout of KD above
//   QT   8192   [4 pairs][64 lanes][8 bf16]  Q~ in the layout of KD above
//   GAM  12288  as GAM above
constexpr int kBRecKD = 0;
constexpr int kBRecWT = 4096;
constexpr int kBRecQT = 8192;
constexpr int kBRecGAM = 12288;
constexpr int kBRecBytes = 12800;

// A 128 x 128 state (or state gradient) of one (chunk, head) in bf16, as 32 MFMA
// fragments of 1 KiB: fragment (ct, ks) at byte ((ct * 4 + ks) * 64 + lane) * 16 holds,
// in lane (c, grp) = (lane % 16, lane / 16), value column 16 ct + c and keys
// 32 ks + 8 grp + e (elements e = 0..7; rows 4grp + i of accumulator tiles 2ks and
// 2ks + 1): the B operand of W S in the recurrent kernel, as that kernel holds it.
constexpr int kStateBytesBf16 = 32768;

// fp32 record for head dimension K: W, QT, KD [16][K]; TB, MM [16][16]; GAM [K] (all fp32).
constexpr size_t rec_bytes_f32(int K) { return 4u * (3u * 16u * (size_t)K + 2u * 256u + (size_t)K); }

struct Geometry {
    int64_t T;
    int H, K, V, N, io;
    bool scalar_gate;        // g is [T, H] (one decay per token and head) instead of [T, H, K]
    int64_t max_chunks;      // upper bound on chunks over all sequences
    size_t off_chunk_off;    // int32 [N + 1]
    size_t off_chunk_seq;    // int32 [max_chunks]
    size_t off_records;      // records [max_chunks][H] (chunk-major: a chunk's heads are contiguous)
    size_t record_bytes;
    size_t total_bytes;
    // backward only (make_backward_geometry): backward records, chunk start states
    // and chunk end-state gradients, each [max_chunks][H] like the records
    size_t off_brecords;
    size_t off_states;
    size_t off_dstates;
    size_t backward_bytes;
};

// The current device's compute units and XCDs, read from the runtime once per device.
struct DeviceShape {
    int cus;   // compute units
    int xccs;  // XCDs (accelerator complex dies); workgroups are dealt to them round robin
};
hipError_t device_shape(DeviceShape *shape);
// Raises kernel `fn`'s dynamic LDS limit to `bytes` on the current device, once per
// (kernel, device); later calls return at once.
hipError_t set_dynamic_lds(const void *fn, int bytes);
// Units (e.g. (sequence, head) pairs) rounded up to a whole number per XCD.
inline int round_to_xccs(int units, int xccs) { return (units + xccs - 1) / xccs * xccs; }

// Fills g from d; returns KDA_OK or a negative status (no device access).
int make_geometry(const kda_dims_t *d, Geometry *g);
// make_geometry plus the backward pass's workspace areas (bf16 io only).
int make_backward_geometry(const kda_dims_t *d, Geometry *g);

hipError_t launch_check_seqlens(const int32_t *cu_seqlens, int num_seqs, int64_t total_tokens, int32_t *result,
                                hipStream_t stream);
hipError_t launch_chunk_table(const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                              hipStream_t stream);
hipError_t launch_intra_bf16(const void *q, const void *k, const float *g, const float *beta,
                             const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                             hipStream_t stream);
hipError_t launch_inter_bf16(const void *v, const int32_t *cu_seqlens, const float *s0, void *out,
                             float *sT, const Geometry &geo, const void *ws, hipStream_t stream);
// Backward pass: records for both directions, the forward recomputed for the chunk
// start states, the reverse state-gradient pass and the token-parallel gradients.
hipError_t launch_intra_bf16_bwd(const void *q, const void *k, const float *g, const float *beta,
                                 const int32_t *cu_seqlens, const Geometry &geo, void *ws, hipStream_t stream);
hipError_t launch_inter_bf16_states(const void *v, const int32_t *cu_seqlens, const float *s0,
                                    const Geometry &geo, void *ws, hipStream_t stream);
// The forward with its output and final state that also saves every chunk's start
// state for the backward (the states and the output of one recurrent pass).
hipError_t launch_inter_bf16_states_out(const void *v, const int32_t *cu_seqlens, const float *s0, void *out,
                                        float *sT, const Geometry &geo, void *ws, hipStream_t stream);
hipError_t launch_state_grad_bf16(const void *d_out, const int32_t *cu_seqlens, const float *dsT, float *ds0,
                                  const Geometry &geo, void *ws, hipStream_t stream);
hipError_t launch_grad_bf16(const void *q, const void *k, const void *v, const float *g, const float *beta,
                            const void *d_out, const int32_t *cu_seqlens, void *dq, void *dk, void *dv, float *dg,
                            float *dbeta, const Geometry &geo, const void *ws, hipStream_t stream);
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
