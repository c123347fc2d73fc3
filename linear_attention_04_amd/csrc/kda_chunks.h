// kda_chunks.h -- device-side view of the chunk decomposition of a (packed) batch.
//
// Chunks are 16 tokens long and aligned to the start of their own sequence, so a
// chunk never straddles two sequences; the last chunk of a sequence may be short.
// With cu_seqlens == NULL there is one sequence and chunk c covers tokens
// [16c, min(16c + 16, T)). Otherwise the chunk table built by kda_chunk_table gives,
// per sequence n, its first chunk chunk_off[n] (chunk_off[N] = number of chunks)
// and, per chunk, its sequence chunk_seq[c] (-1 for unused slots).
// Every value read from the device-resident table or cu_seqlens is clamped so that
// malformed boundaries can give wrong results but never out-of-range accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct SeqChunks {
    int64_t tok_begin;   // first token of the sequence
    int64_t tok_end;     // one past its last token
    int64_t chunk_begin; // first chunk index
    int64_t chunk_end;   // one past its last chunk
};

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

__device__ __forceinline__ SeqChunks seq_chunks(const int32_t *cu_seqlens, const int32_t *chunk_off,
                                                int n, int64_t T, int64_t max_chunks) {
    SeqChunks s;
    if (cu_seqlens == nullptr) {
        s.tok_begin = 0;
        s.tok_end = T;
        s.chunk_begin = 0;
        s.chunk_end = (T + 15) / 16;
    } else {
        s.tok_begin = clamp64(cu_seqlens[n], 0, T);
        s.tok_end = clamp64(cu_seqlens[n + 1], s.tok_begin, T);
        s.chunk_begin = clamp64(chunk_off[n], 0, max_chunks);
        s.chunk_end = clamp64(chunk_off[n + 1], s.chunk_begin, max_chunks);
    }
    return s;
}

// Token range of chunk c; len == 0 marks a slot with no chunk.
__device__ __forceinline__ void chunk_span(const int32_t *cu_seqlens, const int32_t *chunk_off,
                                           const int32_t *chunk_seq, int64_t c, int64_t T,
                                           int num_seqs, int64_t max_chunks, int64_t &start,
                                           int &len) {
    if (cu_seqlens == nullptr) {
        start = c * 16;
        const int64_t rem = T - start;
        len = rem <= 0 ? 0 : (rem >= 16 ? 16 : (int)rem);
        return;
    }
    const int n = chunk_seq[c];
    if (n < 0 || n >= num_seqs) {
        start = 0;
        len = 0;
        return;
    }
    const SeqChunks s = seq_chunks(cu_seqlens, chunk_off, n, T, max_chunks);
    start = s.tok_begin + 16 * (c - s.chunk_begin);
    const int64_t rem = s.tok_end - start;
    len = (c < s.chunk_begin || rem <= 0) ? 0 : (rem >= 16 ? 16 : (int)rem);
}

}  // namespace kda
