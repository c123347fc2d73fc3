// kda_chunk_table.hip -- chunk table of a packed (variable-length) batch.
//
// Sequences packed back to back are cut into 16-token chunks aligned to each
// sequence's own start (the FlashKDA benchmark has a variable-length column:
// tech-noisy.com, section "MoE通信とアテンション:MoonEPとFlashKDA"). The table holds
// chunk_off[n] = sum over m < n of ceil(len_m / 16) (a scan), and for every chunk slot
// the sequence it belongs to (binary search over chunk_off). Small batches take one
// workgroup and one launch; large ones four gridded passes (below). It runs on the
// device so that no host synchronisation is needed.
#include <climits>

#include "kda_internal.h"

namespace kda {

constexpr int kTableThreads = 1024;

__global__ __launch_bounds__(kTableThreads) void kda_chunk_table_kernel(
    const int32_t *__restrict__ cu, int N, int64_t T, int64_t max_chunks,
    int32_t *__restrict__ chunk_off, int32_t *__restrict__ chunk_seq) {
    __shared__ int64_t scan[kTableThreads];
    __shared__ int64_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += kTableThreads) {
        const int n = base + tid;
        int64_t cnt = 0;
        if (n < N) {
            const int64_t a = cu[n] < 0 ? 0 : (cu[n] > T ? T : cu[n]);
            const int64_t b = cu[n + 1] < a ? a : (cu[n + 1] > T ? T : cu[n + 1]);
            cnt = (b - a + 15) / 16;
        }
        scan[tid] = cnt;
        __syncthreads();
        for (int d = 1; d < kTableThreads; d <<= 1) {
            const int64_t add = tid >= d ? scan[tid - d] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        const int64_t excl = carry + scan[tid] - cnt;
        if (n < N) chunk_off[n] = (int32_t)(excl < max_chunks ? excl : max_chunks);
        __syncthreads();
        if (tid == kTableThreads - 1) carry += scan[tid];
        __syncthreads();
    }
    const int64_t total = carry < max_chunks ? carry : max_chunks;
    if (tid == 0) chunk_off[N] = (int32_t)total;
    __syncthreads();
    for (int64_t c = tid; c < max_chunks; c += kTableThreads) {
        int32_t seq = -1;
        if (c < total) {
            // largest n in [0, N) with chunk_off[n] <= c
            int lo = 0, hi = N - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
            }
            seq = lo;
        }
        chunk_seq[c] = seq;
    }
}

// ---------------------------------------------------------------------------
// The same table for large batches, in four gridded passes (the one-workgroup kernel
// above scans 1 024 sequences per step and labels every slot from one workgroup):
//  1. each workgroup scans the chunk counts of 1 024 sequences: chunk_off[n] = offset
//     within the workgroup's block, and the block's total to `block_tot`;
//  2. one workgroup turns the block totals into block offsets (exclusive scan, in place)
//     and writes chunk_off[N];
//  3. chunk_off[n] += its block's offset (clamped to max_chunks);
//  4. every chunk slot is labelled by binary search over chunk_off.
// `block_tot` is the chunk_seq area read as int64: passes 1-3 use it before pass 4
// writes the labels there.

// Inclusive block-wide sum of one value per thread (every thread of the workgroup calls
// it); `total` gets the sum over the whole workgroup.
__device__ __forceinline__ int64_t block_inclusive_sum(int64_t x, int64_t *scan, int64_t &total) {
    const int tid = threadIdx.x;
    scan[tid] = x;
    __syncthreads();
    for (int d = 1; d < kTableThreads; d <<= 1) {
        const int64_t add = tid >= d ? scan[tid - d] : 0;
        __syncthreads();
        scan[tid] += add;
        __syncthreads();
    }
    const int64_t r = scan[tid];
    total = scan[kTableThreads - 1];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kTableThreads) void kda_chunk_counts_kernel(const int32_t *__restrict__ cu, int N,
                                                                         int64_t T, int32_t *__restrict__ chunk_off,
                                                                         int64_t *__restrict__ block_tot) {
    __shared__ int64_t scan[kTableThreads];
    const int tid = threadIdx.x;
    const int n = blockIdx.x * kTableThreads + tid;
    int64_t cnt = 0;
    if (n < N) {
        const int64_t a = cu[n] < 0 ? 0 : (cu[n] > T ? T : cu[n]);
        const int64_t b = cu[n + 1] < a ? a : (cu[n + 1] > T ? T : cu[n + 1]);
        cnt = (b - a + 15) / 16;
    }
    int64_t total;
    const int64_t incl = block_inclusive_sum(cnt, scan, total);
    // within one block of sequences: at most ceil(T / 16) + 1 024, which fits int32
    if (n < N) chunk_off[n] = (int32_t)(incl - cnt);
    if (tid == 0) block_tot[blockIdx.x] = total;
}

__global__ __launch_bounds__(kTableThreads) void kda_chunk_blocks_kernel(int64_t *__restrict__ block_tot,
                                                                         int nblocks, int N, int64_t max_chunks,
                                                                         int32_t *__restrict__ chunk_off) {
    __shared__ int64_t scan[kTableThreads];
    const int tid = threadIdx.x;
    int64_t carry = 0;
    for (int base = 0; base < nblocks; base += kTableThreads) {
        const int i = base + tid;
        const int64_t x = i < nblocks ? block_tot[i] : 0;
        int64_t total;
        const int64_t incl = block_inclusive_sum(x, scan, total);
        if (i < nblocks) block_tot[i] = carry + incl - x;
        carry += total;
    }
    if (tid == 0) chunk_off[N] = (int32_t)(carry < max_chunks ? carry : max_chunks);
}

__global__ __launch_bounds__(256) void kda_chunk_offsets_kernel(const int64_t *__restrict__ block_off, int N,
                                                                int64_t max_chunks,
                                                                int32_t *__restrict__ chunk_off) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const int64_t x = block_off[n / kTableThreads] + chunk_off[n];
    chunk_off[n] = (int32_t)(x < max_chunks ? x : max_chunks);
}

__global__ __launch_bounds__(256) void kda_chunk_labels_kernel(const int32_t *__restrict__ chunk_off, int N,
                                                               int64_t max_chunks, int32_t *__restrict__ chunk_seq) {
    const int64_t total = chunk_off[N];
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < max_chunks; c += stride) {
        int32_t seq = -1;
        if (c < total) {
            int lo = 0, hi = N - 1;  // largest n in [0, N) with chunk_off[n] <= c
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
            }
            seq = lo;
        }
        chunk_seq[c] = seq;
    }
}

// Up to these sizes the one-workgroup kernel builds the table in one launch.
constexpr int kSmallTableSeqs = kTableThreads;
constexpr int64_t kSmallTableChunks = 1 << 16;

hipError_t launch_chunk_table(const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                              hipStream_t stream) {
    char *base = static_cast<char *>(ws);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(base + geo.off_chunk_off);
    int32_t *chunk_seq = reinterpret_cast<int32_t *>(base + geo.off_chunk_seq);
    if (geo.N <= kSmallTableSeqs && geo.max_chunks <= kSmallTableChunks) {
        hipLaunchKernelGGL(kda_chunk_table_kernel, dim3(1), dim3(kTableThreads), 0, stream, cu_seqlens,
                           geo.N, geo.T, geo.max_chunks, chunk_off, chunk_seq);
        return hipGetLastError();
    }
    const int nblocks = (geo.N + kTableThreads - 1) / kTableThreads;
    // the block totals borrow the chunk_seq area (labelled last): it is 256-byte aligned
    // and holds max_chunks >= 15 N / 16 int32, far more than nblocks int64
    if ((size_t)nblocks * sizeof(int64_t) > (size_t)geo.max_chunks * sizeof(int32_t) ||
        geo.off_chunk_seq % alignof(int64_t) != 0)
        return hipErrorInvalidValue;
    int64_t *block_tot = reinterpret_cast<int64_t *>(chunk_seq);
    hipLaunchKernelGGL(kda_chunk_counts_kernel, dim3(nblocks), dim3(kTableThreads), 0, stream, cu_seqlens, geo.N,
                       geo.T, chunk_off, block_tot);
    hipLaunchKernelGGL(kda_chunk_blocks_kernel, dim3(1), dim3(kTableThreads), 0, stream, block_tot, nblocks, geo.N,
                       geo.max_chunks, chunk_off);
    hipLaunchKernelGGL(kda_chunk_offsets_kernel, dim3((geo.N + 255) / 256), dim3(256), 0, stream, block_tot, geo.N,
                       geo.max_chunks, chunk_off);
    const int64_t label_blocks = (geo.max_chunks + 255) / 256;
    hipLaunchKernelGGL(kda_chunk_labels_kernel, dim3((unsigned)(label_blocks < 65536 ? label_blocks : 65536)),
                       dim3(256), 0, stream, chunk_off, geo.N, geo.max_chunks, chunk_seq);
    return hipGetLastError();
}


// Check of packed-sequence boundaries, which the host never reads: the smallest n in
// [0, N] at which cu[0] = 0, cu[n - 1] <= cu[n] or cu[N] = T fails, else -1. The
// prefill kernels do not depend on it (they clamp every boundary they read); it lets
// a caller find malformed boundaries that would otherwise only give wrong numbers.
__global__ __launch_bounds__(kTableThreads) void kda_check_seqlens_kernel(const int32_t *__restrict__ cu, int N,
                                                                          int64_t T, int32_t *__restrict__ result) {
    __shared__ int first;
    const int tid = threadIdx.x;
    if (tid == 0) first = INT_MAX;
    __syncthreads();
    for (int n = tid; n <= N; n += kTableThreads) {
        const int64_t x = cu[n];
        const bool bad = (n == 0 ? x != 0 : x < (int64_t)cu[n - 1]) || (n == N && x != T);
        if (bad) {
            atomicMin(&first, n);  // n grows along the loop: this thread's first failure is its smallest
            break;
        }
    }
    __syncthreads();
    if (tid == 0) *result = first == INT_MAX ? -1 : first;
}

hipError_t launch_check_seqlens(const int32_t *cu_seqlens, int num_seqs, int64_t total_tokens, int32_t *result,
                                hipStream_t stream) {
    hipLaunchKernelGGL(kda_check_seqlens_kernel, dim3(1), dim3(kTableThreads), 0, stream, cu_seqlens, num_seqs,
                       total_tokens, result);
    return hipGetLastError();
}

}  // namespace kda
