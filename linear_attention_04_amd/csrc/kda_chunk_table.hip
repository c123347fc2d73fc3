// kda_chunk_table.hip -- chunk table of a packed (variable-length) batch.
//
// Sequences packed back to back are cut into 16-token chunks aligned to each
// sequence's own start (the FlashKDA benchmark has a variable-length column:
// tech-noisy.com, section "MoE通信とアテンション:MoonEPとFlashKDA"). One workgroup
// computes chunk_off[n] = sum over m < n of ceil(len_m / 16) with a block-wide scan,
// then labels every chunk slot with its sequence by binary search over chunk_off.
// It runs on the device so that no host synchronisation is needed.
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

hipError_t launch_chunk_table(const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                              hipStream_t stream) {
    char *base = static_cast<char *>(ws);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(base + geo.off_chunk_off);
    int32_t *chunk_seq = reinterpret_cast<int32_t *>(base + geo.off_chunk_seq);
    hipLaunchKernelGGL(kda_chunk_table_kernel, dim3(1), dim3(kTableThreads), 0, stream, cu_seqlens,
                       geo.N, geo.T, geo.max_chunks, chunk_off, chunk_seq);
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
