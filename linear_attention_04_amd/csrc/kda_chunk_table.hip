// kda_chunk_table.hip -- chunk table of a packed (variable-length) batch.
//
// Sequences packed back to back are cut into 16-token chunks aligned to each
// sequence's own start (the FlashKDA benchmark has a variable-length column:
// tech-noisy.com, section "MoE通信とアテンション:MoonEPとFlashKDA"). One workgroup
// computes chunk_off[n] = sum over m < n of ceil(len_m / 16) with a block-wide scan,
// then labels every chunk slot with its sequence by binary search over chunk_off.
// It runs on the device so that no host synchronisation is needed.
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

}  // namespace kda
