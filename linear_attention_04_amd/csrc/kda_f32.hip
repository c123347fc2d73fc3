// kda_f32.hip -- fp32-io chunked KDA prefill (K = V in {16, 32, 64, 128}).
//
// Same two-kernel decomposition and the same chunk algebra as the bf16 path (see
// kda_intra_bf16.hip), carried out entirely in fp32 on the vector ALU with LDS
// staging: exponentials of gate differences are taken directly, exp(G_r - G_i),
// and nothing is rounded to bf16. It serves small and accuracy-critical cases;
// the MFMA path is the bf16 one.
//
// Record of one (chunk, head), fp32, row-major:
//   W [16][K] | QT [16][K] | KD [16][K] | TB [16][16] | MM [16][16] | GAM [K]
#include "kda_chunks.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <int K>
struct F32Rec {
    static constexpr int W = 0;
    static constexpr int QT = 16 * K;
    static constexpr int KD = 32 * K;
    static constexpr int TB = 48 * K;
    static constexpr int MM = 48 * K + 256;
    static constexpr int GAM = 48 * K + 512;
    static constexpr int FLOATS = 49 * K + 512;
};

template <int K>
__global__ __launch_bounds__(64) void kda_intra_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off,
    const int32_t *__restrict__ chunk_seq, int64_t T, int H, int N, int64_t max_chunks,
    float *__restrict__ records, int scalar_gate) {
    __shared__ float qs[16 * K], ks[16 * K], G[16 * K];
    __shared__ float A[256], P[256], TB[256], MM[256], bs[16];
    const int tid = threadIdx.x;
    const int64_t chunk = blockIdx.x;
    const int h = blockIdx.y;
    int64_t start;
    int len;
    chunk_span(cu, chunk_off, chunk_seq, chunk, T, N, max_chunks, start, len);
    if (len == 0) return;
    float *rec = records + ((size_t)chunk * H + h) * F32Rec<K>::FLOATS;  // chunk-major

    for (int idx = tid; idx < 16 * K; idx += 64) {
        const int r = idx / K, ch = idx % K;
        const bool ok = r < len;
        const size_t off = ((size_t)(start + r) * H + h) * K + ch;
        qs[idx] = ok ? q[off] : 0.f;
        ks[idx] = ok ? k[off] : 0.f;
        // a scalar gate (g [T, H]) is the same decay for every channel
        const size_t goff = scalar_gate ? (size_t)(start + r) * H + h : off;
        G[idx] = ok ? g[goff] : 0.f;
    }
    if (tid < 16) bs[tid] = tid < len ? beta[(size_t)(start + tid) * H + h] : 0.f;
    __syncthreads();
    for (int ch = tid; ch < K; ch += 64) {
        float run = 0.f;
        for (int r = 0; r < 16; ++r) {
            run += G[r * K + ch];
            G[r * K + ch] = run;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < 256; idx += 64) {
        const int r = idx >> 4, i = idx & 15;
        float a = 0.f, p = 0.f;
        if (i <= r) {
            for (int ch = 0; ch < K; ++ch) {
                const float e = expf(G[r * K + ch] - G[i * K + ch]);
                const float ke = ks[i * K + ch] * e;
                a += ks[r * K + ch] * ke;
                p += qs[r * K + ch] * ke;
            }
        }
        A[idx] = i < r ? bs[r] * a : 0.f;
        P[idx] = p;
    }
    __syncthreads();
    if (tid < 16) {
        const int j = tid;
        float x[16];
        for (int r = 0; r < 16; ++r) {
            float acc = (r == j) ? 1.f : 0.f;
            for (int i = 0; i < r; ++i) acc -= A[r * 16 + i] * x[i];
            x[r] = acc;
        }
        for (int r = 0; r < 16; ++r) TB[r * 16 + j] = x[r] * bs[j];
    }
    __syncthreads();
    for (int idx = tid; idx < 256; idx += 64) {
        const int r = idx >> 4, j = idx & 15;
        float m = 0.f;
        for (int i = 0; i < 16; ++i) m += P[r * 16 + i] * TB[i * 16 + j];
        MM[idx] = m;
        rec[F32Rec<K>::TB + idx] = TB[idx];
    }
    for (int idx = tid; idx < 16 * K; idx += 64) {
        const int ch = idx % K;
        rec[F32Rec<K>::KD + idx] = ks[idx] * expf(G[15 * K + ch] - G[idx]);
    }
    for (int ch = tid; ch < K; ch += 64) rec[F32Rec<K>::GAM + ch] = expf(G[15 * K + ch]);
    __syncthreads();
    for (int idx = tid; idx < 16 * K; idx += 64) {
        const float eg = expf(G[idx]);
        ks[idx] *= eg;  // K+
        qs[idx] *= eg;  // Q+
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * K; idx += 64) {
        const int t = idx / K, ch = idx % K;
        float w = 0.f, pw = 0.f;
        for (int i = 0; i < 16; ++i) {
            const float kp = ks[i * K + ch];
            w += TB[t * 16 + i] * kp;
            pw += MM[t * 16 + i] * kp;
        }
        rec[F32Rec<K>::W + idx] = w;
        rec[F32Rec<K>::QT + idx] = qs[idx] - pw;
    }
    for (int idx = tid; idx < 256; idx += 64) rec[F32Rec<K>::MM + idx] = MM[idx];
}

template <int K>
__global__ __launch_bounds__(K) void kda_inter_f32_kernel(
    const float *__restrict__ v, const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off,
    const float *__restrict__ s0, float *__restrict__ out, float *__restrict__ sT, int64_t T, int H,
    int64_t max_chunks, const float *__restrict__ records) {
    constexpr int V = K;
    __shared__ float R[F32Rec<K>::FLOATS];
    __shared__ float D[16 * V];  // Delta of the current chunk, [token][column]
    const int pair = blockIdx.x;
    const int n = pair / H, h = pair % H;
    const int j = threadIdx.x;  // value column
    const SeqChunks sc = seq_chunks(cu, chunk_off, n, T, max_chunks);
    float S[K];
    const size_t sbase = (size_t)pair * K * V + j;
#pragma unroll
    for (int kk = 0; kk < K; ++kk) S[kk] = s0 ? s0[sbase + (size_t)kk * V] : 0.f;

    for (int64_t ci = sc.chunk_begin; ci < sc.chunk_end; ++ci) {
        const int64_t tok0 = sc.tok_begin + 16 * (ci - sc.chunk_begin);
        const int64_t rem = sc.tok_end - tok0;
        const int len = rem <= 0 ? 0 : (rem >= 16 ? 16 : (int)rem);
        const float *rec = records + ((size_t)ci * H + h) * F32Rec<K>::FLOATS;
        __syncthreads();
        for (int idx = j; idx < F32Rec<K>::FLOATS; idx += V) R[idx] = rec[idx];
        __syncthreads();
        float vv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) vv[t] = t < len ? v[((size_t)(tok0 + t) * H + h) * V + j] : 0.f;
#pragma unroll 1
        for (int t = 0; t < 16; ++t) {
            float u = 0.f, x = 0.f, o = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                u += R[F32Rec<K>::TB + t * 16 + i] * vv[i];
                o += R[F32Rec<K>::MM + t * 16 + i] * vv[i];
            }
#pragma unroll
            for (int kk = 0; kk < K; ++kk) {
                x += R[F32Rec<K>::W + t * K + kk] * S[kk];
                o += R[F32Rec<K>::QT + t * K + kk] * S[kk];
            }
            D[t * V + j] = u - x;
            if (t < len) out[((size_t)(tok0 + t) * H + h) * V + j] = o;
        }
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
            float acc = R[F32Rec<K>::GAM + kk] * S[kk];
#pragma unroll 1
            for (int t = 0; t < 16; ++t) acc += R[F32Rec<K>::KD + t * K + kk] * D[t * V + j];
            S[kk] = acc;
        }
    }
    if (sT) {
#pragma unroll
        for (int kk = 0; kk < K; ++kk) sT[sbase + (size_t)kk * V] = S[kk];
    }
}

template <int K>
hipError_t intra_f32(const float *q, const float *k, const float *g, const float *beta,
                     const int32_t *cu, const Geometry &geo, void *ws, hipStream_t stream) {
    char *base = static_cast<char *>(ws);
    const dim3 grid((unsigned)geo.max_chunks, (unsigned)geo.H);
    hipLaunchKernelGGL(kda_intra_f32_kernel<K>, grid, dim3(64), 0, stream, q, k, g, beta, cu,
                       reinterpret_cast<const int32_t *>(base + geo.off_chunk_off),
                       reinterpret_cast<const int32_t *>(base + geo.off_chunk_seq), geo.T, geo.H, geo.N,
                       geo.max_chunks, reinterpret_cast<float *>(base + geo.off_records), (int)geo.scalar_gate);
    return hipGetLastError();
}

template <int K>
hipError_t inter_f32(const float *v, const int32_t *cu, const float *s0, float *out, float *sT,
                     const Geometry &geo, const void *ws, hipStream_t stream) {
    const char *base = static_cast<const char *>(ws);
    hipLaunchKernelGGL(kda_inter_f32_kernel<K>, dim3(geo.N * geo.H), dim3(K), 0, stream, v, cu,
                       reinterpret_cast<const int32_t *>(base + geo.off_chunk_off), s0, out, sT, geo.T,
                       geo.H, geo.max_chunks, reinterpret_cast<const float *>(base + geo.off_records));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_intra_f32(const float *q, const float *k, const float *g, const float *beta,
                            const int32_t *cu_seqlens, const Geometry &geo, void *ws,
                            hipStream_t stream) {
    if (geo.max_chunks == 0) return hipSuccess;
    switch (geo.K) {
    case 16: return intra_f32<16>(q, k, g, beta, cu_seqlens, geo, ws, stream);
    case 32: return intra_f32<32>(q, k, g, beta, cu_seqlens, geo, ws, stream);
    case 64: return intra_f32<64>(q, k, g, beta, cu_seqlens, geo, ws, stream);
    case 128: return intra_f32<128>(q, k, g, beta, cu_seqlens, geo, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_inter_f32(const float *v, const int32_t *cu_seqlens, const float *s0, float *out,
                            float *sT, const Geometry &geo, const void *ws, hipStream_t stream) {
    switch (geo.K) {
    case 16: return inter_f32<16>(v, cu_seqlens, s0, out, sT, geo, ws, stream);
    case 32: return inter_f32<32>(v, cu_seqlens, s0, out, sT, geo, ws, stream);
    case 64: return inter_f32<64>(v, cu_seqlens, s0, out, sT, geo, ws, stream);
    case 128: return inter_f32<128>(v, cu_seqlens, s0, out, sT, geo, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
