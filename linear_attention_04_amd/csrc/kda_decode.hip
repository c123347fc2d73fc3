// kda_decode.hip -- one-token KDA state update for a batch of sequences (serving).
//
// When a new token arrives, the model updates each head's fixed-size recurrent
// state rather than growing a cache, and a deployment keeps those states between
// calls (augursoft.site "Kimi K3 的三個系統設計", section "第一個設計：把長上下文從
// 「一直累積」改成「持續更新狀態」"). For one token with state S (K x V, fp32):
//   S' = Diag(alpha) S,   delta = beta (v - S'^T k),   S = S' + k delta^T,
//   o  = S^T q = S'^T q + (q . k) delta.
// Every element of S is read once and written once, so the step is bound by HBM
// traffic: 2 * K * V * 4 bytes per (sequence, head), against which the K-long dot
// products are small.
//
// One workgroup of 256 threads per (sequence, head). Thread t holds the four value
// columns 4 (t % 32) .. + 3 of the 16 key rows t / 32 + 8 m (m = 0..15): each wave
// load covers two whole 512-byte rows of S, and the partial k . S' and q . S' of the
// eight row groups are summed through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int KD = 128;
constexpr int VD = 128;
constexpr int kThreads = 256;
constexpr int kColGroups = VD / 4;              // 32 threads span one row
constexpr int kRowGroups = kThreads / kColGroups;  // 8
constexpr int kRowsPerThread = KD / kRowGroups;    // 16

template <typename IO>
__device__ __forceinline__ float load_io(const IO *p, size_t i);
template <>
__device__ __forceinline__ float load_io<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_io<__bf16>(const __bf16 *p, size_t i) { return from_bf16(p[i]); }

template <typename IO>
__device__ __forceinline__ void store_io(IO *p, size_t i, float x);
template <>
__device__ __forceinline__ void store_io<float>(float *p, size_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_io<__bf16>(__bf16 *p, size_t i, float x) { p[i] = to_bf16(x); }

template <typename IO, bool SCALAR_GATE>
__global__ __launch_bounds__(kThreads) void kda_decode_kernel(const IO *__restrict__ q, const IO *__restrict__ k,
                                                              const IO *__restrict__ v, const float *__restrict__ g,
                                                              const float *__restrict__ beta,
                                                              float *__restrict__ state, IO *__restrict__ out) {
    __shared__ float qs[KD], ks[KD], al[KD], vs[VD], dl[VD];
    __shared__ float red_k[kRowGroups][VD], red_q[kRowGroups][VD];
    __shared__ float qk_part[2];
    const int t = threadIdx.x;
    const size_t bh = blockIdx.x;  // sequence * H + head
    const size_t vec = bh * KD;    // q, k, g rows (K == V here)

    if (t < KD) {
        const float qi = load_io(q, vec + t), ki = load_io(k, vec + t);
        qs[t] = qi;
        ks[t] = ki;
        al[t] = __expf(SCALAR_GATE ? g[bh] : g[vec + t]);
        vs[t] = load_io(v, bh * VD + t);
        // q . k over the 128 channels: two waves, one partial each
        float p = qi * ki;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) p += __shfl_xor(p, off, 64);
        if ((t & 63) == 0) qk_part[t >> 6] = p;
    }
    const float b = beta[bh];

    const int cg = t % kColGroups, rg = t / kColGroups;
    float4 *srow = reinterpret_cast<float4 *>(state + bh * KD * VD) + cg;
    float4 s[kRowsPerThread];
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m) s[m] = srow[(size_t)(rg + kRowGroups * m) * (VD / 4)];
    __syncthreads();

    // decay, then this thread's parts of k . S' and q . S' for its four columns
    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m) {
        const int i = rg + kRowGroups * m;
        const float a = al[i], ki = ks[i], qi = qs[i];
        s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
        pk.x += ki * s[m].x; pk.y += ki * s[m].y; pk.z += ki * s[m].z; pk.w += ki * s[m].w;
        pq.x += qi * s[m].x; pq.y += qi * s[m].y; pq.z += qi * s[m].z; pq.w += qi * s[m].w;
    }
    *reinterpret_cast<float4 *>(&red_k[rg][4 * cg]) = pk;
    *reinterpret_cast<float4 *>(&red_q[rg][4 * cg]) = pq;
    __syncthreads();

    if (t < VD) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int r = 0; r < kRowGroups; ++r) {
            sk += red_k[r][t];
            sq += red_q[r][t];
        }
        const float d = b * (vs[t] - sk);
        dl[t] = d;
        store_io(out, bh * VD + t, sq + (qk_part[0] + qk_part[1]) * d);
    }
    __syncthreads();

    const float4 d4 = *reinterpret_cast<const float4 *>(&dl[4 * cg]);
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m) {
        const float ki = ks[rg + kRowGroups * m];
        s[m].x += ki * d4.x; s[m].y += ki * d4.y; s[m].z += ki * d4.z; s[m].w += ki * d4.w;
        // written non-temporal: the next step reads the state back from HBM anyway (the
        // batch's states exceed the caches), and dirty lines left behind would be written
        // back while that step streams its own reads
        __builtin_nontemporal_store(f32x4_t{s[m].x, s[m].y, s[m].z, s[m].w},
                                    reinterpret_cast<f32x4_t *>(srow + (size_t)(rg + kRowGroups * m) * (VD / 4)));
    }
}

template <typename IO>
hipError_t launch_typed(const void *q, const void *k, const void *v, const float *g, const float *beta, float *state,
                        void *out, int64_t B, int H, bool scalar_gate, hipStream_t stream) {
    const int64_t blocks = B * H;
    if (blocks == 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    auto kern = scalar_gate ? kda_decode_kernel<IO, true> : kda_decode_kernel<IO, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), 0, stream, static_cast<const IO *>(q),
                       static_cast<const IO *>(k), static_cast<const IO *>(v), g, beta, state,
                       static_cast<IO *>(out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         float *state, void *out, int64_t B, int H, int io, bool scalar_gate, hipStream_t stream) {
    if (io == KDA_IO_BF16) return launch_typed<__bf16>(q, k, v, g, beta, state, out, B, H, scalar_gate, stream);
    return launch_typed<float>(q, k, v, g, beta, state, out, B, H, scalar_gate, stream);
}

}  // namespace kda
