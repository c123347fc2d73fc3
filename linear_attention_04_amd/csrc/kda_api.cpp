// kda_api.cpp -- C ABI entry points of libkda: argument checks, workspace layout and
// kernel launches. Nothing here touches the device before every check has passed.
#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace kda {

namespace {
std::mutex g_cache_mutex;
std::vector<std::pair<int, DeviceShape>> g_shapes;      // per device
std::vector<std::pair<const void *, int>> g_lds_set;    // (kernel, device) pairs done
}  // namespace

hipError_t device_shape(DeviceShape *shape) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    for (const auto &it : g_shapes) {
        if (it.first == dev) {
            *shape = it.second;
            return hipSuccess;
        }
    }
    DeviceShape s{};
    e = hipDeviceGetAttribute(&s.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (hipDeviceGetAttribute(&s.xccs, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || s.xccs < 1) {
        (void)hipGetLastError();  // an older runtime without the attribute: one die
        s.xccs = 1;
    }
    if (s.cus < 1) s.cus = 1;
    g_shapes.emplace_back(dev, s);
    *shape = s;
    return hipSuccess;
}

hipError_t set_dynamic_lds(const void *fn, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    for (const auto &it : g_lds_set) {
        if (it.first == fn && it.second == dev) return hipSuccess;
    }
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    g_lds_set.emplace_back(fn, dev);
    return hipSuccess;
}

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported(const kda_dims_t *d) {
    if (d->io_dtype == KDA_IO_BF16) return d->head_k == 128 && d->head_v == 128;
    if (d->io_dtype == KDA_IO_F32)
        return d->head_k == d->head_v &&
               (d->head_k == 16 || d->head_k == 32 || d->head_k == 64 || d->head_k == 128);
    return false;
}

int check_pointers(std::initializer_list<const void *> required, std::initializer_list<const void *> optional) {
    for (const void *p : required) {
        if (p == nullptr) return KDA_ERR_ARG;
    }
    for (const void *p : required) {
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    }
    for (const void *p : optional) {
        if (p != nullptr && !aligned16(p)) return KDA_ERR_ALIGN;
    }
    return KDA_OK;
}

int check_common(const kda_dims_t *dims, const int32_t *cu_seqlens, void *ws, size_t ws_bytes, Geometry *geo) {
    const int st = make_geometry(dims, geo);
    if (st != KDA_OK) return st;
    if (cu_seqlens == nullptr && dims->num_seqs != 1) return KDA_ERR_ARG;
    if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_ALIGN;
    if (ws == nullptr || ws_bytes < geo->total_bytes) return KDA_ERR_WORKSPACE;
    if (!aligned16(ws)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH; }

}  // namespace

int make_geometry(const kda_dims_t *d, Geometry *g) {
    if (d == nullptr || g == nullptr) return KDA_ERR_ARG;
    if (d->total_tokens < 0 || d->num_heads < 1 || d->head_k < 1 || d->head_v < 1 || d->num_seqs < 1 ||
        (d->gate_kind != KDA_GATE_CHANNEL && d->gate_kind != KDA_GATE_SCALAR))
        return KDA_ERR_ARG;
    if (d->total_tokens > (int64_t)INT32_MAX || d->num_seqs > kMaxSeqs || d->num_heads > (1 << 16))
        return KDA_ERR_ARG;
    if (!supported(d)) return KDA_ERR_UNSUPPORTED;
    g->T = d->total_tokens;
    g->H = d->num_heads;
    g->K = d->head_k;
    g->V = d->head_v;
    g->N = d->num_seqs;
    g->io = d->io_dtype;
    g->scalar_gate = d->gate_kind == KDA_GATE_SCALAR;
    // sum_n ceil(len_n / 16) <= (T + 15 N) / 16
    g->max_chunks = (g->T + 15 * (int64_t)g->N) / kChunk;
    if (g->max_chunks > (int64_t)INT32_MAX / 2) return KDA_ERR_ARG;
    if ((int64_t)g->N * g->H > (int64_t)INT32_MAX / 64) return KDA_ERR_ARG;
    g->record_bytes = d->io_dtype == KDA_IO_BF16 ? (size_t)kRecBytesBf16 : rec_bytes_f32(g->K);
    g->off_chunk_off = 0;
    g->off_chunk_seq = align_up(sizeof(int32_t) * ((size_t)g->N + 1));
    g->off_records = g->off_chunk_seq + align_up(sizeof(int32_t) * (size_t)g->max_chunks);
    g->total_bytes = g->off_records + (size_t)g->max_chunks * (size_t)g->H * g->record_bytes;
    return KDA_OK;
}

int make_backward_geometry(const kda_dims_t *d, Geometry *g) {
    const int st = make_geometry(d, g);
    if (st != KDA_OK) return st;
    if (g->io != KDA_IO_BF16) return KDA_ERR_UNSUPPORTED;
    const size_t per = (size_t)g->max_chunks * (size_t)g->H;
    g->off_brecords = align_up(g->total_bytes);
    g->off_states = align_up(g->off_brecords + per * kBRecBytes);
    g->off_dstates = align_up(g->off_states + per * kStateBytesBf16);
    g->backward_bytes = g->off_dstates + per * kStateBytesBf16;
    return KDA_OK;
}

}  // namespace kda

using kda::Geometry;

extern "C" {

size_t kda_workspace_bytes(const kda_dims_t *dims) {
    Geometry geo;
    if (kda::make_geometry(dims, &geo) != KDA_OK) return 0;
    return geo.total_bytes;
}

int kda_intra_chunk(const void *q, const void *k, const float *g, const float *beta,
                    const int32_t *cu_seqlens, const kda_dims_t *dims, void *workspace,
                    size_t workspace_bytes, void *stream) {
    Geometry geo;
    int st = kda::check_common(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st != KDA_OK) return st;
    if (geo.T > 0) {
        st = kda::check_pointers({q, k, g, beta}, {});
        if (st != KDA_OK) return st;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (cu_seqlens != nullptr) {
        st = kda::launch_status(kda::launch_chunk_table(cu_seqlens, geo, workspace, s));
        if (st != KDA_OK) return st;
    }
    if (geo.T == 0) return KDA_OK;
    if (geo.io == KDA_IO_BF16)
        return kda::launch_status(kda::launch_intra_bf16(q, k, g, beta, cu_seqlens, geo, workspace, s));
    return kda::launch_status(kda::launch_intra_f32(static_cast<const float *>(q), static_cast<const float *>(k),
                                                    g, beta, cu_seqlens, geo, workspace, s));
}

int kda_inter_chunk(const void *v, const int32_t *cu_seqlens, const float *initial_state, void *out,
                    float *final_state, const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                    void *stream) {
    Geometry geo;
    int st = kda::check_common(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st != KDA_OK) return st;
    if (geo.T > 0) {
        st = kda::check_pointers({v, out}, {initial_state, final_state});
    } else {
        st = kda::check_pointers({}, {v, out, initial_state, final_state});
    }
    if (st != KDA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (geo.io == KDA_IO_BF16)
        return kda::launch_status(
            kda::launch_inter_bf16(v, cu_seqlens, initial_state, out, final_state, geo, workspace, s));
    return kda::launch_status(kda::launch_inter_f32(static_cast<const float *>(v), cu_seqlens, initial_state,
                                                    static_cast<float *>(out), final_state, geo, workspace, s));
}

int kda_chunk_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                      const int32_t *cu_seqlens, const float *initial_state, void *out, float *final_state,
                      const kda_dims_t *dims, void *workspace, size_t workspace_bytes, void *stream) {
    Geometry geo;
    int st = kda::check_common(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st != KDA_OK) return st;
    if (geo.T > 0) {
        st = kda::check_pointers({q, k, v, g, beta, out}, {initial_state, final_state});
    } else {
        st = kda::check_pointers({}, {q, k, v, g, beta, out, initial_state, final_state});
    }
    if (st != KDA_OK) return st;
    st = kda_intra_chunk(q, k, g, beta, cu_seqlens, dims, workspace, workspace_bytes, stream);
    if (st != KDA_OK) return st;
    return kda_inter_chunk(v, cu_seqlens, initial_state, out, final_state, dims, workspace, workspace_bytes,
                           stream);
}

int kda_chunk_prefill_fused(const void *q, const void *k, const void *v, const float *g, const float *beta,
                            const int32_t *cu_seqlens, const float *initial_state, void *out, float *final_state,
                            const kda_dims_t *dims, void *workspace, size_t workspace_bytes, void *stream) {
    Geometry geo;
    int st = kda::check_common(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st != KDA_OK) return st;
    if (geo.io != KDA_IO_BF16) return KDA_ERR_UNSUPPORTED;
    if (geo.T > 0) {
        st = kda::check_pointers({q, k, v, g, beta, out}, {initial_state, final_state});
    } else {
        st = kda::check_pointers({}, {q, k, v, g, beta, out, initial_state, final_state});
    }
    if (st != KDA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (cu_seqlens != nullptr) {
        st = kda::launch_status(kda::launch_chunk_table(cu_seqlens, geo, workspace, s));
        if (st != KDA_OK) return st;
    }
    return kda::launch_status(kda::launch_fused_bf16(q, k, v, g, beta, cu_seqlens, initial_state, out,
                                                     final_state, geo, workspace, s));
}

int kda_decode_step(const void *q, const void *k, const void *v, const float *g, const float *beta,
                    float *state, void *out, const kda_dims_t *dims, void *stream) {
    if (dims == nullptr) return KDA_ERR_ARG;
    if (dims->total_tokens < 0 || dims->num_heads < 1 || dims->num_seqs < 0 ||
        dims->total_tokens != (int64_t)dims->num_seqs ||
        (dims->gate_kind != KDA_GATE_CHANNEL && dims->gate_kind != KDA_GATE_SCALAR) ||
        (dims->io_dtype != KDA_IO_BF16 && dims->io_dtype != KDA_IO_F32))
        return KDA_ERR_ARG;
    if (dims->total_tokens * (int64_t)dims->num_heads > (int64_t)INT32_MAX) return KDA_ERR_ARG;
    if (dims->head_k != 128 || dims->head_v != 128) return KDA_ERR_UNSUPPORTED;
    if (dims->total_tokens == 0) return KDA_OK;
    const int st = kda::check_pointers({q, k, v, g, beta, state, out}, {});
    if (st != KDA_OK) return st;
    return kda::launch_status(kda::launch_decode(q, k, v, g, beta, state, out, dims->total_tokens,
                                                 dims->num_heads, dims->io_dtype,
                                                 dims->gate_kind == KDA_GATE_SCALAR,
                                                 static_cast<hipStream_t>(stream)));
}

size_t kda_backward_workspace_bytes(const kda_dims_t *dims) {
    Geometry geo;
    if (kda::make_backward_geometry(dims, &geo) != KDA_OK) return 0;
    return geo.backward_bytes;
}

namespace {

int check_backward(const kda_dims_t *dims, const int32_t *cu_seqlens, void *ws, size_t ws_bytes, Geometry *geo) {
    const int st = kda::make_backward_geometry(dims, geo);
    if (st != KDA_OK) return st;
    if (cu_seqlens == nullptr && dims->num_seqs != 1) return KDA_ERR_ARG;
    if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_ALIGN;
    if (ws == nullptr || ws_bytes < geo->backward_bytes) return KDA_ERR_WORKSPACE;
    if (!kda::aligned16(ws)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

// Pointers that must be set when there are tokens (all are optional when T = 0).
int check_data(const Geometry &geo, std::initializer_list<const void *> required,
               std::initializer_list<const void *> optional) {
    if (geo.T > 0) return kda::check_pointers(required, optional);
    int st = kda::check_pointers({}, required);
    return st != KDA_OK ? st : kda::check_pointers({}, optional);
}

}  // namespace

int kda_backward_records(const void *q, const void *k, const float *g, const float *beta,
                         const int32_t *cu_seqlens, const kda_dims_t *dims, void *workspace,
                         size_t workspace_bytes, void *stream) {
    Geometry geo;
    int st = check_backward(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st == KDA_OK) st = check_data(geo, {q, k, g, beta}, {});
    if (st != KDA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (cu_seqlens != nullptr) {
        st = kda::launch_status(kda::launch_chunk_table(cu_seqlens, geo, workspace, s));
        if (st != KDA_OK) return st;
    }
    if (geo.T == 0) return KDA_OK;
    return kda::launch_status(kda::launch_intra_bf16_bwd(q, k, g, beta, cu_seqlens, geo, workspace, s));
}

int kda_backward_states(const void *v, const int32_t *cu_seqlens, const float *initial_state,
                        const kda_dims_t *dims, void *workspace, size_t workspace_bytes, void *stream) {
    Geometry geo;
    int st = check_backward(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st == KDA_OK) st = check_data(geo, {v}, {initial_state});
    if (st != KDA_OK || geo.T == 0) return st;
    return kda::launch_status(kda::launch_inter_bf16_states(v, cu_seqlens, initial_state, geo, workspace,
                                                            static_cast<hipStream_t>(stream)));
}

int kda_chunk_prefill_for_backward(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const int32_t *cu_seqlens, const float *initial_state,
                                   void *out, float *final_state, const kda_dims_t *dims, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    Geometry geo;
    int st = check_backward(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st == KDA_OK) st = check_data(geo, {q, k, v, g, beta, out}, {initial_state, final_state});
    if (st != KDA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (cu_seqlens != nullptr) {
        st = kda::launch_status(kda::launch_chunk_table(cu_seqlens, geo, workspace, s));
        if (st != KDA_OK) return st;
    }
    if (geo.T > 0) {
        st = kda::launch_status(kda::launch_intra_bf16_bwd(q, k, g, beta, cu_seqlens, geo, workspace, s));
        if (st != KDA_OK) return st;
    }
    // also with T = 0: the final state of each (empty) sequence is its initial state
    return kda::launch_status(
        kda::launch_inter_bf16_states_out(v, cu_seqlens, initial_state, out, final_state, geo, workspace, s));
}

int kda_backward_state_grad(const void *d_out, const int32_t *cu_seqlens, const float *d_final_state,
                            float *d_initial_state, const kda_dims_t *dims, void *workspace,
                            size_t workspace_bytes, void *stream) {
    Geometry geo;
    int st = check_backward(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st == KDA_OK) st = check_data(geo, {d_out}, {d_final_state, d_initial_state});
    if (st != KDA_OK) return st;
    // also with T = 0: the final-state gradient passes through empty sequences
    return kda::launch_status(kda::launch_state_grad_bf16(d_out, cu_seqlens, d_final_state, d_initial_state, geo,
                                                          workspace, static_cast<hipStream_t>(stream)));
}

int kda_backward_token_grad(const void *q, const void *k, const void *v, const float *g, const float *beta,
                            const void *d_out, const int32_t *cu_seqlens, void *dq, void *dk, void *dv, float *dg,
                            float *dbeta, const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                            void *stream) {
    Geometry geo;
    int st = check_backward(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st == KDA_OK) st = check_data(geo, {q, k, v, g, beta, d_out, dq, dk, dv, dg, dbeta}, {});
    if (st != KDA_OK || geo.T == 0) return st;
    return kda::launch_status(kda::launch_grad_bf16(q, k, v, g, beta, d_out, cu_seqlens, dq, dk, dv, dg, dbeta,
                                                    geo, workspace, static_cast<hipStream_t>(stream)));
}

int kda_chunk_prefill_backward(const void *q, const void *k, const void *v, const float *g, const float *beta,
                               const int32_t *cu_seqlens, const float *initial_state, const void *d_out,
                               const float *d_final_state, void *dq, void *dk, void *dv, float *dg, float *dbeta,
                               float *d_initial_state, const kda_dims_t *dims, void *workspace,
                               size_t workspace_bytes, void *stream) {
    Geometry geo;
    int st = check_backward(dims, cu_seqlens, workspace, workspace_bytes, &geo);
    if (st == KDA_OK)
        st = check_data(geo, {q, k, v, g, beta, d_out, dq, dk, dv, dg, dbeta},
                        {initial_state, d_final_state, d_initial_state});
    if (st != KDA_OK) return st;
    st = kda_backward_records(q, k, g, beta, cu_seqlens, dims, workspace, workspace_bytes, stream);
    if (st == KDA_OK) st = kda_backward_states(v, cu_seqlens, initial_state, dims, workspace, workspace_bytes, stream);
    if (st == KDA_OK)
        st = kda_backward_state_grad(d_out, cu_seqlens, d_final_state, d_initial_state, dims, workspace,
                                     workspace_bytes, stream);
    if (st == KDA_OK)
        st = kda_backward_token_grad(q, k, v, g, beta, d_out, cu_seqlens, dq, dk, dv, dg, dbeta, dims, workspace,
                                     workspace_bytes, stream);
    return st;
}

int kda_check_seqlens(const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t *result,
                      void *stream) {
    if (cu_seqlens == nullptr || result == nullptr) return KDA_ERR_ARG;
    if (num_seqs < 1 || num_seqs > kda::kMaxSeqs || total_tokens < 0 || total_tokens > (int64_t)INT32_MAX)
        return KDA_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0 || (reinterpret_cast<uintptr_t>(result) & 3u) != 0)
        return KDA_ERR_ALIGN;
    return kda::launch_status(
        kda::launch_check_seqlens(cu_seqlens, num_seqs, total_tokens, result, static_cast<hipStream_t>(stream)));
}

const char *kda_status_string(int status) {
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_ARG: return "invalid argument (NULL pointer, bad sizes, or num_seqs != 1 without cu_seqlens)";
    case KDA_ERR_UNSUPPORTED: return "unsupported head size / io dtype combination";
    case KDA_ERR_ALIGN: return "a data pointer is misaligned (16 bytes; 4 for int32 arrays)";
    case KDA_ERR_WORKSPACE: return "workspace missing or smaller than kda_workspace_bytes()";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
    case KDA_ERR_CAPACITY: return "problem larger than kda_chunk_prefill_noalloc's fixed scratch buffer";
    default: return "unknown status";
    }
}

int kda_version(void) { return 200; }

}  // extern "C"
