/*
 * kda.h -- C ABI of the MI355X (gfx950) chunked KDA prefill library (libkda.so).
 *
 * Kimi Delta Attention (KDA) keeps one fixed-size K x V recurrent state per head;
 * every token updates it instead of appending to a key/value cache
 * (akiraxclaw.com "Kimi K3 開源基礎設施：三個專案怎麼分工？", section
 * "FlashKDA：先把 KDA kernel 跑快"; augursoft.site "Kimi K3 的三個系統設計",
 * section "第一個設計"). For token t of a sequence, with alpha_t = exp(g_t):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t.
 *
 * Prefill evaluates this over whole sequences in 16-token chunks with two kernels,
 * one token-parallel over (chunk, head) and one that carries the state from chunk
 * to chunk (augursoft.site "Kimi K3 的三個系統設計", section
 * "為什麼 FlashKDA 選擇 16-token chunks": 16-token chunks, a 16 x 16 matrix
 * inversion, and work split into two kernels by parallelism). The fast path is
 * head dimension K = V = 128 (tech-noisy.com, section
 * "MoE通信とアテンション:MoonEPとFlashKDA", which states that restriction).
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller. The library
 *    allocates and frees no device memory and is reentrant; its only global state
 *    is a per-device cache of the compute-unit and XCD counts and of the kernels'
 *    LDS limits, filled on a device's first launch (thread-safe).
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    default stream) and the call returns without waiting. Buffers must stay
 *    alive until the stream has passed the call.
 *  - Argument checks happen on the host before anything is enqueued; a negative
 *    status means nothing was launched. No C++ exception crosses the ABI.
 *  - Contents of cu_seqlens are not read on the host (they live on the device);
 *    they must satisfy cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = T.
 *
 * Layouts (row-major, contiguous, T = total_tokens over all packed sequences):
 *    q, k     [T, H, K]      io dtype     (q already scaled; the library applies none)
 *    v        [T, H, V]      io dtype
 *    out      [T, H, V]      io dtype     (bf16 results are rounded to nearest even)
 *    g        [T, H, K]      fp32         natural-log per-channel decay, alpha = exp(g)
 *             [T, H]         fp32         with gate_kind = KDA_GATE_SCALAR: one decay per
 *                                         token and head, the same for every channel
 *    beta     [T, H]         fp32
 *    states   [N, H, K, V]   fp32         initial_state (read), final_state (written)
 *    cu_seqlens [N + 1]      int32        sequence boundaries; NULL means one sequence
 * Every data pointer must be 16-byte aligned (cu_seqlens: 4-byte).
 *
 * Gate range. Any finite g <= 0 (a decay, of any strength) gives finite results
 * that are exact up to the kernels' rounding. Inside each 16-token chunk the bf16
 * kernels factor the pairwise decay exp(G_r - G_i) (G the running in-chunk sum of g)
 * around the chunk's 8th token; a chunk in which the running gate of any channel
 * moves more than 72 away from that token's (e.g. per-token g below -9 throughout)
 * is computed pair by pair instead, without factoring, at a higher cost for that
 * chunk alone. The pages say only that the gate range at 16-token chunks suits bf16
 * (augursoft.site "Kimi K3 的三個系統設計", section "為什麼 FlashKDA 選擇
 * 16-token chunks"). g > 0 (growth) is accepted and exact while the true states
 * and outputs stay inside fp32's range. NaN or infinite g are not supported.
 *
 * Size limits (KDA_ERR_ARG beyond them, and kda_workspace_bytes returns 0):
 * 0 <= T <= 2^31 - 1, 1 <= H <= 2^16, 1 <= N <= 2^20 and N * H < 2^25. (The
 * workspace holds a record for every chunk slot a batch may need, (T + 15 N) / 16
 * per head: at N = 2^20 that is already ~15 GB per head.)
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* io dtype of q, k, v and out */
#define KDA_IO_BF16 0
#define KDA_IO_F32 1

/* layout of g. KDA_GATE_SCALAR is the scalar-gated delta rule (Gated DeltaNet), the
 * other chunked delta-rule kernel FlashKDA's benchmark is compared with
 * (tech-noisy.com, section "MoE通信とアテンション:MoonEPとFlashKDA"); it is KDA with
 * g_t broadcast over the K channels, computed by the same kernels. */
#define KDA_GATE_CHANNEL 0 /* g [T, H, K] */
#define KDA_GATE_SCALAR 1  /* g [T, H]    */

/* status codes */
#define KDA_OK 0
#define KDA_ERR_ARG (-1)         /* NULL required pointer, bad sizes, or num_seqs != 1 with NULL cu_seqlens */
#define KDA_ERR_UNSUPPORTED (-2) /* (K, V, io dtype) combination without a kernel */
#define KDA_ERR_ALIGN (-3)       /* a data pointer is not 16-byte aligned */
#define KDA_ERR_WORKSPACE (-4)   /* workspace NULL or smaller than kda_workspace_bytes() */
#define KDA_ERR_LAUNCH (-5)      /* the HIP runtime reported an error at launch */
#define KDA_ERR_CAPACITY (-6)    /* larger than kda_chunk_prefill_noalloc's fixed scratch buffer */

/* Problem sizes. Supported: io bf16 with K = V = 128; io fp32 with K = V in {16, 32, 64, 128}. */
typedef struct kda_dims {
    int64_t total_tokens; /* T >= 0, summed over the packed sequences */
    int32_t num_heads;    /* H >= 1 */
    int32_t head_k;       /* K */
    int32_t head_v;       /* V */
    int32_t num_seqs;     /* N >= 1 */
    int32_t io_dtype;     /* KDA_IO_BF16 or KDA_IO_F32 */
    int32_t gate_kind;    /* KDA_GATE_CHANNEL (0) or KDA_GATE_SCALAR */
} kda_dims_t;

/* Bytes of device workspace kda_chunk_prefill / kda_intra_chunk / kda_inter_chunk need
 * for these sizes, or 0 if the sizes are invalid or unsupported. Host-only. */
size_t kda_workspace_bytes(const kda_dims_t *dims);

/* Whole prefill: chunk table (packed input only), intra-chunk kernel, then the
 * recurrent inter-chunk kernel, all on `stream`.
 *  initial_state NULL: every sequence starts from S = 0.
 *  final_state NULL: final states are not written.
 * Returns KDA_OK or a negative status. */
int kda_chunk_prefill(const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const int32_t *cu_seqlens,
                      const float *initial_state, void *out, float *final_state,
                      const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                      void *stream);

/* First half of kda_chunk_prefill: builds the chunk table (if cu_seqlens is not NULL)
 * and, for every 16-token chunk of every head, the in-chunk gate prefix sums, the
 * 16 x 16 unit lower triangular inverse and the chunk factors, written to
 * `workspace` in the library's own layout (not part of the ABI; read it only
 * through kda_inter_chunk with the same dims and cu_seqlens). */
int kda_intra_chunk(const void *q, const void *k, const float *g, const float *beta,
                    const int32_t *cu_seqlens, const kda_dims_t *dims, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Second half: consumes the workspace written by kda_intra_chunk (same dims, same
 * cu_seqlens, enqueued after it), carries each (sequence, head) state across its
 * chunks, writes out and, if not NULL, final_state. */
int kda_inter_chunk(const void *v, const int32_t *cu_seqlens, const float *initial_state,
                    void *out, float *final_state, const kda_dims_t *dims,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Single-kernel form of kda_chunk_prefill, kept for the ablation that compares it
 * with the two-kernel split (augursoft.site "Kimi K3 的三個系統設計", section
 * "為什麼 FlashKDA 選擇 16-token chunks": FlashKDA's split into a token-parallel and a
 * recurrent kernel beat one fused kernel). One launch; each recurrent workgroup
 * builds the intra-chunk factors of its own head in LDS, so nothing but inputs,
 * outputs and states goes through device memory. Same arguments, layouts, workspace
 * and results as kda_chunk_prefill (bitwise: the same arithmetic in the same order);
 * bf16 io only (KDA_ERR_UNSUPPORTED otherwise). The workspace holds only the chunk
 * table here. */
int kda_chunk_prefill_fused(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const int32_t *cu_seqlens,
                            const float *initial_state, void *out, float *final_state,
                            const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                            void *stream);

/* One decode step (serving): a batch of B sequences, one new token each, updates
 * every (sequence, head) state in place and writes that token's output. A deployment
 * keeps each head's fixed-size state between calls and updates it per token instead
 * of growing a cache (augursoft.site "Kimi K3 的三個系統設計", section
 * "第一個設計：把長上下文從「一直累積」改成「持續更新狀態」"). Per (sequence, head):
 *     S <- Diag(alpha) S,  delta = beta (v - S^T k),  S <- S + k delta^T,  o = S^T q.
 * dims: total_tokens = num_seqs = B (B = 0 does nothing), num_heads = H,
 *       head_k = head_v = 128, io_dtype KDA_IO_BF16 or KDA_IO_F32, gate_kind either.
 * Layouts: q, k [B, H, K] and v, out [B, H, V] in the io dtype; g [B, H, K] or [B, H]
 *          (scalar gate) and beta [B, H] fp32; state [B, H, K, V] fp32, read and
 *          overwritten. The arithmetic is fp32; bf16 out is rounded to nearest even.
 * No workspace. Returns KDA_ERR_ARG (bad sizes, NULL pointer), KDA_ERR_UNSUPPORTED
 * (K or V not 128), KDA_ERR_ALIGN, KDA_ERR_LAUNCH, or KDA_OK. `state` must not alias
 * any other argument. */
int kda_decode_step(const void *q, const void *k, const void *v, const float *g, const float *beta,
                    float *state, void *out, const kda_dims_t *dims, void *stream);

/* Workspace bytes for kda_chunk_prefill_backward with these dims (0 if invalid or
 * unsupported). Larger than the forward's: it also holds every chunk's start state
 * and end-state gradient (bf16, 32 KiB each per (chunk, head)). */
size_t kda_backward_workspace_bytes(const kda_dims_t *dims);

/* Backward of kda_chunk_prefill for training: the gradients of
 *     L = sum_t <d_out_t, out_t> + sum_n <d_final_state_n, S_n>
 * with respect to q, k, v, g, beta and initial_state, for the recurrence the
 * forward computes (S <- Diag(exp(g_t)) S, S <- S + beta_t k_t (v_t - S^T k_t)^T,
 * out_t = S^T q_t). The pages describe only the forward kernel, and say that the
 * released libraries ran Kimi K3's training as well as its inference (tech-noisy.com,
 * section "Moonshot AIが公開した3本のライブラリ"); the gradients here are the plain
 * derivatives of that recurrence, formed
 * chunk by chunk (16 tokens) like the forward: the forward is recomputed to obtain
 * each chunk's start state, a reverse pass over the chunks carries the state
 * gradient, and a token-parallel pass forms the per-token gradients.
 * dims, cu_seqlens, q, k, v, g, beta, initial_state: as kda_chunk_prefill (bf16 io,
 *       K = V = 128 only; KDA_ERR_UNSUPPORTED otherwise).
 * d_out [T, H, V] bf16; d_final_state [N, H, K, V] fp32 or NULL (zero).
 * Outputs (written, never read): dq, dk [T, H, K] and dv [T, H, V] bf16 (rounded to
 *       nearest even); dg fp32 with g's shape ([T, H, K], or [T, H] for a scalar gate:
 *       the sum over the key channels); dbeta [T, H] fp32; d_initial_state
 *       [N, H, K, V] fp32 or NULL (not computed).
 * Arithmetic: fp32 accumulation with bf16 MFMA operands; chunk states and state
 * gradients are held as bf16 between the passes.
 * workspace: device memory of at least kda_backward_workspace_bytes(dims) bytes, owned
 * by the caller; no other call may use it until this one has completed on `stream`.
 * Returns KDA_OK or an error status as kda_chunk_prefill (nothing is enqueued on an
 * argument error). Outputs must not alias inputs or each other. */
int kda_chunk_prefill_backward(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const int32_t *cu_seqlens,
                               const float *initial_state, const void *d_out,
                               const float *d_final_state, void *dq, void *dk, void *dv,
                               float *dg, float *dbeta, float *d_initial_state,
                               const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                               void *stream);


/* The four stages of kda_chunk_prefill_backward as separate calls, for callers that
 * time or schedule them apart. Enqueued in this order on one stream with one
 * workspace (of kda_backward_workspace_bytes) and the same dims and cu_seqlens, they
 * do exactly what kda_chunk_prefill_backward does; arguments, layouts and status
 * codes are that function's.
 *   kda_backward_records: builds the chunk table and each chunk's factors (the
 *       forward record and the backward record) from q, k, g, beta.
 *   kda_backward_states: runs the forward recurrence again from initial_state
 *       and stores every chunk's start state (no output).
 *   kda_backward_state_grad: the reverse pass over the chunks from d_final_state,
 *       storing every chunk's end-state gradient and writing d_initial_state (if
 *       not NULL).
 *   kda_backward_token_grad: dq, dk, dv, dg, dbeta from the stored states.
 * The states and state_grad stages read only what the records stage wrote, not each
 * other's results, so they may run in either order; token_grad needs all three. */
int kda_backward_records(const void *q, const void *k, const float *g, const float *beta,
                         const int32_t *cu_seqlens, const kda_dims_t *dims, void *workspace,
                         size_t workspace_bytes, void *stream);
int kda_backward_states(const void *v, const int32_t *cu_seqlens, const float *initial_state,
                        const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                        void *stream);
int kda_backward_state_grad(const void *d_out, const int32_t *cu_seqlens,
                            const float *d_final_state, float *d_initial_state,
                            const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                            void *stream);
int kda_backward_token_grad(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const void *d_out, const int32_t *cu_seqlens,
                            void *dq, void *dk, void *dv, float *dg, float *dbeta,
                            const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                            void *stream);

/* A forward for training: kda_chunk_prefill that also leaves in a backward
 * workspace what the backward's last two stages read. It writes out and final_state
 * (bitwise equal to kda_chunk_prefill's) and runs the records stage and a recurrence
 * that outputs and saves every chunk's start state in the same pass. The backward of
 * the same inputs is then kda_backward_state_grad followed by
 * kda_backward_token_grad, with the same dims, cu_seqlens and workspace, and gives
 * exactly kda_chunk_prefill_backward's gradients. Skipping its records and states
 * stages is the saving.
 * Arguments: as kda_chunk_prefill (bf16 io, K = V = 128 only), except workspace: at
 * least kda_backward_workspace_bytes(dims) bytes, owned by the caller and left
 * untouched by other calls until the backward stages have run on it. Status codes as
 * kda_chunk_prefill_backward. */
int kda_chunk_prefill_for_backward(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const int32_t *cu_seqlens,
                                   const float *initial_state, void *out, float *final_state,
                                   const kda_dims_t *dims, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* Checks packed-sequence boundaries on the device (the other entry points never read
 * them on the host; their kernels clamp every boundary they read, so malformed ones
 * give wrong numbers, never out-of-range accesses). Sequences are packed back to back
 * as in the variable-length column of the FlashKDA benchmark (tech-noisy.com, section
 * "MoE通信とアテンション:MoonEPとFlashKDA").
 *   cu_seqlens [num_seqs + 1] int32, device, 4-byte aligned
 *   result     one int32, device, 4-byte aligned: written with the smallest n in
 *              [0, num_seqs] at which cu_seqlens[0] = 0, cu_seqlens[n - 1] <=
 *              cu_seqlens[n] or cu_seqlens[num_seqs] = total_tokens fails, else -1.
 * Asynchronous on `stream` like every entry point: read *result after the stream has
 * passed the call. KDA_ERR_ARG for NULL pointers, num_seqs outside [1, 2^20] or
 * total_tokens outside [0, 2^31 - 1]; KDA_ERR_ALIGN for misaligned pointers. */
int kda_check_seqlens(const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t *result,
                      void *stream);

/* Bytes of the device buffer kda_chunk_prefill_noalloc works in (64 MiB). The library
 * holds one on every device it runs on, from the first launch there until the process
 * ends. */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kda_chunk_prefill without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation). Arguments, layouts and results as kda_chunk_prefill, bitwise. The
 * workspace is a fixed buffer of KDA_NOALLOC_SCRATCH_BYTES that the library keeps on
 * each device; this call allocates and frees nothing.
 *  - When kda_workspace_bytes(dims) fits the buffer, the call is one
 *    kda_chunk_prefill.
 *  - A single sequence (num_seqs = 1) that does not fit runs in segments of whole
 *    16-token chunks, carrying the fp32 state between them inside the buffer. With
 *    num_seqs = 1 the boundaries are taken as [0, T) and cu_seqlens is not read.
 *    Each segment is two launches.
 *  - A packed batch that does not fit, or a head count whose two fp32 state carriers
 *    and one chunk's records do not fit, returns KDA_ERR_CAPACITY before anything is
 *    enqueued.
 * Every call on a device uses that device's one buffer and leaves its contents behind
 * (nothing in it needs to start at zero). Calls that overlap on one device, from
 * several streams or host threads, race on it and give wrong results: serialise them. */
int kda_chunk_prefill_noalloc(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const int32_t *cu_seqlens,
                              const float *initial_state, void *out, float *final_state,
                              const kda_dims_t *dims, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
