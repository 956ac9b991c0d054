/*
 * cpla.h -- C ABI of the chunkwise context-parallel linear-attention library
 * (libcpla.so, gfx950 / MI355X).
 *
 * The calls follow the local-backend protocol of the Megatron-Core API page
 * "core.ssm.context_parallel.chunkwise" (class LinearAttentionCPBackend):
 *   cp_forward_prepare   - the state summary of each contiguous shard with zero
 *                          incoming state (S_out = M S_in + delta_S);
 *   cp_forward_apply     - compose the preceding summaries, then compute the
 *                          local output;
 *   cp_backward_prepare  - gamma of each shard with zero outgoing-state gradient
 *                          (dS_in = M^T dS_out + gamma);
 *   cp_backward_apply    - compose the reverse-causal suffix, then finish the
 *                          local input gradients;
 * plus build_packed_sequence_cp_metadata (same page, function of that name and
 * class PackedSequenceCPMetadata).
 *
 * On one GPU the CP "ranks" are P contiguous segments of the same sequence in
 * the same HBM; one call handles the shards [rank_begin, rank_end) of every
 * (b, h) row. The library performs no communication.
 *
 * Method (per (b, h) row; g is the log-decay, a_t = exp(g_t)):
 *   S_t = diag(a_t) S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t,  S_{-1} = S_init,
 *   and S_{t-1} := 0 where token t starts a packed sequence.
 *
 * Conventions shared by every call
 *   - Every pointer is caller-owned. Device pointers point to HBM; the library
 *     calls no allocator (the one buffer of its own is the static scratch array
 *     of cp_forward_apply_noalloc), keeps no caller pointer after returning, and
 *     enqueues all device work on `stream` without synchronising the host
 *     (cpla_check_decay_range, which returns a count, synchronises `stream`).
 *   - Tensors are dense row-major with the last index fastest:
 *       q, k      [B, T, H, dk]   dtype (bf16 or fp32)
 *       v, o, dO  [B, T, H, dv]   dtype
 *       g, dg     scalar decay [B, T, H] fp32; diagonal decay [B, T, H, dk]
 *                 fp32; no decay: NULL. g <= 0 (log of a decay in (0, 1]).
 *                 Diagonal decay: within every 64-token chunk the running
 *                 sum of g per key dim must stay at or above
 *                 CPLA_DIAG_GAMMA_MIN = -80 (the kernels factor the decay into
 *                 exp(+-sum), which must stay finite in fp32), i.e. an average
 *                 of -1.25 per token over a whole chunk; stronger decays are
 *                 outside the supported range, and cpla_check_decay_range
 *                 reports them (the calls themselves do not read g on the host).
 *       states    [B, H, dk, dv] fp32 (S_init, final state and their grads)
 *       summaries [P, B, H, W] fp32, W = cpla_summary_width(): the first
 *                 m_slot entries hold the transition M (dk values for a
 *                 diagonal decay, else one value followed by 3 zero pads),
 *                 then dk*dv entries hold delta_S (or gamma), row = key dim.
 *                 M is 0 for a shard that contains a packed-sequence start.
 *       per-shard states [P, B, H, dk, dv] fp32
 *       chunk states [B, H, n_chunks, dk, dv] fp32: the state entering every
 *                 64-token chunk of every shard, the shards' chunks in order
 *                 (n_chunks = sum over shards of ceil(shard length / 64));
 *                 saved by the forward for the backward
 *   - Shard r covers tokens [r*L, min((r+1)*L, T)) of every row, L = ceil(T/P)
 *     (torch.chunk's division: the last non-empty shard may be shorter and
 *     trailing shards empty).
 *   - Alignment: every device pointer 16-byte aligned.
 *   - Validation happens on the host before any launch. On failure a call
 *     returns a non-zero cpla_status, launches nothing, and sets a message
 *     readable through cpla_last_error(). Kernel launch failures return
 *     CPLA_E_HIP. Device kernels trust packed metadata produced by
 *     build_packed_sequence_cp_metadata / cpla_packed_rank_slices.
 */
#ifndef CPLA_H
#define CPLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#define CPLA_ABI_VERSION 6

/* Largest cpla_problem.num_shards the calls accept. */
#define CPLA_MAX_SHARDS 1024

/* Lower bound of the running log-decay within a 64-token chunk, per key dim, that
 * the diagonal-decay kernels support (see the layout notes above). */
#define CPLA_DIAG_GAMMA_MIN (-80.0f)

typedef enum {
  CPLA_OK = 0,
  CPLA_E_INVALID = 1,      /* null pointer where one is required, bad enum  */
  CPLA_E_SHAPE = 2,        /* sizes not positive or inconsistent            */
  CPLA_E_DTYPE = 3,        /* unknown dtype                                  */
  CPLA_E_ALIGN = 4,        /* a pointer is not 16-byte aligned               */
  CPLA_E_UNSUPPORTED = 5,  /* valid request this build does not implement   */
  CPLA_E_METADATA = 6,     /* malformed packed-sequence metadata             */
  CPLA_E_HIP = 7           /* a HIP launch or runtime call failed            */
} cpla_status;

typedef enum { CPLA_F32 = 0, CPLA_BF16 = 1 } cpla_dtype;
typedef enum { CPLA_DECAY_NONE = 0, CPLA_DECAY_SCALAR = 1, CPLA_DECAY_DIAG = 2,
               CPLA_DECAY_DELTA = 3 /* gated delta rule: the _delta calls below */ } cpla_decay;

typedef struct {
  int64_t B, T, H, dk, dv;   /* packed sequences: each of the B rows is a stream of T
                                tokens with its own packing. Head dims: dk == dv in
                                {16, 64, 128} (bf16) or {16, 64} (fp32); dk != dv:
                                bf16 (64, 128) or (128, 64); others CPLA_E_UNSUPPORTED */
  int32_t num_shards;        /* P <= 1024 shards of any T: torch.chunk's division (shard
                                size ceil(T/P), the last non-empty shard shorter, trailing
                                shards empty when T is short; a shard's last chunk may be
                                partial), the graceful division the mixle page relies on */
  int32_t chunk;             /* chunk length C; this build supports 64 only            */
  int32_t rank_begin;        /* shards handled by this call: [rank_begin, rank_end)    */
  int32_t rank_end;          /*   (0 and P on one GPU)                                  */
  int32_t dtype;             /* cpla_dtype of q, k, v, o, dO, dq, dk, dv                */
  int32_t decay;             /* cpla_decay                                              */
  int32_t qk_heads;          /* heads of q and k: 0 (or H) = one per head; G with
                                H % G == 0 = q and k are [B,T,G,dk] and head h reads
                                their head h / (H / G) (Mamba2's B and C, shared by a
                                group of heads). dq and dk stay per head [B,T,H,dk]
                                (a group's sum is the gradient of the shared tensor).
                                Scalar decay only (the others and the _delta calls take
                                0 or H)                                                */
} cpla_problem;

/* Packed sequences. Passing NULL for the whole struct means "not packed": every
 * row is one sequence that starts from S_init, the forward prefix of rank r is
 * [0, r) and the backward suffix is (r, P). Device pointers, row-major with one
 * row per batch row b: each row is packed on its own (B == 1 is the usual
 * single packed stream), and its slices are those cpla_packed_rank_slices gives
 * for that row's ids. */
typedef struct {
  const int32_t* seq_idx;               /* [B, T] global sequence id of each token in
                                           its row (>= 0, as cpla_seq_idx_from_cu_seqlens
                                           writes)                                       */
  const int32_t* preceding_rank_start;  /* [B, P] inclusive start of rank r's prefix   */
  const int32_t* following_rank_stop;   /* [B, P] exclusive end of rank r's suffix     */
} cpla_packed;

/* Floats per (shard, b, h) summary record: m_slot + dk*dv (see layout above). */
int64_t cpla_summary_width(const cpla_problem* p);

/* Bytes of the chunk-state buffer the forward saves for the backward: one fp32
 * dk x dv state per (b, h) and per 64-token chunk of every shard, the shards'
 * chunks in order ([B,H,n_chunks,dk,dv]). -1 for an invalid problem. */
int64_t cpla_chunk_states_bytes(const cpla_problem* p);

/* cp_forward_prepare: for every handled shard, run the shard from a zero state
 * and write its map (M, delta_S) to fwd_summary[r]. With packed sequences the
 * summary covers the shard's last sequence segment. Reads k, v, g. */
cpla_status cp_forward_prepare(const cpla_problem* p, const cpla_packed* packed,
                               const void* k, const void* v, const float* g,
                               float* fwd_summary, hipStream_t stream);

/* cp_forward_apply: compose the summaries of the preceding shards (the prefix
 * [preceding_rank_start, r), started from initial_state when it starts at rank 0,
 * else from zero) into shard_in_state[r], then run every handled shard from its
 * incoming state and write o. final_state (nullable) receives the state after
 * the last shard. chunk_states (nullable) receives the state entering every
 * chunk; it is required later by cp_backward_apply. initial_state must be NULL
 * with packed sequences. */
cpla_status cp_forward_apply(const cpla_problem* p, const cpla_packed* packed,
                             const void* q, const void* k, const void* v, const float* g,
                             const float* fwd_summary, const float* initial_state,
                             void* o, float* shard_in_state, float* final_state,
                             void* chunk_states, hipStream_t stream);

/* cp_forward_apply_noalloc: cp_forward_apply for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). It computes exactly what cp_forward_apply computes,
 * with the same kernels (same bits in o, final_state and chunk_states), but the
 * composed incoming state of every shard -- the shard_in_state buffer that
 * cp_forward_apply takes from the caller -- lives in a scratch array inside the
 * library: one per GPU, cpla_noalloc_scratch_bytes() (32 MiB) in size, allocated
 * when the library's code is loaded on that GPU and held until the process ends.
 * The call itself allocates and frees nothing. It rejects with
 * CPLA_E_UNSUPPORTED (launching nothing) a problem whose composed states need
 * more: P * B * H * dk * dv * 4 bytes (the diagonal-decay workload B=4 H=16
 * d=128 with 8 shards needs exactly 32 MiB). Every call on one GPU shares that
 * GPU's scratch: calls that may overlap on one GPU (several streams, several
 * host threads) race and must be serialised by the caller; the composed states
 * are not returned (use cp_forward_apply to keep them). Other arguments, errors
 * and ordering on `stream` as for cp_forward_apply. */
cpla_status cp_forward_apply_noalloc(const cpla_problem* p, const cpla_packed* packed,
                                     const void* q, const void* k, const void* v, const float* g,
                                     const float* fwd_summary, const float* initial_state,
                                     void* o, float* final_state, void* chunk_states,
                                     hipStream_t stream);

/* cpla_check_decay_range: opt-in validation of a diagonal log-decay g against
 * the supported range (the layout notes above): counts, over the chunks of the
 * handled shards [rank_begin, rank_end), the (chunk, key dim) pairs whose running
 * sum of g from the chunk's first token falls below CPLA_DIAG_GAMMA_MIN (or is
 * NaN), and returns CPLA_E_INVALID with that count in cpla_last_error() if any
 * does. `count` is a caller-owned device int32 (16-byte aligned) the call
 * overwrites. Unlike the other calls it synchronises `stream` (it reads the count
 * back), so it is meant for debugging and input validation, not for the hot
 * path. For no decay or a scalar decay (applied without a factorisation) it
 * returns CPLA_OK without launching anything. */
cpla_status cpla_check_decay_range(const cpla_problem* p, const float* g, int32_t* count,
                                   hipStream_t stream);

/* Size in bytes of the per-GPU scratch of cp_forward_apply_noalloc. */
int64_t cpla_noalloc_scratch_bytes(void);

/* cp_backward_prepare: for every handled shard, the gradient w.r.t. its
 * incoming state when no gradient arrives at its end (gamma), and its
 * transition, into bwd_summary[r]. With packed sequences it covers the shard's
 * first sequence segment. Reads q, g, dO. */
cpla_status cp_backward_prepare(const cpla_problem* p, const cpla_packed* packed,
                                const void* q, const float* g, const void* dO,
                                float* bwd_summary, hipStream_t stream);

/* cp_backward_apply: compose the reverse-causal suffix (r, following_rank_stop)
 * of backward summaries, started from d_final_state (nullable = zero; must be
 * NULL with packed sequences) when it reaches the last rank, into
 * shard_out_grad[r]; then walk every handled shard backwards from it and write
 * dq, dk, dv and dg (fp32, like g; NULL iff no decay). d_initial_state
 * (nullable, unpacked only) receives the gradient w.r.t. S_init. chunk_states
 * is the buffer cp_forward_apply filled. */
cpla_status cp_backward_apply(const cpla_problem* p, const cpla_packed* packed,
                              const void* q, const void* k, const void* v, const float* g,
                              const void* dO, const void* chunk_states,
                              const float* bwd_summary, const float* d_final_state,
                              void* dq, void* dk, void* dv, float* dg,
                              float* shard_out_grad, float* d_initial_state,
                              hipStream_t stream);

/* Weighted variants (scalar decay only): each token's input k_t v_t^T enters the
 * state weighted by w_t > 0, w [B,T,H] fp32 (device; NULL = 1):
 *   S_t = exp(g_t) S_{t-1} + w_t k_t v_t^T.
 * The weight is applied in fp32 inside the walks (in the score tile and the
 * tail factor of the state update), never folded into the bf16 k or v. With w,
 * cp_backward_apply_weighted also writes dw [B,T,H] fp32 (nullable): dw_t =
 * k_t^T dS_t v_t, formed as (dv_t . v_t) / w_t from dv in fp32 before its
 * rounding. cp_backward_prepare does not depend on w. Mamba2's dt is such a
 * weight (see the SSD calls below). grad_dtype is the cpla_dtype of dq, dk, dv:
 * the input dtype, or CPLA_F32 with bf16 inputs and a scalar decay (gradients a
 * caller sums further before rounding). Errors as for the unweighted calls; a
 * weight with another decay is CPLA_E_INVALID, another grad_dtype
 * CPLA_E_DTYPE. */
cpla_status cp_forward_prepare_weighted(const cpla_problem* p, const cpla_packed* packed,
                                        const void* k, const void* v, const float* g, const float* w,
                                        float* fwd_summary, hipStream_t stream);
cpla_status cp_forward_apply_weighted(const cpla_problem* p, const cpla_packed* packed,
                                      const void* q, const void* k, const void* v, const float* g,
                                      const float* w, const float* fwd_summary,
                                      const float* initial_state, void* o, float* shard_in_state,
                                      float* final_state, void* chunk_states, hipStream_t stream);
cpla_status cp_backward_apply_weighted(const cpla_problem* p, const cpla_packed* packed,
                                       const void* q, const void* k, const void* v, const float* g,
                                       const float* w, const void* dO, const void* chunk_states,
                                       const float* bwd_summary, const float* d_final_state,
                                       void* dq, void* dk, void* dv, float* dg, float* dw,
                                       float* shard_out_grad, float* d_initial_state,
                                       int32_t grad_dtype, hipStream_t stream);

/* build_packed_sequence_cp_metadata (host memory, pure, thread-safe): rank-local
 * packed metadata from the global per-token sequence ids (length T, starting at
 * 0, each step 0 or 1), the rank's shard being torch.chunk's slice (see
 * cpla_problem.num_shards; L = its length, at most ceil(T/cp_size)).
 * local_seq_idx [L] receives the rank's ids rebased to start at 0;
 * local_cu_seqlens (capacity L + 1) receives 0, each interior id
 * change and L, and *num_local_seqs its number of sequences; *preceding_rank_start
 * is the rank holding the first token of the sequence live at the rank's first
 * token, *following_rank_stop one past the rank holding the last token of the
 * sequence live at its last token. An empty shard gets local_cu_seqlens {0},
 * no sequences and the slice [r, r + 1) (it composes nothing). Malformed ids
 * return CPLA_E_METADATA. */
cpla_status build_packed_sequence_cp_metadata(const int32_t* global_seq_idx, int64_t T,
                                              int32_t cp_rank, int32_t cp_size,
                                              int32_t* local_seq_idx, int32_t* local_cu_seqlens,
                                              int32_t* num_local_seqs,
                                              int32_t* preceding_rank_start,
                                              int32_t* following_rank_stop);

/* preceding_rank_start and following_rank_stop of every rank at once (host). */
cpla_status cpla_packed_rank_slices(const int32_t* global_seq_idx, int64_t T, int32_t cp_size,
                                    int32_t* preceding_rank_start, int32_t* following_rank_stop);

/* Sequence id of every token from cu_seqlens [n_seqs + 1] (host): strictly
 * increasing, 0 first, T last. */
cpla_status cpla_seq_idx_from_cu_seqlens(const int32_t* cu_seqlens, int32_t n_seqs, int64_t T,
                                         int32_t* seq_idx);

/* ---- The gated delta rule: a dense state transition -------------------------------
 * The Megatron-Core page core.ssm.context_parallel.chunkwise states the shard maps
 * for a general transition M (classes CPForward*Summary: S_out = M S_in + delta_S;
 * CPBackward*Summary: dS_in = M^T dS_out + gamma), and the axolotl-ringmaster
 * README (Status table) validates gated-DeltaNet linear attention on that state
 * passing. Here the recurrence is
 *   S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  a_t = exp(g_t),
 *   o_t = S_t^T q_t,  S_{t-1} := 0 where token t starts a packed sequence,
 * so M is a full d_k x d_k matrix (zero for a shard holding a start) and the
 * composition multiplies matrices (M^T backwards). Problem: decay =
 * CPLA_DECAY_DELTA, dk == dv in {16, 32, 64} (fp32 or bf16) or 128 (bf16); g and beta
 * [B,T,H] fp32 (beta is the write strength, usually in (0, 1); keys are usually
 * L2-normalised by the caller, and q carries any scale). Summary records
 * (cpla_summary_width = dk*dk + dk*dv floats): [M (dk x dk, row-major) | delta_S
 * (forward) or gamma (backward) (dk x dv)]. The four calls follow the protocol of
 * the calls above; their local context lives in a caller-owned workspace of
 * cpla_delta_workspace_bytes() bytes (16-byte aligned), which must be the same
 * buffer, unchanged, across the four calls of one step: forward prepare fills the
 * per-chunk solves, forward apply the chunk states, backward prepare reads them,
 * backward apply writes the chunk-end gradients. Packing, rank ranges and error
 * behaviour as for the calls above; the gradients dg and dbeta are fp32 [B,T,H],
 * dq, dk, dv in the input dtype. */
int64_t cpla_delta_workspace_bytes(const cpla_problem* p);   /* -1 for an invalid problem */

cpla_status cp_forward_prepare_delta(const cpla_problem* p, const cpla_packed* packed, const void* k,
                                     const void* v, const float* g, const float* beta, float* fwd_summary,
                                     void* workspace, hipStream_t stream);
cpla_status cp_forward_apply_delta(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                   const void* k, const void* v, const float* g, const float* beta,
                                   const float* fwd_summary, const float* initial_state, void* o,
                                   float* shard_in_state, float* final_state, void* workspace,
                                   hipStream_t stream);
cpla_status cp_backward_prepare_delta(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                      const void* k, const float* g, const float* beta, const void* dO,
                                      const float* fwd_summary, float* bwd_summary, void* workspace,
                                      hipStream_t stream);
cpla_status cp_backward_apply_delta(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                    const void* k, const void* v, const float* g, const float* beta,
                                    const void* dO, const float* bwd_summary, const float* d_final_state,
                                    void* dq, void* dk, void* dv, float* dg, float* dbeta, float* shard_out_grad,
                                    float* d_initial_state, void* workspace, hipStream_t stream);

/* ---- Mamba2 (SSD) parametrisation of the scalar-decay path ------------------------
 * The axolotl-ringmaster README (Status table, Layout) runs Mamba2 SSM context
 * parallelism through the same exact CP linear scan as linear attention. Mamba2's
 * selective state space, for head h of group gr = h / (H / G):
 *   h_t = exp(dt_t A_h) h_{t-1} + dt_t B_t x_t^T   (state N x P),   y_t = h_t^T C_t
 * is the weighted scalar-decay recurrence above with q = C[gr], k = B[gr], v = x,
 * g = A dt and w = dt: run cpla_ssd_inputs, the weighted cp_* calls (and
 * cp_backward_prepare) with q = C, k = B, qk_heads = G, v = x and w = dt, then
 * cpla_ssd_input_grads (run with per-head copies q, k and qk_heads = 0 instead,
 * they give the same results).
 * Shapes: x and y [B,T,H,P], B, C [B,T,G,N] in `dtype` (copies q, k [B,T,H,N]); dt, g
 * [B,T,H] and A [H] fp32 (dt already positive: any softplus or bias is the
 * caller's); the state is N x P per head, so the cp_* calls run with dk = N and
 * dv = P (bf16: N = P in {16, 64, 128} or (N, P) = (64, 128), (128, 64); fp32:
 * N = P in {16, 64}; other pairs are rejected by those calls). All pointers
 * are device memory owned by the caller, 16-byte aligned; work is enqueued on
 * `stream`; invalid arguments return an error and launch nothing. */
typedef struct {
  int64_t B, T, H;           /* batch, tokens, heads                                   */
  int64_t G;                 /* groups sharing B and C: H % G == 0                     */
  int64_t N;                 /* state size (B, C, q, k): a multiple of 4, N/4 a power
                                of two up to 64                                       */
  int64_t P;                 /* head dim (x, y): a multiple of 4, at most 256         */
  int32_t dtype;             /* cpla_dtype of x, B, C, q, k, dx, dB, dC                */
} cpla_ssd_problem;

/* g = A dt (fp32), and, when q and k are both non-NULL, per-head copies
 * q[b,t,h] = C[b,t,gr], k[b,t,h] = B[b,t,gr]. With both NULL the cp_* calls read B
 * and C in place: pass k = B, q = C and cpla_problem.qk_heads = G. */
cpla_status cpla_ssd_inputs(const cpla_ssd_problem* p, const float* dt, const float* A,
                            const void* B, const void* C, void* q, void* k, float* g,
                            hipStream_t stream);

/* The chain rule from the gradients of cp_backward_apply_weighted, run with
 * grad_dtype CPLA_F32 (dq, dk, dv, dg, dw all fp32), to the Mamba2 inputs:
 * dx = dv (dtype [B,T,H,P]), d_dt = dw + A dg (fp32 [B,T,H]), dA = sum over
 * (b, t) of dt dg (fp32 [H], summed in a fixed order: the same on every run),
 * dB = sum over the group's heads of dk and dC of dq (dtype [B,T,G,N], summed in
 * fp32 and rounded once). */
cpla_status cpla_ssd_input_grads(const cpla_ssd_problem* p, const float* dt, const float* A,
                                 const float* dq, const float* dk, const float* dv, const float* dg,
                                 const float* dw, void* dx, float* d_dt, float* dA, void* dB, void* dC,
                                 hipStream_t stream);

/* Message of the last failure on the calling thread; valid until its next call. */
const char* cpla_last_error(void);

int cpla_abi_version(void);

/* Testing aid for the divided apply walks (no decay or a scalar decay): on grids
 * too small to fill the GPU, cp_forward_apply and cp_backward_apply divide each
 * shard's walk among up to four workgroups, each replaying the state (or adjoint)
 * up to its own chunks, which gives the bits of the undivided walk. parts = 1, 2
 * or 4 forces that division (halved until every part holds a chunk), 0 restores
 * the automatic choice. Process-wide; returns the previous setting, or -1 (and
 * changes nothing) for any other value. */
int cpla_set_apply_parts(int parts);

#ifdef __cplusplus
}
#endif

#endif /* CPLA_H */
