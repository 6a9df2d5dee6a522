/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) core.
 *
 * KDA is a gated delta rule with per-channel diagonal decay. For every
 * (sequence, head) the recurrent state S (Dk x Dv, fp32) evolves per token t as
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,              alpha_t = exp(g_t)  (g_t <= 0, per key channel)
 *
 * Sources: the delta rule as one correction step on the L2 value-retrieval
 * error and KDA's diagonal (per-channel) forgetting factor are described in the
 * Kimi K3 report (xxquant, English and Chinese editions), "Methodology notes"
 * (DeltaNet and Delta Rule; Kimi Delta Attention) and in the SemiAnalysis
 * Kimi K3 digest, section 1 (KDA). The same pages describe the prefill as a
 * chunked rewrite with two kernels -- tensor preparation (decayed queries and
 * keys, an inverse "UT" transform, causal matrices) and a blockwise recurrence
 * (pseudo-values, outputs, updated state) -- and the decode step as constant
 * cost, about 7*D^2 FLOPs and 8*D^2 bytes of fp32 state traffic per head and
 * token (report, "Key data").
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains caller memory. Scratch memory
 *     is passed in through `workspace` (size from kda_prefill_workspace_size),
 *     except for kda_prefill_chunked_noalloc, which uses a fixed array the
 *     library holds on each device instead.
 *   - All work is enqueued asynchronously on `stream` (0 = the null stream);
 *     no entry point synchronises. Results are visible after the caller
 *     synchronises the stream. Only kernels are enqueued (no allocation,
 *     memset or copy), so calls may be captured in a HIP graph.
 *   - Layouts are dense row-major (C order) with the last index contiguous:
 *       q, k  [tokens, H, Dk]     v, o  [tokens, H, Dv]
 *       g     [tokens, H, Dk]     beta  [tokens, H]
 *       state [seqs, H, Dk, Dv]   (row i = key channel, column j = value channel)
 *   - q, k, v are fp32 (KDA_F32) or bf16 (KDA_BF16, raw 16-bit patterns);
 *     g, beta, states and o are always fp32.
 *   - q and k are expected to be L2-normalised per (token, head) by the
 *     caller; the library uses them as given and applies no attention scale.
 *     The *_ex entry points can instead apply KDA's parameter-free input
 *     transforms themselves (KDA_FRONT_* below).
 *   - Tensor pointers must be 16-byte aligned; workspace 256-byte aligned.
 *   - Arguments are validated on the host BEFORE any HIP call. On any error
 *     nothing is enqueued and no output is touched, except KDA_ERR_HIP, which
 *     reports a failed launch (outputs then undefined).
 *   - Device-side preconditions that are documented but not checked (their
 *     violation gives unspecified results, never an out-of-bounds access,
 *     because sequence ranges are clamped to [0, total_tokens) on the device):
 *     cu_seqlens non-decreasing with cu_seqlens[num_seqs] == total_tokens;
 *     g <= 0, where any such value is valid, -inf (alpha = 0) included; every
 *     other input finite. With bf16 q/k/v the matrix-core operands are fp16,
 *     so every element of v, of the states (the initial state and the state
 *     at each 64-token chunk boundary) and of the pseudo-values
 *     U = Ainv diag(beta) (V - K_decayed S) must have magnitude below 65504.
 *   - Decay range: every decay factor the prefill forms stays inside its
 *     operand type's range: inside a 16-token block, channels that decay by
 *     less than 2^12 (bf16 q/k/v; 2^60 with fp32) over the block share one
 *     reference row there (factors up to that bound), and every other factor
 *     is at most 1, so KDA's per-channel forgetting is handled down to
 *     alpha = 0 in any channel. It floors the per-token log-decay at -16 nats
 *     with bf16 q/k/v and at -64 nats with fp32 q/k/v (alpha >= 1.1e-7 resp.
 *     1.6e-28): each state column moves by at most that fraction of its
 *     norm, and later steps never enlarge the difference, so results change
 *     by about 1e-7 of the state's magnitude. The decode step applies exp(g)
 *     as given.
 *   - The library keeps no global state besides the loaded code object, the
 *     device attributes it caches per device on first use, and the scratch
 *     array of kda_prefill_chunked_noalloc. It is reentrant; calls on
 *     different streams may run concurrently if they write disjoint outputs
 *     and workspaces (calls of kda_prefill_chunked_noalloc on one device
 *     share its array and must not overlap).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,  /* NULL required pointer, bad size, misalignment  */
    KDA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dims, chunk size)   */
    KDA_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than required        */
    KDA_ERR_HIP = 4           /* a HIP launch or runtime call failed            */
} kda_status_t;

typedef enum kda_dtype {
    KDA_F32 = 0,              /* q, k, v in fp32                                 */
    KDA_BF16 = 1              /* q, k, v in bf16                                 */
} kda_dtype_t;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int kda_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *kda_status_string(kda_status_t status);

/*
 * Bytes of device workspace kda_prefill_chunked needs for these sizes.
 * Returns 0 when the sizes are invalid or unsupported (the same checks as
 * kda_prefill_chunked). The size depends only on the arguments. It includes
 * the buffers of the chunk-parallel scan when that scan applies to these
 * sizes (kda_prefill_scan_segments); a smaller workspace that still holds the
 * plain path's buffers is accepted and runs the plain scan. An allocation of
 * this size is valid for every call with the same or smaller sizes.
 */
size_t kda_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                  int32_t Dk, int32_t Dv, int32_t chunk_size,
                                  kda_dtype_t in_dtype);

/*
 * Segments of the chunk-parallel scan that kda_prefill_chunked (and the _ex
 * variant) uses for these sizes on the current device, given a workspace of
 * kda_prefill_workspace_size(...) bytes; 1 = the plain scan.
 *
 * The blockwise recurrence is sequential over chunks, and one sequence with
 * few heads gives it too few (head, 16-column) blocks to fill the device.
 * Each chunk step is an affine map of the state (the chunk algebra behind the
 * report's FlashKDA note, "Methodology notes"), so the library then cuts the
 * sequence into P segments of whole chunks, scans them all at once (once for
 * the values, once from the identity to get each segment's linear map),
 * chains the segment end states in fp32 and adds each segment's start-state
 * term to its outputs. Used only with cu_seqlens == NULL (one sequence), both
 * phases in one call, no checkpoints and no positions, and only when the
 * workspace holds the extra buffers (the plain path runs otherwise, with
 * identical semantics). Host-only query (reads the device's CU count); 0 for
 * invalid sizes.
 */
int32_t kda_prefill_scan_segments(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                  int32_t Dk, int32_t Dv, int32_t chunk_size,
                                  kda_dtype_t in_dtype);

/*
 * Chunked KDA prefill over one or more packed sequences.
 *
 * Computes, for every sequence s, head h and token t of s, o_t = S_t^T q_t of
 * the recurrence above, starting from initial_state[s, h] (zeros if NULL), and
 * optionally the state after the last token (final_state) and after every
 * ckpt_interval tokens of each sequence (ckpt_states).
 *
 *   q, k, v, in_dtype  inputs as in the layout conventions ([total_tokens, H, D])
 *   g                  [total_tokens, H, Dk] fp32 log-decay (alpha = exp(g))
 *   beta               [total_tokens, H] fp32 write strengths
 *   cu_seqlens         device int32 [num_seqs + 1]: sequence s owns tokens
 *                      cu_seqlens[s] .. cu_seqlens[s+1]-1; cu_seqlens[0] = 0.
 *                      NULL means one sequence of total_tokens (num_seqs must
 *                      be 1). Zero-length sequences are allowed: their final
 *                      state equals their initial state.
 *   num_seqs, total_tokens, H, Dk, Dv   sizes; Dk, Dv in {64, 128};
 *                      H * max(Dk, Dv) * 64 <= 2^31 - 1 (else KDA_ERR_UNSUPPORTED)
 *   chunk_size         must be 64
 *   initial_state      [num_seqs, H, Dk, Dv] fp32 or NULL (zeros)
 *   final_state        [num_seqs, H, Dk, Dv] fp32 or NULL (not written)
 *   ckpt_interval      0 = no checkpoints; otherwise a positive multiple of
 *                      chunk_size. Checkpoint m (m = 1, 2, ...) of sequence s
 *                      is the state after its first m*ckpt_interval tokens.
 *   ckpt_states        [ckpt_rows, H, Dk, Dv] fp32; required iff
 *                      ckpt_interval > 0. Row c = base_s + m - 1 holds
 *                      checkpoint m of sequence s, base_s = sum over earlier
 *                      sequences of floor(L / ckpt_interval).
 *   ckpt_rows          rows available in ckpt_states (the caller knows the
 *                      lengths; the library does not read them on the host).
 *                      Checkpoints whose row would be >= ckpt_rows are not
 *                      written.
 *   o                  [total_tokens, H, Dv] fp32 output
 *   workspace          device scratch of at least
 *                      kda_prefill_workspace_size(...) bytes, 256-byte aligned;
 *                      its contents need no initialisation and are garbage
 *                      afterwards. It must not be shared by concurrent calls.
 *   stream             HIP stream the kernels are enqueued on
 *
 * Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE
 * (validated before any launch) or KDA_ERR_HIP (launch failure).
 * total_tokens == 0 is valid: only final_state (= initial state) is written.
 */
kda_status_t kda_prefill_chunked(
    const void *q, const void *k, const void *v, kda_dtype_t in_dtype,
    const float *g, const float *beta, const int32_t *cu_seqlens,
    int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
    int32_t chunk_size, const float *initial_state, float *final_state,
    int64_t ckpt_interval, float *ckpt_states, int64_t ckpt_rows, float *o,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Phases of the chunked prefill (bit mask for kda_prefill_chunked_phases). */
#define KDA_PHASE_PREPARE 1u  /* chunk tensor preparation: writes the workspace   */
#define KDA_PHASE_SCAN 2u     /* blockwise recurrence: reads the workspace, writes
                                 o and the states                                 */

/*
 * kda_prefill_chunked split into its two phases. Same arguments and
 * validation as kda_prefill_chunked, plus `phases`, a non-zero subset of
 * KDA_PHASE_PREPARE | KDA_PHASE_SCAN (both = kda_prefill_chunked).
 * PREPARE reads q, k, g, beta and cu_seqlens and fills the workspace; SCAN
 * reads v, cu_seqlens, initial_state and that workspace and writes o,
 * final_state and ckpt_states. A SCAN-only call must follow a PREPARE of the
 * same inputs into the same workspace, ordered before it (same stream, or an
 * event); the library does not check this. Lets a caller time the phases or
 * overlap the preparation of one batch with the scan of another on a second
 * stream (each batch with its own workspace).
 */
kda_status_t kda_prefill_chunked_phases(
    const void *q, const void *k, const void *v, kda_dtype_t in_dtype,
    const float *g, const float *beta, const int32_t *cu_seqlens,
    int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
    int32_t chunk_size, const float *initial_state, float *final_state,
    int64_t ckpt_interval, float *ckpt_states, int64_t ckpt_rows, float *o,
    void *workspace, size_t workspace_bytes, uint32_t phases, hipStream_t stream);

/*
 * Parameter-free input transforms applied inside the kernels: bit mask
 * `frontend` of kda_prefill_chunked_ex and kda_decode_step_ex. KDA normalises
 * queries and keys to unit L2 norm and drives its per-channel decay through a
 * gate (Kimi K3 report, "Methodology notes", Kimi Delta Attention bullet);
 * the pages give no formulas, and these are the library's reading:
 *   KDA_FRONT_L2NORM_QK     every q and k row (one token, one head) is scaled
 *                           by 1 / sqrt(sum_c x_c^2 + 1e-6), in fp32, where it
 *                           enters the computation (a zero row stays zero)
 *   KDA_FRONT_GATE          g holds u; the log-decay used is -exp(u)
 *   KDA_FRONT_BETA_SIGMOID  beta holds logits b; the write strength used is
 *                           1 / (1 + exp(-b))
 * Tensors keep their shapes, dtypes and layouts, and are only read. The
 * weighted parts of KDA's input path (short convolution, low-rank gate
 * projection, output gate) are the caller's.
 */
#define KDA_FRONT_L2NORM_QK 1u
#define KDA_FRONT_GATE 2u
#define KDA_FRONT_BETA_SIGMOID 4u

/*
 * kda_prefill_chunked_phases with a `frontend` mask (a subset of the
 * KDA_FRONT_* bits; 0 = kda_prefill_chunked_phases). The transforms act in
 * the PREPARE phase, the only one that reads q, k, g and beta here; a
 * SCAN-only call ignores them. The decay floor then applies to -exp(u)
 * (u = +inf gives alpha = 0). Returns KDA_ERR_INVALID_ARG for unknown bits,
 * otherwise as kda_prefill_chunked_phases.
 */
kda_status_t kda_prefill_chunked_ex(
    const void *q, const void *k, const void *v, kda_dtype_t in_dtype,
    const float *g, const float *beta, const int32_t *cu_seqlens,
    int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
    int32_t chunk_size, const float *initial_state, float *final_state,
    int64_t ckpt_interval, float *ckpt_states, int64_t ckpt_rows, float *o,
    void *workspace, size_t workspace_bytes, uint32_t phases, uint32_t frontend,
    hipStream_t stream);

/*
 * kda_prefill_chunked_ex that also returns states at arbitrary positions,
 * for example prompt boundaries whose state a serving system caches
 * (the Kimi K3 report's deployment notes mention caching the recurrent
 * state at prompt boundaries).
 *
 *   pos_offsets  device int32 [num_seqs + 1]: the positions of sequence s
 *                are pos_values[pos_offsets[s] .. pos_offsets[s + 1])
 *                (non-decreasing offsets; pos_offsets[num_seqs] = num_pos)
 *   pos_values   device int32 [num_pos]: token counts P, 0 <= P <= L_s,
 *                non-decreasing within a sequence (P = 0 is the initial
 *                state, P = L_s the final state)
 *   num_pos      number of positions (>= 0); 0 = kda_prefill_chunked_ex and
 *                the three position arguments are ignored
 *   pos_states   [num_pos, H, Dk, Dv] fp32: slot j receives the state after
 *                the first pos_values[j] tokens of its sequence
 *
 * The scan stores the state at the start of the chunk that holds each P and
 * a small kernel applies the remaining P mod 64 tokens to it: with bf16
 * inputs in chunk form on the matrix cores, from that chunk's prepared
 * tensors in the workspace and its k, v, g (the same fp16-operand numerics as
 * the scan); with fp32 inputs token by token in fp32 (also reading beta).
 * Both belong to the SCAN phase, so a split call must pass the same
 * `frontend` bits to both phases.
 * Device-side (unchecked) preconditions: P outside [0, L_s] is clamped into
 * it; offsets outside [0, num_pos] are clamped; out-of-order positions give
 * unspecified states in their slots (never an out-of-bounds access).
 * Returns KDA_ERR_INVALID_ARG for num_pos < 0, or num_pos > 0 with a NULL or
 * misaligned position argument; otherwise as kda_prefill_chunked_ex.
 */
kda_status_t kda_prefill_chunked_at(
    const void *q, const void *k, const void *v, kda_dtype_t in_dtype,
    const float *g, const float *beta, const int32_t *cu_seqlens,
    int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
    int32_t chunk_size, const float *initial_state, float *final_state,
    int64_t ckpt_interval, float *ckpt_states, int64_t ckpt_rows, float *o,
    const int32_t *pos_offsets, const int32_t *pos_values, int32_t num_pos,
    float *pos_states, void *workspace, size_t workspace_bytes, uint32_t phases,
    uint32_t frontend, hipStream_t stream);

/*
 * kda_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Its scratch is a fixed 128 MiB device
 * array inside the library (one per device, held until the process ends,
 * never allocated or freed by this call). Sizes whose
 * kda_prefill_workspace_size-style need exceeds it are refused with
 * KDA_ERR_WORKSPACE before any launch: with bf16 q/k/v, H = 32 and
 * Dk = Dv = 128 that allows one sequence of up to 4,224 tokens. Every call on
 * a device shares that device's array: calls that overlap in time on one
 * device (different streams or threads) race and give undefined results. The
 * array keeps the last call's contents, which no later call reads. Other
 * arguments and results as kda_prefill_chunked; KDA_ERR_HIP if the array's
 * address cannot be obtained.
 */
kda_status_t kda_prefill_chunked_noalloc(
    const void *q, const void *k, const void *v, kda_dtype_t in_dtype,
    const float *g, const float *beta, const int32_t *cu_seqlens,
    int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t Dk, int32_t Dv,
    int32_t chunk_size, const float *initial_state, float *final_state,
    int64_t ckpt_interval, float *ckpt_states, int64_t ckpt_rows, float *o,
    hipStream_t stream);

/*
 * One KDA decode step for B independent sequences (one new token each).
 *
 * For each (b, h): S <- (I - beta k k^T) Diag(exp(g)) S + beta k v^T and
 * o = S^T q with the UPDATED S. The state is read and written in place
 * (one read and one write of every element).
 *
 *   q, k   [B, H, Dk] (in_dtype); v [B, H, Dv] (in_dtype)
 *   g      [B, H, Dk] fp32;  beta [B, H] fp32
 *   state  [B, H, Dk, Dv] fp32, updated in place; must not overlap inputs or o
 *   o      [B, H, Dv] fp32
 *   Dk, Dv in {64, 128}; B, H >= 1 (B == 0 is a valid no-op).
 *
 * Each (b, h)'s output and new state are bitwise the same whatever B and H
 * (the work is split differently for small batches, with every sum in the
 * same order), and the call enqueues kernels only, so it may be captured in
 * a HIP graph.
 *
 * Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP.
 */
kda_status_t kda_decode_step(
    const void *q, const void *k, const void *v, kda_dtype_t in_dtype,
    const float *g, const float *beta, int32_t B, int32_t H, int32_t Dk, int32_t Dv,
    float *state, float *o, hipStream_t stream);

/*
 * kda_decode_step with a `frontend` mask (a subset of the KDA_FRONT_* bits;
 * 0 = kda_decode_step). Returns KDA_ERR_INVALID_ARG for unknown bits,
 * otherwise as kda_decode_step.
 */
kda_status_t kda_decode_step_ex(
    const void *q, const void *k, const void *v, kda_dtype_t in_dtype,
    const float *g, const float *beta, int32_t B, int32_t H, int32_t Dk, int32_t Dv,
    float *state, float *o, uint32_t frontend, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
