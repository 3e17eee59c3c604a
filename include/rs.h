/*
 * rs.h -- ReplaySSM decode / speculative verify for Gated DeltaNet (GDN) and KDA layers
 * on AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes, no C++ or torch types.
 *
 * The method (from three public pull-request pages):
 *   - LightLLM, "feat: add ReplaySSM state modes for GDN and KDA" (PR description; commit
 *     messages on lazy compaction, the on-device overflow decision, the cursor kernel,
 *     the shared cursor advanced after the last layer, fp32 delta history, the key-group
 *     fold barrier and program order);
 *   - vLLM, "[Feature][MRV2] Enable Qwen3.5 GDN ReplaySSM standard decode" (Overview,
 *     Claims: no GPU-to-CPU reads, persistent graph buffers);
 *   - sglang, GDN ReplaySSM spec verify for DFLASH/DSPARK (commit 1: ring length check and
 *     null state slots; commit 3: causal terms selected, commit loads masked; commit 4:
 *     the ring commit folds the accepted window; commit 5: history skipped when
 *     write_pos is 0; Modifications; Behavior changes).
 *
 * The recurrence (gated delta rule; KDA when the decay is a vector over dk), with the
 * state stored as S[dk][dv] per value head:
 *     S' = alpha (.) S        (GDN: scalar alpha; KDA: key row i scaled by alpha[i])
 *     d  = beta * (v - S'^T k)            the "delta", kept in fp32 history
 *     S  = S' + k d^T,        o = scale S^T q  (post-update state; dims->scale)
 * Value head h reads key head h / (hv / hk).
 *
 * ReplaySSM: the canonical state S of a slot stays in place.  A verify of T draft tokens
 * replays the slot's committed history records (k, d, alpha) over S without writing S,
 * and appends the T draft records to the slot's ring at [write_pos, write_pos + T).  The
 * per-slot cursor counts committed records; it is shared by every layer and advanced
 * once per step, after the last layer, by rs_cursor_advance.  When a verify's window
 * would overflow the ring (cursor + T > L) the verify first folds the whole committed
 * prefix into S in-kernel and writes its window at 0.  rs_commit_fold folds at commit
 * time by policy.
 *
 * Ownership and execution.  The caller owns every buffer (contiguous, row-major, device
 * memory, 16-byte aligned).  The library allocates nothing, keeps no state between calls
 * and is reentrant.  Every call validates its arguments on the host, enqueues kernels on
 * the given stream and returns; it never synchronises and never copies device data to
 * the host, so a whole decode step can be captured in a HIP graph.
 *
 * Device-side contract (not checkable without a sync): live slots in slot_idx are
 * distinct; 0 <= accept_len <= T; 0 <= cursor <= L; a slot restored from a checkpoint
 * or written by prefill has cursor 0 (LightLLM: the restored slot's replay cursor is
 * cleared); each verify of a layer is followed by one rs_cursor_advance before that
 * layer's next verify.  For memory safety the kernels clamp out-of-contract values:
 * slots >= num_slots are treated as null, cursors are clamped to [0, L] and accept
 * lengths to [0, T].
 */
#ifndef RS_H_
#define RS_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RS_OK = 0,
    RS_E_NULLPTR = 1,         /* a required pointer is NULL */
    RS_E_SHAPE = 2,           /* unsupported or inconsistent dimensions */
    RS_E_DTYPE = 3,           /* unsupported dtype */
    RS_E_RING_TOO_SMALL = 4,  /* ring_cap < T: the ring cannot hold the draft window */
    RS_E_LAUNCH = 5,          /* the kernel launch failed (hipGetLastError) */
    RS_E_VALUE = 6,           /* a scalar argument is out of range (dims->scale) */
    RS_E_SCRATCH = 7          /* too large for rs_gdn_verify_noalloc's static workspace */
} rs_status;

typedef enum { RS_F32 = 0, RS_BF16 = 1 } rs_dtype;

/* Fold policy applied by rs_cursor_advance (sglang commit 4; LightLLM force_compress). */
typedef enum {
    RS_FOLD_NONE = 0,          /* never fold at commit; verify folds in-kernel on overflow */
    RS_FOLD_EVERY_COMMIT = 1,  /* fold every accepted window at commit */
    RS_FOLD_LAZY = 2,          /* fold when the next verify (width next_T) would overflow */
    RS_FOLD_FORCE = 3          /* fold rows in force_mask (every live row if NULL) */
} rs_fold_policy;

/* Shapes.  batch B: request rows; T: verify window, 1..16; hk, hv: key and value heads
 * (hv % hk == 0; KDA needs hv == hk); dk in {16,32,...,256} and dv a multiple of 16;
 * ring_cap L >= T, L <= 256; num_slots: size of the slot pools; act_dtype: q, k, v, beta,
 * gate and ring keys; state_dtype: S.  scale: the query scale, o = scale S^T q (1.0 for
 * none, dk^-1/2 for the usual attention scale); read by the verifies only, which return
 * RS_E_VALUE unless it is finite and nonzero (a zero-initialised struct is refused rather
 * than silently producing zero outputs).  tile_v: value columns per workgroup (16, 32, 64
 * or 128, dividing dv), or 0 for the library's choice. */
typedef struct {
    int32_t batch, T, hk, hv, dk, dv, ring_cap, num_slots;
    rs_dtype act_dtype, state_dtype;
    float scale;
    int32_t tile_v;
} rs_dims;

/*
 * rs_gdn_verify -- verify (T >= 1) or decode (T == 1) of one GDN layer.
 *   q, k        [B*T, hk, dk]  act dtype (token t of row r at r*T + t)
 *   v           [B*T, hv, dv]  act dtype
 *   beta, gate  [B*T, hv]      act dtype; gate is the linear decay alpha in (0, 1]
 *   state       [num_slots, hv, dk, dv] state dtype; written only for rows that fold
 *               (bf16: round-to-nearest-even on every write)
 *   ring_k      [num_slots, L, hk, dk] act dtype  (exact copies of k)
 *   ring_d      [num_slots, L, hv, dv] fp32        (deltas)
 *   ring_g      [num_slots, L, hv]     fp32        (exact upcasts of gate)
 *   cursor      [num_slots] int32, read only
 *   slot_idx    [B] int32; a negative slot is a null row: nothing is read or written
 *   out         [B*T, hv, dv] fp32; null rows are not written
 *   write_pos_out [B] int32 or NULL: write_pos of each live row (0 after a fold)
 *   group_counter [B, hk] int32 workspace, zeroed once by the caller; every call leaves
 *               it zeroed.  It orders the fused fold's rewrite of the shared ring keys
 *               and gates after every workgroup of the key group has read them (LightLLM
 *               commit on the key-group fold barrier), with no spinning.
 * Rows folding in-kernel: S <- fold(S, ring[0:cursor]), then write_pos = 0.  Otherwise
 * write_pos = cursor and the history [0, cursor) is replayed without writing S.  The T
 * draft records go to ring rows [write_pos, write_pos + T).  Causal terms are selected,
 * never multiplied by zero, so non-finite inputs at draft t reach no output before t.
 *   out[t] = dims->scale * S_t^T q_t, S_t the state after draft t.
 * Errors: RS_E_NULLPTR, RS_E_SHAPE, RS_E_DTYPE, RS_E_RING_TOO_SMALL, RS_E_VALUE,
 * RS_E_LAUNCH.
 */
rs_status rs_gdn_verify(const rs_dims* dims,
                        const void* q, const void* k, const void* v,
                        const void* beta, const void* gate,
                        void* state, void* ring_k, float* ring_d, float* ring_g,
                        const int32_t* cursor, const int32_t* slot_idx,
                        float* out, int32_t* write_pos_out, int32_t* group_counter,
                        hipStream_t stream);

/*
 * rs_gdn_verify_noalloc -- rs_gdn_verify for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without group_counter, the same kernels and the same results.  The
 * fold counters it needs live in a static device array inside the library, 65536 int32
 * (256 KiB) on each GPU the library runs on, held until the process ends; the call clears
 * the batch * hk counters it uses (a fill kernel on the stream) and allocates nothing.
 * Every call on one GPU shares that GPU's array: calls whose executions overlap on one
 * GPU (concurrent streams, or host threads) race on it and must be ordered by the caller.
 * Errors: as rs_gdn_verify; RS_E_SCRATCH when batch * hk > 65536.
 */
rs_status rs_gdn_verify_noalloc(const rs_dims* dims,
                                const void* q, const void* k, const void* v,
                                const void* beta, const void* gate,
                                void* state, void* ring_k, float* ring_d, float* ring_g,
                                const int32_t* cursor, const int32_t* slot_idx,
                                float* out, int32_t* write_pos_out, hipStream_t stream);

/*
 * rs_kda_verify -- as rs_gdn_verify for KDA (LightLLM: KDA gets the same windowed
 * reconstruction): hv == hk, the decay is per key channel.
 *   gate    [B*T, hv, dk] act dtype
 *   ring_g  [num_slots, L, hv, dk] fp32
 * Every other argument as for rs_gdn_verify.
 */
rs_status rs_kda_verify(const rs_dims* dims,
                        const void* q, const void* k, const void* v,
                        const void* beta, const void* gate,
                        void* state, void* ring_k, float* ring_d, float* ring_g,
                        const int32_t* cursor, const int32_t* slot_idx,
                        float* out, int32_t* write_pos_out, int32_t* group_counter,
                        hipStream_t stream);

/*
 * rs_gdn_verify_varlen, rs_kda_verify_varlen -- as rs_gdn_verify / rs_kda_verify with
 * ragged verify windows: each request row verifies its own number of draft tokens, and
 * the tokens of all rows are packed into one list (LightLLM commit: decode reads every
 * request window from the cumulative lengths, with q, k, v laid out [tokens, heads, dim];
 * sglang Modifications: per-request verify lengths packed into one token list).
 *   cu_seqlens  [B + 1] int32 device memory: row r owns packed tokens
 *               [cu_seqlens[r], cu_seqlens[r + 1]), its window width T_r; the caller
 *               keeps cu_seqlens nondecreasing, cu_seqlens[B] <= total_tokens and every
 *               T_r in [0, dims->T] (dims->T is the widest window of the batch, 1..16).
 *   total_tokens  rows of the packed inputs and outputs (>= 0)
 *   q, k        [total_tokens, hk, dk]; v [total_tokens, hv, dv]; beta [total_tokens, hv];
 *   gate        [total_tokens, hv] (GDN) or [total_tokens, hv, dk] (KDA)
 *   out         [total_tokens, hv, dv] fp32; packed token j of row r is draft t = j - cu[r]
 * Every per-row rule reads the row's own T_r: the row folds in-kernel when
 * cursor + T_r > L, and its records go to ring rows [write_pos, write_pos + T_r).  A row
 * with T_r = 0 reports write_pos = cursor and reads or writes nothing else.  For memory
 * safety the kernels clamp out-of-contract lengths to [0, total_tokens] and to dims->T.
 * Every other argument, and the errors, as for rs_gdn_verify; also RS_E_NULLPTR when
 * cu_seqlens is NULL (batch > 0) and RS_E_SHAPE when total_tokens < 0.
 */
rs_status rs_gdn_verify_varlen(const rs_dims* dims, const int32_t* cu_seqlens,
                               int32_t total_tokens, const void* q, const void* k,
                               const void* v, const void* beta, const void* gate, void* state,
                               void* ring_k, float* ring_d, float* ring_g,
                               const int32_t* cursor, const int32_t* slot_idx, float* out,
                               int32_t* write_pos_out, int32_t* group_counter,
                               hipStream_t stream);
rs_status rs_kda_verify_varlen(const rs_dims* dims, const int32_t* cu_seqlens,
                               int32_t total_tokens, const void* q, const void* k,
                               const void* v, const void* beta, const void* gate, void* state,
                               void* ring_k, float* ring_d, float* ring_g,
                               const int32_t* cursor, const int32_t* slot_idx, float* out,
                               int32_t* write_pos_out, int32_t* group_counter,
                               hipStream_t stream);

/*
 * rs_cursor_advance -- once per step, after every layer's verify (LightLLM: the shared
 * cursor is advanced only after the last layer; MTP verify trims the rejected tail).
 * For each live row r with slot s: write_pos = (cursor[s] + T > L) ? 0 : cursor[s];
 * m = write_pos + accept_len[r]; fold_len[s] = m if the policy folds the row, else 0;
 * cursor[s] = fold_len[s] ? 0 : m.  LAZY folds when m + next_T > L; FORCE folds rows with
 * force_mask[r] != 0 (every live row when force_mask is NULL).  Null rows are skipped
 * (sglang commit 1).
 *   cursor [num_slots] int32 (in/out); fold_len [num_slots] int32 (out, live slots only)
 *   slot_idx [B] int32; accept_len [B] int32 in [0, T]; force_mask [B] uint8 or NULL
 * Errors: RS_E_NULLPTR, RS_E_SHAPE, RS_E_RING_TOO_SMALL, RS_E_LAUNCH.
 */
rs_status rs_cursor_advance(const rs_dims* dims, int32_t* cursor, int32_t* fold_len,
                            const int32_t* slot_idx, const int32_t* accept_len,
                            rs_fold_policy policy, int32_t next_T,
                            const uint8_t* force_mask, hipStream_t stream);

/*
 * rs_cursor_advance_varlen -- rs_cursor_advance after ragged verifies: cu_seqlens and
 * total_tokens exactly as the step's rs_*_verify_varlen calls received them.  Row r's
 * write_pos is recomputed with its own window width T_r, and accept_len[r] is in
 * [0, T_r] (clamped to it).  Errors as for rs_cursor_advance; also RS_E_NULLPTR when
 * cu_seqlens is NULL (batch > 0) and RS_E_SHAPE when total_tokens < 0.
 */
rs_status rs_cursor_advance_varlen(const rs_dims* dims, const int32_t* cu_seqlens,
                                   int32_t total_tokens, int32_t* cursor, int32_t* fold_len,
                                   const int32_t* slot_idx, const int32_t* accept_len,
                                   rs_fold_policy policy, int32_t next_T,
                                   const uint8_t* force_mask, hipStream_t stream);

/*
 * rs_commit_fold -- compact commit: S[s] <- fold(S[s], ring[s, 0:fold_len[s]]) for each
 * live row with fold_len > 0.  Reads fold_len, never the cursor, so layers sharing one
 * cursor all fold the same prefix after it was reset (sglang commits 3 and 4: the ring
 * loads are masked to the committed history).  bf16 states are rounded once, on write.
 *   is_kda: 0 = GDN (ring_g [num_slots, L, hv]), 1 = KDA (ring_g [num_slots, L, hv, dk])
 * Errors: RS_E_NULLPTR, RS_E_SHAPE, RS_E_DTYPE, RS_E_LAUNCH.
 */
rs_status rs_commit_fold(const rs_dims* dims, int is_kda, void* state, const void* ring_k,
                         const float* ring_d, const float* ring_g, const int32_t* fold_len,
                         const int32_t* slot_idx, hipStream_t stream);

/*
 * rs_materialize -- the accepted state fold(S[s], ring[s, 0:cursor[s]]) of each live row
 * into out_state [B, hv, dk, dv] fp32 (LightLLM: accepted-state materialization; a
 * read-only fold).  S, rings and cursors are not modified; null rows are not written.
 * Errors: RS_E_NULLPTR, RS_E_SHAPE, RS_E_DTYPE, RS_E_LAUNCH.
 */
rs_status rs_materialize(const rs_dims* dims, int is_kda, const void* state,
                         const void* ring_k, const float* ring_d, const float* ring_g,
                         const int32_t* cursor, const int32_t* slot_idx, float* out_state,
                         hipStream_t stream);

/*
 * rs_snapshot_verify, rs_snapshot_commit -- the snapshot-verify baseline that ReplaySSM
 * replaces, for comparison in time and memory (sglang PR, Behavior changes and Speed
 * Tests: the snapshot verify writes one full state per draft token, 72.6 GB against
 * 3.04 GB of ring at TP1 with 128 requests, and the commit scatters the accepted
 * snapshot).  No ring and no cursor: the verify runs the recurrence token by token from
 * S[slot] and writes S after every draft token; the commit copies the accepted one back.
 *   is_kda      0 = GDN (gate [B*T, hv]), 1 = KDA (hv == hk, gate [B*T, hv, dk])
 *   q, k, v, beta, gate, out   as for rs_gdn_verify / rs_kda_verify
 *   state       [num_slots, hv, dk, dv] state dtype; read by the verify, written by the
 *               commit (slot of each live row with accept_len > 0)
 *   snapshots   [B, T, hv, dk, dv] state dtype: snapshots[r, t] = S after draft t of row r
 *               (bf16: round-to-nearest-even); caller-owned, written by the verify
 *   accept_len  [B] int32 in [0, T]; 0 leaves the state as it is
 * Null rows (slot < 0) are skipped by both.  dims->ring_cap must still be >= T (the
 * dims are shared with the ring calls); dims->tile_v = 0 or a width up to 64; outputs are
 * scaled by dims->scale as in rs_gdn_verify.
 * Errors: RS_E_NULLPTR, RS_E_SHAPE, RS_E_DTYPE, RS_E_RING_TOO_SMALL, RS_E_VALUE (verify),
 * RS_E_LAUNCH.
 */
rs_status rs_snapshot_verify(const rs_dims* dims, int is_kda, const void* q, const void* k,
                             const void* v, const void* beta, const void* gate,
                             const void* state, void* snapshots, const int32_t* slot_idx,
                             float* out, hipStream_t stream);
rs_status rs_snapshot_commit(const rs_dims* dims, void* state, const void* snapshots,
                             const int32_t* slot_idx, const int32_t* accept_len,
                             hipStream_t stream);

/*
 * rs_gdn_prefill -- chunked prefill of one GDN layer (LightLLM commit messages: prefill
 * writes the canonical SSM directly and leaves the cursor at zero).  Row r's prompt, the
 * packed tokens [cu_seqlens[r], cu_seqlens[r+1]) (any length, 0 allowed; clamped to
 * [0, total_tokens]), runs from the slot's canonical state S through the gated delta rule;
 * S is overwritten with the state after the last prompt token and cursor[slot] set to 0.
 * The ring is not read: a slot with pending records must have them folded first (a FORCE
 * rs_cursor_advance and rs_commit_fold), so that S is its committed state; a new request's
 * S is zeroed by the caller; a long prompt may be split over calls.
 *   q, k   [total_tokens, hk, 128] bf16;  v [total_tokens, hv, dv] bf16
 *   beta, gate [total_tokens, hv] bf16;   out [total_tokens, hv, dv] fp32 (scale S^T q)
 *   state  [num_slots, hv, 128, dv] state dtype (bf16: one rounding at the end)
 *   cursor [num_slots] int32 (written: 0 for live rows); slot_idx [B] (null rows skipped)
 * Covers dk = 128, bf16 inputs and dv a multiple of 64; dims->T, ring_cap and tile_v are
 * not used.  The state stays on chip across the prompt, in chunks of 16 tokens.
 * Errors: RS_E_NULLPTR, RS_E_SHAPE (other shapes, total_tokens < 0), RS_E_DTYPE,
 * RS_E_VALUE (scale), RS_E_LAUNCH.
 */
rs_status rs_gdn_prefill(const rs_dims* dims, const int32_t* cu_seqlens, int32_t total_tokens,
                         const void* q, const void* k, const void* v, const void* beta,
                         const void* gate, void* state, int32_t* cursor,
                         const int32_t* slot_idx, float* out, hipStream_t stream);

/*
 * The short causal convolution a GDN layer applies to its mixed q/k/v channels before the
 * recurrence, with its per-slot window state, and the rollback of that window at commit
 * (LightLLM PR description: Conv/SSM state management with MTP accept and rollback;
 * commit messages: page save and PD/DP copy "the accepted conv window" with the canonical
 * SSM, a restored slot receives the canonical conv and SSM state; sglang PR commit 4: the
 * GDN ring commit includes the conv rollback).  The pages do not give the convolution;
 * this library takes the depthwise causal form
 *     y_t[c] = act( sum_{j<K} weight[c][j] * x_{t-K+1+j}[c] + bias[c] ),
 * tap K-1 on the current input, act = none or SiLU, where the inputs before the window
 * come from the slot's conv state: its last K-1 committed inputs, oldest first.
 *
 * rs_conv_dims:  batch B; T the verify window (1..16; the widest window with cu_seqlens);
 * channels C (a multiple of 8); width K (2, 3 or 4); num_slots; act_dtype of x, weight,
 * bias and state; out_dtype of y (bf16: round to nearest even); activation.
 */
typedef enum { RS_ACT_NONE = 0, RS_ACT_SILU = 1 } rs_activation;

typedef struct {
    int32_t batch, T, channels, width, num_slots;
    rs_dtype act_dtype, out_dtype;
    rs_activation activation;
} rs_conv_dims;

/*
 * rs_conv_verify -- the window's conv outputs; the conv state is read, never written.
 *   cu_seqlens  NULL: row r's T inputs are tokens [r*T, r*T + T); else row r owns tokens
 *               [cu_seqlens[r], cu_seqlens[r+1]) of total_tokens packed tokens (at most T;
 *               clamped as for rs_gdn_verify_varlen), a width-0 window writes nothing
 *   x           [tokens, C] act dtype (tokens = B*T, or total_tokens)
 *   weight      [C, K] act dtype;  bias [C] act dtype or NULL
 *   conv_state  [num_slots, K-1, C] act dtype, oldest input first
 *   slot_idx    [B]; a negative slot is a null row: nothing is read or written
 *   y           [tokens, C] out dtype; rows of null rows are not written
 * Buffers are device memory, 16-byte aligned.  Enqueued on stream, no synchronisation.
 * Errors: RS_E_NULLPTR, RS_E_SHAPE, RS_E_DTYPE, RS_E_VALUE (activation), RS_E_LAUNCH.
 */
rs_status rs_conv_verify(const rs_conv_dims* dims, const int32_t* cu_seqlens,
                         int32_t total_tokens, const void* x, const void* weight,
                         const void* bias, const void* conv_state, const int32_t* slot_idx,
                         void* y, hipStream_t stream);

/*
 * rs_conv_commit -- the conv rollback after a step's verifies: for each live row with
 * accept length a > 0 (clamped to [0, T_r]), the slot's state becomes inputs [a, a + K - 1)
 * of state ++ window, i.e. the K-1 inputs ending at the last accepted draft; a = 0 leaves
 * it.  cu_seqlens, total_tokens and x exactly as the step's rs_conv_verify calls received
 * them; accept_len [B] int32.  A bit copy: no arithmetic.
 *   layers      1..65535: one launch rolls back this many layers whose conv states
 *               ([layers, num_slots, K-1, C]) and window inputs ([layers, tokens, C]) sit
 *               back to back, layer-major (the rollback follows the last layer, as the
 *               cursor advance does, so the layers' bytes share one launch's latency)
 * Errors as rs_conv_verify; also RS_E_SHAPE for layers out of range.
 */
rs_status rs_conv_commit(const rs_conv_dims* dims, const int32_t* cu_seqlens,
                         int32_t total_tokens, int32_t layers, void* conv_state,
                         const void* x, const int32_t* slot_idx, const int32_t* accept_len,
                         hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* rs_status_str(rs_status status);

/* Workgroup count and dynamic LDS bytes the verify launches for these dims, for
 * profiling and tests.  Returns RS_OK or the validation error. */
rs_status rs_verify_launch_info(const rs_dims* dims, int is_kda, int32_t* tile_v,
                                int32_t* workgroups, int32_t* lds_bytes);

/* Measurement aid, not part of the method: the read-bandwidth reference the verify is
 * compared with.  Streams `bytes` bytes of src with the load instructions and workgroup
 * size the verify uses for its state tiles (non-temporal 16-byte vector loads, 256
 * threads, 16 KiB per workgroup) and does nothing else.
 *   src   device memory, 16-byte aligned, bytes > 0 and a multiple of 16; only read.
 *   sink  device memory of 256 floats that the kernel may write (contents unspecified),
 *         so that the loads are kept.
 * Enqueued on stream; no synchronisation.
 * Errors: RS_E_NULLPTR, RS_E_SHAPE (size or alignment), RS_E_LAUNCH. */
rs_status rs_stream_read(const void* src, uint64_t bytes, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* RS_H_ */
