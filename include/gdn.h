/*
 * gdn.h - C ABI of the MI355X (gfx950) chunked gated delta rule prefill scan
 * (and the single-token decode step that continues from its state).
 *
 * The operation ("flashinfer.gdn_prefill": chunk_gated_delta_rule is the
 * chunked GDN scan that builds the recurrent state from a whole prompt before
 * decoding takes over; "flashinfer.cudnn.cudnn_chunk_gated_delta_rule" gives
 * its arguments).  Per token t of a sequence and per value head h:
 *
 *     S_t = a_t * S_{t-1} * (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * S is the [V = 128, K = 128] state, stored V-major (S[v][k]) as on the
 * "flashinfer.cudnn" page, section "Linear attention".  a_t is the forget
 * gate in linear space (Parameters: g), b_t the post-sigmoid update gate
 * (Parameters: beta).  Value head h reads query/key head h / (Hv / Hqk).
 *
 * Everything here is plain C: device pointers, element sizes and element
 * strides.  No caller pointer is kept after a call returns.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of a gdn_tensor. */
enum gdn_dtype {
    GDN_F32 = 0,
    GDN_BF16 = 1,
    GDN_F16 = 2,
    GDN_I32 = 3,
    GDN_I64 = 4
};

/* Return codes.  Invalid inputs and unsupported configurations fail closed,
 * with no fallback to another implementation ("flashinfer.gdn_prefill", Cake
 * GDN CP context-parallel backend: invalid inputs and unsupported
 * architectures fail closed); like the engine that declines a graph it cannot
 * serve while the reason is logged ("flashinfer.cudnn", Linear attention), a
 * refused call returns a code and gdn_last_error() gives the reason.  A
 * non-zero code means nothing was enqueued and nothing was written. */
enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1, /* NULL required tensor, bad ndim/shape/stride/dtype */
    GDN_ERR_UNSUPPORTED = 2,      /* head_dim != 128, head relation, dtype combination */
    GDN_ERR_ALIAS = 3,            /* output_state->data == initial_state->data */
    GDN_ERR_NO_DEVICE = 4,        /* no HIP device visible */
    GDN_ERR_ARCH = 5,             /* current device is not gfx950 */
    GDN_ERR_HIP = 6               /* a HIP runtime call failed (launch, allocation) */
};

/* A strided view of device memory.  sizes/strides are in elements; entries
 * beyond ndim are ignored.  The innermost dimension must have stride 1. */
typedef struct gdn_tensor {
    void *data;
    int32_t dtype;      /* enum gdn_dtype */
    int32_t ndim;
    int64_t sizes[4];
    int64_t strides[4];
} gdn_tensor;

/*
 * gdn_chunk_prefill - runs the scan over a packed varlen batch.
 *
 * Argument meanings follow "flashinfer.cudnn.cudnn_chunk_gated_delta_rule",
 * Parameters (T = total tokens, N = sequences, d = 128):
 *   q, k            [T, Hqk, 128], F32 or BF16 (both the same), innermost
 *                   contiguous.  Token and head strides: non-negative, a
 *                   multiple of 16 bytes, the token stride at least 128
 *                   elements and below 32 MiB; data 16-byte aligned (the
 *                   pages pass any strides through; these limits come from
 *                   the 16-byte row loads here, GDN_ERR_UNSUPPORTED).
 *   v               [T, Hv, 128], q's dtype, same stride rule; Hv % Hqk == 0.
 *   g               NULL (all ones) or [T, Hv] forget gate in linear space,
 *                   F32, BF16 or F16, innermost stride 1 not required.
 *                   Values in [0, 1]; a zero gate resets the state (the
 *                   kernels clamp ln(a) at -80).
 *   beta            NULL (all ones) or [T, Hv] post-sigmoid gate, F32 or q's
 *                   dtype.
 *   scale           query scale; exactly 0.0 means 1/sqrt(128); must be finite.
 *   cu_seqlens      [N + 1] I32 or I64 in device memory, contiguous; required.
 *                   cu[0] = 0, non-decreasing, cu[N] = T.  These contents are
 *                   an unchecked precondition (they are never read on the
 *                   host); empty sequences are allowed.
 *   initial_state   NULL (zero state) or [N, Hv, 128, 128] F32 or BF16,
 *                   V-major, innermost (K) stride 1; data and the other
 *                   strides 16-byte aligned, rows at least 128 elements apart.
 *   output_state    NULL (no state written at all) or the same shape, F32 or
 *                   BF16 (each state buffer carries its own dtype; the scan
 *                   accumulates in fp32).  Must not overlap initial_state:
 *                   equal data pointers are rejected with GDN_ERR_ALIAS;
 *                   partial overlap is an unchecked precondition.  An empty
 *                   sequence copies its initial state (or zeros) here.
 *   use_qk_l2norm   non-zero: q and k rows are scaled by 1/sqrt(sum x^2 + 1e-6)
 *                   inside the kernel before use.
 *   batch_invariant non-zero: every sequence is scanned by one work item per
 *                   head in a fixed order, so its output and final state are
 *                   bitwise independent of the rest of the batch.  Zero
 *                   allows splitting one long sequence across work items
 *                   (segment scan, then a state fix-up), which may change the
 *                   last bits.
 *   out             [T, Hv, 128], q's dtype, written in place (the library
 *                   allocates no output); strides as for q, and no two
 *                   elements at one address (e.g. a head stride below 128
 *                   elements is rejected, GDN_ERR_UNSUPPORTED).  Overlap of
 *                   out with q, k, v, g or beta is an unchecked precondition.
 *   stream          a hipStream_t (NULL = the default stream).  The call is
 *                   asynchronous: it validates on the host, enqueues on
 *                   `stream` and returns without synchronising.  A long
 *                   GDN_PLAN_PREPARED_SCAN call also enqueues part of its
 *                   work on a side stream the library keeps for `stream`,
 *                   forked from `stream` and joined back into it by events:
 *                   to the caller the call is ordered on `stream` as any
 *                   other.
 *
 * Ownership: every tensor is caller-owned device memory; the library writes
 * only `out`, `output_state` and its own workspace (cached per device and
 * stream, grown on demand; see gdn_release_workspace).  Calls on different
 * streams may be made from different threads at once; calls on one stream
 * must come from one thread at a time (they share that stream's workspace,
 * side stream and events, and each call's kernels must stay together in the
 * stream's order).
 * Graph capture: a call whose plan (gdn_prefill_plan) is GDN_PLAN_SPLIT or
 * GDN_PLAN_PREPARED_SCAN uses the workspace of its stream; after one eager call of the largest shape on
 * that stream, calls enqueue kernels only and can be captured.  A call that
 * would grow the workspace while the stream is capturing is refused with
 * GDN_ERR_UNSUPPORTED.  A captured graph keeps the capture stream's workspace
 * address: its replays share that memory with eager split calls on the
 * capture stream, so the two must not run at the same time, and growing the
 * workspace later keeps the old buffer alive for the graph.  The side stream
 * of a prepared call is created by the first eager call on `stream`; a
 * captured prepared call without one runs on `stream` alone, with bitwise the
 * same results.
 * Errors: validation happens before any enqueue; an invalid call writes
 * nothing and returns a gdn_status (no fallback path exists).
 */
int gdn_chunk_prefill(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                      const gdn_tensor *g, const gdn_tensor *beta, float scale,
                      const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                      const gdn_tensor *output_state, int use_qk_l2norm,
                      int batch_invariant, const gdn_tensor *out, void *stream);

/*
 * gdn_chunk_prefill_noalloc - gdn_chunk_prefill for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, plan, kernels and
 * results; the split path's workspace is a fixed 128 MiB array in the
 * library's device memory instead of a cached allocation, so no call
 * allocates or frees anything.  Every GPU holds its own copy of the array
 * from its first use to the end of the process.  On a 256-CU gfx950 part
 * every split plan fits (at most 120 MiB); a plan needing more is refused
 * with GDN_ERR_UNSUPPORTED.  All calls on one GPU share the array: calls
 * that overlap in time on one GPU (other streams, or another thread) race
 * and must be serialised by the caller.  Ownership and errors otherwise as
 * for gdn_chunk_prefill.
 */
int gdn_chunk_prefill_noalloc(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                              const gdn_tensor *g, const gdn_tensor *beta, float scale,
                              const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                              const gdn_tensor *output_state, int use_qk_l2norm,
                              int batch_invariant, const gdn_tensor *out, void *stream);

/*
 * gdn_chunk_prefill_checkpointed - gdn_chunk_prefill that also writes the
 * state at fixed token intervals of every sequence (the state checkpointing
 * that "flashinfer.cudnn", Linear attention, lists among the arguments the
 * routing layer handles before cuDNN is called).
 *
 *   checkpoints               [N * P, Hv, 128, 128] F32 or BF16 (required),
 *                             V-major like the states, rows 16-byte aligned;
 *                             must not share its data pointer with
 *                             initial_state or output_state.
 *   checkpoints_per_sequence  P >= 1.
 *   checkpoint_interval       I tokens, a positive multiple of 64.
 *
 * Slot n * P + i receives the state of sequence n after its first (i + 1) * I
 * tokens, for every i < P with (i + 1) * I <= length of sequence n; other
 * slots are left as they are (a checkpoint at the sequence end equals the
 * final state).  All other arguments, ownership and errors as for
 * gdn_chunk_prefill.
 */
int gdn_chunk_prefill_checkpointed(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                                   const gdn_tensor *g, const gdn_tensor *beta, float scale,
                                   const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                                   const gdn_tensor *output_state, int use_qk_l2norm,
                                   int batch_invariant, const gdn_tensor *checkpoints,
                                   int32_t checkpoints_per_sequence, int64_t checkpoint_interval,
                                   const gdn_tensor *out, void *stream);

/*
 * gdn_chunk_prefill_pooled - gdn_chunk_prefill on an indexed state pool,
 * updated in place (the indexed state pools that "flashinfer.cudnn", Linear
 * attention, lists among the arguments the routing layer handles before cuDNN
 * is called).
 *
 *   state_pool      [S, Hv, 128, 128] F32 or BF16, V-major, rows 16-byte
 *                   aligned (required): both the initial and the final states.
 *   state_indices   [N] I32 or I64 in device memory, contiguous (required).
 *                   Sequence n starts from state_pool[state_indices[n]] and
 *                   its final state is written back there.  An entry outside
 *                   [0, S) means a zero initial state and no state written.
 *                   Entries in [0, S) must be distinct (an unchecked
 *                   precondition: they are never read on the host).
 *
 * Rows of the pool no sequence names are left as they are.  All other
 * arguments, ownership and errors as for gdn_chunk_prefill.
 */
int gdn_chunk_prefill_pooled(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                             const gdn_tensor *g, const gdn_tensor *beta, float scale,
                             const gdn_tensor *cu_seqlens, const gdn_tensor *state_pool,
                             const gdn_tensor *state_indices, int use_qk_l2norm, int batch_invariant,
                             const gdn_tensor *out, void *stream);

/*
 * gdn_decode_step - one recurrent step for a batch of N sequences, one new
 * token each: the decode-side update that continues from the state a prefill
 * hands over ("flashinfer.gdn_prefill": the chunked scan initialises the
 * recurrent state before the decode loop takes over; "flashinfer.cudnn",
 * Linear attention: the state crosses V-major, float32 or bfloat16).  Per
 * sequence n and value head h it applies the same recurrence as above to the
 * single token:
 *
 *     S' = a S (I - b k k^T) + b v k^T,   o = scale S' q
 *
 *   q, k            [N, Hqk, 128], F32 or BF16 (both the same), innermost
 *                   contiguous, rows 16-byte aligned.
 *   v               [N, Hv, 128], q's dtype; Hv % Hqk == 0.
 *   g, beta         NULL (ones) or [N, Hv]; g F32, BF16 or F16, beta F32 or
 *                   q's dtype (as for gdn_chunk_prefill).
 *   scale           as for gdn_chunk_prefill (0.0 means 1/sqrt(128)).
 *   state_in        NULL (zero state) or [N, Hv, 128, 128] F32 or BF16,
 *                   V-major, rows 16-byte aligned.
 *   state_out       NULL (no state written) or the same shape, F32 or BF16.
 *                   It may be state_in itself (the identical view: same
 *                   pointer, dtype and strides) for an in-place update; the
 *                   same pointer with another dtype or strides is rejected
 *                   with GDN_ERR_ALIAS, other overlap is an unchecked
 *                   precondition.
 *   use_qk_l2norm   as for gdn_chunk_prefill.
 *   out             [N, Hv, 128], q's dtype.
 *   stream          as for gdn_chunk_prefill (asynchronous).
 *
 * Ownership and errors as for gdn_chunk_prefill; no workspace is used.
 */
int gdn_decode_step(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                    const gdn_tensor *g, const gdn_tensor *beta, float scale,
                    const gdn_tensor *state_in, const gdn_tensor *state_out,
                    int use_qk_l2norm, const gdn_tensor *out, void *stream);

/*
 * gdn_decode_step_pooled - gdn_decode_step on an indexed state pool, updated
 * in place: sequence n reads and rewrites state_pool[state_indices[n]]
 * (state_pool [S, Hv, 128, 128] F32 or BF16, state_indices [N] I32 or I64 in
 * device memory; entries outside [0, S) mean a zero state and no write;
 * entries in [0, S) must be distinct, an unchecked precondition).  Other
 * arguments, ownership and errors as for gdn_decode_step.
 */
int gdn_decode_step_pooled(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                           const gdn_tensor *g, const gdn_tensor *beta, float scale,
                           const gdn_tensor *state_pool, const gdn_tensor *state_indices,
                           int use_qk_l2norm, const gdn_tensor *out, void *stream);

/* What a gdn_chunk_prefill call (or its checkpointed and pooled forms) runs,
 * decided on the host from host-known sizes only (the "split/segment plan" of
 * "flashinfer.gdn_prefill", Cake GDN CP context-parallel backend: T precompute
 * -> MN precompute -> state fixup -> CP prefill, taken here only when splitting
 * few long sequences pays off, and never with batch_invariant).
 *   GDN_PLAN_SCAN            one launch of the four-wave fused scan
 *   GDN_PLAN_PIPELINED_SCAN  one launch of the eight-wave pipelined scan (bf16,
 *                            no checkpoints, more than half as many work items
 *                            as CUs and at most one per CU, or fewer work items
 *                            when the prepared chunks would take more than
 *                            8 GiB, about 208 bytes per token and value head);
 *                            bitwise the results of GDN_PLAN_SCAN
 *   GDN_PLAN_SPLIT           segment table, the two segment maps, the state
 *                            fix-up and the per-segment scan, with segments
 *                            of *segment_length tokens
 *   GDN_PLAN_PREPARED_SCAN   the state-independent preparation of every chunk
 *                            in one parallel pass ("T precompute"), then the
 *                            scan that consumes it with each head's state rows
 *                            spread over two or four CUs (bf16, no checkpoints,
 *                            at most half as many work items as CUs); when
 *                            the scan takes at most half the CUs and the
 *                            sequences average 64 or more chunks, in four
 *                            ranges of chunks, the later ranges prepared on a
 *                            side stream while the earlier ones are scanned;
 *                            bitwise the results of GDN_PLAN_SCAN.
 *                            gdn_chunk_prefill_noalloc runs
 *                            GDN_PLAN_PIPELINED_SCAN instead (no workspace).
 */
enum gdn_plan_kind { GDN_PLAN_SCAN = 0, GDN_PLAN_PIPELINED_SCAN = 1, GDN_PLAN_SPLIT = 2, GDN_PLAN_PREPARED_SCAN = 3 };

/* The plan for num_seqs sequences of num_tokens tokens in total, num_v_heads
 * value heads, q/k/v of io_dtype (GDN_F32 or GDN_BF16), with or without
 * checkpoints, on a device with num_cus compute units.  A pure host function
 * (no device needed).  Writes *kind (enum gdn_plan_kind) and *segment_length
 * (0 unless GDN_PLAN_SPLIT).  Returns GDN_OK, GDN_ERR_INVALID_ARGUMENT for
 * NULL outputs, negative sizes, num_v_heads or num_cus below 1, or another
 * dtype, and GDN_ERR_UNSUPPORTED for sizes gdn_chunk_prefill refuses (more
 * than 2^40 tokens, 65536 value heads or 2^24 sequences, or a grid of
 * (sequence, value head) work items beyond one launch). */
int gdn_prefill_plan(int64_t num_seqs, int64_t num_tokens, int64_t num_v_heads, int io_dtype,
                     int checkpoints, int batch_invariant, int num_cus, int *kind,
                     int64_t *segment_length);

/* The reason for the last non-zero return of a gdn_* call on this thread
 * ("" if none): the counterpart of the per-engine reason that the frontend
 * logs when an engine declines a graph ("flashinfer.cudnn", Linear attention).
 * The pointer stays valid until the next call on the thread. */
const char *gdn_last_error(void);

/* Frees every cached workspace, current and superseded, on all devices and
 * streams (the workspace the dispatcher caches with the shape-specific plan,
 * "flashinfer.gdn_prefill", Cake GDN CP context-parallel backend; nothing is
 * kept for the process lifetime unless the caller keeps calling), and the side
 * streams and events of prepared calls.  The caller must ensure that no
 * enqueued gdn work is still running and that no graph captured from a split
 * or prepared call is replayed afterwards. */
void gdn_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
