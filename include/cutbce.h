/*
 * cutbce.h -- C ABI of the MI355X (gfx950) fused full-vocabulary binary cross-entropy library (libcutbce.so).
 *
 * The operation ("Cut Binary Cross Entropy", Li, Ning, Hammad):
 *   rows r < R carry hidden states H[r] (D values), items v < V carry embeddings E[v]; the logit is
 *   z_rv = H[r] . E[v] (Section III-A). Row r's positive items are a list of ids; y_rv = 1 iff v is in the
 *   list (a repeated id counts once). Rows with row_mask[r] == 0 are padding and take no part.
 *   Valid rows may carry weights w_r (row_weight; w_r = 1 when it is NULL). With W = sum of w_r over the
 *   valid rows (R_v, the number of valid rows, without weights) and s = 1 / (W * V):
 *     loss   = s * sum_{valid r} w_r sum_v [ max(z,0) + log(1 + exp(-|z|)) - y*z ]  (Eq. (2)-(3) and the
 *                                                                                   averaging after Eq. (4))
 *     dH[r]  = g * s * w_r * sum_v (sigma(z_rv) - y_rv) * E[v]    for valid r, 0 for masked r   (Eq. (4))
 *     dE[v]  = g * s * sum_{valid r} w_r (sigma(z_rv) - y_rv) * H[r]                          (Eq. (4))
 *   where g is the cotangent of the scalar loss. W = 0 gives loss 0 and zero gradients. The weights are the
 *   per-position `weights` of the paper's API call (Listing 1), which the pages do not define: here they turn
 *   the average over positions into a weighted average; 0/1 weights are the padding mask itself.
 *   The logits Z and their gradient are never written to memory (Section III-B, Table I): every kernel forms
 *   its [rows x items] tile in registers and reduces it on chip.
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) must point to device memory of the GPU that is current on the calling thread;
 *     pointers marked (host) to host memory. The caller owns and allocates all memory; the library never
 *     allocates device memory and keeps no state between calls (apart from the opt-in timing records of
 *     cutbce_profile_enable and the fixed per-GPU scratch array of cutbce_forward_noalloc).
 *   - H [R][D], E [V][D], dH [R][D], dE [V][D] are dense row-major, in the problem's element type, 16-byte
 *     aligned. row_offsets int32 [R+1] (row_offsets[0] = 0, non-decreasing, row_offsets[R] <= nnz); item_ids
 *     int32 [nnz], any order within a row, repeats allowed, entries from row_offsets[R] on unused (so a
 *     capacity-sized buffer from cutbce_targets_to_csr can be passed as is); row_mask uint8 [R]
 *     (0 = padding, else valid).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs asynchronously; no call
 *     synchronises with the host. Scalars that the device produces or consumes (loss, grad_loss) stay in
 *     device memory.
 *   - Host-side argument checks run before anything is enqueued; on any error nothing is enqueued and the
 *     outputs are untouched. Ids outside [0, V) are skipped by the compute entry points, and row offsets are
 *     clamped into [0, nnz] (a decreasing range is empty), so malformed targets never cause reads outside
 *     item_ids; cutbce_validate_targets reports them on the device.
 *   - Results are deterministic: the same inputs on the same device give bitwise identical outputs (no
 *     floating-point atomics).
 *   - The workspace (device, cutbce_workspace_size() bytes, 256-byte aligned) is scratch: its contents on
 *     entry are ignored (except by cutbce_backward_reuse, which reads what cutbce_forward left) and on return
 *     are unspecified. Concurrent calls must use distinct workspaces.
 *   - The first compute call of a problem type on a device also sets up per-kernel launch data (dynamic LDS
 *     limit, resident workgroups per CU). Later calls enqueue kernel launches only (no memset or memcpy), so a
 *     caller can capture them into a HIP graph and replay it; the replays read the inputs anew.
 */
#ifndef CUTBCE_H
#define CUTBCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CUTBCE_OK = 0,
    CUTBCE_ERR_NULL = 1,        /* a required pointer is NULL */
    CUTBCE_ERR_SHAPE = 2,       /* R < 1, V < 1, nnz < 0, or sizes overflow the supported range */
    CUTBCE_ERR_DTYPE = 3,       /* unknown element type */
    CUTBCE_ERR_ALIGN = 4,       /* H, E, dH, dE, dh_saved not 16-byte aligned, the workspace not 256-byte
                                 * aligned, or int / float arrays not 4-byte aligned */
    CUTBCE_ERR_WORKSPACE = 5,   /* workspace smaller than cutbce_workspace_size() */
    CUTBCE_ERR_UNSUPPORTED = 6, /* (dtype, D) combination without a kernel: see cutbce_problem */
    CUTBCE_ERR_HIP = 7          /* a HIP launch or runtime call failed */
} cutbce_status;

typedef enum {
    CUTBCE_F32 = 0, /* IEEE float32 inputs, float32 MFMA, float32 gradients */
    CUTBCE_BF16 = 1 /* bfloat16 inputs, bf16 MFMA for the logits with float32 accumulation; the gradient GEMMs
                     * run on f16 operands (the logit gradients, and copies of H or E scaled by a power of two);
                     * bfloat16 gradients */
} cutbce_dtype;

/* Problem description (host struct). Supported: bf16 with D in {64, 128, 256, 512}; f32 with D in
 * {64, 128, 256}. 1 <= R, V <= 2^31 - 1025 (the library pads both to a multiple of 256 and keeps 32-bit
 * indices); 0 <= nnz <= 2^31 - 1. */
typedef struct {
    int64_t rows;  /* R = B*N positions (Section III-A flattens batch and sequence) */
    int64_t vocab; /* V items */
    int64_t nnz;   /* length of item_ids */
    int32_t dim;   /* D */
    int32_t dtype; /* cutbce_dtype */
} cutbce_problem;

/* Bytes of device workspace that cutbce_forward and cutbce_backward need for this problem (host call).
 * Grows with V*D (one re-laid-out copy of E for the forward's gradient GEMM), R*D and nnz; never with R*V. */
cutbce_status cutbce_workspace_size(const cutbce_problem *p, size_t *bytes);

/* Forward (Section III-A, Eq. (2)-(3); Section III-C's forward sweep over vocabulary blocks).
 *   row_weight (device) float [R] or NULL: the weights w_r of the rows (finite, >= 0; read for valid rows
 *             only). NULL weighs every valid row 1. A valid row of weight 0 adds nothing but is still swept.
 *   loss      (device) float [1]: the scalar loss above.
 *   row_loss  (device) float [R] or NULL: sum_v [softplus(z_rv) - y_rv z_rv] per valid row (neither weighted
 *             nor divided by W*V), 0 for masked rows.
 *   dh_saved  (device) float [R][D] or NULL: when given, the same sweep also forms
 *             s * w_r * sum_v (sigma(z_rv) - y_rv) E[v] (the dH of Eq. (4) for g = 1; 0 for masked rows) so
 *             that cutbce_backward can return dH without recomputing the logits for it.
 *   metrics   (device) int32 [R][4] or NULL: Cut Metrics (Section III-D), counted in the same sweep from the
 *             same float32 logits: TP, FP, FN, TN over the V items of each valid row, an item being predicted
 *             positive iff z_rv > 0 (the section names no threshold: sigma(z) > 1/2 is used); all four are 0
 *             for masked rows. A repeated id counts once; ids outside [0, V) are not positives.
 * Numerics (bf16, D <= 128): rows whose logits are all bounded by 0.8 in magnitude (checked per group of 32 rows
 * through max ||H[r]|| * max ||E[v]||) take the loss terms and sigma(z) - 1/2 from truncated alternating series
 * (error at most 1.4e-5 of each loss term, 2.9e-6 absolute on the logit gradient); other rows use exp / log.
 */
cutbce_status cutbce_forward(const cutbce_problem *p, const void *H, const void *E,
                             const int32_t *row_offsets, const int32_t *item_ids, const uint8_t *row_mask,
                             const float *row_weight, float *loss, float *row_loss, float *dh_saved,
                             int32_t *metrics, void *workspace, size_t workspace_bytes, void *stream);

/* Size of the scratch array behind cutbce_forward_noalloc (per GPU). */
#define CUTBCE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* cutbce_forward for callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, computation and outputs as cutbce_forward, except that
 * the workspace is a device array of the library, CUTBCE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held until
 * the process ends; nothing is allocated. Its device address is looked up on the first call on each device
 * (hipGetSymbolAddress), so a caller that captures should make one call on the device before capturing.
 * Errors as for cutbce_forward, and CUTBCE_ERR_WORKSPACE when cutbce_workspace_size() of the problem exceeds
 * the array (roughly: R * D * 4 * (vocabulary splits, up to 64) plus 2 * V * D + O(R * D + nnz) bytes).
 * All calls on one GPU share the array and each leaves its contents behind: calls that may overlap on a GPU
 * (several streams, or several host threads) race and must be serialised by the caller. */
cutbce_status cutbce_forward_noalloc(const cutbce_problem *p, const void *H, const void *E,
                                     const int32_t *row_offsets, const int32_t *item_ids,
                                     const uint8_t *row_mask, const float *row_weight, float *loss,
                                     float *row_loss, float *dh_saved, int32_t *metrics, void *stream);

/* Backward (Section III-B, Eq. (4); the custom VJP recomputes logit tiles on chip).
 *   row_weight (device) float [R] or NULL: as for cutbce_forward (the same weights as the forward call).
 *   grad_loss (device) float [1]: the cotangent g.
 *   dh_saved  (device) float [R][D] or NULL: the forward's dh_saved for these same inputs. When NULL and dH
 *             is requested, dH is computed here by recomputing the logits.
 *   dH        (device) [R][D] in the element type, or NULL to skip: overwritten with g * (dH of Eq. (4)).
 *   dE        (device) [V][D] in the element type, or NULL to skip: overwritten with g * (dE of Eq. (4)).
 */
cutbce_status cutbce_backward(const cutbce_problem *p, const void *H, const void *E,
                              const int32_t *row_offsets, const int32_t *item_ids, const uint8_t *row_mask,
                              const float *row_weight, const float *grad_loss, const float *dh_saved, void *dH,
                              void *dE, void *workspace, size_t workspace_bytes, void *stream);

/* cutbce_backward after the cutbce_forward it belongs to, on the same workspace: the backward of a training step
 * (Section III-B's custom VJP), reusing the row compaction (valid rows, their weights and id ranges, s) and the H
 * preparation (compacted rows, column sums, row norms) that cutbce_forward left in the workspace instead of
 * recomputing them. Arguments, outputs and errors as for cutbce_backward, and the results are the same bits.
 * Precondition (not checkable without a host synchronisation): the last call on `workspace` was cutbce_forward
 * with the same problem, H, row_offsets, item_ids, row_mask and row_weight, none of which has changed since (E is
 * not part of what is reused; the forward need not have been given dh_saved). If the precondition
 * does not hold the gradients are wrong, but every read stays inside the arrays and every loop ends: the kernels
 * clamp the valid-row count to R and the id ranges to [0, nnz]. */
cutbce_status cutbce_backward_reuse(const cutbce_problem *p, const void *H, const void *E,
                                    const int32_t *row_offsets, const int32_t *item_ids, const uint8_t *row_mask,
                                    const float *row_weight, const float *grad_loss, const float *dh_saved,
                                    void *dH, void *dE, void *workspace, size_t workspace_bytes, void *stream);

/* Device-side check of the targets: writes to *bad (device int32) the number of ids outside [0, V) plus
 * the number of rows whose offsets decrease, plus 1 if row_offsets[0] != 0 or row_offsets[R] > nnz (ids are
 * checked up to min(row_offsets[R], nnz)).
 * 0 means the targets are well formed. Needs no workspace. */
cutbce_status cutbce_validate_targets(const cutbce_problem *p, const int32_t *row_offsets,
                                      const int32_t *item_ids, int32_t *bad, void *stream);

/* Full-vocabulary top-k scoring (the evaluation of Section III-E: hidden states projected onto every item, items
 * ranked, Hit@k). For each valid row r, the k items with the largest logits z_rv = H[r] . E[v], ranked by logit
 * (descending) and, among equal logits, by item id (ascending); the logits are never written to memory.
 *   k          1 <= k <= 8 and k <= V.
 *   top_vals   (device) float [R][k], written: the float32 logits of the ranked items; -inf for masked rows.
 *   top_ids    (device) int32 [R][k], written: the ranked item ids; -1 for masked rows.
 *   hits       (device) int32 [R] or NULL: how many of the row's k items are among its positives (row_offsets /
 *              item_ids as in cutbce_forward; a repeated id counts once). Hit@k of a set of rows is the fraction
 *              with hits > 0. 0 for masked rows.
 * Uses the same workspace as cutbce_forward. Errors as for cutbce_forward; SHAPE for k out of range. */
cutbce_status cutbce_topk(const cutbce_problem *p, const void *H, const void *E, const int32_t *row_offsets,
                          const int32_t *item_ids, const uint8_t *row_mask, int32_t k, float *top_vals,
                          int32_t *top_ids, int32_t *hits, void *workspace, size_t workspace_bytes, void *stream);

/* Dense padded targets -> CSR positives (the [B, N, L] target slots of the paper's Listing 1).
 *   rows        R = B*N rows; slots L >= 0 id slots per row.
 *   targets     (device) int32 [R][L], row-major; a slot equal to pad_id is padding and is dropped.
 *   row_offsets (device) int32 [R+1], written: row_offsets[0] = 0, row_offsets[r+1] - row_offsets[r] = kept
 *               slots of row r; row_offsets[R] = nnz, the number of kept slots.
 *   item_ids    (device) int32 [R*L] (capacity), written: the kept ids of each row in slot order, rows in order;
 *               entries from nnz on are left untouched. Repeated ids are kept (the loss counts them once).
 * Errors: SHAPE when R < 1, L < 0 or R*L >= 2^31; NULL for a missing pointer; ALIGN for a pointer that is not
 * 4-byte aligned. Needs no workspace; asynchronous on `stream`. */
cutbce_status cutbce_targets_to_csr(int64_t rows, int32_t slots, const int32_t *targets, int32_t pad_id,
                                    int32_t *row_offsets, int32_t *item_ids, void *stream);

/* Opt-in kernel timing for benchmarks (host calls). While enabled, every launch of the logit-tile sweeps
 * (kind 0: forward rows sweep, kind 1: backward dE sweep, kind 2: the scoring sweep of cutbce_topk) is
 * bracketed by HIP events recorded on the launch stream. cutbce_profile_read waits for those events and
 * returns, per kind, the summed milliseconds and the number of launches since the last enable/read, then
 * clears them. Besides the launch data cached per kernel and device (see the conventions above), this is the
 * only state the library keeps across calls; it is off by default. Enabling (on != 0) clears previous records; at most 65536 launches are
 * recorded (later ones are not timed). Not thread-safe. */
cutbce_status cutbce_profile_enable(int on);
cutbce_status cutbce_profile_read(double *ms, int64_t *launches, int n_kinds);

/* MFMA-only ceiling of the device (a measurement, not part of the loss): launches `blocks` workgroups of
 * `waves_per_block` waves (1..16), each wave running `iters` rounds of four independent
 * v_mfma_f32_32x32x16_bf16 -- the sweeps' instruction -- on register operands, with no memory traffic.
 * One round is 4 * 32768 flops. Lane 0 of wave w writes stamps[4w .. 4w+3] = (s_memtime before, after,
 * s_memrealtime before, after): shader-clock ticks and 100 MHz reference ticks, so the clock the device held is
 * 0.1 GHz * (t1 - t0) / (r1 - r0).
 *   stamps (device) int64 [4 * blocks * waves_per_block], 8-byte aligned.
 * Errors: SHAPE for counts out of range, NULL, ALIGN. Asynchronous on `stream`. */
cutbce_status cutbce_mfma_ceiling(int blocks, int waves_per_block, int iters, long long *stamps, void *stream);

/* The same ceiling on random operands (a measurement, not part of the loss): each wave holds four register sets
 * of random bf16 values in [-1, 1), one per accumulator tile, like the sweeps' operand tiles; the multipliers'
 * power on such values lowers the clock the device holds. Arguments, stamps, flops per round and errors as for
 * cutbce_mfma_ceiling. */
cutbce_status cutbce_mfma_ceiling_random(int blocks, int waves_per_block, int iters, long long *stamps,
                                         void *stream);

/* Static description of a status code (host). */
const char *cutbce_status_string(cutbce_status s);

/* Library version as major*10000 + minor*100 + patch (host). 0.2.0 added row_weight to cutbce_forward and
 * cutbce_backward. */
int cutbce_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CUTBCE_H */
