/*
 * sdm.h — C ABI of the MI355X (gfx950) chunked sparse-delta-memory (SDM) forward.
 *
 * The operation. P streams each own a bank of M rows by head_dim columns. Every token
 * writes W weighted slots and then reads R weighted slots:
 *     each written row decays by exp(log_decay), the retrieved vector is the weighted
 *     sum of the decayed written rows, the write error is beta * (v - retrieved), each
 *     written row gains weight * error, and the reading is the weighted sum of the read
 *     rows after the write.
 * This is the per-token definition in the SDMWriteRead class docstring (memory_ops.py,
 * sparse-delta-memory 2.0.0 wheel, diffend page 21). The library computes it in the
 * chunked three-part form of that module's docstring: Phase 1 (per-slot log-decays,
 * dedup groups, gather weights, Gram matrices A and QK), the solve
 * X = (I + tril(beta A, -1))^-1, QX = QK X (wy_solve.py docstring, page 23), and Phase 2,
 * Nt sequential steps of gather, dual matmul and decay-and-write (phase2_kernels.py
 * docstring, page 23).
 *
 * Conventions shared by every entry point:
 *   - Pointers named "device" are HIP device (or managed) memory on the current device;
 *     the library never dereferences them on the host, never allocates device memory
 *     and never synchronizes. Work is enqueued on exec->stream (a hipStream_t; NULL is
 *     the null stream) and runs asynchronously; a fault in it surfaces at the caller's
 *     next synchronization.
 *   - All arrays are dense row-major with no padding. Token arrays are stream-major:
 *     element (p, t, j) of a [P, T, J] array sits at ((p * T) + t) * J + j.
 *   - Every argument is checked on the host before anything is enqueued; on a failed
 *     check nothing is enqueued and a negative SDM_ERR_* code is returned
 *     (sdm_last_error() then describes it). The pages raise TypeError / ValueError /
 *     UnsupportedConfigurationError before any work for the same classes of mistakes
 *     (_layout and _admit in memory_ops.py, page 21).
 *   - Caller contract NOT checked (it would need a device read): every slot id lies in
 *     [0, M), and the W write slots of a token are distinct (sdm_write_read's docstring
 *     requires distinct write slots). A violation gives unspecified (but in-bounds for
 *     reads of ids in range) results.
 *   - Results are bitwise reproducible for fixed inputs and shapes on one GPU type: every
 *     bank element has one writer per step and every sum runs in a fixed order (the
 *     determinism contract of memory_ops.py and phase2_kernels.py). A stream's results do
 *     not depend on the other streams, on the column slicing, or on the workspace size.
 *   - Calls that share a workspace or a bank must be ordered on one stream.
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SDM_OK = 0,
    SDM_ERR_DTYPE = -1,       /* bank dtype not SDM_F32 / SDM_BF16 */
    SDM_ERR_SHAPE = -2,       /* P, T, W, R, head_dim, M < 1; W or R > 256; gate width not 1 or W */
    SDM_ERR_RANGE = -3,       /* chunk outside [16, 256]; P*M >= 2^31 rows; P*Nt*C >= 2^31; head_dim > 2^20 */
    SDM_ERR_NULL = -4,        /* a required pointer is NULL */
    SDM_ERR_ALIGN = -5,       /* a device pointer is not aligned to its element size (16 B for vector rows) */
    SDM_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than one step needs */
    SDM_ERR_UNSUPPORTED = -7, /* no kernel plan for this shape on this device */
    SDM_ERR_HIP = -8          /* a HIP runtime call failed (launch, attribute query) */
};

typedef enum { SDM_F32 = 0, SDM_BF16 = 1 } sdm_dtype;

/* Slot ids, device int32 or int64 (sdm_write_read takes either, page 21, memory_ops.py,
 * _layout). write: [P, T, W]; read: [P, T, R]. Rows in [0, M) of the stream's bank, or of
 * the one bank in shared mode (sdm_bank.shared).
 * write_id_bytes, read_id_bytes: 4 (int32; 0 means 4) or 8 (int64); an int64 id must lie in
 * [0, M) like an int32 one (not checked on the device). */
typedef struct {
    const void *write;
    const void *read;
    int32_t W;
    int32_t R;
    int32_t write_id_bytes;
    int32_t read_id_bytes;
} sdm_slots;

/* Slot weights, device, in the bank dtype. write: [P, T, W] (k_val); read: [P, T, R] (q_val). */
typedef struct {
    const void *write;
    const void *read;
} sdm_weights;

/* The bank, device, in dtype; read and advanced in place to its final state.
 * shared = 0: [P, rows, head_dim]; stream p owns rows [p * rows, (p + 1) * rows) of the
 *   flat [P * rows, head_dim] array (sdm_write_read's per-stream slot ranges,
 *   num_memory_slots = rows).
 * shared = 1: one [rows, head_dim] bank read and written by every stream (sdm_write_read
 *   with shared_bank=True, page 21, memory_ops.py docstring): the streams' slot sets must
 *   be disjoint over the whole call (caller contract, not checked). */
typedef struct {
    void *data;
    int64_t rows;
    int32_t head_dim;
    int32_t dtype; /* sdm_dtype */
    int32_t shared;
} sdm_bank;

/* Where and with what scratch the call runs. stream: hipStream_t (NULL = null stream).
 * workspace: device scratch of workspace_bytes, 256-byte aligned, owned by the caller,
 * no initial contents required; the call uses the largest slab of steps that fits.
 * events: optional (NULL = none) array of num_events >= SDM_TIMING_EVENTS hipEvent_t
 * created by the caller; sdm_fwd then records them on `stream` at the kernel boundaries
 * of its first slab, in order: before the radix sort, before the group scan, before the
 * read lookup, before the cold-pair Gram kernel, before the dense (hot-slot) Gram kernel,
 * before the solve, before Phase 2, after Phase 2.
 * Recording is asynchronous; the caller reads the elapsed times after synchronizing. */
typedef struct {
    void *stream;
    void *workspace;
    size_t workspace_bytes;
    void **events;
    int32_t num_events;
    /* optional device int64 counter (NULL = none): sdm_fwd adds the number of live write
     * entries that repeat a slot of their own token (the counter sdm_write_read keeps for
     * repeated_write_slots, page 21, memory_ops.py; such calls break the distinct-slots
     * contract and their results are unspecified). Ordered on `stream`; the caller zeroes
     * and reads it. */
    int64_t *repeated_writes;
    /* CUs the Phase-2 launch geometry may plan for (0 = all of the device; larger values are
     * clamped to it; negative is SDM_ERR_SHAPE). sdm_fwd and sdm_fwd_phase2 size their
     * column slices so that Phase 2's workgroups fill this many CUs; a caller that runs
     * another batch's sdm_fwd_phase1 beside this Phase 2 can leave that Phase 1 the rest of
     * the device. Results never depend on it. Ignored by the other entry points. */
    int32_t phase2_cus;
} sdm_exec;

#define SDM_TIMING_EVENTS 8

/*
 * Workspace bytes sdm_fwd needs to run its steps in slabs of `slab_steps` steps
 * (0 = all Nt = ceil(tokens / chunk) steps in one slab). A slab holds every Phase-1
 * quantity and both solve outputs of its P * slab_steps chunks (112 B per write entry,
 * 24 B per read entry, 16 B per chunk-matrix element, a slot search index of up to
 * 64 KiB and dense hot-slot operands of up to 12 * chunk * 256 B per chunk) (the pages
 * budget the same kinds of state, SLAB_BYTES in memory_ops.py).
 * Returns 0 for arguments sdm_fwd would reject with SDM_ERR_SHAPE or SDM_ERR_RANGE.
 * Results never depend on the slab size.
 */
size_t sdm_fwd_workspace_bytes(int32_t streams, int32_t tokens, int32_t chunk, int32_t W, int32_t R,
                               int32_t head_dim, int32_t slab_steps);

/*
 * The SDM forward (sdm_write_read's no-grad forward, memory_ops.py, page 21).
 *   streams P >= 1, tokens T >= 1, chunk C in [16, 256] (T need not be a multiple of C).
 *   slots, weights: as above. beta: device float32 [P, T]. log_decay: device float32
 *   [P, T, gate_width], gate_width 1 (one log-decay per token, applied to each of its
 *   writes) or W (one per write slot).
 *   v: device [P, T, head_dim] in the bank dtype. bank: in/out.
 *   valid_tokens: device int32 [P], each in [0, T], or NULL (= T for every stream).
 *     Tokens t >= valid_tokens[p] are padding: they touch no bank row and read 0.
 *   out: device [P, T, head_dim] in the bank dtype; every element is written (padding
 *     rows +0). out must not overlap the bank or any input.
 * Arithmetic: inputs widened to float32; accumulation in float32; the readings and each
 * written bank row are rounded once to the bank dtype (round to nearest even for bf16).
 */
int sdm_fwd(int32_t streams, int32_t tokens, int32_t chunk, const sdm_slots *slots,
            const sdm_weights *weights, const float *beta, const float *log_decay,
            int32_t gate_width, const void *v, const sdm_bank *bank,
            const int32_t *valid_tokens, void *out, const sdm_exec *exec);

/*
 * sdm_fwd for callers that cannot allocate (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc): the same arguments, checks and result bits as sdm_fwd,
 * but the workspace is a static device array inside the library, SDM_NOALLOC_SCRATCH_BYTES
 * on each GPU it runs on (held from the library's first call on that device until the
 * process ends). exec->workspace must be NULL and exec->workspace_bytes 0; the other exec
 * fields are as for sdm_fwd. The call uses the largest slab of steps that fits the scratch;
 * shapes whose single step needs more (sdm_fwd_workspace_bytes(..., 1) > the scratch size)
 * are refused with SDM_ERR_WORKSPACE before any work. Nothing is allocated and the
 * scratch needs no initial contents (it keeps the last call's). Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (different streams with no
 * ordering between them) race and give undefined results.
 */
#define SDM_NOALLOC_SCRATCH_BYTES (64u << 20)
int sdm_fwd_noalloc(int32_t streams, int32_t tokens, int32_t chunk, const sdm_slots *slots,
                    const sdm_weights *weights, const float *beta, const float *log_decay,
                    int32_t gate_width, const void *v, const sdm_bank *bank,
                    const int32_t *valid_tokens, void *out, const sdm_exec *exec);

/*
 * The forward in two calls, for callers that overlap the Phase 1 of one batch with the
 * Phase 2 of another (Phase 1 reads only the slot ids, weights, gates, beta and
 * valid_tokens, never the bank, v or out). Both take exactly sdm_fwd's arguments and
 * checks; exec->workspace must hold all Nt steps (sdm_fwd_workspace_bytes(..., 0)), else
 * SDM_ERR_WORKSPACE; exec->events is ignored.
 * sdm_fwd_phase1: Phase 1 and the solve for every chunk, into the workspace (and the
 *   repeated-writes counter); v, bank->data and out are not accessed (may be NULL).
 * sdm_fwd_phase2: Phase 2 from that workspace; the caller orders it after the
 *   sdm_fwd_phase1 call with the same arguments and workspace (same stream, or an event),
 *   and keeps the workspace unchanged between the two. Phase 2 keeps bookkeeping of its
 *   own in the workspace: every sdm_fwd_phase2 call needs an sdm_fwd_phase1 call of its
 *   own before it.
 * The pair computes exactly sdm_fwd's result (same bits).
 */
int sdm_fwd_phase1(int32_t streams, int32_t tokens, int32_t chunk, const sdm_slots *slots,
                   const sdm_weights *weights, const float *beta, const float *log_decay,
                   int32_t gate_width, const void *v, const sdm_bank *bank,
                   const int32_t *valid_tokens, void *out, const sdm_exec *exec);
int sdm_fwd_phase2(int32_t streams, int32_t tokens, int32_t chunk, const sdm_slots *slots,
                   const sdm_weights *weights, const float *beta, const float *log_decay,
                   int32_t gate_width, const void *v, const sdm_bank *bank,
                   const int32_t *valid_tokens, void *out, const sdm_exec *exec);

/*
 * Phase 1 and the solve only, for every chunk, into caller buffers (for checking the
 * intermediates; sdm_fwd keeps them in its workspace). Chunk (p, ti) is n = p * Nt + ti.
 *   rows, head_dim, dtype: the bank the call would run on (rows bounds the ids; dtype is
 *   the weights' dtype).
 *   A, QK, X, QX: device float32 [P * Nt, C, C]. A: strict lower triangle of the
 *   decay-weighted write x write Gram matrix, +0 elsewhere; QK: lower triangle (diagonal
 *   included) of the read x write Gram matrix, +0 above; X = (I + tril(beta A, -1))^-1,
 *   QX = QK X, both +0 above the diagonal (wy_solve.py docstring, page 23).
 *   gw: device float32 [P * Nt, C, W] gather weights k * exp(L) of the write entries;
 *   gr: device float32 [P * Nt, C, R] gather weights q * exp(L) of the read entries;
 *   0 for padding tokens.
 *   exec->workspace must hold sdm_fwd_workspace_bytes(..., slab_steps = 1).
 */
int sdm_chunk_mats(int32_t streams, int32_t tokens, int32_t chunk, const sdm_slots *slots,
                   const sdm_weights *weights, const float *beta, const float *log_decay,
                   int32_t gate_width, int64_t rows, int32_t head_dim, int32_t dtype,
                   const int32_t *valid_tokens, float *A, float *QK, float *X, float *QX,
                   float *gw, float *gr, const sdm_exec *exec);

/*
 * Phase 1's integer records of every chunk, verbatim (for checking the grouping, dedup and
 * read lookups exactly; sdm_fwd keeps them in its workspace). Same arguments and checks as
 * sdm_chunk_mats; E = chunk * W, F = chunk * R; chunk (p, ti) is n = p * Nt + ti.
 *   meta: device int32 [P * Nt, 8]: live tokens, live write entries, write groups (the
 *     writes of one slot in the chunk), hot groups, groups of at least 16 members, the hot
 *     count rounded up to 16, -, 1 if the chunk's Phase 1 sorted every write entry in memory
 *     (else it ran in LDS slot partitions).
 *   spk: device int32 [P * Nt, E, 4]: the write entries in group order, each group's members
 *     in token order (positions < live write entries): {slot, token, bits of k, bits of L}.
 *   grec: device int32 [P * Nt, E, 4]: group g < meta[2]: {slot, first member's position |
 *     (members - 1) << 16 | first member's token << 24, bits of exp(L_last), bits of the first
 *     member's k exp(L_last - L)}.
 *   ecr: device int32 [P * Nt, C, W, 4]: live write entry (t, w) at position m: {position of
 *     its group's first member, m, bits of k, bits of L}, or {m, m, 0, 0} if its group is hot
 *     (its pair terms go to the dense products).
 *   rcr: device int32 [P * Nt, C, R, 4]: read entry (t, r) whose slot has a write at a token
 *     <= t in a group that is not hot: {first member's position, 1 + position of the latest
 *     such write, bits of q, bits of that write's L}; otherwise zeros.
 * Entries past meta[1] / meta[2] and of padding tokens are unspecified (rcr: zeros).
 */
int sdm_chunk_records(int32_t streams, int32_t tokens, int32_t chunk, const sdm_slots *slots,
                      const sdm_weights *weights, const float *beta, const float *log_decay,
                      int32_t gate_width, int64_t rows, int32_t head_dim, int32_t dtype,
                      const int32_t *valid_tokens, int32_t *meta, int32_t *spk, int32_t *grec,
                      int32_t *ecr, int32_t *rcr, const sdm_exec *exec);

/*
 * The per-chunk solve on its own (wy_solve, wy_solve.py, page 23):
 *   X = (I + tril(beta[:, None] * A, -1))^-1 and QX = QK @ X for each of n chunks.
 *   A, QK: device float32 [n, C, C]; only the strict lower triangle of A and the lower
 *   triangle (diagonal included) of QK are read. beta: device float32 [n, C].
 *   X, QX: device float32 [n, C, C], +0 above the diagonal; must not overlap the inputs
 *   (not checked).
 *   C in [1, 256]. exec->workspace is not used (may be NULL).
 */
int sdm_wy_solve(int64_t n, int32_t chunk, const float *A, const float *beta, const float *QK,
                 float *X, float *QX, const sdm_exec *exec);

/*
 * The launch plan sdm_fwd takes for these shapes on the current device, for reports and
 * tuning (the results never depend on it). It assumes 16-byte aligned v, bank and out, as
 * sdm_fwd does when it picks `vec`. Returns SDM_OK, or the error sdm_fwd would return for
 * these shapes (SDM_ERR_SHAPE, SDM_ERR_RANGE, SDM_ERR_DTYPE), or SDM_ERR_HIP.
 */
typedef struct {
    int32_t vec;               /* bank elements per vector access: 16 bytes' worth (4 float32,
                                  8 bfloat16); 4 bfloat16 (8 bytes) when a bank slice held in
                                  LDS is narrowed to 4 columns because one 16-byte vector per
                                  slice would still leave more than half of the CUs idle; 1 when
                                  head_dim is not a multiple of the 16-byte count */
    int32_t slice_vectors;     /* vectors per column slice of Phase 2 */
    int32_t slices;            /* column slices per stream */
    int32_t phase2_mode;       /* 0: Phase-2 arrays and bank rows read from memory; 1: the chunk's
                                  Phase-2 block staged in LDS; 2: staged, and the workgroup's
                                  column slice of the bank held in LDS for the whole call */
    int32_t phase2_lds_bytes;  /* LDS per Phase-2 workgroup */
    int32_t phase1_fused;      /* 1: Phase 1 and the solve run as one kernel, one workgroup per chunk */
    int32_t phase1_partitions_log2; /* >= 0: chunks not fused run Phase 1 in 2^this slot partitions
                                  held in LDS one after another (one workgroup per chunk); -1: by
                                  sorting every write entry of a chunk in memory */
    int32_t lds_limit;         /* LDS bytes per workgroup the plan may use */
    int32_t lds_default;       /* the device's default per-workgroup LDS limit */
    int32_t phase2_team;       /* workgroups per (stream, slice): Phase 2 runs streams * slices *
                                  phase2_team workgroups; 2 or 4 (memory mode only) split each
                                  chunk's tokens and DW groups among them, exchanging u through
                                  the workspace */
} sdm_plan;

int sdm_fwd_plan(int32_t streams, int32_t tokens, int32_t chunk, int32_t W, int32_t R, int32_t head_dim,
                 int64_t rows, int32_t dtype, sdm_plan *plan);

/*
 * Exact top-k over all sums of one value from each product-key factor (product_key_topk,
 * page 23, product_key_topk.py docstring): the slot selection that feeds write and read
 * slot ids.
 *   raw: device [rows, sum(factors)] in dtype (SDM_F32 or SDM_BF16), the factors side by
 *     side. factors: HOST array of num_factors (1..8) widths, each 1..65535 columns (the
 *     pages' two- to four-factor kernels take up to 65535), their product below 2^55.
 *     k: 1..256; kk = min(k, product of the factors).
 *   val: device [rows, kk] in dtype: the selected slots' scores (float32 sums of their
 *     factor values in factor order; bfloat16 with more than two factors rounds each
 *     partial sum to bfloat16 before the next factor), rounded to dtype.
 *   lin: device int64 [rows, kk]: the selected slots (c_0 .. c_{F-1}) as
 *     (..(c_0 factors[1] + c_1) ..) factors[F-1] + c_{F-1}, strictly ascending per row.
 *   Selection (exact ties included): (1) scores compare as float32 with negative zero
 *   beneath positive zero and NaN as negative infinity; (2) a factor's columns are ordered
 *   by value, highest first, the higher column index first among equal values; (3) stage
 *   f >= 1 pairs a surviving rank i < n with a rank j < m = min(k, factors[f]) of factor f
 *   where (i + 1)(j + 1) <= c = min(k, n m) and keeps the c best; an exact tie goes to the
 *   greater i + j, then to the greater i.
 *   exec->stream only (no workspace). rows = 0 does nothing. Returns SDM_OK or a negative
 *   SDM_ERR_* before any launch (SDM_ERR_UNSUPPORTED for factors past the limits).
 */
int sdm_product_key_topk(int64_t rows, const void *raw, int32_t dtype, const int32_t *factors,
                         int32_t num_factors, int32_t k, void *val, int64_t *lin,
                         const sdm_exec *exec);

/*
 * The sparse backward of sdm_product_key_topk (the pages' top-k is differentiable in raw,
 * with a deterministic backward, page 23, product_key_topk.py): the gradient of a raw column
 * is the sum of grad_val over the selected slots that use it (d val / d raw is 1 at each
 * factor column of a slot; roundings pass the gradient through). Sums run in float32 over
 * the slots in their output order (ascending lin), rounded once to dtype.
 *   lin: device int64 [rows, kk] as returned by sdm_product_key_topk (entries must be below
 *   the slot count; not checked). grad_val: device [rows, kk] in dtype. grad_raw: device
 *   [rows, sum(factors)] in dtype, every element written. factors, num_factors: as for the
 *   forward; kk: 1..min(256, slot count). exec->stream only.
 */
int sdm_product_key_topk_backward(int64_t rows, const int64_t *lin, const void *grad_val, int32_t dtype,
                                  const int32_t *factors, int32_t num_factors, int32_t kk, void *grad_raw,
                                  const sdm_exec *exec);

/*
 * The backward of sdm_fwd (sdm_write_read is differentiable in the slot weights, v, beta,
 * the log-decays and the bank: SDMWriteRead, page 21, memory_ops.py; the pages name their
 * backward's stages without listing them, so this is the derivative of the per-token loop
 * that defines the forward, evaluated in float32). For the objective
 *     J = sum(grad_out * readings) + sum(grad_bank_final * final bank)
 * it returns dJ/d(each float input) at the given inputs:
 *   grads->bank       [P, rows, head_dim] ([rows, head_dim] for a shared bank)
 *                     in: grad_bank_final (zeros for none);
 *                     out: the gradient w.r.t. the bank the forward started from
 *   grads->v          [P, T, head_dim]
 *   grads->beta       [P, T]
 *   grads->log_decay  [P, T, gate_width]
 *   grads->write      [P, T, W]   (write slot weights)
 *   grads->read       [P, T, R]   (read slot weights)
 * All device float32 whatever the bank dtype, every element written (padding tokens:
 * zeros); none may overlap an input. slots, weights, beta, log_decay, gate_width, v,
 * valid_tokens: exactly as given to sdm_fwd (weights and v in the bank dtype).
 * grad_out: device [P, T, head_dim] in the bank dtype.
 * bank: as for sdm_fwd (float32 or bfloat16; per stream, or shared with the streams' slot
 * sets disjoint), holding the bank the forward STARTED from. The call replays the forward
 * on it in float32 and walks it back, restoring every written row from a saved copy: a
 * float32 bank is used as the working state and holds exactly its entry contents again on
 * return; a bfloat16 bank is only read (its rows are widened into float32 working rows).
 * exec->workspace: sdm_bwd_workspace_bytes(...) bytes, 256-byte aligned (it keeps each
 * write entry's row as it was before its token, 4 * W * head_dim bytes per token (2 with
 * bfloat16 snapshot rows), rounded
 * up to whole column slices of 4..64 columns, plus 8 * R bytes per token, one float per
 * token, column slice and dot product, and for a bfloat16 bank the float32 working rows,
 * 4 * head_dim bytes per bank row).
 * snapshot_quant: storage of the saved rows (the snapshot the pages' sdm_write_read keeps
 *   for its backward, argument snapshot_quant, page 21, memory_ops.py):
 *   SDM_SNAP_NONE  float32 rows; the bank is restored exactly.
 *   SDM_SNAP_BF16  on a float32 bank, bfloat16 rows (round to nearest even, half the snapshot
 *                  bytes): the reverse sweep recomputes each token's decayed rows from the
 *                  widened bfloat16 rows and restores every written bank row to them, so the
 *                  bank holds, on return, its entry rows rounded to bfloat16 where the forward
 *                  wrote them (its other rows exactly); a bfloat16 bank runs it as NONE.
 *   SDM_SNAP_FP8, SDM_SNAP_INT4  refused with SDM_ERR_UNSUPPORTED (the pages fix their row
 *                  widths, head_dim bytes of float8_e4m3fn and (head_dim + 1) / 2 bytes, not
 *                  how values are scaled into them); any other value is SDM_ERR_SHAPE.
 * exec->events: optional, num_events >= SDM_BWD_TIMING_EVENTS hipEvent_t recorded on the
 * stream before the read-slot fold, before the replay-and-reverse sweep, before the
 * reduction of the per-slice dots, and after it. exec->repeated_writes is not used.
 * Sums run in a fixed order: results are bitwise reproducible. Errors as for sdm_fwd.
 */
#define SDM_BWD_TIMING_EVENTS 4
#define SDM_SNAP_NONE 0
#define SDM_SNAP_FP8 1
#define SDM_SNAP_INT4 2
#define SDM_SNAP_BF16 3

typedef struct {
    float *bank;
    float *v;
    float *beta;
    float *log_decay;
    float *write;
    float *read;
} sdm_grads;

/* Workspace bytes sdm_bwd needs for these shapes, bank rows (per stream, or of the shared
 * bank), bank dtype, sharing and snapshot mode (0 for arguments sdm_bwd rejects with
 * SDM_ERR_SHAPE, SDM_ERR_RANGE, SDM_ERR_DTYPE or SDM_ERR_UNSUPPORTED). */
size_t sdm_bwd_workspace_bytes(int32_t streams, int32_t tokens, int32_t W, int32_t R, int32_t head_dim,
                               int64_t rows, int32_t dtype, int32_t shared, int32_t snapshot_quant);

int sdm_bwd(int32_t streams, int32_t tokens, const sdm_slots *slots, const sdm_weights *weights,
            const float *beta, const float *log_decay, int32_t gate_width, const void *v,
            const sdm_bank *bank, const int32_t *valid_tokens, const void *grad_out,
            const sdm_grads *grads, int32_t snapshot_quant, const sdm_exec *exec);

/* Static text for an SDM_* code. */
const char *sdm_error_string(int code);

/* Description of the last error returned on the calling thread ("" if none). */
const char *sdm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H */
