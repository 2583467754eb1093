/*
 * lora.h — C ABI of the MI355X (gfx950) LoRA low-rank-adapter library.
 *
 * The library computes the LoRA hot path on one AMD GPU with hand-written HIP
 * kernels:
 *   - single adapter, forward and backward, as defined by the API pages
 *     "nemo_automodel.components._peft.lora_kernel" (NeMo Automodel):
 *     lora_forward_kernel / lora_forward_wrapper, lora_da_dx_kernel /
 *     lora_da_dx_update_wrapper, lora_db_kernel / lora_db_update_wrapper;
 *   - slot-addressed multi-adapter serving ops, as defined by the API page
 *     "mstar.engine.resources.lora.ops" (M* engine), class LoraOpsBackend:
 *     shrink, expand_fused, gather_shrink.
 *
 * Conventions (all entry points):
 *   - Every tensor pointer is a DEVICE pointer. Sizes, strides, out_slices and
 *     the descriptors themselves live in host memory.
 *   - Strides are in ELEMENTS (as in the pages' stride_*_m / stride_*_k pairs).
 *   - The caller owns every buffer, including the workspace. The library keeps
 *     no state between calls, allocates nothing, never synchronises the stream
 *     and never reads device data on the host.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream). Results are ready when the stream reaches that point.
 *   - Return value: LORA_OK (0) or a negative LORA_ERR_* code. Every argument
 *     check happens on the host BEFORE any launch; a failing call launches
 *     nothing and touches no buffer. LORA_ERR_LAUNCH reports a HIP launch error
 *     (hipGetLastError after the launches).
 *   - Empty problems (M, K, L or T equal to 0) launch nothing and return
 *     LORA_OK (with K = 0 the forward adds zero, i.e. leaves res unchanged; the
 *     backward then writes zero gradients where they have nonzero size).
 *   - Reductions run in a fixed order: results are bitwise reproducible from
 *     run to run for the same inputs and shapes.
 *   - Floating-point inputs are bfloat16 or float32 (all inputs of one call have
 *     the same dtype); accumulation is float32; every output is float32 (the
 *     pages' wrappers default to dtype=torch.float32).
 *   - Data anomalies that the host cannot see (slot ids outside [0, S), ranks
 *     outside [0, r_max], token ids outside [0, V)) are defined behaviour, not
 *     errors: such tokens, rank rows or ids add no term.
 */
#ifndef LORA_MI355X_LORA_H
#define LORA_MI355X_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 1

/* Element types. */
typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/* Status codes. */
enum {
  LORA_OK = 0,
  LORA_ERR_NULL = -1,      /* a required pointer is NULL */
  LORA_ERR_SHAPE = -2,     /* operand shapes disagree, a size is negative or unsupported, or an
                              operand (dims and strides) spans more than 2^47 bytes or has a
                              negative stride */
  LORA_ERR_DTYPE = -3,     /* unsupported dtype or mixed input dtypes */
  LORA_ERR_STRIDE = -4,    /* unsupported stride or alignment of a streamed operand */
  LORA_ERR_RANK = -5,      /* rank outside [1, 128] (single adapter) or r_max outside [1, 128] */
  LORA_ERR_WORKSPACE = -6, /* workspace NULL or smaller than lora_workspace_bytes() */
  LORA_ERR_LAUNCH = -7,    /* a HIP launch failed */
  LORA_ERR_LIMIT = -8      /* a size exceeds a documented library limit (e.g. S > 1024) */
};

/* A 2-D matrix view: element (i, j) is at ptr + i*stride_row + j*stride_col. */
typedef struct {
  void* ptr;
  int32_t dtype; /* lora_dtype */
  int32_t reserved;
  int64_t rows, cols;
  int64_t stride_row, stride_col;
} lora_mat;

/* A 3-D tensor view: element (i, j, k) is at ptr + i*s0 + j*s1 + k*s2. */
typedef struct {
  void* ptr;
  int32_t dtype; /* lora_dtype */
  int32_t reserved;
  int64_t d0, d1, d2;
  int64_t s0, s1, s2;
} lora_t3;

/*
 * Token-to-slot addressing of one batch (the pages' LoraAddressing, whose
 * fields the page does not print; this is the library's reading of it).
 *   token_slot[T]     in:  slot id of each token (any int32; ids outside
 *                           [0, S) make the token inactive).
 *   counts[S]         out: number of active tokens per slot.
 *   offsets[S+1]      out: exclusive prefix sum of counts; offsets[S] =
 *                           n_active.
 *   sorted_tokens[T]  out: the active tokens grouped by slot, ascending token
 *                           index within a slot, in entries [0, n_active);
 *                           entries past n_active are unspecified.
 * A token is active iff 0 <= token_slot[t] < S and the slot's rank, clamped
 * to [0, r_max], is positive (rank 0 = the zero adapter). All arrays are
 * device memory owned by the caller; lora_addressing_build writes the
 * outputs, and the multi-adapter ops read them.
 */
typedef struct {
  const int32_t* token_slot;
  int32_t T;
  int32_t S;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_tokens;
} lora_addressing;

/* Operation ids for lora_workspace_bytes. */
enum { LORA_OP_FWD = 0, LORA_OP_BWD_DX_DA = 1, LORA_OP_BWD_DB = 2 };

/* ABI version (LORA_ABI_VERSION) of the loaded library. */
int lora_abi_version(void);

/*
 * Kernel timing, for measurement tools (not one of the LoRA operations).
 * While recording, every kernel the library launches is dispatched with
 * hipExtLaunchKernel and a pair of HIP events that the dispatch stamps at the
 * kernel's start and end, so a duration covers the kernel alone, without the
 * command-processor latency that event records around a call add.
 *   lora_timing_begin   forgets earlier records and starts recording.
 *   lora_timing_pause   stops recording (launches run untimed);
 *   lora_timing_resume  starts it again, keeping the records.
 *   lora_timing_read    waits for every recorded kernel to finish and returns
 *                       the sum of their durations (ms) and their number;
 *                       -1 for NULL outputs, -7 if an event query fails.
 *   lora_timing_reserve creates event pairs up front until `pairs` exist (on
 *                       the current device), so that timed launches reuse
 *                       them instead of creating events while being timed;
 *                       -2 for a negative count, -7 if creation fails.
 * The state is process-wide: launches from any thread or stream while
 * recording are included. Events are created (once, then reused) on the
 * device current at the first timed launch, so one recording session must
 * time launches on one device. Records stay valid until the next
 * lora_timing_begin.
 */
int lora_timing_begin(void);
int lora_timing_pause(void);
int lora_timing_resume(void);
int lora_timing_read(double* total_ms, int64_t* launches);
int lora_timing_reserve(int64_t pairs);

/* Static text for a status code. */
const char* lora_status_string(int status);

/*
 * Workspace bytes that `op` needs for a problem of M tokens, K in-features,
 * L out-features, rank r and input dtype `dtype`, whatever the operand
 * strides. Returns 0 when the sizes are invalid. The workspace is device
 * memory of at least this size, 256-byte aligned, owned by the caller; its
 * contents on entry do not matter and are clobbered.
 */
size_t lora_workspace_bytes(int op, int64_t M, int64_t K, int64_t L, int32_t r, int32_t dtype);

/*
 * Single-adapter forward (lora_forward_kernel / lora_forward_wrapper: the
 * matmul D = A x B x C with N, the LoRA dimension, within one block, added to
 * the output):
 *     res += scale * (x @ lora_A) @ lora_B
 *   x       M x K   input activations (bf16 or f32); stride_col must be 1,
 *                   stride_row*elt and ptr 16-byte aligned, K a multiple of 8
 *                   (bf16) or 4 (f32).
 *   lora_A  K x r   any strides (a view of an r x K weight with stride_row 1
 *                   and a 16-byte aligned row is read in place; other layouts
 *                   are packed into the workspace first).
 *   lora_B  r x L   any strides (a view of an L x r weight with stride_row 1
 *                   is read in place; others are packed).
 *   res     M x L   accumulated in place (the page's `res`; pass a zeroed
 *                   buffer when there is none): float32, or bfloat16 when x,
 *                   lora_A and lora_B are bfloat16 (the page's output dtype:
 *                   the float32 sum of res and the update is rounded once to
 *                   the nearest bfloat16, ties to even). stride_col 1, row
 *                   16-byte aligned, L a multiple of 4.
 *   1 <= r <= 128.
 *   The library picks one of two schedules from the shapes: fused (one
 *   workgroup per token tile computes the rank-r intermediate and expands it,
 *   the intermediate never leaves registers and LDS) for K <= 8192 and an
 *   output below 256 MB; else split (a shrink kernel writes the
 *   intermediate to the workspace as MFMA operand fragments, 1 KB per 16
 *   tokens and 16 ranks, and each workgroup of the expand owns a band of 256
 *   output columns over a few token tiles). Both give the same results up to
 *   float32 summation order.
 *   workspace: lora_workspace_bytes(LORA_OP_FWD, ...) bytes (an upper bound
 *   over all layouts and output dtypes). It is needed only when a weight must
 *   be packed (a layout other than the two read in place) or the split
 *   schedule runs; otherwise the call uses none and workspace may be NULL
 *   with workspace_bytes 0, as for the page's lora_forward_wrapper, which
 *   takes only x, lora_A, lora_B, res and scale. LORA_ERR_WORKSPACE when one
 *   is needed and missing or too small.
 */
int lora_fwd(const lora_mat* x, const lora_mat* lora_A, const lora_mat* lora_B, const lora_mat* res,
             float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Single-adapter backward for x and lora_A (lora_da_dx_kernel /
 * lora_da_dx_update_wrapper: DYB = DY x B, DX = DY * B * A, and the token
 * reduction that gives dlora_A), in the page's frame:
 *   xt      K x M   input activations transposed (a view of row-major x:
 *                   stride_row must be 1; stride_col*elt and ptr 16-byte
 *                   aligned; K a multiple of 8 (bf16) or 4 (f32)).
 *   dy      M x L   output gradient; stride_col 1, 16-byte aligned rows, L a
 *                   multiple of 8 (bf16) or 4 (f32).
 *   lora_B  L x r   any strides.
 *   lora_A  r x K   any strides. bf16 weights in the nn.Linear layouts
 *                   (stride_col 1 for both, rows of a multiple of 8 elements
 *                   starting 16-byte aligned, r a multiple of 8) are read in
 *                   place; other layouts are packed into the workspace first
 *                   (one more kernel launch, same results bit for bit).
 *   dx      M x K   out (overwritten): dx = scale * (dy @ lora_B) @ lora_A.
 *                   stride_col 1, 16-byte aligned rows.
 *   dA      K x r   out (overwritten), any strides:
 *                   dA = scale * xt @ (dy @ lora_B).
 *   dx and dA each float32, or bfloat16 with bfloat16 inputs (the page's
 *   wrapper takes a dtype for its outputs): a bfloat16 element is the float32
 *   result rounded once to the nearest bfloat16 (ties to even).
 *   LORA_ERR_DTYPE for a bfloat16 output with float32 inputs.
 *   1 <= r <= 128; workspace of lora_workspace_bytes(LORA_OP_BWD_DX_DA, ...).
 */
int lora_bwd_dx_da(const lora_mat* xt, const lora_mat* dy, const lora_mat* lora_B, const lora_mat* lora_A,
                   float scale, const lora_mat* dx, const lora_mat* dA, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * lora_bwd_dx_da with dx accumulated instead of overwritten (the page's
 * wrapper takes a dtype for its outputs and leaves open whether dx is a fresh
 * buffer; a training step usually adds the adapter's input gradient to the
 * base layer's, which this does without a separate add over M x K):
 *   dx += scale * (dy @ lora_B) @ lora_A, every element read once and written
 *   once (float32 add of the float32 product; in a bfloat16 dx the float32
 *   sum rounded once); dA is overwritten as in
 *   lora_bwd_dx_da. Same arguments, layouts, workspace and errors; with M or
 *   L zero dx is left unchanged and dA set to zero.
 */
int lora_bwd_dx_da_accumulate(const lora_mat* xt, const lora_mat* dy, const lora_mat* lora_B,
                              const lora_mat* lora_A, float scale, const lora_mat* dx, const lora_mat* dA,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Single-adapter backward for lora_B (lora_db_kernel: AXT = A x X^T;
 * lora_db_update_wrapper multiplies it by dy), in the page's frame:
 *   lora_A  r x K   any strides.
 *   xt      K x M   input transposed (stride_row 1, as for lora_bwd_dx_da).
 *   dy      M x L   output gradient (stride_col 1, as for lora_bwd_dx_da).
 *   dB      r x L   out (overwritten), any strides:
 *                   dB = scale * (lora_A @ xt) @ dy. float32, or bfloat16
 *                   with bfloat16 inputs (rounded once, as for dA).
 *   1 <= r <= 128; workspace of lora_workspace_bytes(LORA_OP_BWD_DB, ...).
 */
int lora_bwd_db(const lora_mat* lora_A, const lora_mat* xt, const lora_mat* dy, float scale, const lora_mat* dB,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Token-to-slot grouping (the addressing every multi-adapter op takes; the
 * M* page's ops neither wait on the host nor size anything from device data,
 * so the grouping runs on the device). Writes addr->counts, offsets
 * and sorted_tokens from addr->token_slot and ranks[S] (device int32).
 *   1 <= r_max <= 128; 0 <= S <= 1024 (LORA_ERR_LIMIT above); T >= 0.
 */
int lora_addressing_build(const lora_addressing* addr, const int32_t* ranks, int32_t r_max, void* stream);

/*
 * Multi-adapter shrink (LoraOpsBackend.shrink: h[t] = x[t] @ a[slot(t)]^T):
 *   x   T x K                  bf16 or f32; stride_col 1, 16-byte aligned
 *                              rows, K a multiple of 8 (bf16) / 4 (f32).
 *   a   S x (num_slices*r_max) x K, same dtype as x; s2 must be 1 and s1*elt,
 *                              s0*elt and ptr 16-byte aligned. Rows
 *                              i*r_max + j hold slice i, rank row j.
 *   h   T x num_slices x r_max float32 out; s2 must be 1.
 *   For active t on slot s with rank rho, every slice i and j < rho:
 *   h[t, i, j] = sum_k x[t, k] * a[s, i*r_max + j, k]. Entries of inactive
 *   tokens and j >= rho are left unwritten (the page leaves them
 *   unspecified); rows j >= rho of a are never read.
 *   addr must have been built by lora_addressing_build with the same ranks
 *   and r_max (stream order).
 */
int lora_shrink(const lora_mat* x, const lora_t3* a, const lora_addressing* addr, const int32_t* ranks,
                int32_t num_slices, int32_t r_max, const lora_t3* h, void* stream);

/*
 * Multi-adapter expand over fused output slices (LoraOpsBackend.expand_fused:
 * y[t, slice i] += scalings[slot(t)] * h[t, slice i] @ b[slot(t), slice i]^T,
 * in place on y):
 *   h          T x num_slices x r_max float32; s2 must be 1, s1 and s0 multiples
 *              of 4, ptr 16-byte aligned.
 *   b          S x sum(out_slices) x r_max, bf16 or f32; s2 must be 1.
 *   scalings   float32[S], device.
 *   y          T x sum(out_slices), updated in place: float32, or bfloat16
 *              when b is bfloat16 (the float32 sum of y and the update is
 *              rounded once to the nearest bfloat16, ties to even);
 *              stride_col 1, 16-byte aligned rows.
 *   out_slices int64[num_slices], HOST memory: widths of the output slices
 *              (each a multiple of 4), concatenated along y's columns and b's
 *              rows.
 *   Columns j >= rank of h and b are never read; rows of y of inactive
 *   tokens are never written.
 */
int lora_expand_fused(const lora_t3* h, const lora_t3* b, const lora_addressing* addr, const int32_t* ranks,
                      const float* scalings, const lora_mat* y, const int64_t* out_slices, int32_t num_slices,
                      int32_t r_max, void* stream);

/*
 * Multi-adapter linear target (LoraOpsBackend.apply_linear_: shrink then
 * expand into y, for a linear target; the page lets a backend fuse them):
 *   x, a       as for lora_shrink.
 *   b, scalings, y, out_slices
 *              as for lora_expand_fused (num_slices = number of out_slices).
 *   h          T x num_slices x r_max float32 WORKSPACE owned by the caller,
 *              with the layout rules of both calls; its contents after the
 *              call are unspecified.
 *   y[t, slice i] += scalings[slot(t)] * (x[t] @ a[s, slice i]^T) @ b[s, slice i]^T
 *   for active t on slot s (ranks as in the two calls). Batches of 512 tokens
 *   or more whose token tiles and 1024-column chunks fit one round
 *   of the GPU's 256 CUs (tiles estimated as if the tokens spread evenly over
 *   the S slots), with x, a and b of one dtype, run as ONE launch that keeps
 *   the rank intermediate on chip and leaves h unwritten; the others run the
 *   shrink into h and the expand back to back on the stream. Both forms give
 *   the same bits where the shrink takes the pipelined kernel (batches below
 *   1024 tokens, and larger ones with few slots). The arguments of both
 *   operations are checked before anything launches: a failing call launches
 *   nothing.
 */
int lora_apply_linear(const lora_mat* x, const lora_t3* a, const lora_t3* b, const lora_addressing* addr,
                      const int32_t* ranks, const float* scalings, const lora_mat* y, const int64_t* out_slices,
                      int32_t num_slices, int32_t r_max, const lora_t3* h, void* stream);

/*
 * lora_apply_linear without a caller workspace, for callers that cannot
 * allocate (code under HIP graph capture, serving loops that must not call
 * hipMalloc, harnesses that forbid allocation). The rank intermediate h lives
 * in a device array of the library (32 MiB per GPU, allocated when the library's
 * code object loads on that GPU and held until the process ends), laid out
 * T x num_slices x r_max float32; the call allocates and frees nothing.
 *   Arguments as for lora_apply_linear, without h; results are bit for bit
 *   those of lora_apply_linear (the same kernels).
 *   T * num_slices * r_max * 4 bytes must not exceed 32 MiB: LORA_ERR_LIMIT
 *   (before anything is launched) otherwise.
 *   Every call on one GPU uses that GPU's one array, which keeps the last
 *   call's contents: calls that overlap on one GPU (on different streams, or
 *   from different threads without ordering) race and give wrong results;
 *   calls ordered on one stream do not.
 */
int lora_apply_linear_noalloc(const lora_mat* x, const lora_t3* a, const lora_t3* b, const lora_addressing* addr,
                              const int32_t* ranks, const float* scalings, const lora_mat* y,
                              const int64_t* out_slices, int32_t num_slices, int32_t r_max, void* stream);

/*
 * Multi-adapter embedding gather (LoraOpsBackend.gather_shrink:
 * h[t] = a[slot(t)][:, ids[t]], i.e. column ids[t] of the token's adapter):
 *   ids  int32[T] device.
 *   a    S x r_max x V, bf16 or f32, any strides (64-bit offsets; a table
 *        stored with the rank index contiguous, s1 = 1, is read coalesced).
 *   h    T x 1 x r_max float32 out; s2 must be 1.
 *   For active t with rank rho: h[t, 0, j] = a[s, j, ids[t]] for j < rho, an
 *   exact copy, or +0.0 when ids[t] lies outside [0, V). Other entries are
 *   left unwritten.
 */
int lora_gather_shrink(const int32_t* ids, const lora_t3* a, const lora_addressing* addr, const int32_t* ranks,
                       int32_t r_max, const lora_t3* h, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_LORA_H */
