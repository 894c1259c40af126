/*
 * rglru.h - C ABI of the MI355X (gfx950) RG-LRU library.
 *
 * The library computes the fused RG-LRU (Hawk) gated linear recurrence and its
 * backward on one GPU, plus the block-diagonal gate projection that feeds it.
 * The Fattori comparison page lists what the fused operator covers: both
 * sigmoid gates, softplus(a_param) with a dynamic decay and the stationary
 * square-root factor, the input-gated write, a sequential state-stationary
 * recurrence, and a custom backward with the reverse recurrence and pointwise
 * derivatives. Its "Semantic limits" list names what a canonical version adds
 * (reset tokens, a nonzero initial state, any width, any length), and its
 * closing paragraph names an exact parallel chunk forward and backward with
 * partial chunks. Per batch row b, channel w and step t:
 *
 *   i = sigmoid(gate_x)   r = sigmoid(gate_a)   s = softplus(lambda[w])
 *   a = exp(-c * s * r)   m = sqrt(1 - a^2)
 *   h[t] = a * h[t-1] + m * i * x           (ordinary token)
 *   h[t] = i * x                            (reset token: state cleared, multiplier 1)
 *   h[-1] = h0 (or 0)
 *
 * Conventions shared by every entry point:
 *  - All tensors are dense, row-major and owned by the caller. Sequence
 *    tensors are [B, L, W] with channels contiguous; reset flags are uint8
 *    [B, L] (nonzero = reset token, shared by all channels of that token).
 *  - "io" tensors are float32 or bf16 (bit pattern, uint16) per
 *    rglru_shape_t.io_dtype. lambda, h0, h_last, ckpt, dlambda and dh0 are
 *    always float32. The carry is float32; bf16 outputs are rounded to nearest
 *    even.
 *  - Pointers are device pointers unless stated. Every pointer must be aligned
 *    to its element size; wider alignment (and W a multiple of 4) selects
 *    wider vector loads, it never changes results beyond rounding.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream). The library never allocates, frees or synchronises.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error the call returns a status and writes nothing.
 *  - Outputs must not alias inputs unless an entry point says otherwise.
 *  - Workspaces: a caller-owned device buffer of at least the queried size,
 *    aligned to 256 bytes, ZERO-FILLED BEFORE ITS FIRST USE. Every completed
 *    call leaves it ready for the next one; no clearing between calls is
 *    needed. One workspace may serve forward and backward calls of any shape
 *    (size it for the largest), but calls that use the same workspace must not
 *    overlap in time (same stream, or ordered by events).
 *    Layout of its first 16 bytes (read-only for callers): a 64-bit counter
 *    (high half: completed calls, which skips 0xFFFFFFFF; low half: tiles
 *    handed out during a forward), a 32-bit count of finished workgroups, and
 *    a 32-bit sticky error word. Bit 0 is set if a wait for another
 *    workgroup's published prefix (the look-back across tiles) exceeded its
 *    spin limit; bit 1 if a wait between the waves of one workgroup (on a
 *    flag in LDS) exceeded its spin limit; bit 2 if the segment offsets of a
 *    packed-sequence call were invalid. Any of them makes the outputs of that
 *    call invalid; bits 0 and 1 cannot happen while every launched workgroup
 *    makes progress. The library never clears the word; the caller reads it
 *    (after the call has completed) to check, and zero-fills the workspace to
 *    clear it.
 */
#ifndef RGLRU_H_
#define RGLRU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RGLRU_ABI_VERSION 1
/* The forward checkpoints the float32 carry every RGLRU_CKPT_STEPS steps. */
#define RGLRU_CKPT_STEPS 8

typedef enum {
  RGLRU_IO_F32 = 0,
  RGLRU_IO_BF16 = 1
} rglru_io_t;

typedef enum {
  RGLRU_OK = 0,
  RGLRU_ERR_INVALID_ARGUMENT = 1,  /* bad shape, NULL required pointer, bad enum */
  RGLRU_ERR_MISALIGNED = 2,        /* a pointer not aligned to its element size */
  RGLRU_ERR_WORKSPACE_TOO_SMALL = 3,
  RGLRU_ERR_UNSUPPORTED = 4,       /* a valid request this build does not implement */
  RGLRU_ERR_HIP = 5,               /* the HIP runtime refused a launch */
  RGLRU_ERR_SCRATCH_TOO_SMALL = 6  /* rglru_fwd_scratch: the shape needs more than RGLRU_SCRATCH_BYTES */
} rglru_status_t;

/* Size limits (beyond them RGLRU_ERR_INVALID_ARGUMENT, and size queries
 * return 0): B <= 2^24, W <= 2^24, L <= 2^34, and ceil(W / 64) * B *
 * ceil(L / 8) < 2^31 (the count of 64-channel, 8-step units indexed in 32
 * bits). */
typedef struct {
  int64_t batch;    /* B >= 1 */
  int64_t length;   /* L >= 1 */
  int64_t width;    /* W >= 1, any value */
  int32_t io_dtype; /* rglru_io_t */
  int32_t chunk;    /* requested time tile of the parallel scan: 0 = library
                       default, or one of 8, 16, 32, 64, 128, 256 (anything
                       else is RGLRU_ERR_INVALID_ARGUMENT). Results depend on
                       it only through floating-point rounding. The request is
                       an upper bound that each direction clamps to the
                       longest tile it implements for the call:
                         forward : default 128; at most 128 for bf16 io whose
                                   rows (W * 2 bytes) are a multiple of 16
                                   bytes with x, gate_x, gate_a 16-byte aligned,
                                   at most 64 otherwise.
                         backward: default 64; at most 64 under the same
                                   bf16 condition (dh aligned too), at most 32
                                   otherwise.
                       A clamped request is not an error: it runs the
                       clamped tile and returns RGLRU_OK. */
  float c;          /* decay scale of a = exp(-c * softplus(lambda) * r); 8 in the method */
  int32_t reserved; /* must be 0 */
} rglru_shape_t;

/* Number of float32 elements of the forward's carry checkpoint:
 * B * ceil(L / RGLRU_CKPT_STEPS) * W. Element [b, k, w] holds the carry
 * entering step k * RGLRU_CKPT_STEPS (so [b, 0, w] = h0 or 0). Returns 0 for
 * an invalid shape. */
size_t rglru_ckpt_elems(const rglru_shape_t* shape);

/* Workspace bytes for rglru_fwd, rglru_bwd, and for either (the maximum).
 * Return 0 for an invalid shape. */
size_t rglru_fwd_workspace_bytes(const rglru_shape_t* shape);
size_t rglru_bwd_workspace_bytes(const rglru_shape_t* shape);
size_t rglru_workspace_bytes(const rglru_shape_t* shape);

/* Forward scan (the operator of the Fattori comparison page: sigmoid gates,
 * softplus dynamic decay, stationary square-root multiplier, input-gated write,
 * state-stationary recurrence; canonical reset tokens and initial state as its
 * "Semantic limits" list describes; an exact chunked parallel form).
 *
 *   x, gate_x, gate_a : [B, L, W] io, required.
 *   lambda            : [W] float32, required (the per-channel a_param).
 *   reset             : [B, L] uint8 or NULL (no reset tokens).
 *   h0                : [B, W] float32 or NULL (zero initial state).
 *   h                 : [B, L, W] io, required output: the state after every step.
 *   h_last            : [B, W] float32 or NULL: the float32 state after step L-1.
 *   ckpt              : rglru_ckpt_elems() float32 or NULL. Required if a
 *                       backward will follow (training); NULL for inference.
 *   workspace         : see Conventions.
 */
rglru_status_t rglru_fwd(const rglru_shape_t* shape,
                         const void* x, const void* gate_x, const void* gate_a,
                         const float* lambda, const uint8_t* reset, const float* h0,
                         void* h, float* h_last, float* ckpt,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Backward scan (the custom backward of the same page: reverse recurrence,
 * pointwise derivatives recomputed from the inputs instead of saved gates,
 * a_param gradient reduced over batch and time). The loss is taken to be
 * <dh, h> + <dh_last, h_last>.
 *
 *   x, gate_x, gate_a, lambda, reset : exactly as passed to rglru_fwd.
 *   ckpt              : filled by rglru_fwd with the same shape, required.
 *                       (It carries h0, so h0 is not passed again.)
 *   dh                : [B, L, W] io, required: gradient on every h[t].
 *   dh_last           : [B, W] float32 or NULL: gradient on h_last.
 *   dx, dgate_x, dgate_a : [B, L, W] io, required outputs.
 *   dlambda           : [W] float32, required output, overwritten (not accumulated).
 *   dh0               : [B, W] float32 or NULL: gradient on h0 (0 where t = 0 is a reset).
 *   workspace         : see Conventions.
 */
rglru_status_t rglru_bwd(const rglru_shape_t* shape,
                         const void* x, const void* gate_x, const void* gate_a,
                         const float* lambda, const uint8_t* reset, const float* ckpt,
                         const void* dh, const float* dh_last,
                         void* dx, void* dgate_x, void* dgate_a,
                         float* dlambda, float* dh0,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Block-diagonal gate projections (the two BlockDiagonalLinear maps the
 * Fattori comparison page says the caller computes before the operator):
 *   gate_x[:, blk k] = x[:, blk k] @ w_x[k] + b_x[blk k]   (and likewise for gate_a)
 * with blk k = columns [k*block, (k+1)*block).
 *
 *   tokens, width, block : T >= 1 rows; width = nblocks * block; block = 256 in this build.
 *   x                 : [T, width] bf16, required.
 *   w_x, w_a          : [width/block, block, block] bf16, read as [block, in, out], required.
 *   b_x, b_a          : [width] bf16 or NULL (zero bias).
 *   gate_x, gate_a    : [T, width] bf16 outputs (float32 accumulation, rounded once).
 */
rglru_status_t rglru_blockdiag_gate_proj_fwd(int64_t tokens, int64_t width, int64_t block,
                                             const void* x,
                                             const void* w_x, const void* b_x,
                                             const void* w_a, const void* b_a,
                                             void* gate_x, void* gate_a, void* stream);

/* Backward of the projections:
 *   dx_out = dx_in + dgate_x @ w_x^T + dgate_a @ w_a^T   (per block; dx_in may be NULL)
 *   dw_x[k] = x_blk^T @ dgate_x_blk,  dw_a likewise     (float32, overwritten)
 *   db_x = column sums of dgate_x,    db_a likewise     (float32, overwritten; NULL skips)
 *
 *   x, w_x, w_a       : as in the forward.
 *   dgate_x, dgate_a  : [T, width] bf16, required.
 *   dx_in             : [T, width] bf16 or NULL; dx_out may equal dx_in.
 *   dx_out            : [T, width] bf16, required.
 *   dw_x, dw_a        : [width/block, block, block] float32, required.
 *   db_x, db_a        : [width] float32 or NULL.
 *   workspace         : at least rglru_blockdiag_gate_proj_bwd_workspace_bytes(); any content.
 */
size_t rglru_blockdiag_gate_proj_bwd_workspace_bytes(int64_t tokens, int64_t width, int64_t block);
rglru_status_t rglru_blockdiag_gate_proj_bwd(int64_t tokens, int64_t width, int64_t block,
                                             const void* x, const void* w_x, const void* w_a,
                                             const void* dgate_x, const void* dgate_a,
                                             const void* dx_in, void* dx_out,
                                             float* dw_x, float* db_x, float* dw_a, float* db_a,
                                             void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status. Never NULL. */
/* Forward scan with both block-diagonal gate projections computed inside it
 * (the step the Fattori comparison page says prior art leaves to the caller:
 * two BlockDiagonalLinear projections of x ahead of the fused operator), so
 * the logits need not pass through HBM. The result is bitwise that of
 * rglru_blockdiag_gate_proj_fwd followed by rglru_fwd with chunk 64 on its
 * logits; the logits themselves are written too when gate_x / gate_a are
 * given (training: rglru_bwd and rglru_blockdiag_gate_proj_bwd take them).
 *
 *   shape          : io_dtype bf16, width a multiple of 256, chunk 0 or 64
 *                    (the call runs 64-step tiles); anything else is
 *                    RGLRU_ERR_UNSUPPORTED.
 *   x              : [B, L, W] bf16, 16-byte aligned.
 *   w_x, w_a       : [W/256, 256, 256] bf16 weights, read as [block, in, out].
 *   b_x, b_a       : [W] bf16 or NULL (zero bias).
 *   lambda, reset, h0, h, h_last, ckpt : as for rglru_fwd (h 16-byte aligned).
 *   gate_x, gate_a : [B, L, W] bf16 (8-byte aligned) or NULL.
 *   workspace      : rglru_blockdiag_fused_fwd_workspace_bytes() bytes,
 *                    zero-filled before its first use, as for rglru_fwd; it
 *                    also holds a transposed copy of both weights, rebuilt by
 *                    every call. */
size_t rglru_blockdiag_fused_fwd_workspace_bytes(const rglru_shape_t* shape);
rglru_status_t rglru_blockdiag_fused_fwd(const rglru_shape_t* shape, const void* x,
                                         const void* w_x, const void* b_x, const void* w_a, const void* b_a,
                                         const float* lambda, const uint8_t* reset, const float* h0,
                                         void* h, float* h_last, float* ckpt, void* gate_x, void* gate_a,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Packed variable-length sequences (the cu_seqlens convention of the
 * linear-attention reference oracles, recurrent_delta_rule_reference and
 * chunk_gdn_reference: offsets into one packed row, per-sequence initial and
 * final states, gradients through the initial states). n_seqs sequences lie end to end in one row of T tokens, sequence s
 * holding tokens [cu_seqlens[s], cu_seqlens[s+1]). Each sequence is computed
 * exactly as its own batch row would be: its first token starts from h0[s]
 * (zero if h0 is NULL) with the ordinary write, its last token's float32
 * state is h_last[s]; reset tokens inside a sequence keep their meaning (a
 * reset on a sequence's first token ignores h0[s]). A sequence with no
 * tokens has h_last[s] = h0[s] and dh0[s] = dh_last[s].
 *
 *   shape       : batch = 1, length = T >= 1 (all tokens), width, io_dtype,
 *                 chunk, c as for rglru_fwd.
 *   cu_seqlens  : [n_seqs + 1] int32, device, 0 = cu[0] <= cu[1] <= ... <=
 *                 cu[n_seqs] = T. Not checked on the host (that would need a
 *                 synchronisation); invalid offsets set bit 2 of the
 *                 workspace error word and give unspecified (but in-bounds)
 *                 results.
 *   n_seqs      : 1 <= n_seqs < 2^30.
 *   x, gate_x, gate_a, h, dh, dx, dgate_x, dgate_a : [T, W] io.
 *   reset       : [T] uint8 or NULL.
 *   h0, h_last, dh_last, dh0 : [n_seqs, W] float32 or NULL.
 *   ckpt        : rglru_ckpt_elems() of the shape, as for rglru_fwd.
 *   workspace   : rglru_varlen_workspace_bytes() bytes (serves both
 *                 directions), zero-filled before its first use, as for
 *                 rglru_fwd; it also holds the per-token segment words,
 *                 rebuilt by every call.
 * The backward takes h0 again (segment starts inside the row need it). */
size_t rglru_varlen_workspace_bytes(const rglru_shape_t* shape, int64_t n_seqs);
rglru_status_t rglru_fwd_varlen(const rglru_shape_t* shape, const int32_t* cu_seqlens, int64_t n_seqs,
                                const void* x, const void* gate_x, const void* gate_a,
                                const float* lambda, const uint8_t* reset, const float* h0,
                                void* h, float* h_last, float* ckpt,
                                void* workspace, size_t workspace_bytes, void* stream);
rglru_status_t rglru_bwd_varlen(const rglru_shape_t* shape, const int32_t* cu_seqlens, int64_t n_seqs,
                                const void* x, const void* gate_x, const void* gate_a,
                                const float* lambda, const uint8_t* reset, const float* h0,
                                const float* ckpt, const void* dh, const float* dh_last,
                                void* dx, void* dgate_x, void* dgate_a, float* dlambda, float* dh0,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Forward scan without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * results (bitwise) and errors as rglru_fwd, minus the workspace: the library
 * uses a static device array of RGLRU_SCRATCH_BYTES in its place, one per GPU,
 * which it holds from the first call on that GPU until the process ends
 * (zero-filled when the library's code object loads; every completed call
 * leaves it ready for the next one). Returns RGLRU_ERR_SCRATCH_TOO_SMALL,
 * writing nothing, when rglru_fwd_workspace_bytes(shape) exceeds
 * RGLRU_SCRATCH_BYTES: B * ceil(L / T) * W' must stay under about 2.79e6,
 * with T = min(chunk, 64) (64 for the default chunk) and W' = W rounded up to
 * a multiple of 512 (B=1, L=32768, W=4096 needs 2097152). Returns
 * RGLRU_ERR_HIP if the runtime cannot give the array's address.
 * Runs on the current device. Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race and must be ordered by the caller. */
#define RGLRU_SCRATCH_BYTES (((size_t)64) << 20)
rglru_status_t rglru_fwd_scratch(const rglru_shape_t* shape,
                                 const void* x, const void* gate_x, const void* gate_a,
                                 const float* lambda, const uint8_t* reset, const float* h0,
                                 void* h, float* h_last, float* ckpt, void* stream);

const char* rglru_status_string(rglru_status_t status);

/* RGLRU_ABI_VERSION of the loaded library. */
int rglru_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RGLRU_H_ */
