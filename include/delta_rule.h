/* Gated delta rule forward (GDN and KDA), token-recurrent form, on gfx950.
 *
 * The operation is the one the linear_attention reference page
 * (modelopt.torch.quantization.linear_attention.reference) names
 * recurrent_delta_rule_reference: GDN (one decay per value head) or KDA (one
 * decay per key channel), natural-log gates, inputs already normalized, an
 * optional initial state, packed sequences through cu_seqlens, and the output
 * together with the final state. For value head h (key head h / (Hv / Hk))
 * and each token t, with S the [Dk, Dv] state:
 *
 *     S   <- diag(exp(g_t)) S                  (GDN: exp(g_t) S)
 *     S   <- S + k_t (beta_t (v_t - S^T k_t))^T
 *     o_t  = scale S^T q_t
 *
 * The state is carried in float32; q, k, v and o are float32 or bf16.
 */
#ifndef RGLRU_DELTA_RULE_H_
#define RGLRU_DELTA_RULE_H_

#include "rglru.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RGLRU_DELTA_GDN = 0,  /* g [.., Hv]: one decay per value head and token */
  RGLRU_DELTA_KDA = 1   /* g [.., Hv, Dk]: one decay per key channel, value head and token */
} rglru_delta_decay_t;

/* Limits beyond which the call returns RGLRU_ERR_INVALID_ARGUMENT:
 * batch, length >= 0 with batch * length < 2^40; 1 <= k_heads <= v_heads <
 * 2^16 with v_heads a multiple of k_heads; 1 <= k_dim, v_dim <= 2^16; finite
 * scale; state_v_first 0 or 1; and n_seqs * v_heads * ceil(v_dim / 16) <
 * 2^31 (the workgroups of one call). Within them, k_dim > 256, or k_dim or
 * v_dim not a multiple of 8, is RGLRU_ERR_UNSUPPORTED. */
typedef struct {
  int64_t batch;          /* B; 1 with cu_seqlens */
  int64_t length;         /* T tokens per batch row (with cu_seqlens: all tokens) */
  int32_t k_heads;        /* Hk, heads of q and k */
  int32_t v_heads;        /* Hv, heads of v, g, beta, o and the state */
  int32_t k_dim;          /* Dk */
  int32_t v_dim;          /* Dv */
  int32_t io_dtype;       /* rglru_io_t of q, k, v and o */
  int32_t decay;          /* rglru_delta_decay_t */
  int32_t state_v_first;  /* 0: states [N, Hv, Dk, Dv]; 1: [N, Hv, Dv, Dk] */
  float scale;            /* read-out scale (the reference's default is 1 / sqrt(Dk)) */
} rglru_delta_shape_t;

/* Forward of the gated delta rule over every token, on `stream` (a
 * hipStream_t; NULL = the null stream). All pointers are device memory,
 * owned by the caller, dense row-major:
 *
 *   cu_seqlens : NULL (B independent rows of T tokens, N = B) or [n_seqs + 1]
 *                int32 with 0 = cu[0] <= ... <= cu[n_seqs] = T and B = 1
 *                (N = n_seqs packed sequences, 1 <= n_seqs < 2^30). Offsets
 *                are read on the device and clamped into [0, T], so invalid
 *                offsets give unspecified but in-bounds results.
 *   q, k       : [B, T, Hk, Dk] io, 16-byte aligned.
 *   v, o       : [B, T, Hv, Dv] io, 16-byte aligned; o is written.
 *   g          : float32 natural-log decays, [B, T, Hv] (GDN, 4-byte aligned)
 *                or [B, T, Hv, Dk] (KDA, 16-byte aligned).
 *   beta       : [B, T, Hv] float32 write strengths.
 *   h0         : NULL (zero initial states) or [N, Hv, Dk, Dv] float32
 *                ([N, Hv, Dv, Dk] with state_v_first), 16-byte aligned.
 *   h_last     : NULL or the final states, same layout and alignment as h0; a
 *                sequence with no tokens gets its initial state.
 *   ckpt       : NULL (inference) or rglru_delta_ckpt_elems(shape, n) float32
 *                (n = n_seqs with cu_seqlens, else 0), 16-byte aligned: the
 *                state entering every 8th token of each sequence, which
 *                rglru_delta_rule_bwd needs; each slot column-major (the Dk
 *                values of a state column contiguous, whatever state_v_first).
 * q, k, v, g, beta and o may be NULL only when B * T = 0. Returns
 * RGLRU_ERR_INVALID_ARGUMENT, RGLRU_ERR_MISALIGNED or RGLRU_ERR_UNSUPPORTED
 * without launching anything, RGLRU_ERR_HIP if the launch fails. Outputs
 * must not overlap inputs. */
rglru_status_t rglru_delta_rule_fwd(const rglru_delta_shape_t* shape, const int32_t* cu_seqlens,
                                    int64_t n_seqs, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const float* h0, void* o,
                                    float* h_last, float* ckpt, void* stream);

/* Float32 elements of the forward's checkpoint: per value head, ceil(T / 8)
 * slots per batch row (B rows), or ceil(T / 8) + n_seqs slots for packed
 * sequences, of Dk * Dv each. 0 for an invalid shape. */
size_t rglru_delta_ckpt_elems(const rglru_delta_shape_t* shape, int64_t n_seqs);

/* Backward of rglru_delta_rule_fwd (token form, GDN or KDA) for the loss
 * <do, o> + <dh_last, final state>: the reverse-mode steps of the same
 * recurrence (the page's recurrent oracle keeps gradients through every input
 * and the initial state). The forward must have run with ckpt on the same
 * inputs; h0 is not needed again (the checkpoint holds it).
 *
 *   q, k, v, g, beta, cu_seqlens, n_seqs : as for the forward.
 *   ckpt       : the forward's checkpoint (16-byte aligned).
 *   d_o        : [B, T, Hv, Dv] io, 16-byte aligned: the gradient of o.
 *   dh_last    : NULL (zero) or the gradient of the final state, layout of h0.
 *   dq, dk     : [B, T, Hk, Dk] io (summed over the value heads of each key head).
 *   dv         : [B, T, Hv, Dv] io, 16-byte aligned.
 *   dg         : float32, the shape of g.  dbeta : [B, T, Hv] float32.
 *   dh0        : NULL or the gradient of the initial state, layout of h0.
 *   workspace  : rglru_delta_bwd_workspace_bytes(shape, n) bytes (n as for
 *                the checkpoint), 256-byte aligned, no initial contents
 *                required: per-column-block partial sums, which a second
 *                launch adds in a fixed order, so results are bitwise
 *                reproducible.
 * Restrictions (RGLRU_ERR_UNSUPPORTED otherwise): k_dim at most 128, k_dim
 * and v_dim multiples of 8. Invalid offsets give unspecified (in-bounds)
 * results. Returns as the forward does. */
size_t rglru_delta_bwd_workspace_bytes(const rglru_delta_shape_t* shape, int64_t n_seqs);
rglru_status_t rglru_delta_rule_bwd(const rglru_delta_shape_t* shape, const int32_t* cu_seqlens,
                                    int64_t n_seqs, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const float* ckpt, const void* d_o,
                                    const float* dh_last, void* dq, void* dk, void* dv, float* dg,
                                    float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* The same forward for GDN in chunk form (chunk_gdn_reference on the same
 * page: within each chunk of 64 tokens, a unit-lower-triangular solve gives
 * the WY operands W = T diag(beta e^Gc) K and U~ = T diag(beta) V, with T the
 * inverse of I plus the strictly lower, decay-weighted beta K K^T; the state
 * then advances once per chunk; packed sequences through cu_seqlens). The
 * dense products run on bf16 MFMA with float32 accumulation: T, W, U~, the
 * corrected writes, the masked Q K^T, the decayed and scaled K and Q and the
 * state's operand copy are rounded to bf16 where they enter a product, so
 * results match the token recurrence to bf16-operand accuracy, not bitwise;
 * the state itself is float32 throughout.
 *
 * Arguments as for rglru_delta_rule_fwd (cu_seqlens NULL with n_seqs
 * ignored, or n_seqs >= 1 packed sequences with B = 1; offsets read on the
 * device and clamped into [0, T]), with these restrictions
 * (RGLRU_ERR_UNSUPPORTED otherwise): decay RGLRU_DELTA_GDN, io bf16, k_dim
 * 64 or 128, v_dim a multiple of 32 and at most 256. o needs only 2-byte,
 * h0 and h_last only 4-byte alignment here. workspace: device memory of at least
 * rglru_delta_chunk_workspace_bytes(shape, n) bytes (n = n_seqs with
 * cu_seqlens, else 0), 256-byte aligned, owned by the caller, no initial
 * contents required; it holds the WY operands between the launches (and
 * the chunk map of packed sequences); it may be NULL when B * T = 0 without
 * cu_seqlens (then only the final state is written, from h0 or zeros). The
 * size query returns 0 for an invalid or unsupported shape. */
size_t rglru_delta_chunk_workspace_bytes(const rglru_delta_shape_t* shape, int64_t n_seqs);
rglru_status_t rglru_delta_chunk_fwd(const rglru_delta_shape_t* shape, const int32_t* cu_seqlens,
                                     int64_t n_seqs, const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, const float* h0, void* o,
                                     float* h_last, void* workspace, size_t workspace_bytes,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* RGLRU_DELTA_RULE_H_ */
