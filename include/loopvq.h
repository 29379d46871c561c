/*
 * loopvq.h -- C ABI of the LoopVQ hot path on MI355X (gfx950).
 *
 * LoopVQ (review of arXiv 2611.05304 on jaehun.me, "paper-2611-05304v1") stores
 * a looped transformer's per-step KV cache as one b-bit code per joint vector
 * that spans c = G/T_c channels at each of T_c consecutive loop steps
 * (section 3.1, eq. 4/5).  Two calls mirror the two things a user of the method
 * does (section 3.4): encode a block of per-step K or V into index rows, and
 * run decode attention over the index rows with codebooks resident on chip.
 *
 * Conventions shared by every entry point
 *   - Pointers named "device" point to GPU memory of the current HIP device;
 *     the geometry / pre-transform structs are host memory, read during the
 *     call only.  The caller owns every buffer; the library allocates no device
 *     memory in these calls (decode scratch comes from the caller's workspace).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous; they never synchronize.  Faults raised
 *     while kernels run surface at the caller's next synchronization.
 *   - All argument checks happen on the host before any HIP call.  A failed
 *     check returns LOOPVQ_EINVAL (bad value) or LOOPVQ_ENOTSUP (legal but not
 *     built, e.g. D != 128); a failed launch returns LOOPVQ_EHIP.  The message
 *     is available from loopvq_last_error() (thread-local).  No C++ exception
 *     crosses this boundary.
 *   - bf16 and fp16 tensors are passed as raw 16-bit storage.
 *   - Multi-dimensional buffers are dense, row-major, in the order given.
 */
#ifndef LOOPVQ_H
#define LOOPVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOOPVQ_ABI_VERSION 4

typedef enum {
  LOOPVQ_OK = 0,
  LOOPVQ_EINVAL = -1,
  LOOPVQ_ENOTSUP = -2,
  LOOPVQ_EHIP = -3,
  LOOPVQ_EWORKSPACE = -4
} loopvq_status;

/* Geometry of one attention layer (section 3.1 notation).
 *   D          head dim (even; this build supports D = 128)
 *   T          loop steps; T_c steps per block, T % T_c == 0, n_blk = T / T_c
 *   G          joint-vector length, G % T_c == 0, c = G / T_c, D % c == 0;
 *              this build supports G in {16, 32} with D/2 % c == 0
 *   K          codebook entries, 2 <= K <= 256 (one uint8 index per code)
 *   n_kv_heads, n_q_heads   n_q_heads % n_kv_heads == 0; q-head hq reads
 *              kv-head hq / (n_q_heads / n_kv_heads)
 *   rope_theta RoPE base (rotate-half pairs (d, d + D/2), angle
 *              pos * theta^(-2d/D)) */
typedef struct {
  int32_t D, T, T_c, G, K, n_kv_heads, n_q_heads;
  float rope_theta;
} loopvq_geom;

/* Channel pre-transform for keys (section 3.3, appendix B eq. 10).
 *   w      device fp32 [n_kv_heads][D], every entry > 0
 *   perm   device int16 [n_kv_heads][D], a permutation of 0..D-1 per head;
 *          transformed channel d' holds raw channel perm[d']
 *   sigma  device fp16 [B][N_cap][T]: per-(token, step) RMS of the layer's raw
 *          pre-RoPE key over all n_kv_heads * D channels, rounded to fp16
 *          (round to nearest even).  loopvq_encode writes it for the tokens it
 *          encodes; loopvq_decode_attn reads it.  4-byte aligned (decode
 *          reads the two steps of a half block as one word; EINVAL otherwise)
 *   N_cap  token capacity of sigma
 * The transformed key is z[d'] = (w[perm[d']] * k[perm[d']]) / sigma. */
typedef struct {
  const float* w;
  const int16_t* perm;
  uint16_t* sigma;
  int32_t N_cap;
} loopvq_pretransform;

/* loopvq_encode -- nearest-codeword encode of loop-axis joint vectors
 * (section "terms" eq. 2 with the joint vector of section 3.1 eq. 4).
 *
 * For every batch b < B, kv-head h, block beta < n_blk, token j < N and chunk
 * q < D/c, the joint vector is z[i*T_c + m] = x[b][h][beta*T_c + m][j][q*c + i]
 * (i < c, m < T_c), or its pre-transformed value when pt != NULL, and
 *   idx[b][h][beta][tok0 + j][q] = argmin_r ||z - e_r||^2
 * over the entries e_r = codebook[h][beta][r][0..G) (lowest r on exact ties).
 * Distances are screened with bf16 MFMA tiles and every code whose best two
 * candidates lie within the screening error bound is re-scored in fp64, so the
 * result equals the exact argmin.
 *
 *   g          geometry (host)
 *   x          device bf16, element (b, h, t, j, d) at
 *              b*xs[0] + h*xs[1] + t*xs[2] + j*xs[3] + d   (xs = x_strides,
 *              in elements; each row of D channels is contiguous)
 *   codebook   device bf16 [n_kv_heads][n_blk][K][G], coordinate i*T_c + m
 *   B, N, tok0 batch size, tokens to encode, first destination token
 *   idx        device uint8 [B][n_kv_heads][n_blk][N_cap][D/c]
 *   N_cap      token capacity of idx, tok0 + N <= N_cap
 *   pt         NULL for values and plain keys; for pre-transformed keys also
 *              writes pt->sigma[b][tok0 + j][t] for every step t < T
 * Errors: EINVAL for NULL pointers, bad geometry, N < 0, tok0 < 0,
 * tok0 + N > N_cap (or > pt->N_cap), non-positive strides; ENOTSUP for D != 128
 * or G not in {16, 32}.  N == 0 is a no-op returning LOOPVQ_OK. */
loopvq_status loopvq_encode(const loopvq_geom* g, const void* x, const int64_t x_strides[4],
                            const void* codebook, int32_t B, int32_t N, int32_t tok0,
                            uint8_t* idx, int32_t N_cap, const loopvq_pretransform* pt,
                            void* stream);

/* loopvq_rope_table -- the per-position sin/cos table the decode kernel reads
 * (section 3.4, step 3).  For position p and frequency f < D/2 the angle is
 * phi = p * theta^(-2f/D), evaluated in fp64 on the GPU; cos(phi) and sin(phi)
 * are rounded once to fp16 (round to nearest even).
 *   table   device fp16 [n_pos][D/8][8]: entry [p][f/4] holds
 *           cos of frequencies 4*(f/4) .. +3, then their sines
 * Errors: EINVAL for NULL table, n_pos < 1, D not a positive multiple of 8,
 * theta <= 0. */
loopvq_status loopvq_rope_table(float theta, int32_t D, int32_t n_pos, void* table,
                                void* stream);

/* loopvq_decode_attn_workspace -- bytes of scratch loopvq_decode_attn needs
 * for this shape (split-context partials).  Same argument rules as
 * loopvq_decode_attn; *bytes may be 0. */
loopvq_status loopvq_decode_attn_workspace(const loopvq_geom* g, int32_t B, int32_t N,
                                           int32_t step0, int32_t n_steps, size_t* bytes);

/* loopvq_decode_attn -- fused decode attention over the compressed cache
 * (section 3.4 step 3; RoPE after dequant, section 3.1).
 *
 * For every batch b, q-head hq and loop step t in [step0, step0 + n_steps):
 * with kv-head h = hq / (n_q_heads / n_kv_heads), block beta = t / T_c and
 * m = t % T_c, the keys are the n_s bf16 sinks sink_k[b][h][t][s] at position
 * s, the dequantized tokens j < N_b, whose channel q*c + i is
 * k_cb[h][beta][k_idx[b][h][beta][j][q]][i*T_c + m] (inverse pre-transform
 * applied when pt != NULL), at position n_s + j, and the n_r bf16 tokens of
 * the recent window recent_k[b][h][t][r] at position n_s + N_b + r (section
 * 3.4 step 1: sinks and the newest tokens stay bf16); every key is rotated
 * (RoPE) at its position; values likewise from v_idx / v_cb / sink_v /
 * recent_v (no RoPE).
 * The result is softmax attention with scale 1/sqrt(D):
 *   out[b][hq][t - step0][0..D)  (fp32)
 *   lse[b][hq][t - step0]        (fp32, natural log-sum-exp of the scaled
 *                                 scores; may be NULL)
 * so a caller can merge it with attention over other keys (Flash-Decoding
 * log-sum-exp combine).  Each index row is decoded once for every step of its
 * block that lies in the requested range.
 *
 *   q          device bf16 [B][n_q_heads][n_steps][D], already rotated
 *   k_idx, v_idx  device uint8 [B][n_kv_heads][n_blk][N_cap][D/c]
 *   k_cb, v_cb device bf16 [n_kv_heads][n_blk][K][G]
 *   sink_k, sink_v  device bf16 [B][n_kv_heads][T][n_s][D], pre-RoPE; may be
 *              NULL when n_s == 0
 *   recent_k, recent_v  device bf16 [B][n_kv_heads][T][R_cap][D], pre-RoPE;
 *              the first n_r tokens are attended; may be NULL when n_r == 0
 *   N          quantized tokens in the cache (N <= N_cap)
 *   seq_len    device int32 [B] or NULL; batch b attends min(seq_len[b], N)
 *              quantized tokens (negative values count as 0)
 *   pt         keys' pre-transform (reads w, perm, sigma) or NULL
 *   rope_table device fp16 table written by loopvq_rope_table for this D and
 *              theta, with n_pos >= n_s + N + n_r positions
 *   workspace  device scratch of at least loopvq_decode_attn_workspace() bytes
 * Alignment: q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, recent_k, recent_v,
 * rope_table and
 * workspace must be 16-byte aligned.
 * A row with no keys at all (n_s == 0, N_b == 0 and n_r == 0) yields out = 0 and
 * lse = -inf.
 * Range: the fast kernels compute in fp16 after power-of-two rescaling of
 * the queries, of each block's codebooks together with the bf16 sinks and
 * recent rows, and of the values; the scales are folded back into the fp32
 * scores and outputs (fp32), so no fp16 value overflows for finite bf16
 * inputs (with keys pre-transformed, the keys' range is taken after the
 * weights w, the queries' after division by them).  Inputs must be finite.
 * Errors: EINVAL for NULL pointers, bad geometry, step range outside [0, T),
 * N > N_cap, n_r > R_cap, n_pos too small; EWORKSPACE for a short workspace; ENOTSUP as for
 * loopvq_encode. */
loopvq_status loopvq_decode_attn(const loopvq_geom* g, const void* q, int32_t step0,
                                 int32_t n_steps, const uint8_t* k_idx, const uint8_t* v_idx,
                                 int32_t N_cap, const void* k_cb, const void* v_cb,
                                 const void* sink_k, const void* sink_v, int32_t n_s,
                                 const void* recent_k, const void* recent_v, int32_t n_r,
                                 int32_t R_cap, int32_t B, int32_t N, const int32_t* seq_len,
                                 const loopvq_pretransform* pt, const void* rope_table,
                                 int32_t n_pos, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* loopvq_decode_attn_noalloc -- loopvq_decode_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * loopvq_decode_attn, without the workspace: the split-context partials go
 * to a static device array of LOOPVQ_NOALLOC_SCRATCH_BYTES, one per GPU,
 * held until the process ends.  The call allocates nothing (its first call
 * on a device looks up that device's array with hipGetSymbolAddress).
 * Every call on one GPU shares that GPU's array: calls that may run at the
 * same time on one GPU (different streams, or one stream fed by several
 * host threads without ordering) race and give wrong results.  Nothing in
 * the array needs clearing: each call writes every partial it reads.
 * Errors: as loopvq_decode_attn; EWORKSPACE when the shape's partials
 * (loopvq_decode_attn_workspace) exceed LOOPVQ_NOALLOC_SCRATCH_BYTES. */
#define LOOPVQ_NOALLOC_SCRATCH_BYTES (8u << 20)
loopvq_status loopvq_decode_attn_noalloc(const loopvq_geom* g, const void* q, int32_t step0,
                                         int32_t n_steps, const uint8_t* k_idx, const uint8_t* v_idx,
                                         int32_t N_cap, const void* k_cb, const void* v_cb,
                                         const void* sink_k, const void* sink_v, int32_t n_s,
                                         const void* recent_k, const void* recent_v, int32_t n_r,
                                         int32_t R_cap, int32_t B, int32_t N, const int32_t* seq_len,
                                         const loopvq_pretransform* pt, const void* rope_table,
                                         int32_t n_pos, float* out, float* lse, void* stream);

/* loopvq_tasq_covariance -- statistics for deriving the keys' channel
 * permutation (section 3.3: the permutation is taken from the T_c*D x T_c*D
 * covariance of a block's stacked step keys).  For every (kv-head, block) it
 * computes, in fp64, the mean and the covariance (centred, divided by B*N) of
 * the scaled keys y[s*D + d] = w[h][d] * k[d] / sigma at block step s, over
 * the B*N (batch entry, token) pairs.  sigma is the same per-(token, step) RMS
 * as in loopvq_encode and is written here first.
 *   x, x_strides  raw bf16 pre-RoPE keys [B][H_kv][T][N] rows of D (as encode)
 *   w             device fp32 [H_kv][D], entries > 0
 *   sigma         device fp16 [B][sig_cap][T], written for tokens 0..N-1
 *   mean          device fp64 [H_kv][T/T_c][T_c*D], written
 *   cov           device fp64 [H_kv][T/T_c][T_c*D][T_c*D], written
 * Errors: EINVAL for NULL pointers, B < 1, N < 1, sig_cap < N, bad strides or
 * geometry; ENOTSUP for D != 128 or T_c*D > 1024.  Stream-ordered, does not
 * synchronize; the result does not depend on launch order (no atomics). */
loopvq_status loopvq_tasq_covariance(const loopvq_geom* g, const void* x, const int64_t x_strides[4],
                                     int32_t B, int32_t N, const float* w, uint16_t* sigma, int32_t sig_cap,
                                     double* mean, double* cov, void* stream);

/* loopvq_tasq_pair_permutation -- host-side grouping of one block's
 * covariance (as written by loopvq_tasq_covariance, copied to host memory)
 * into a channel permutation whose chunks of c channels each hold c/2 whole
 * RoPE pairs {u, u + D/2} (section 3.3).  Pairs u, v < D/2 are scored by the
 * sum of |correlation| over their two channels each and every (step, step)
 * combination; groups are built one at a time: the free pair with the largest
 * score to all free pairs seeds a group, then the free pair with the largest
 * summed score to the group's members joins, until c/2 pairs; ties go to the
 * lowest pair number.  Chunk q is the q-th group, its pairs in joining order,
 * each as (u, u + D/2).
 *   cov   host fp64 [T_c*D][T_c*D]
 *   perm  host int16 [D], written: transformed channel d' holds raw channel
 *         perm[d'] (the loopvq_pretransform convention)
 * Errors: EINVAL for NULL pointers, T_c < 1, odd D, odd c or c not dividing D. */
loopvq_status loopvq_tasq_pair_permutation(const double* cov, int32_t T_c, int32_t D, int32_t c,
                                           int16_t* perm);

/* loopvq_kmeans_accumulate -- the update half of one step of the
 * importance-weighted k-means that builds the codebooks ("codebook and
 * calibration", eq. 3: joint vector n weighs omega_n = ||dL/dz_n||^2, summed
 * over the T_c steps it covers).  The assignment is loopvq_encode's exact
 * argmin of the same vectors.  For every joint vector n of the B x N tokens
 * with index r = idx[n] < K it adds, in fp64,
 *     sums[h][beta][r][u] += omega_n * z_n[u]   (u = i*T_c + m, eq. 4 layout)
 *     wsum[h][beta][r]    += omega_n
 * where z_n is the bf16 joint vector, or with pt the pre-transformed key
 * w[p(d')] * k[p(d')] / sigma in fp64 (sigma as written by loopvq_encode).
 *   x, x_strides  the encoded bf16 cache [B][H_kv][T][N] rows of D (as encode)
 *   idx, N_cap    indices written by loopvq_encode for the same x
 *   weight        device fp32 [B][H_kv][T/T_c][N][D/c] (omega per joint
 *                 vector) or NULL for all ones
 *   sums, wsum    device fp64 [H_kv][T/T_c][K][G] and [H_kv][T/T_c][K];
 *                 accumulated (zero them before the first call of a step)
 * The fp64 sums are accumulated with atomics, so their last bits depend on
 * the order of execution.  Errors: EINVAL for NULL pointers, negative B or N,
 * N > N_cap, bad strides, an undersized pt->N_cap; ENOTSUP for D != 128 or G
 * not in {16, 32}.  N == 0 or B == 0 is a no-op. */
loopvq_status loopvq_kmeans_accumulate(const loopvq_geom* g, const void* x, const int64_t x_strides[4],
                                      int32_t B, int32_t N, const uint8_t* idx, int32_t N_cap,
                                      const float* weight, const loopvq_pretransform* pt, double* sums,
                                      double* wsum, void* stream);

/* loopvq_kmeans_finalize -- the new codebook of the step: every entry with
 * wsum > 0 becomes sums / wsum rounded to bf16 (to nearest, ties to even,
 * from the fp64 quotient); entries with zero weight keep their value.
 *   codebook  device bf16 [H_kv][T/T_c][K][G], updated in place
 * Errors: EINVAL for NULL pointers; ENOTSUP as for the geometry. */
loopvq_status loopvq_kmeans_finalize(const loopvq_geom* g, const double* sums, const double* wsum,
                                    void* codebook, void* stream);

/* ---- loop-aware codebook fine-tuning (section 3.2, eq. 6) ----
 * The objective compares the model's outputs with the precise cache and with
 * the cache rebuilt from the codebooks at every position after the sinks,
 * with all loop steps reading the rebuilt cache; the codebook entries get
 * exact gradients by backpropagation (the assignment is a constant of each
 * iteration).  The two calls below are that attention and its backward pass;
 * the model around them and the optimizer are the caller's. */

/* loopvq_rope_table_f32 -- fp32 RoPE table for the calls below.
 *   table  device fp32 [n_pos][D/2][2]: cos and sin of p * theta^(-2f/D),
 *          evaluated in fp64 on the GPU, rounded once to fp32
 * Errors: EINVAL for NULL table, n_pos < 1, odd D, theta <= 0. */
loopvq_status loopvq_rope_table_f32(float theta, int32_t D, int32_t n_pos, float* table, void* stream);

/* loopvq_prefill_attn -- causal attention of the N positions after the sinks
 * over the compressed cache of those N tokens.
 *
 * For every batch b, q-head hq and loop step t in [step0, step0 + n_steps),
 * with kv-head h = hq / (n_q_heads / n_kv_heads), block beta = t / T_c and
 * m = t % T_c: query i (i < N) sits at position n_s + i and attends to the
 * n_s bf16 sinks sink_k[b][h][t][s] (position s) and to the tokens j <= i,
 * whose channel q*c + i' is k_cb[h][beta][k_idx[b][h][beta][j][q]][i'*T_c + m]
 * (section 3.1 eq. 5) at position n_s + j (with pt, the inverse
 * pre-transform is applied first: raw channel p(d') is coordinate d' times
 * sigma[b][j][t] / w[h][p(d')]); keys are rotated (RoPE) at their positions,
 * values come from v_idx / v_cb / sink_v; scale 1/sqrt(D).
 *   q          device fp32 [B][n_q_heads][n_steps][N][D], already rotated
 *   k_idx, v_idx  device uint8 [B][n_kv_heads][n_blk][N_cap][D/c]
 *   k_cb, v_cb device bf16 [n_kv_heads][n_blk][K][G]
 *   sink_k, sink_v  device bf16 [B][n_kv_heads][T][n_s][D], pre-RoPE; may be
 *              NULL when n_s == 0
 *   pt         keys' pre-transform (reads w, perm and the sigma the encode
 *              wrote for tokens 0..N-1) or NULL
 *   rope_table device fp32 table of loopvq_rope_table_f32 with
 *              n_pos >= n_s + N positions
 *   out        device fp32 [B][n_q_heads][n_steps][N][D], written
 *   lse        device fp32 [B][n_q_heads][n_steps][N], written (natural log)
 * Alignment: q, sinks, rope_table and out 16-byte aligned.
 * Errors: EINVAL for NULL pointers, bad geometry, step range outside [0, T),
 * N > N_cap, n_pos too small, misalignment; ENOTSUP as for loopvq_encode.
 * B == 0 or N == 0 is a no-op (the tensor pointers may then be NULL).
 * Deterministic. */
loopvq_status loopvq_prefill_attn(const loopvq_geom* g, const float* q, int32_t step0, int32_t n_steps,
                                  int32_t B, int32_t N, const uint8_t* k_idx, const uint8_t* v_idx,
                                  int32_t N_cap, const void* k_cb, const void* v_cb, const void* sink_k,
                                  const void* sink_v, int32_t n_s, const loopvq_pretransform* pt,
                                  const float* rope_table, int32_t n_pos, float* out, float* lse, void* stream);

/* loopvq_prefill_attn_backward_workspace -- bytes of scratch the backward
 * needs: B * n_q_heads * n_steps * N floats. */
loopvq_status loopvq_prefill_attn_backward_workspace(const loopvq_geom* g, int32_t B, int32_t N,
                                                     int32_t step0, int32_t n_steps, size_t* bytes);

/* loopvq_prefill_attn_backward -- gradients of loopvq_prefill_attn for a
 * given d_out (same arguments as the forward, plus its out and lse):
 *   d_q        device fp32 like q, written
 *   d_k_cb, d_v_cb  device fp32 [n_kv_heads][n_blk][K][G], overwritten with
 *              the gradient with respect to the bf16 codebook entries the
 *              forward read (summed over every batch entry, q-head, step and
 *              token of the call; keys pass back through the rotation and,
 *              with pt, the inverse pre-transform)
 *   workspace  device scratch of loopvq_prefill_attn_backward_workspace()
 *              bytes, 16-byte aligned
 * Alignment: as the forward, plus out, d_out and d_q 16-byte aligned.
 * Errors: as the forward; EWORKSPACE for a short workspace.  The codebook
 * gradients are summed with fp32 atomics, so their last bits depend on the
 * order of execution; d_q is deterministic.  B == 0 or N == 0 zeroes
 * d_k_cb and d_v_cb (which must not be NULL; the other tensors may be). */
loopvq_status loopvq_prefill_attn_backward(const loopvq_geom* g, const float* q, int32_t step0,
                                           int32_t n_steps, int32_t B, int32_t N, const uint8_t* k_idx,
                                           const uint8_t* v_idx, int32_t N_cap, const void* k_cb,
                                           const void* v_cb, const void* sink_k, const void* sink_v,
                                           int32_t n_s, const loopvq_pretransform* pt, const float* rope_table,
                                           int32_t n_pos, const float* out, const float* lse, const float* d_out,
                                           float* d_q, float* d_k_cb, float* d_v_cb, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* Thread-local text of the last non-OK status ("" if none). */
const char* loopvq_last_error(void);

/* LOOPVQ_ABI_VERSION of the built library. */
int32_t loopvq_abi_version(void);

/* loopvq_precise_attn / loopvq_precise_attn_backward -- the same causal
 * attention as loopvq_prefill_attn (query i of a step at position n_s + i
 * attends to the sinks and to tokens j <= i) over the PRECISE cache, and its
 * gradients, for the importance weights of the codebook k-means ("codebook
 * and calibration", eq. 3: omega_n = ||dL/dz_n||^2 of the precise cache's
 * joint vectors).
 *   q             device fp32 [B][n_q_heads][n_steps][N][D], post-RoPE
 *   k, v          device bf16 [B][n_kv_heads][T][N_x][D], the stored cache
 *                 (keys pre-RoPE), tokens 0..N-1 attended, N <= N_x
 *   sink_k, sink_v, rope_table (fp32 table of loopvq_rope_table_f32),
 *   out, lse      as in loopvq_prefill_attn
 * Backward: d_q (fp32 like q) is written; the gradients of the loss with
 * respect to every attended cached key (before RoPE) and value of the served
 * steps are ADDED into d_k and d_v (fp32 [B][n_kv_heads][T][N_x][D]; zero them
 * before the first call; q-heads of a GQA group add into their kv-head's
 * tokens, in an order that may vary in the last bits).  workspace: at least
 * loopvq_prefill_attn_backward_workspace() bytes.
 * Errors: EINVAL for NULL pointers, N > N_x, bad geometry or step range, a
 * short rope table, misaligned tensors (16 bytes for q, k, v, sinks, tables,
 * out, d_out, d_q); EWORKSPACE for a short workspace. */
loopvq_status loopvq_precise_attn(const loopvq_geom* g, const float* q, int32_t step0, int32_t n_steps,
                                  int32_t B, int32_t N, const void* k, const void* v, int32_t N_x,
                                  const void* sink_k, const void* sink_v, int32_t n_s, const float* rope_table,
                                  int32_t n_pos, float* out, float* lse, void* stream);
loopvq_status loopvq_precise_attn_backward(const loopvq_geom* g, const float* q, int32_t step0, int32_t n_steps,
                                           int32_t B, int32_t N, const void* k, const void* v, int32_t N_x,
                                           const void* sink_k, const void* sink_v, int32_t n_s,
                                           const float* rope_table, int32_t n_pos, const float* out,
                                           const float* lse, const float* d_out, float* d_q, float* d_k,
                                           float* d_v, void* workspace, size_t workspace_bytes, void* stream);

/* loopvq_fisher_weights -- importance of every joint vector for the weighted
 * k-means ("codebook and calibration", eq. 3; section 3.1: a loop-axis joint
 * vector covers T_c steps): omega_n = sum over the G coordinates of z_n of
 * (dL/dz_n)^2, where coordinate i*T_c + m of chunk q is channel q*c + i at
 * block step m.  With the keys' pre-transform (pt, section 3.3) the key
 * vector is z[d'] = w[perm[d']] k[perm[d']] / sigma, so dL/dz[d'] =
 * d_k[perm[d']] * sigma / w[perm[d']] (sigma fixed, as stored).
 *   d_k, d_v        device fp32 [B][n_kv_heads][T][N_x][D] (as written by
 *                   loopvq_precise_attn_backward over every step)
 *   omega_k, omega_v  device fp32 [B][n_kv_heads][T/T_c][N][D/c], written;
 *                   the `weight` input of loopvq_kmeans_accumulate
 * Each omega is summed in fp64 and rounded once to fp32.
 * Errors: EINVAL for NULL pointers, N > N_x, bad geometry or pre-transform. */
loopvq_status loopvq_fisher_weights(const loopvq_geom* g, const float* d_k, const float* d_v, int32_t B, int32_t N,
                                    int32_t N_x, const loopvq_pretransform* pt, float* omega_k, float* omega_v,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LOOPVQ_H */
