/*
 * kda.h -- C ABI of libkda.so: the Kimi Delta Attention (KDA) mixer's hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "colibri/c/kimi_k3.c", file header comment "KDA per-head
 * recurrence"), per sequence and head, head dim D = 128:
 *
 *   q,k,v = SiLU(ShortConv4(x))        depthwise causal conv, 4 taps, oldest tap first,
 *                                      no bias; x_{t<0} taken from the carried conv state
 *   q,k   L2-normalised over the head's D channels, eps added inside the sqrt;
 *         q *= q_scale (D^-0.5)
 *   gk    = gate_lower_bound * sigmoid(exp(A_log[h]) * (z + dt_bias)),  alpha = exp(gk)
 *   beta  = sigmoid(b)
 *   S     = (I - beta k k^T) Diag(alpha) S + beta k v^T       S[key][value], fp32
 *   o     = S^T q                                             with the updated S
 *   out   = sigmoid(g) * RMSNorm(o)                           RMSNorm weight norm_w[D],
 *                                                             shared by all heads
 *
 * The projections that produce the pre-conv q/k/v and the z/b/g logits, and the output
 * projection, are not part of this library.
 *
 * Layouts (row-major; every array dense except q, k, v, whose rows are qkv_row_stride
 * elements apart):
 *   per-token activations q, k, v, z, g   [tokens, H*D]   channel h*D+i of head h
 *   beta logits b                         [tokens, H]
 *   conv_w                                [3*H*D, 4]      rows: the q block (H*D), then
 *                                                         k, then v; taps oldest first
 *   A_log [H], dt_bias [H*D], norm_w [D]
 *   state                                 [B, H, D, D]    S[key][value], fp32
 *   conv_state                            [B, 3*H*D, 3]   the 3 previous pre-conv inputs
 *                                                         of each channel, oldest first
 *   out                                   [tokens, H*D]   fp32, or bf16 (raw bit
 *                                                         patterns, round to nearest
 *                                                         even) with KDA_OUT_BF16
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers (HIP) unless stated; the caller owns every buffer.
 *     The library allocates and frees nothing and never synchronises: all work is
 *     queued on the given HIP stream (NULL = the default stream), so a call may be
 *     captured into a HIP graph.
 *   - Arguments are checked on the host before anything is queued; a rejected call
 *     queues nothing and leaves every buffer untouched.  Values inside device buffers
 *     (e.g. cu_seqlens) cannot be checked on the host; the kernels clamp them so that
 *     no access leaves the buffers the sizes describe.
 *   - The library never exits or aborts.  A device fault surfaces at the caller's next
 *     synchronisation.
 *   - Calls on different streams that touch different buffers may run concurrently;
 *     calls that write the same state buffer must be ordered by the caller.
 *   - qkv_row_stride: element distance between consecutive token rows of q, k and v (0
 *     means dense, H*D).  Otherwise it must be >= H*D, a multiple of 8 and at most 2^24,
 *     so that q, k and v can be row-strided views of one fused [tokens, 3*H*D]
 *     projection output (the header comment "KDA per-head recurrence" derives q, k and v
 *     from the three projections W{q,k,v} x, which one GEMM produces side by side).  The
 *     three views may overlap each other: they are only read.
 *   - Outputs never overlap inputs or each other (KDA_ERR_OVERLAP), except the exact
 *     in-place aliases an entry point names (e.g. final_state == initial_state).  Extents
 *     are the byte ranges the sizes describe; q, k, v span (rows-1)*stride + H*D
 *     elements.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 11

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_ARG = 1,   /* a required pointer is NULL */
    KDA_ERR_BAD_CONFIG = 2, /* head_dim != 128, conv_size != 4, num_heads outside
                               1..65536, bad eps, prefill_path outside 0..2 (kda_prefill),
                               out_dtype or precision outside 0..1 */
    KDA_ERR_BAD_SHAPE = 3,  /* negative or inconsistent sizes, or sizes past the limits */
    KDA_ERR_MISALIGNED = 4, /* a pointer is not 16-byte aligned (workspace: 256-byte) */
    KDA_ERR_WORKSPACE = 5,  /* workspace smaller than kda_prefill_workspace_bytes() */
    KDA_ERR_LAUNCH = 6,     /* the HIP runtime refused a kernel launch or a copy */
    KDA_ERR_OVERLAP = 7     /* an output buffer overlaps an input or another output (other
                               than an exact in-place alias the entry point allows) */
} kda_status;

/* Mixer constants.  Fill with kda_config_default() and set num_heads. */
typedef struct {
    int32_t num_heads;      /* H, 1 .. 65536 */
    int32_t head_dim;       /* D; must be 128 (the pages' KDA head dim) */
    int32_t conv_size;      /* ShortConv taps; must be 4 */
    float gate_lower_bound; /* gmin of the decay gate; the pages' value is -5 */
    float l2_eps;           /* added to sum(x^2) inside the sqrt of the q/k L2 norm; 1e-6 */
    float rms_eps;          /* eps of the per-head RMSNorm of o; the loader's rms default 1e-5 */
    float q_scale;          /* scale of the normalised q; <= 0 selects D^-0.5 */
    int32_t prefill_path;   /* KDA_PREFILL_AUTO, _FUSED or _CHUNKED (kda_prefill only) */
    int32_t out_dtype;      /* KDA_OUT_F32 or KDA_OUT_BF16: element type of every `out` */
    int32_t precision;      /* KDA_PRECISION_STANDARD or _HIGH (kda_prefill only) */
    int32_t decode_multi_form; /* KDA_MULTI_BLOCK or _SEQUENTIAL (kda_decode_multi only) */
} kda_config;

/* How kda_decode_multi evaluates its tokens (both fp32, the same recurrence):
 *   KDA_MULTI_BLOCK       blocks of eight tokens in the chunk form of the recurrence, with
 *                         the state products on fp32 MFMAs; agrees with the same number
 *                         of kda_decode_step calls to fp32 rounding (about 3e-6
 *                         relative), not bit for bit.  About 1.6x faster at 8 tokens.
 *   KDA_MULTI_SEQUENTIAL  token by token with kda_decode_step's arithmetic in the same
 *                         order: n tokens give the bits of n kda_decode_step calls. */
#define KDA_MULTI_BLOCK 0
#define KDA_MULTI_SEQUENTIAL 1

/* Operand precision of kda_prefill's chunked algebra (decode is fp32 throughout).
 *   KDA_PRECISION_STANDARD  bf16 MFMA operands with fp32 accumulation, the operands that
 *                           decide the state's and the output's error split into bf16
 *                           hi + lo.  Within 2e-2 (outputs) and 5e-3 (states, relative) of
 *                           the fp64 recurrence for gates with decay; with no decay and
 *                           beta -> 1 on every token (the plain delta rule, where no
 *                           rounding is ever forgotten) the output error grows to about
 *                           2e-2 at 1K tokens and 3e-2 at 8K.
 *   KDA_PRECISION_HIGH      every MFMA operand of the chunk algebra split into bf16 hi +
 *                           lo (about 16 significant bits each): about 1e-4 in that regime
 *                           too.  Costs more MFMA and VALU work per chunk, and the chunked
 *                           layout's records grow from 111,616 to 144,384 bytes. */
#define KDA_PRECISION_STANDARD 0
#define KDA_PRECISION_HIGH 1

/* Element type of the output buffers.  With KDA_OUT_BF16 each output is the fp32 result
 * rounded to the nearest bf16 (ties to even), at half the bytes; states and conv windows
 * stay fp32 either way. */
#define KDA_OUT_F32 0
#define KDA_OUT_BF16 1

/* How kda_prefill lays out its work (the result is the same up to rounding order):
 *   KDA_PREFILL_FUSED    one workgroup per (sequence, head) walks the sequence chunk by
 *                        chunk; no workspace.  Fills the GPU when B*H is large.
 *   KDA_PREFILL_CHUNKED  one workgroup per (64-token chunk, head) computes the chunk's
 *                        state-independent products into the workspace, then one
 *                        workgroup per (sequence, head) carries the state through them
 *                        (two, each owning half the value columns, when B*H <= 128 in
 *                        the standard precision).  Fills the GPU when B*H is small (a
 *                        few long sequences).  For B*H <= 128 (either precision),
 *                        where the device has at least 2*B*H compute units
 *                        and an estimate predicts it faster, the
 *                        carries run in the same launch as the chunk workgroups and
 *                        follow the records as they are written (same bits).  A carry
 *                        waits for a record a few seconds at most; if other work on
 *                        the device kept the chunk workgroups from running that long,
 *                        the outputs and final states of the call would be NaN.
 *   KDA_PREFILL_AUTO     the one an estimate of both times on MI355X predicts faster,
 *                        from B, H and N (the sequences taken as equal in length): CHUNKED
 *                        for a few long sequences (e.g. B*H = 96 or 288 units), FUSED when
 *                        B*H fills whole rounds of 256 workgroups (e.g. 192, 384, 1536). */
#define KDA_PREFILL_AUTO 0
#define KDA_PREFILL_FUSED 1
#define KDA_PREFILL_CHUNKED 2

/* Defaults: H = 96, D = 128, conv 4, gmin -5, l2_eps 1e-6, rms_eps 1e-5, q_scale D^-0.5
 * (page "colibri/c/kimi_k3.c": header comment "KDA per-head recurrence" and the
 * config loader's rms_norm_eps default), prefill_path KDA_PREFILL_AUTO, out_dtype
 * KDA_OUT_F32, precision KDA_PRECISION_STANDARD. */
kda_config kda_config_default(void);

/*
 * kda_decode_step -- one new token for each of B sequences against resident states.
 *
 * Follows the header comment "KDA per-head recurrence" (page "colibri/c/kimi_k3.c")
 * for a single token: the conv window of every channel is advanced by one input, the
 * state is decayed, corrected and written, and the gated, normalised readout is
 * returned.  The state is streamed once: each 64 KiB head state is read and written
 * exactly once per call.
 *
 *   batch                  B >= 0 (0: nothing queued, KDA_OK)
 *   q, k, v                [B, H*D] fp32 pre-conv inputs of the new token, rows
 *                          qkv_row_stride elements apart (0: dense)
 *   z                      [B, H*D] fp32 decay logits, before dt_bias
 *   b                      [B, H]   fp32 beta logits
 *   g                      [B, H*D] fp32 output-gate logits
 *   conv_w, A_log, dt_bias, norm_w   fp32 parameters (layouts above)
 *   state                  [B, H, D, D] fp32, read and overwritten in place
 *   conv_state             [B, 3*H*D, 3] fp32, read and overwritten in place
 *   out                    [B, H*D] fp32 or bf16 (cfg->out_dtype), written
 *   stream                 hipStream_t or NULL
 * state, conv_state and out must not overlap each other or any input (KDA_ERR_OVERLAP).
 * Alignment: every pointer 16-byte aligned.  Limits: B*H <= 16,777,215 (one
 * workgroup of 256 lanes per (sequence, head) in one dispatch).
 */
kda_status kda_decode_step(const kda_config *cfg, int32_t batch,
                           const float *q, const float *k, const float *v, int64_t qkv_row_stride,
                           const float *z, const float *b, const float *g,
                           const float *conv_w, const float *A_log, const float *dt_bias,
                           const float *norm_w,
                           float *state, float *conv_state, void *out,
                           void *stream);

/*
 * kda_decode_step_slots -- kda_decode_step for a batch whose states live in a pool:
 * batch row r (its token inputs and output row r) advances pool entry slots[r] of
 * state_pool and conv_pool.  The per-row step is exactly kda_decode_step's (the same
 * kernel, so the same bits).  This is the multiplexed decode step of the serving
 * engine, where each batch row is one token of one of several parked conversations and
 * carries its own recurrent state (page "colibri/c/kimi_k3.c": the K3Seq / K3Row
 * structures and the multiplexed step over them), with the states held in one device
 * pool rather than a dense [B, ...] batch.
 *
 *   batch                  B >= 0 rows (0, or pool_size 0: nothing queued, KDA_OK)
 *   slots                  device int32 [B]: the pool entry of row r.  A row whose slot
 *                          lies outside [0, pool_size) is skipped: its pool entries are
 *                          not touched and its output row is left as it was.  Two rows
 *                          must not name the same slot (their updates race; the
 *                          result for that slot is unspecified, every access still
 *                          stays inside the pool)
 *   pool_size              P >= 0 entries in state_pool and conv_pool
 *   q, k, v, z, g          [B, H*D] fp32 (q, k, v rows qkv_row_stride apart);  b [B, H]
 *                          fp32 (row r is slot slots[r]'s token)
 *   conv_w, A_log, dt_bias, norm_w   fp32 parameters (layouts above)
 *   state_pool             [P, H, D, D] fp32, entries of valid slots read and
 *                          overwritten in place
 *   conv_pool              [P, 3*H*D, 3] fp32, likewise
 *   out                    [B, H*D] fp32 or bf16 (cfg->out_dtype)
 *   stream                 hipStream_t or NULL
 * state_pool, conv_pool and out must not overlap each other or any input.
 * Alignment: every fp32 pointer 16-byte aligned, slots 4-byte aligned.
 * Limits: B*H <= 16,777,215.
 */
kda_status kda_decode_step_slots(const kda_config *cfg, int32_t batch, const int32_t *slots, int32_t pool_size,
                                 const float *q, const float *k, const float *v, int64_t qkv_row_stride,
                                 const float *z, const float *b, const float *g,
                                 const float *conv_w, const float *A_log, const float *dt_bias,
                                 const float *norm_w,
                                 float *state_pool, float *conv_pool, void *out,
                                 void *stream);

/*
 * kda_decode_multi -- up to `tokens` new tokens for each of B sequences in one call:
 * the state is read once, carried through the tokens, and written once.  This is the
 * decode step for several known tokens (speculative verification, or a short chunk of
 * a prompt against a resident state); each token follows the header comment "KDA
 * per-head recurrence" (page "colibri/c/kimi_k3.c").  cfg->decode_multi_form picks how:
 * KDA_MULTI_BLOCK (default) evaluates blocks of eight tokens in the chunk form of that
 * recurrence (the same terms summed in another order), so n tokens agree with n
 * kda_decode_step calls to fp32 rounding (about 3e-6 relative), not bit for bit, and a
 * call with n_tokens = a repeats, bit for bit, the outputs of the first a tokens of a
 * call with more tokens; KDA_MULTI_SEQUENTIAL runs kda_decode_step's arithmetic token by
 * token, so n tokens give the bits of n kda_decode_step calls.  The final conv windows
 * are exact either way.
 *
 * Verify and roll back (the engine's multi-token verify and rollback are not
 * implemented on the pages; this is this library's form of it): call with
 * state_out != state_in, so that state_in keeps the state before the candidates; after
 * accepting a prefix of a_s tokens of sequence s, call again from state_in with
 * n_tokens = a to commit exactly the accepted prefix (state_out may then be state_in).
 *
 *   batch                  B >= 0 (0: nothing queued, KDA_OK)
 *   tokens                 T >= 1 when B > 0: the token slots per sequence
 *   n_tokens               device int32 [B]: tokens to apply to sequence s (clamped to
 *                          [0, T]; the rest of its slots are ignored), or NULL for T each
 *   q, k, v, z, g          [B, T, H*D] fp32 (row s*T + t is token t of sequence s; the
 *                          rows of q, k, v are qkv_row_stride elements apart)
 *   b                      [B, T, H] fp32
 *   conv_w, A_log, dt_bias, norm_w   fp32 parameters (layouts above)
 *   state_in, state_out    [B, H, D, D] fp32; either the same buffer (update in place)
 *                          or disjoint
 *   conv_state_in, conv_state_out   [B, 3*H*D, 3] fp32; the same buffer or disjoint
 *   out                    [B, T, H*D] fp32 or bf16 (cfg->out_dtype): rows of applied
 *                          tokens are written, the others are left untouched
 *   stream                 hipStream_t or NULL
 * A sequence with n_tokens 0 copies its state and windows to the outputs.
 * state_out, conv_state_out and out must not overlap each other or any input other than
 * their own exact alias (state_out == state_in, conv_state_out == conv_state_in).
 * Alignment: every fp32 pointer 16-byte aligned, n_tokens 4-byte aligned.
 * Limits: B*H <= 16,777,215; B*T <= 2^31-1.
 */
kda_status kda_decode_multi(const kda_config *cfg, int32_t batch, int32_t tokens, const int32_t *n_tokens,
                            const float *q, const float *k, const float *v, int64_t qkv_row_stride,
                            const float *z, const float *b, const float *g,
                            const float *conv_w, const float *A_log, const float *dt_bias,
                            const float *norm_w,
                            const float *state_in, float *state_out,
                            const float *conv_state_in, float *conv_state_out,
                            void *out, void *stream);

/*
 * kda_decode_multi_slots -- kda_decode_multi for states held in pools, as
 * kda_decode_step_slots is for kda_decode_step: batch row r (its tokens, its n_tokens
 * entry and its output rows) reads entry slots[r] of state_in / conv_state_in and writes
 * entry slots[r] of state_out / conv_state_out.  The per-row work is exactly
 * kda_decode_multi's (the same kernel), so verify and roll back work the same way over a
 * pool: candidates into a second pool (state_out != state_in), then the accepted
 * prefixes committed in place.
 *
 *   slots                  device int32 [B]; a row whose slot lies outside
 *                          [0, pool_size) is skipped (its pool entries and output rows are
 *                          not touched); two rows must not name the same slot
 *   pool_size              P >= 0 entries in each of the four pools (0: nothing queued)
 *   state_in, state_out    [P, H, D, D] fp32; the same buffer or disjoint
 *   conv_state_in, conv_state_out   [P, 3*H*D, 3] fp32; the same buffer or disjoint
 *   all other arguments    as for kda_decode_multi ([B, T, ...] token rows, out [B, T, H*D])
 * Alignment: every fp32 pointer 16-byte aligned, n_tokens and slots 4-byte aligned.
 * Limits: B*H <= 16,777,215; B*T <= 2^31-1.
 */
kda_status kda_decode_multi_slots(const kda_config *cfg, int32_t batch, int32_t tokens, const int32_t *n_tokens,
                                  const int32_t *slots, int32_t pool_size,
                                  const float *q, const float *k, const float *v, int64_t qkv_row_stride,
                                  const float *z, const float *b, const float *g,
                                  const float *conv_w, const float *A_log, const float *dt_bias,
                                  const float *norm_w,
                                  const float *state_in, float *state_out,
                                  const float *conv_state_in, float *conv_state_out,
                                  void *out, void *stream);

/*
 * kda_prefill -- a packed batch of whole sequences (varlen), processed in chunks of
 * 64 tokens with the chunked (WY / UT-transform) form of the same recurrence; returns
 * every token's output and each sequence's final state and conv state.  The work
 * layout follows cfg->prefill_path (see KDA_PREFILL_*).
 *
 * Follows the header comment "KDA per-head recurrence" (page "colibri/c/kimi_k3.c");
 * the engine's prefill also runs in token chunks (same page, ENV K3_CHUNK).  The
 * chunked form gives the token recurrence's result up to rounding.
 *
 *   num_seqs               B >= 0 (0: nothing queued)
 *   total_tokens           N >= 0, the packed token count
 *   cu_seqlens             device int32 [B+1]: sequence s holds tokens
 *                          cu_seqlens[s] .. cu_seqlens[s+1]-1; must start at 0, be
 *                          non-decreasing and end at N (values are clamped to [0, N])
 *   q, k, v, z, g          [N, H*D] bf16 (raw bit patterns); the rows of q, k, v are
 *                          qkv_row_stride elements apart (0: dense)
 *   b                      [N, H]   bf16
 *   conv_w, A_log, dt_bias, norm_w   fp32 parameters
 *   initial_state          [B, H, D, D] fp32, or NULL for zeros
 *   initial_conv_state     [B, 3*H*D, 3] fp32, or NULL for zeros
 *   out                    [N, H*D] fp32 or bf16 (cfg->out_dtype), written
 *   final_state            [B, H, D, D] fp32, written; may be the same pointer as
 *                          initial_state (in-place carry), must not partially overlap it
 *                          (KDA_ERR_OVERLAP)
 *   final_conv_state       [B, 3*H*D, 3] fp32, written; may equal initial_conv_state,
 *                          must not partially overlap it
 *   workspace              device scratch of workspace_bytes >=
 *                          kda_prefill_workspace_bytes(cfg, B, N), 256-byte aligned;
 *                          may be NULL when that is 0.  Contents on entry are ignored
 *                          and on return are unspecified; two calls that overlap in
 *                          time must not share it.
 *   stream                 hipStream_t or NULL
 * A sequence of length 0 copies its initial state and conv state to the final ones.
 * out, final_state, final_conv_state and the workspace must not overlap each other or
 * any input other than the two exact aliases above.
 * Alignment: every fp32/bf16 array pointer 16-byte aligned, cu_seqlens 4-byte aligned.
 * Limits: N <= 2^31-1; B*H <= 8,388,607 (one workgroup of 512 lanes per (sequence,
 * head) in one dispatch); for the chunked layout also (floor(N/64) + B)*H <= 8,388,607
 * and (floor((floor(N/64) + B)/4) + B)*H <= 8,388,607
 * (KDA_PREFILL_AUTO falls back to FUSED past it; an explicit CHUNKED returns
 * KDA_ERR_BAD_SHAPE).
 */
kda_status kda_prefill(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens,
                       const int32_t *cu_seqlens,
                       const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t qkv_row_stride,
                       const uint16_t *z, const uint16_t *b, const uint16_t *g,
                       const float *conv_w, const float *A_log, const float *dt_bias,
                       const float *norm_w,
                       const float *initial_state, const float *initial_conv_state,
                       void *out, float *final_state, float *final_conv_state,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_prefill_gate_proj -- kda_prefill with the decay logits formed inside the library
 * from the low-rank decay projection: instead of z = W_fb(W_fa x) the caller passes
 * f = W_fa x, shared by all heads, and the second factor W_fb; each chunk forms its
 * logits z = W_fb f with bf16 MFMAs (fp32 accumulation) before the gate.  The page
 * "colibri/c/kimi_k3.c" gives the gate's argument as W_fb(W_fa x) + dt_bias (header
 * comment "KDA per-head recurrence") and the two factors as the `Kda` struct's decay
 * low-rank pair `fa, fb`.  This reads 256 bytes per token (f) instead of 256 bytes per
 * token and head (z).
 *
 *   f                      [N, 128] bf16 (raw bit patterns): W_fa x of each token
 *   w_fb                   [H*D, 128] bf16: row h*D + i is channel i of head h
 *   all other arguments    as for kda_prefill (z is not taken; the rank is 128)
 * The logits are not rounded to bf16 (kda_prefill takes them as bf16), so the results
 * match kda_prefill's only up to that rounding.  Alignment: f and w_fb 16-byte aligned.
 */
kda_status kda_prefill_gate_proj(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens,
                                 const int32_t *cu_seqlens,
                                 const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t qkv_row_stride,
                                 const uint16_t *f, const uint16_t *w_fb,
                                 const uint16_t *b, const uint16_t *g,
                                 const float *conv_w, const float *A_log, const float *dt_bias,
                                 const float *norm_w,
                                 const float *initial_state, const float *initial_conv_state,
                                 void *out, float *final_state, float *final_conv_state,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_prefill_noalloc -- kda_prefill for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation (the same kernels, so the same bits) with no workspace
 * arguments: the chunked layout's workspace is a scratch array the library holds in
 * each device's memory (KDA_NOALLOC_SCRATCH_BYTES = 256 MiB, kept until the process
 * ends), never a caller buffer; the call allocates nothing.
 *
 *   all arguments          as for kda_prefill
 * Layout: cfg->prefill_path as for kda_prefill, except that KDA_PREFILL_AUTO takes the
 * chunked layout only when its workspace (kda_prefill_workspace_bytes with
 * KDA_PREFILL_CHUNKED) fits in the scratch array, and the fused layout (no workspace)
 * otherwise.  An explicit KDA_PREFILL_CHUNKED that needs more than
 * KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_WORKSPACE.
 * The first call on a device looks up that device's array (hipGetSymbolAddress, with
 * the device current); KDA_ERR_LAUNCH if the runtime refuses.  Every call on one device
 * uses the same array and leaves its contents behind: two calls that overlap in time on
 * one device (e.g. on two streams) race, so the caller must order them.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
kda_status kda_prefill_noalloc(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens,
                               const int32_t *cu_seqlens,
                               const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t qkv_row_stride,
                               const uint16_t *z, const uint16_t *b, const uint16_t *g,
                               const float *conv_w, const float *A_log, const float *dt_bias,
                               const float *norm_w,
                               const float *initial_state, const float *initial_conv_state,
                               void *out, float *final_state, float *final_conv_state, void *stream);

/* Device scratch kda_prefill needs for these sizes with cfg->prefill_path and
 * cfg->precision: 0 for the fused layout; for the chunked one a table of 2(B+1) int32
 * (padded to 256 bytes); where the carries run in the chunk workgroups' launch (B*H <=
 * 128, when the estimate prefers it), 4 bytes per (chunk, head) of
 * records' ready words (padded to 256 bytes) and, for B > 1, 4 bytes per chunk-kernel
 * segment of the segments' order (padded to 256 bytes); otherwise, for B*H <= 128 in the
 * standard precision, 4,096 bytes per (sequence, head) for the two-workgroup carry's row
 * sums; then one record per (chunk, head) (111,616 bytes, or 144,384 with
 * KDA_PRECISION_HIGH) for floor(N/64) + B chunks (the most that B sequences of N tokens
 * in total can need).  Returns 0 for arguments kda_prefill would reject. */
size_t kda_prefill_workspace_bytes(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens);

/*
 * kda_state_copy -- copy whole (sequence) entries of recurrent state and conv windows
 * between two state buffers: entry src_slots[i] of (src_state, src_conv) to entry
 * dst_slots[i] of (dst_state, dst_conv), for i = 0 .. n-1, in that order.
 *
 * The serving engine on page "colibri/c/kimi_k3.c" keeps "photos" of the KDA recurrent
 * state and its three conv windows at turn boundaries (ENV COLI_K3_CKPT /
 * COLI_K3_CKPT_DIR in the header comment) and resumes a divergent prompt from the
 * deepest valid photo instead of prefilling again.  This call takes such a photo of pool
 * entries into host memory, restores one into any pool entries, or copies entries
 * inside the device (fork a sequence, compact a pool, keep a pre-verify snapshot).
 *
 *   n                      entries to copy, >= 0 (0: nothing queued)
 *   src_state, src_conv    [src_entries, H, D, D] and [src_entries, 3*H*D, 3] fp32
 *   src_entries            entries in the source buffers
 *   src_slots              HOST int32 [n], each in [0, src_entries)
 *   dst_state, dst_conv    [dst_entries, H, D, D] and [dst_entries, 3*H*D, 3] fp32
 *   dst_entries, dst_slots the same for the destination
 *   stream                 hipStream_t or NULL
 * Each buffer is device memory or host memory; with pinned host memory (hipHostMalloc)
 * the copies are asynchronous on the stream, with pageable host memory the runtime may
 * complete them before returning.  A source and a destination buffer are either the same
 * buffer or do not overlap (KDA_ERR_OVERLAP otherwise); within one buffer the copies run
 * in slot-list order, and an entry copied onto itself is left as it is (the state and the
 * conv entry are each decided on their own).  Every slot is checked before anything is queued; a
 * KDA_ERR_LAUNCH (the runtime refused a copy) can leave the entries before the failing
 * one copied.
 * Alignment: the four buffer pointers 16-byte aligned.
 */
kda_status kda_state_copy(const kda_config *cfg, int32_t n,
                          const float *src_state, const float *src_conv, int32_t src_entries,
                          const int32_t *src_slots,
                          float *dst_state, float *dst_conv, int32_t dst_entries,
                          const int32_t *dst_slots, void *stream);

/* Test hook for the bounded wait of the chunked prefill's two-workgroup carry (the form
 * used for B*H <= 128 in the standard precision, whose two workgroups of a (sequence,
 * head) pair exchange each output row's RMS sums).  publish = 0 makes both workgroups
 * skip publishing their sums, so that every wait times out; max_polls > 0 bounds each
 * wait to that many polls (0: the library's bound, about a second).  A wave that times
 * out writes NaN for that chunk's outputs and every later chunk's of the call without
 * waiting again; states and conv windows are unaffected.  Process-wide, read when a
 * prefill call is made; for tests of that path only.  kda_test_split_carry(1, 0)
 * restores normal operation. */
void kda_test_split_carry(int32_t publish, int32_t max_polls);

/* Test hook for the chunked prefill whose carries run in the chunk workgroups' launch
 * (B*H <= 128, either precision; each carry reads a record once its ready word is set).
 * mode 0: the library's choice; 1: never that form; 2: that form wherever it can run
 * (B*H <= 128, 2*B*H <= compute units), chosen
 * before kda_prefill_workspace_bytes sizes the workspace, so query the size after
 * setting it.  publish = 0 makes the chunk workgroups skip the ready words, so that every
 * carry's wait times out; max_polls > 0 bounds each wait to that many polls (0: the
 * library's bound, a few seconds).  A wave that times out sets its columns of the state
 * to NaN, so every later output and those columns of the final state are NaN, and does
 * not wait again.  Process-wide, read when a prefill call or a workspace query is made;
 * for tests only.  kda_test_pipeline(0, 1, 0) restores normal operation. */
void kda_test_pipeline(int32_t mode, int32_t publish, int32_t max_polls);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_str(kda_status s);

/* KDA_ABI_VERSION of the built library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
