/*
 * damp.h -- C ABI of libdamp.so: the per-token decode update of Gated DeltaNet (GDN) and Kimi
 * Delta Attention (KDA) recurrent states on AMD Instinct MI355X (gfx950), with the state held
 * in DAMP's mixed-precision layout, plus the FP32-state and uniform-INT8-state updates the
 * DAMP pages compare against.
 *
 * Sources (web pages):
 *  [C2]   "STEPQuant: When and Where Errors Matter in Delta-Rule Recurrent State Quantization"
 *         (thelatestinai.com listing), appendix Table C2, one persistent decode step. It takes
 *         the compressed state, q_t, k_t, v_t, the gate D_t, beta_t and a frozen precision map.
 *         Step 1 rebuilds S_hat (codes times scales; FP16 rows as stored); step 2 forms
 *         X = D_t S_hat + beta_t k_t (v_t^T - k_t^T D_t S_hat); step 3 takes the readout
 *         y_t = X^T q_t before any requantization; step 6 writes the new codes, scales and FP16
 *         rows, leaving the previous copy intact for readers that still use it.
 *  [DAMP] "DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization", abstract (arXiv v1
 *         on news.chathome.org; later version on mlsanity.com): high-risk key channels chosen
 *         offline are kept in FP16, the remaining key channels in INT8, under a fixed storage
 *         budget; states are otherwise FP32; the update is memory-bandwidth bound; the gate is
 *         a scalar per head (GDN) or one decay per key channel (KDA).
 *
 * Notation. A "unit" is one (slot, head) state S of d_k x d_v floats; row i is key channel i,
 * column j is value dimension j. D_t = alpha * I (GDN, one alpha per unit) or diag(alpha)
 * (KDA, alpha[d_k] per unit). The library neither normalises q or k nor scales q; callers do
 * that before the call. Supported sizes: d_k == d_v in {16, 32, 64, 128}; anything else
 * returns DAMP_ERR_UNSUPPORTED.
 *
 * INT8 rows (the pages only say "INT8"; this rule is the library's): symmetric, one fp32 scale
 * per row, scale = fl32(max_j |X_ij| / 127), code = round-half-to-even of fl32(X_ij / scale),
 * codes in [-127, 127]; a row whose scale is 0 (an all-zero row, or an absmax below
 * 127 * 2^-150, where the quotient rounds to zero) has codes 0. A subnormal scale (absmax below
 * 127 * 2^-126 ~ 1.5e-36) follows the same rule. damp_state_quantize and
 * uniform_int8_quantize follow this rule bit for bit. Inside the decode steps the code is the
 * round-half-to-even of X_ij * rcp(scale) (hardware reciprocal, 1 ulp), which can differ by one
 * from the rule where X_ij / scale lies within ~2e-5 of a half-integer (a few codes in 10^5).
 * FP16 rows: IEEE binary16, round to nearest even. Reconstruction: code * scale, or the
 * binary16 value.
 *
 * Execution model. Every call that takes a `stream` (a hipStream_t, e.g. torch's
 * torch.cuda.current_stream().cuda_stream; NULL = the default stream) only validates its
 * arguments on the host and enqueues work: it returns before the GPU has run. The return value
 * covers host-side validation and launch errors; a fault inside a kernel surfaces at the next
 * synchronisation of that stream (as a HIP error of the caller's runtime). States are updated
 * in place: within one call each listed slot must appear once (duplicates race; the result is
 * undefined), and only listed slots are read or written. A slot index outside [0, num_slots) is
 * skipped by the kernels: nothing of that request is read or written (its readout rows are left
 * as they were), so a bad index cannot send an access outside the pool. With the environment
 * variable DAMP_DEBUG=1 the calls copy slot_idx to the host first (synchronising the stream) and
 * return DAMP_ERR_SLOT_INDEX for an index outside [0, num_slots) or a repeated one.
 *
 * Pointers. "dev" pointers are device (HBM) addresses, "host" pointers host memory. The caller
 * owns every array it passes. No call keeps a pointer after it returns except damp_state_alloc,
 * whose handle keeps `pool` (which must outlive the handle). No exception crosses this ABI;
 * every non-OK status stores a message retrievable with damp_last_error().
 */
#ifndef DAMP_H
#define DAMP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum damp_status {
  DAMP_OK = 0,
  DAMP_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, misaligned pointer, bad enum */
  DAMP_ERR_UNSUPPORTED = -2,      /* a size the kernels are not built for */
  DAMP_ERR_OUT_OF_MEMORY = -3,    /* the library's small device allocation failed */
  DAMP_ERR_SLOT_INDEX = -4,       /* DAMP_DEBUG=1 only: slot index out of range or repeated, or
                                     an order that is not a permutation of the batch */
  DAMP_ERR_HIP = -5               /* a HIP runtime call or kernel launch failed */
} damp_status;

/* Gate form ([C2] step 2, "For KDA" remark; [DAMP]). */
typedef enum damp_decay {
  DAMP_DECAY_SCALAR = 0,  /* GDN: alpha is [B][H] */
  DAMP_DECAY_PER_KEY = 1  /* KDA: alpha is [B][H][d_k] */
} damp_decay;

/* Element type of q, k, v. beta, alpha and the readout are always fp32. */
typedef enum damp_dtype { DAMP_F32 = 0, DAMP_BF16 = 1 } damp_dtype;

/* Shape of a DAMP state pool: num_slots request slots x num_heads heads, each a d_k x d_v
 * state with num_fp16_rows FP16 key rows per head (the same rows for every slot: the frozen
 * precision map of [C2] / [DAMP]) and d_k - num_fp16_rows INT8 rows. */
typedef struct damp_layout {
  int32_t num_slots;
  int32_t num_heads;
  int32_t d_k;
  int32_t d_v;
  int32_t num_fp16_rows;
} damp_layout;

/* Opaque host handle: the layout, the per-head row map and the pool pointer. */
typedef struct damp_state damp_state;

/* ---------------------------------------------------------------------------------------
 * DAMP pool layout. The pool is an array of blocks, block (slot, head) at byte offset
 * (slot * num_heads + head) * damp_block_bytes(layout). With r = num_fp16_rows, D = d_k = d_v:
 *   [0, 2 r D)                        the r FP16 key rows, r x D binary16, ascending key index
 *   [2 r D, 2 r D + (D - r) D)        the D - r INT8 key rows, (D - r) x D int8, ascending key index
 *   [.., + 4 (D - r))                 the fp32 scales of the INT8 rows, same order
 *   zero padding up to a multiple of 256 bytes (never read or written by the kernels)
 * At D = 128, r = 24: 6,144 + 13,312 + 416 = 19,872 data bytes (9.70 bits per state value,
 * 69.7% below FP32), block stride 19,968 bytes.
 * ------------------------------------------------------------------------------------- */

/* Bytes of one block (the block stride), or 0 for an invalid or unsupported layout. */
size_t damp_block_bytes(const damp_layout* layout);

/* Data bytes of one block, without the padding (what a step reads and writes), or 0. */
size_t damp_block_data_bytes(const damp_layout* layout);

/* Device bytes a pool needs: num_slots * num_heads * damp_block_bytes, or 0 if invalid.
 * (Library infrastructure: no page defines it; the storage it counts is [DAMP]'s layout.) */
size_t damp_state_bytes(const damp_layout* layout);

/* Bind a caller-owned device pool to a layout and a frozen row map.
 *   fp16_rows  host int32 [num_heads][num_fp16_rows]: the FP16 key rows of each head, strictly
 *              ascending, each in [0, d_k). May be NULL when num_fp16_rows == 0.
 *   pool       dev, >= damp_state_bytes(layout) bytes (pool_bytes says how many), 256-byte
 *              aligned. Not initialised or touched by this call.
 *   out        receives the handle; *out is set to NULL on failure.
 * Allocates a small device copy of the row map (num_heads * d_k bytes) and copies it with a
 * synchronous hipMemcpy on the current device. Errors: INVALID_ARGUMENT (null pointer, bad
 * size, unsorted/duplicate/out-of-range row, pool too small or misaligned), UNSUPPORTED (d_k),
 * OUT_OF_MEMORY, HIP. */
damp_status damp_state_alloc(const damp_layout* layout, const int32_t* fp16_rows, void* pool,
                             size_t pool_bytes, damp_state** out);

/* Release the handle and its row-map copy (not the pool). NULL is accepted. Synchronises
 * nothing: the caller must not free while work that uses the handle is still queued.
 * (Library infrastructure: no page defines it.) */
damp_status damp_state_free(damp_state* state);

/* Layout of a handle (copied to *layout). */
damp_status damp_state_layout(const damp_state* state, damp_layout* layout);

/* Pack fp32 states into the pool ([C2] step 6 with the rule above):
 *   S        dev fp32 [n][num_heads][d_k][d_v], key rows in their original order
 *   slot_idx dev int32 [n]: block slot of S[i]; distinct, in [0, num_slots)
 * n == 0 is a no-op. Errors: INVALID_ARGUMENT, SLOT_INDEX (debug), HIP. */
damp_status damp_state_quantize(damp_state* state, const float* S, const int32_t* slot_idx,
                                int32_t n, void* stream);

/* Reconstruct fp32 states from the pool ([C2] step 1): S[i] = state of slot slot_idx[i],
 * code * scale (one fp32 rounding) for INT8 rows, the binary16 value for FP16 rows, in the
 * original key-row order. Does not modify the pool. */
damp_status damp_state_dequantize(const damp_state* state, float* S, const int32_t* slot_idx,
                                  int32_t n, void* stream);

/* One decode step of B requests on a DAMP pool, fused in one kernel ([C2] steps 1, 2, 3, 6):
 * for each b < B and head h, unit (slot_idx[b], h):
 *   reconstruct S_hat, S' = D_t S_hat, u = S'^T k, delta = beta (v - u),
 *   X = S' + k delta^T, out = X^T q (from X, before requantization), requantize X in place.
 *   slot_idx dev int32 [B], distinct, in [0, num_slots)
 *   q, k, v  dev [B][num_heads][d] of qkv_dtype (fp32 or bf16), contiguous
 *   alpha    dev fp32 [B][num_heads] (DAMP_DECAY_SCALAR) or [B][num_heads][d_k] (PER_KEY)
 *   beta     dev fp32 [B][num_heads]
 *   out      dev fp32 [B][num_heads][d_v], 16-byte aligned
 * B == 0 is a no-op. Errors: INVALID_ARGUMENT, SLOT_INDEX (debug), HIP. */
damp_status damp_decode_step(damp_state* state, const int32_t* slot_idx, int32_t B,
                             const void* q, const void* k, const void* v, damp_dtype qkv_dtype,
                             const float* alpha, damp_decay decay, const float* beta,
                             float* out, void* stream);

/* damp_decode_step with the pre-step fused into it: the arguments are what a GDN / KDA layer's
 * projections give, and the kernel forms the step's inputs while it stages them:
 *   q, k        unnormalised; the step uses q / ||q||_2 and k / ||k||_2 over the d_k entries of
 *               each (b, head) (a zero vector stays zero), the norms summed in fp32
 *   gate_logit  g, same shapes as alpha; the step uses alpha = exp(-softplus(g)) = 1 / (1 + e^g)
 *   beta_logit  b, [B][num_heads]; the step uses beta = 1 / (1 + e^-b)
 * Everything else as damp_decode_step. It saves the separate launches (and HBM round trips of
 * q, k and the gates) that would form these inputs before the step. The [C2] step takes unit
 * q_t, k_t and gates in (0, 1); how a layer makes them is the library's reading: L2
 * normalisation and the gate activations named here, no 1/sqrt(d) query scale. */
damp_status damp_decode_step_fused(damp_state* state, const int32_t* slot_idx, int32_t B,
                                   const void* q, const void* k, const void* v,
                                   damp_dtype qkv_dtype, const float* gate_logit,
                                   damp_decay decay, const float* beta_logit, float* out,
                                   void* stream);

/* ---------------------------------------------------------------------------------------
 * Processing order. The pages keep one state per concurrent request in a pool that grows with
 * the number of requests ([C2] abstract and Fig. 1a); which slots a batch holds is up to the
 * caller's scheduler, so they can lie anywhere in the pool. A step reads and writes each listed
 * block once in any order, but HBM delivers the blocks faster when those a launch has in flight
 * together lie close in the pool. damp_batch_order makes that order and the *_ordered steps
 * take the batch in it; the pages define no order, and no result depends on it.
 * ------------------------------------------------------------------------------------- */

/* order[0..B) = a permutation of [0, B) listing the batch positions by ascending slot bucket,
 * bucket = min(max(slot_idx[b], 0), num_slots - 1) >> shift, with the smallest shift that gives
 * at most 4,096 buckets (shift = 0, an exact sort, for pools of up to 4,096 slots). Positions in
 * one bucket come in no fixed order. Any slot_idx values give a permutation (repeated or
 * out-of-range entries included). One single-workgroup kernel on `stream`. A batch that keeps
 * its slots can reuse the order for every later step and layer.
 *   slot_idx dev int32 [B]
 *   order    dev int32 [B], written; caller-owned, must not overlap slot_idx
 * B == 0 is a no-op. Errors: INVALID_ARGUMENT (B < 0, num_slots <= 0, NULL or misaligned
 * pointers, overlap), HIP. */
damp_status damp_batch_order(const int32_t* slot_idx, int32_t B, int32_t num_slots, int32_t* order,
                             void* stream);

/* damp_decode_step with the batch positions taken in the order `order` lists them (the units of
 * order[0] first, then those of order[1], ...). For any permutation, the results are exactly
 * those of damp_decode_step, bit for bit. Uniform and per-head layouts.
 *   order dev int32 [B]: a permutation of [0, B), e.g. from damp_batch_order. The units of an
 *         entry outside [0, B) are skipped (no memory is touched for them). A repeated entry
 *         updates its units twice at once: undefined, like a repeated slot. With DAMP_DEBUG=1 a
 *         non-permutation returns DAMP_ERR_SLOT_INDEX.
 * Other arguments and errors as damp_decode_step (order NULL or misaligned: INVALID_ARGUMENT). */
damp_status damp_decode_step_ordered(damp_state* state, const int32_t* slot_idx, const int32_t* order,
                                     int32_t B, const void* q, const void* k, const void* v,
                                     damp_dtype qkv_dtype, const float* alpha, damp_decay decay,
                                     const float* beta, float* out, void* stream);

/* damp_decode_step_fused with the batch positions taken in the order `order` lists them, as
 * damp_decode_step_ordered does for damp_decode_step: bit-identical results for any permutation.
 * Arguments and errors as damp_decode_step_fused, plus `order` as in damp_decode_step_ordered. */
damp_status damp_decode_step_fused_ordered(damp_state* state, const int32_t* slot_idx,
                                           const int32_t* order, int32_t B, const void* q,
                                           const void* k, const void* v, damp_dtype qkv_dtype,
                                           const float* gate_logit, damp_decay decay,
                                           const float* beta_logit, float* out, void* stream);

/* Largest batch damp_decode_step_sorted takes: the entries of its library-held order buffer. */
#define DAMP_SORTED_MAX_B 65536

/* For callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. damp_batch_order followed by
 * damp_decode_step_ordered, with the order kept in a buffer the library holds instead of a
 * caller-owned one: a file-scope device array of DAMP_SORTED_MAX_B int32 (256 KiB) on each GPU
 * the library runs on, held until the process ends. The call allocates nothing, issues no memset
 * and enqueues the two kernels on `stream`; its results (readouts and pool) are those of
 * damp_decode_step, bit for bit. The first call on a device looks the buffer's address up once
 * (with that device current), on the device that runs `stream`.
 * Every call on one device shares that buffer, which keeps the last call's order: calls that
 * overlap on one device (on other streams, or from other threads) race and must be serialized
 * by the caller.
 * Errors: UNSUPPORTED for B > DAMP_SORTED_MAX_B (checked first, before any other argument); the
 * rest as damp_decode_step. */
damp_status damp_decode_step_sorted(damp_state* state, const int32_t* slot_idx, int32_t B,
                                    const void* q, const void* k, const void* v,
                                    damp_dtype qkv_dtype, const float* alpha, damp_decay decay,
                                    const float* beta, float* out, void* stream);

/* ---------------------------------------------------------------------------------------
 * Per-window requantization (the LeapQuant page, abstract: the low-bit state stays fixed for a
 * window of tokens, the window's updates are held in high precision, outputs are computed from
 * both, and the state is quantized once at the window's end). Within a window the state of a
 * unit is diag(a) S_hat + sum over the window's tokens of K_tau E_tau^T: S_hat the stored DAMP
 * state (not written until the window ends), a its cumulative row decay, K_tau the token's key
 * decayed by the later gates and E_tau its delta, held in a window buffer in fp32 (a key of the
 * DAMP_DECAY_SCALAR form that came from bf16 inputs is a bf16 value, and is held as bf16, which
 * is exact). Each unit has its
 * own window position, so the requests of one batch may be at different points of their windows.
 * ------------------------------------------------------------------------------------- */

/* Bytes of the window buffers of a whole pool (num_slots * num_heads units) for windows of
 * `window` tokens, 1 <= window <= 8; 0 if invalid. Per unit: round_up(4 (4 + d + 2 window d), 256).
 * The caller allocates them (256-byte aligned) and fills them with zero bytes once: a zero buffer
 * is a unit at the start of a window. A buffer whose token count lies outside [0, window) (not
 * zero-filled, or last used with another window length) is read as a unit at the start of a
 * window; no access leaves the unit's buffer whatever the buffer holds. */
size_t damp_window_bytes(const damp_layout* layout, int32_t window);

/* One token of a window for B requests, same arguments as damp_decode_step plus the window
 * buffers and the window length. For each unit: u and the readout come from the stored state and
 * the buffered tokens (the readout from X before any requantization, as in the step); the token
 * is appended to the buffer; if it is the window's window-th token, X is stored in the unit's
 * rule (FP16 rows RNE, INT8 rows absmax / 127) and the buffer emptied. Otherwise the pool is only
 * read. window = 1 is the per-token step (the same arithmetic as damp_decode_step up to fp32
 * rounding order). A given buffer must always be used with the same window length, and within
 * one window with the same decay mode: with DAMP_DECAY_SCALAR the buffer holds the decay as
 * scalars (one for the window, one per buffered key) and the keys as appended (bf16 or fp32, as
 * each call's inputs give them), with DAMP_DECAY_PER_KEY as row gains and decayed keys. A flag in the buffer, set by the window's
 * tokens and cleared when the window ends (or is flushed), tells a flush which form it holds.
 * Errors: INVALID_ARGUMENT, SLOT_INDEX (debug), HIP. */
damp_status damp_window_step(damp_state* state, void* window_buf, int32_t window,
                             const int32_t* slot_idx, int32_t B, const void* q, const void* k,
                             const void* v, damp_dtype qkv_dtype, const float* alpha,
                             damp_decay decay, const float* beta, float* out, void* stream);

/* damp_window_step with the batch positions taken in the order `order` lists them, as
 * damp_decode_step_ordered does for damp_decode_step: bit-identical results (readouts, pool and
 * window buffers) for any permutation. Arguments and errors as damp_window_step, plus `order` as
 * in damp_decode_step_ordered. */
damp_status damp_window_step_ordered(damp_state* state, void* window_buf, int32_t window,
                                     const int32_t* slot_idx, const int32_t* order, int32_t B,
                                     const void* q, const void* k, const void* v,
                                     damp_dtype qkv_dtype, const float* alpha, damp_decay decay,
                                     const float* beta, float* out, void* stream);

/* End the windows of n slots now: every listed unit with buffered tokens stores its state in the
 * unit's rule and empties its buffer (units with none are left as they are). Use before reading
 * the pool with damp_state_dequantize, or when a request ends. */
damp_status damp_window_flush(damp_state* state, void* window_buf, int32_t window,
                              const int32_t* slot_idx, int32_t n, void* stream);

/* The same step on an FP32 state pool: the format the states are commonly kept in and that the
 * DAMP storage and kernel speedups are measured against ([DAMP], both abstracts).
 *   pool dev fp32 [num_slots][num_heads][d_k][d_v], 16-byte aligned. Other arguments as in
 *   damp_decode_step. No requantization: X is stored as fp32. */
damp_status fp32_decode_step(float* pool, int32_t num_slots, int32_t num_heads, int32_t d_k,
                             int32_t d_v, const int32_t* slot_idx, int32_t B, const void* q,
                             const void* k, const void* v, damp_dtype qkv_dtype,
                             const float* alpha, damp_decay decay, const float* beta,
                             float* out, void* stream);

/* The same step on a uniform-INT8 state (every key row INT8 with its own fp32 scale): the
 * uniform quantization DAMP improves on, with no high-risk channels kept at higher precision
 * ([DAMP], both abstracts: uniform INT8 already costs reasoning accuracy).
 *   codes  dev int8 [num_slots][num_heads][d_k][d_v], 16-byte aligned
 *   scales dev fp32 [num_slots][num_heads][d_k], 16-byte aligned
 * Bit-identical to damp_decode_step with num_fp16_rows = 0 on the same values. */
damp_status uniform_int8_decode_step(int8_t* codes, float* scales, int32_t num_slots,
                                     int32_t num_heads, int32_t d_k, int32_t d_v,
                                     const int32_t* slot_idx, int32_t B, const void* q,
                                     const void* k, const void* v, damp_dtype qkv_dtype,
                                     const float* alpha, damp_decay decay, const float* beta,
                                     float* out, void* stream);

/* Pack fp32 states S[n][num_heads][d][d] into the uniform-INT8 arrays at slot_idx[n]. */
damp_status uniform_int8_quantize(int8_t* codes, float* scales, int32_t num_slots,
                                  int32_t num_heads, int32_t d_k, int32_t d_v, const float* S,
                                  const int32_t* slot_idx, int32_t n, void* stream);

/* ---------------------------------------------------------------------------------------
 * Per-head DAMP layout. The DAMP abstracts keep the high-risk key channels in FP16 under a
 * fixed total storage budget; spent where the calibration scores are highest (see
 * damp_allocate_rows), that budget gives each head its own FP16 row count r_h. Head h's block
 * has the block format above with r = r_h; within a slot the heads' blocks follow each other,
 * head h at byte offset off_h = sum over h' < h of round_up(data_bytes(r_h'), 256), and slot
 * s starts at s * slot_bytes, slot_bytes = sum over h of round_up(data_bytes(r_h), 256).
 * layout->num_fp16_rows is not used by these calls; damp_state_layout reports -1 for it.
 * Every other entry point accepts a per-head handle like a uniform one.
 * ------------------------------------------------------------------------------------- */

/* Device bytes a per-head pool needs (num_slots * slot_bytes), or 0 if the layout or an r_h
 * (host int32 [num_heads], each in [0, d_k]) is invalid. */
size_t damp_state_bytes_per_head(const damp_layout* layout, const int32_t* r_per_head);

/* Bind a caller-owned pool to a per-head layout.
 *   r_per_head host int32 [num_heads], each in [0, d_k]
 *   row_map    host int32 [num_heads][d_k]: row h lists head h's r_h FP16 key rows strictly
 *              ascending, then its other key rows strictly ascending (a permutation of
 *              0 .. d_k-1; the format damp_allocate_rows writes)
 *   pool       dev, >= damp_state_bytes_per_head bytes, 256-byte aligned, not touched
 * Allocates a small device table (num_heads * (d_k + 8) bytes), copied synchronously.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (d_k), OUT_OF_MEMORY, HIP. */
damp_status damp_state_alloc_per_head(const damp_layout* layout, const int32_t* r_per_head,
                                      const int32_t* row_map, void* pool, size_t pool_bytes,
                                      damp_state** out);

/* Per-head facts of any handle (uniform handles report r = num_fp16_rows for every head):
 *   r_out       host int32 [num_heads] or NULL: r_h
 *   offset_out  host int64 [num_heads] or NULL: off_h, the byte offset of head h's block in
 *               a slot
 *   slot_bytes  host int64 or NULL: the bytes of one slot (num_heads * block bytes when
 *               uniform) */
damp_status damp_state_head_info(const damp_state* state, int32_t* r_out, int64_t* offset_out,
                                 int64_t* slot_bytes);

/* ---------------------------------------------------------------------------------------
 * Offline calibration on the device: the DAMP abstracts choose the high-risk key channels
 * from quantization-error energy together with decay-based error retention, once, from
 * calibration data. The library reads the error energy of key row i of head h as the squared
 * error of storing that row with the INT8 rule above, and the retention as 1 / (1 - abar) for
 * a channel of mean gate abar (a gate that scales the state by abar per step keeps an error
 * for a geometric series of steps).
 * ------------------------------------------------------------------------------------- */

/* Risk scores from n calibration states:
 *   S          dev fp32 [n][num_heads][d][d], key rows in their original order
 *   abar       dev fp32 [num_heads][d]: mean gate of each key channel, in [0, 1) (GDN: the
 *              head's mean gate in every entry)
 *   row_error  dev fp64 [n][num_heads][d] (output, also a workspace): sum over j of
 *              (S[s][h][i][j] - scale * code_j)^2 for the INT8 rule's (code, scale) of that
 *              row, in binary64 with j ascending
 *   score      dev fp64 [num_heads][d] (output): (sum over s ascending of row_error[s][h][i])
 *              / n / (1 - abar[h][i]), each operation one binary64 rounding
 * Deterministic (no atomics). n >= 1. Errors: INVALID_ARGUMENT, UNSUPPORTED (d), HIP. */
damp_status damp_risk_scores(const float* S, int32_t n, int32_t num_heads, int32_t d,
                             const float* abar, double* row_error, double* score, void* stream);

/* FP16 rows, summed over the num_heads heads of one slot, that fit bits_per_value data bits
 * per state value (FP16 rows, INT8 rows and their fp32 scales; padding not counted): the
 * largest R, a multiple of g and at most num_heads * r_max, with
 * num_heads * (d^2 + 4 d) + (d - 4) * R <= bits_per_value * num_heads * d^2 / 8.
 * Returns -1 if not even R = 0 fits or an argument is invalid (d <= 4, g < 1, r_max outside
 * [0, d]). Host only. At d = 128 with 32 heads, 9.9 bits gives R = 872 (27.25 rows per head). */
int64_t damp_budget_rows(int32_t d, int32_t num_heads, double bits_per_value, int32_t g,
                         int32_t r_max);

/* Hand R FP16 rows (R % g == 0) to the heads in groups of g rows by score:
 *   score   dev fp64 [num_heads][d]
 *   r_out   dev int32 [num_heads] (output): r_h, a multiple of g, at most r_max
 *   map_out dev int32 [num_heads][d] (output): head h's r_h FP16 rows ascending, then its other
 *           rows ascending (the row_map of damp_state_alloc_per_head)
 * Per head the rows are ranked by score, larger first, ties to the lower row index; group j of
 * head h is ranks j*g .. j*g+g-1 and its gain the sum of their scores in rank order; groups
 * past r_max / g are never taken; the R / g largest gains are taken (ties to the lower head,
 * then the lower group), so each head keeps a prefix of its ranking and the total score kept in
 * FP16 is the largest any allocation of R rows in groups of g can keep. One workgroup of the
 * device does it. Limits: num_heads * d <= 8192 and num_heads * (r_max / g) <= 4096 groups
 * (else UNSUPPORTED). Errors: INVALID_ARGUMENT, UNSUPPORTED, HIP. */
damp_status damp_allocate_rows(const double* score, int32_t num_heads, int32_t d, int64_t R,
                               int32_t g, int32_t r_max, int32_t* r_out, int32_t* map_out,
                               void* stream);

/* ---------------------------------------------------------------------------------------
 * STEPQuant-style state ([C2] Table C2 steps 1-6; Table C1: for KDA the allocation unit is the
 * key row and the integer widths at a 6-bit budget are {4, 6, 8}; Table D3: FP16 scales and
 * pivots). Each key row of a head is a pivot kept in FP16 or an integer row of 8, 6 or 4 bits,
 * fixed per head by a frozen precision map; the integer rows carry one FP16 row factor each and
 * share one FP16 column-scale vector per (slot, head); entry (i, j) of an integer row is
 * code * rf_i * cs_j. Each step refits the scales to the new state X, for the integer rows N:
 *   cs_j = fp16( sqrt( sum_{i in N} w_i^2 X_ij^2 / sum_{i in N} w_i^2 ) )
 *   rf_i = fp16( max_{j: cs_j > 0} (|X_ij| / cs_j) / qmax_i ),   qmax = 2^(b - 1) - 1
 *   code = clamp(rint(X_ij / (rf_i cs_j)), -qmax, qmax), 0 where rf_i cs_j = 0
 * with w_i the frozen row-impact score (all w_i = 0 in a head means equal weights), the column
 * scales' sums, division and square root in binary64 rounded once to binary16, the other
 * divisions in binary32, binary16 round-to-nearest-even. The page names this fit (a dual-axis fit
 * aware of key rows, one column-scale vector per head weighted by squared row-impact scores) but
 * prints no formula: the formulas are the library's reading. stq_state_quantize takes every
 * decision as written (its sums add in another order than a sequential loop, which can only
 * matter within ~1e-15 of a binary16 tie). Inside stq_decode_step (d = 128) the column sums
 * u = S'^T k and p = S'^T q are exact integer sums on the matrix cores of the codes times the row
 * weights gate_i rf_i k_i (q_i), each split into four 7-bit pieces below a power of two (weights
 * kept to 2^-27 of the largest in their wave), recombined in binary32; X is formed in units of
 * the old column scale, Y_ij = X_ij / cs_j; each thread's partial sum of (w_i Y_ij)^2 over its 8
 * rows is binary32 and the column thread multiplies the binary64 total by cs_j^2, so a column
 * scale can differ from the binary64 fit of the same X only within a few binary32 ulps of a
 * binary16 tie; the row maximum and the codes use Y_ij RN(cs_j / cs'_j) and a rounded reciprocal
 * of the row factor, so a code can differ by one where its quotient lies within a few ulps of a
 * half-integer. At d = 64 X is formed directly and the same bounds hold.
 * Block of (slot, head): storage rows ordered pivots, 8-bit, 6-bit, 4-bit (each by ascending key
 * index): FP16 pivot rows (2 d bytes each) | 8-bit rows (d bytes) | 6-bit rows (3 d / 4 bytes: d / 2
 * bytes of low nibbles, then d / 4 bytes of the top two bits: column c at bits 4 (c mod 2) of byte
 * c / 2 and 2 (c mod 4) of byte c / 4) | 4-bit rows (d / 2 bytes, nibbles as in the 6-bit rows' low
 * plane) | FP16 row factors of the integer rows (storage order) | FP16 column scales (d) | zero
 * padding to 256 bytes. Each region after the pivots starts at the next multiple of 128 bytes,
 * and the 6- and 4-bit rows start at the group of 4 storage rows holding their first row (lead
 * rows of padding before it); padding is never read or written. Codes are two's complement. A
 * slot is its heads' blocks in order.
 * Supported: d_k = d_v = d in {64, 128}.
 * ------------------------------------------------------------------------------------- */
typedef struct stq_state stq_state;

/* Device bytes of a pool of num_slots slots for the precision map row_bits (host uint8
 * [num_heads][d], each 16 (pivot), 8, 6 or 4), or 0 if invalid. */
size_t stq_state_bytes(int32_t num_slots, int32_t num_heads, int32_t d, const uint8_t* row_bits);

/* Bind a caller-owned pool (256-byte aligned, >= stq_state_bytes) to a precision map and the
 * row-impact scores impact (host fp32 [num_heads][d], finite, >= 0). Allocates a device table of
 * num_heads * (5 d + 16) bytes, copied synchronously. Errors: INVALID_ARGUMENT, UNSUPPORTED (d),
 * OUT_OF_MEMORY, HIP. */
damp_status stq_state_alloc(int32_t num_slots, int32_t num_heads, int32_t d,
                            const uint8_t* row_bits, const float* impact, void* pool,
                            size_t pool_bytes, stq_state** out);

damp_status stq_state_free(stq_state* state);

/* Byte offset of each head's block inside a slot (host int64 [num_heads] or NULL) and the bytes
 * of a slot (or NULL). */
damp_status stq_state_head_info(const stq_state* state, int64_t* offset_out, int64_t* slot_bytes);

/* Pack fp32 states S[n][num_heads][d][d] (key rows in original order) with the fit above, into
 * the slots slot_idx[n]; and the reverse (code * rf * cs in binary32, FP16 pivots widened). */
damp_status stq_state_quantize(stq_state* state, const float* S, const int32_t* slot_idx,
                               int32_t n, void* stream);
damp_status stq_state_dequantize(const stq_state* state, float* S, const int32_t* slot_idx,
                                 int32_t n, void* stream);

/* One decode step on the STEPQuant-style state ([C2] Table C2 steps 1-6): reconstruct, decay,
 * update, readout y = X^T q before requantization, refit and pack. dst_pool: NULL writes the new
 * state in place; otherwise a second pool of the same layout receives it and the state bound to
 * the handle is only read (step 6: the previous copy stays intact while readers still use it;
 * the caller then binds the other pool or copies). Other arguments as in damp_decode_step.
 * At d = 128 the step holds the stored codes and forms X twice (environment variable
 * DAMP_STQ_STEP=x, read once per process, selects the kernel that holds X instead; both
 * satisfy the bounds above). */
damp_status stq_decode_step(stq_state* state, void* dst_pool, const int32_t* slot_idx, int32_t B,
                            const void* q, const void* k, const void* v, damp_dtype qkv_dtype,
                            const float* alpha, damp_decay decay, const float* beta, float* out,
                            void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). The string
 * is owned by the library and valid until the thread's next call. (Library infrastructure: no
 * page defines it.) */
const char* damp_last_error(void);

/* ABI version: (major << 16) | minor. (Library infrastructure: no page defines it.) */
int32_t damp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DAMP_H */
