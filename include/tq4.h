/*
 * tq4.h -- C ABI of the TQ4_1S ("Config-I") dequantize-and-multiply library
 * for AMD Instinct MI355X (gfx950).
 *
 * Format (Nemotron-TheHobbit-30B-A3B model card, section What "Config-I"
 * means: a Walsh-Hadamard rotation per 32-weight block, a 16-level Lloyd-Max
 * codebook, two half-block scales, about 5 bits per weight).  The details the
 * card leaves open are fixed here as follows:
 *   - a block is 32 consecutive input features (k) of one output row n;
 *   - z = H32 (s .* w) / sqrt(32): s_i = -1 where bit i of sign_bits is set,
 *     H32 is the Sylvester-ordered Hadamard matrix H[i][j] = (-1)^popcount(i&j);
 *     one sign vector serves every block of every tensor;
 *   - codebook c_0 < ... < c_15: the 16-level Lloyd-Max quantizer of N(0,1),
 *     stored as fp32 (tq4_codebook);
 *   - per half-block h (z elements 0-15, 16-31): S_h = bf16(fp32(max|z| / c_15)),
 *     both roundings to nearest-even;
 *   - code q_j = #{k in 0..14 : z_j > S_h * (c_k + c_{k+1}) / 2}, evaluated in
 *     fp64 (a value exactly on a midpoint takes the lower code);
 *   - block bytes: 16 code bytes (byte i = q_{2i} | q_{2i+1} << 4), then the
 *     bf16 bit patterns of S_0 and S_1, little-endian: 20 bytes per block;
 *     a packed matrix is [n][k/32][20], row-major, contiguous.
 *
 * Conventions for every entry point below:
 *   - Pointers named as device pointers are device memory owned by the caller;
 *     the library never frees them.  Host pointers are named as such.
 *   - All GPU work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and nothing waits on the host: outputs are ready when the stream
 *     reaches that point.  The library never allocates device memory; the
 *     calls that need scratch space take a caller-provided workspace.
 *   - Argument errors are reported synchronously by the return value before
 *     any GPU work is enqueued.  A failed launch returns TQ4_E_DEVICE.
 *   - Outputs are overwritten, never accumulated into.
 *   - Two calls that share a workspace must not run concurrently.
 *
 * Numeric range of the TQ4_1S products (tq4_linear*, tq4_moe_*).  They
 * multiply 16-bit fp16 operands with fp32 accumulation; fp16 has 11
 * significant bits (the error bar below needs them) but an exponent range of
 * 2^-14 .. 65504 only, so every operand is shifted by an exact power of two
 * that the fp32 result undoes.  Inside this domain each output meets
 * relative Frobenius error <= 2e-3 and max |error| <= 1e-2 * rms(y) against
 * the exact product of the decoded weights:
 *   - weights: every half-block scale S <= 93.6, i.e. every rotated block
 *     value |z| <= 255 (guaranteed when every |w| <= 45).  Scales below about
 *     2e-6 (weights of rms below about 3e-6) lose precision gradually to
 *     fp16 subnormals rather than failing;
 *   - activations: for every 32-block of a row, |sum_i +-x_i| < 370000 over
 *     every sign pattern (guaranteed when every |x| <= 11579).  Rows whose
 *     rotated values are all below about 6e-5 lose precision gradually;
 *   - MoE hidden rows: the up products u satisfy, per 32-block,
 *     |sum_i +-relu(u_i)^2| < 5.9e6 (guaranteed when every |u| <= 430);
 *     rows whose squares are all below about 1e-3 lose precision gradually.
 * Outside it an output may be less accurate or infinite; nothing is checked
 * on the device (no host synchronization).  The fp8 entry points use MXFP8
 * operands with their own per-block exponents and have no such limit.
 */
#ifndef TQ4_H
#define TQ4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ4_BLOCK 32        /* weights per block, along k                  */
#define TQ4_BLOCK_BYTES 20  /* 16 code bytes + two bf16 half-block scales  */
#define TQ4_LEVELS 16

typedef enum {
  TQ4_OK = 0,
  TQ4_E_NULL = 1,        /* a required pointer is NULL                          */
  TQ4_E_SHAPE = 2,       /* a size is out of range (k % 32 != 0, topk > E, ...) */
  TQ4_E_ALIGN = 3,       /* a pointer is not aligned as its argument requires   */
  TQ4_E_WORKSPACE = 4,   /* workspace NULL or smaller than the size query says  */
  TQ4_E_DEVICE = 5,      /* a HIP call or kernel launch failed                  */
  TQ4_E_TOO_LARGE = 6    /* sizes need more than the static scratch holds       */
} tq4_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *tq4_status_string(int status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int tq4_version(void);

/* Host-only (no GPU call): writes the 16 stored codebook levels, ascending, to
 * the host array out[16].  The levels are the 16-level Lloyd-Max quantizer of
 * N(0,1) (model card, What "Config-I" means: "16-level Lloyd-Max") rounded to
 * fp32.  Returns TQ4_E_NULL if out is NULL. */
int tq4_codebook(float *out);

/* Bytes of a packed [n, k] matrix: n * (k/32) * 20; 0 if n < 0, k < 0 or
 * k % 32 != 0. */
size_t tq4_packed_size(int64_t n, int64_t k);

/* Encode W (fp32, [n, k] row-major, device, 16-byte aligned) into `packed`
 * (device, [n][k/32][20], 4-byte aligned).  Model card, What "Config-I"
 * means (rotation, codebook, dual half-block scales); offline quantizer of
 * section Reproduction.  All arithmetic is fp64, so the codes are exactly
 * those of the rule in the header comment.  `nonfinite_count` (device int32,
 * optional): increased by the number of blocks holding a NaN or infinity;
 * such blocks are still encoded by the same IEEE rule.
 * Errors: TQ4_E_NULL (w/packed NULL with n*k > 0), TQ4_E_SHAPE (n < 0, k < 0,
 * k % 32 != 0), TQ4_E_ALIGN, TQ4_E_DEVICE.  n == 0 or k == 0 is a no-op. */
int tq4_pack(const float *w, int64_t n, int64_t k, uint32_t sign_bits,
             uint8_t *packed, int32_t *nonfinite_count, void *stream);

/* tq4_pack for BF16 weights (the form the checkpoint ships in; model card,
 * Reproduction: quantizing both BF16 towers): w_bf16 is [n, k] bf16 bit
 * patterns, row-major, device, 16-byte aligned.  Every bf16 value is exact in
 * fp32, so the result is byte-identical to tq4_pack on the same values
 * widened to fp32.  Other arguments and errors as tq4_pack. */
int tq4_pack_bf16(const uint16_t *w_bf16, int64_t n, int64_t k, uint32_t sign_bits,
                  uint8_t *packed, int32_t *nonfinite_count, void *stream);

/* Rotate activations per 32-block: xt[m, :] = R x[m, :] with
 * R = H32 diag(s) / sqrt(32) on each block, fp32 arithmetic, result rounded to
 * fp16.  x: bf16 bit patterns [m, k] (device, 16-byte aligned); xt: fp16 bit
 * patterns [m, k] (device, 16-byte aligned).  Because R is orthogonal,
 * x . W_hat^T = (R x) . Z_hat^T blockwise, where Z_hat holds S_h * c_q: the
 * rotation moves from the weights to the activations.  Errors as tq4_pack. */
int tq4_act_rht(const uint16_t *x_bf16, int64_t m, int64_t k, uint32_t sign_bits,
                uint16_t *xt_f16, void *stream);

/* Workspace bytes that suffice for both tq4_linear and tq4_linear_rotated at
 * these sizes (0 if the sizes are invalid or the call is empty).  No initial
 * contents are required. */
size_t tq4_linear_workspace_size(int64_t m, int64_t k, int64_t n);

/* The on-the-fly dequantizing linear layer (model card, section Running it):
 * y[m, n] = sum_k x[m, k] * W_hat[n, k], W_hat the decoded packed weights,
 * without bias or activation.
 *   x_bf16  : [m, k] bf16 bit patterns, device, 16-byte aligned
 *   packed  : [n][k/32][20], device, 4-byte aligned (from tq4_pack)
 *   y       : [m, n] fp32, device, 4-byte aligned, overwritten
 *   workspace / workspace_bytes : device scratch of at least
 *             tq4_linear_workspace_size(m, k, n) bytes, 256-byte aligned
 *             (may be NULL when that size is 0, as for m <= 16)
 * The rotation is applied to the activations (R x, see tq4_act_rht) and the
 * product runs on 16-bit MFMA with fp32 accumulation; results are
 * deterministic.  For m <= 16 and k <= 4096 this is a single kernel.
 * Errors: TQ4_E_NULL, TQ4_E_SHAPE (negative sizes, k % 32 != 0),
 * TQ4_E_ALIGN, TQ4_E_WORKSPACE, TQ4_E_DEVICE.  m == 0 or n == 0 is a no-op;
 * k == 0 writes zeros. */
int tq4_linear(const uint16_t *x_bf16, int64_t m, int64_t k,
               const uint8_t *packed, int64_t n, uint32_t sign_bits, float *y,
               void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the library's static device scratch used by tq4_linear_noalloc
 * (32 MiB; each GPU the library runs on holds one copy until the process
 * ends). */
#define TQ4_NOALLOC_SCRATCH_BYTES (32u << 20)

/* tq4_linear for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * result equals tq4_linear's bit for bit; the scratch that tq4_linear takes
 * as its workspace is instead a device array inside the library (one per GPU,
 * TQ4_NOALLOC_SCRATCH_BYTES), so the call allocates and frees nothing.  The
 * array's device address is looked up on the first call on each device.
 *   arguments as tq4_linear, without the workspace
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (no call relies on them): calls that may overlap on one GPU (other
 * streams, other host threads) race and must be serialized by the caller.
 * Errors: as tq4_linear, plus TQ4_E_TOO_LARGE when
 * tq4_linear_workspace_size(m, k, n) exceeds TQ4_NOALLOC_SCRATCH_BYTES (for
 * example m * k above about 16.7 M rotated activations), and TQ4_E_DEVICE if
 * the array's address cannot be looked up. */
int tq4_linear_noalloc(const uint16_t *x_bf16, int64_t m, int64_t k,
                       const uint8_t *packed, int64_t n, uint32_t sign_bits, float *y,
                       void *stream);

/* The same product with the activations already rotated: y = xt . Z_hat^T,
 * where xt = tq4_act_rht(x) (fp16 bit patterns [m, k], device, 16-byte
 * aligned) and Z_hat[n, 32b + j] = S_h * c_q of the packed block (n, b).
 * One rotation can then serve several projections of the same activations
 * (model card, Running it: every quantized Linear of a layer reads the same
 * input).  Same workspace, errors and determinism as tq4_linear. */
int tq4_linear_rotated(const uint16_t *xt_f16, int64_t m, int64_t k,
                       const uint8_t *packed, int64_t n, float *y, void *workspace,
                       size_t workspace_bytes, void *stream);

/* tq4_linear with the layer's additive tail fused into the product's final
 * store: y[m, n] = sum_k x[m, k] * W_hat[n, k] + bias[n] + residual[m, n], in
 * fp32 (the product, then + bias, then + residual).  The quantized Linear
 * modules of the model card (section Running it) replace nn.Linear, whose
 * optional bias this is; the residual add is the sum every block of the
 * layer stack feeds into.
 *   bias     : [n] fp32, device, 4-byte aligned, or NULL (no bias)
 *   residual : [m, n] fp32, device, 4-byte aligned, or NULL (no residual);
 *              it may be y itself (each element is read before it is
 *              written, by the same thread), but must not otherwise overlap y
 * Everything else (arguments, workspace, errors, determinism) as tq4_linear,
 * plus TQ4_E_SHAPE for a residual that overlaps y without being y.  With both
 * NULL the result equals tq4_linear's bit for bit.  k == 0 writes bias +
 * residual. */
int tq4_linear_epilogue(const uint16_t *x_bf16, int64_t m, int64_t k,
                        const uint8_t *packed, int64_t n, uint32_t sign_bits,
                        const float *bias, const float *residual, float *y,
                        void *workspace, size_t workspace_bytes, void *stream);

/* tq4_linear_epilogue with a bf16 residual stream and bf16 output, the form
 * the next layer reads (the model runs in BF16; model card, Reproduction):
 * y_bf16[m, n] = bf16(product + bias[n] + residual[m, n]), the sum taken in
 * fp32 as in tq4_linear_epilogue and rounded once, to nearest even.  The
 * result is the bf16 rounding of tq4_linear_epilogue's fp32 result on the
 * same inputs (residual widened exactly), bit for bit.
 *   bias          : [n] fp32, device, 4-byte aligned, or NULL
 *   residual_bf16 : [m, n] bf16 bit patterns, device, 2-byte aligned, or
 *                   NULL; may be y_bf16 itself, must not otherwise overlap it
 *   y_bf16        : [m, n] bf16 bit patterns, device, 2-byte aligned
 * The rounding adds at most 2^-9 of |y| per element to the fp32 result's
 * error.  Workspace, errors and determinism as tq4_linear_epilogue; k == 0
 * writes bf16(bias + residual). */
int tq4_linear_epilogue_bf16(const uint16_t *x_bf16, int64_t m, int64_t k,
                             const uint8_t *packed, int64_t n, uint32_t sign_bits,
                             const float *bias, const uint16_t *residual_bf16,
                             uint16_t *y_bf16, void *workspace, size_t workspace_bytes,
                             void *stream);

/* ---- fp8 weight cache ----------------------------------------------------
 * The card's proposed alternative (model card, Help wanted): decode the
 * weights once into a resident fp8 copy, about 63 GB for both towers, so
 * that no forward pass decodes.  Encoding (MXFP8): OCP e4m3 codes (sign, 4
 * exponent bits with bias 7, 3 mantissa bits, subnormals, NaN only at 0x7F
 * and 0xFF, largest 448) with one power-of-two scale 2^e per 32 consecutive
 * k of a row -- the same 32-weight blocks -- stored as the E8M0 byte e + 127;
 * e is the smallest integer in [-127, 127] with max|block| <= 448 * 2^e
 * (e = -127 for an all-zero block), and an element v is stored as the e4m3
 * code nearest to v / 2^e, ties to the even code, sign kept.  Rows are
 * padded to kp = k rounded up to a multiple of 128 with zero codes and zero
 * scale bytes, which add nothing to a product.  A cache of an [n, k] matrix
 * is the codes [n][kp] followed by the scale bytes [n][kp/32]. */

/* Bytes of the fp8 cache of an [n, k] matrix: n * kp + n * kp / 32 (0 if the
 * sizes are invalid or empty). */
size_t tq4_fp8_cache_size(int64_t n, int64_t k);

/* Build the cache from a packed [n][k/32][20] matrix (device, 4-byte
 * aligned): the decoded weights W_hat (rotation undone, fp64 arithmetic)
 * encoded as above.  cache: device, 16-byte aligned, tq4_fp8_cache_size
 * bytes.  The codes are exactly those of the rule above whenever the two
 * half-block scales of each block are within a factor 2^12 of each other
 * (then every sum of the inverse rotation is exact in fp64).  A block whose
 * decoded values are not finite (a NaN or infinite scale) gets unspecified
 * codes.  Offline, like tq4_pack.  Errors: TQ4_E_NULL, TQ4_E_SHAPE (negative
 * sizes, k % 32 != 0, kp >= 2^23), TQ4_E_ALIGN, TQ4_E_DEVICE.  n == 0 or
 * k == 0 is a no-op. */
int tq4_fp8_cache(const uint8_t *packed, int64_t n, int64_t k, uint32_t sign_bits,
                  uint8_t *cache, void *stream);

/* Quantize bf16 activations [m, k] (device, 16-byte aligned) the same way:
 * codes [m][kp] (device, 16-byte aligned) and scale bytes [m][kp/32]
 * (device).  Non-finite inputs give unspecified codes.  Errors as
 * tq4_fp8_cache. */
int tq4_act_mxfp8(const uint16_t *x_bf16, int64_t m, int64_t k, uint8_t *codes,
                  uint8_t *scales, void *stream);

/* Workspace bytes for tq4_linear_fp8 (the quantized activations). */
size_t tq4_linear_fp8_workspace_size(int64_t m, int64_t k, int64_t n);

/* y[m, n] = sum_k xq[m, k] wq[n, k] with both operands dequantized from the
 * fp8 encoding: x is quantized per call (tq4_act_mxfp8, into the workspace),
 * the weights come from a cache built by tq4_fp8_cache; the product runs on
 * the block-scaled fp8 MFMA with fp32 accumulation, deterministic.  Against
 * the exact TQ4_1S product the fp8 rounding of both operands (at most 2^-4
 * relative each) dominates the error.
 *   x_bf16 : [m, k] bf16 bit patterns, device, 16-byte aligned
 *   cache  : from tq4_fp8_cache for this [n, k], device, 16-byte aligned
 *   y      : [m, n] fp32, device, 4-byte aligned, overwritten
 *   workspace : tq4_linear_fp8_workspace_size(m, k, n) bytes, 256-byte
 *               aligned
 * Errors: as tq4_linear.  k == 0 writes zeros. */
int tq4_linear_fp8(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *cache,
                   int64_t n, float *y, void *workspace, size_t workspace_bytes,
                   void *stream);

/* tq4_linear_fp8 with the activations already quantized by tq4_act_mxfp8
 * (x_codes [m][kp], device, 16-byte aligned; x_scales [m][kp/32], device,
 * 4-byte aligned), so one quantization can serve several projections of the
 * same input.  No workspace.  Errors as tq4_linear_fp8. */
int tq4_linear_fp8_quantized(const uint8_t *x_codes, const uint8_t *x_scales, int64_t m,
                             int64_t k, const uint8_t *cache, int64_t n, float *y,
                             void *stream);

/* Workspace bytes tq4_moe_grouped_fp8 needs (0 if the sizes are invalid). */
size_t tq4_moe_grouped_fp8_workspace_size(int64_t t, int32_t topk, int32_t n_experts,
                                          int64_t n1, int64_t k);

/* The MoE layer of tq4_moe_grouped on fp8 expert caches (model card, Help
 * wanted: the resident fp8 copy; Running it: the sync-free MoE):
 *   out[t, :] = sum_j topk_w[t, j] * dq(q(h_tj)) . dq(W2c_e)^T,
 *   h_tj = relu(dq(q(x[t, :])) . dq(W1c_e)^T)^2,  e = topk_ids[t, j],
 * where q is the MXFP8 quantization of tq4_act_mxfp8 (per row and 32-block)
 * and dq its value; ids outside [0, n_experts) contribute nothing.
 *   x_bf16   : [t, k] bf16 bit patterns, device, 16-byte aligned
 *   topk_ids : [t, topk] int32, device;  topk_w : [t, topk] fp32, device
 *   w1_cache : tq4_fp8_cache of the experts' up projections stacked as one
 *              [n_experts * n1, k] matrix (expert e = rows e*n1 ...), device,
 *              16-byte aligned, tq4_fp8_cache_size(n_experts * n1, k) bytes
 *   w2_cache : the same for the down projections, [n_experts * k, n1]
 *   out      : [t, k] fp32, device, 16-byte aligned, overwritten
 *   workspace: tq4_moe_grouped_fp8_workspace_size(...) bytes, device,
 *              256-byte aligned, no initial contents required
 * Steps: activation quantization, bucketing, grouped up projection whose
 * epilogue squares the positive part in fp32 and quantizes it per 32-block
 * (the quantization of tq4_act_mxfp8 on those fp32 values), grouped down
 * projection, and the per-token weighted sum in slot order.  Deterministic.
 * Errors: as tq4_moe_grouped, plus TQ4_E_SHAPE when t * kp, t * topk *
 * n1p or 256 * kp reach 2^31 (kp, n1p: k, n1 padded to 128). */
int tq4_moe_grouped_fp8(const uint16_t *x_bf16, int64_t t, int64_t k,
                        const int32_t *topk_ids, const float *topk_w, int32_t topk,
                        int32_t n_experts, const uint8_t *w1_cache, int64_t n1,
                        const uint8_t *w2_cache, float *out, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Stable bucketing of the t*topk (token, slot) pairs by expert, the routing
 * step of the sync-free MoE (model card, Running it; 128 experts, top-6 in
 * The model underneath).  Pair p = token * topk + slot.
 *   topk_ids : [t, topk] int32, device
 *   counts   : [n_experts] int32, device  -- pairs per expert
 *   offsets  : [n_experts + 1] int32, device -- exclusive prefix of counts
 *   perm     : [t * topk] int32, device  -- perm[offsets[e] + r] is the r-th
 *              pair (in increasing p) routed to e; entries past offsets[E]
 *              are left untouched
 *   inv      : [t * topk] int32, device  -- inv[perm[i]] = i; -1 for pairs
 *              whose id is outside [0, n_experts)
 * No host synchronization and no memory besides the outputs: one kernel up
 * to 8191 pairs; above, three (per-chunk counts, kept in inv until the last
 * launch overwrites them; one scan; per-chunk scatter).  Results are the
 * same either way.  Errors: TQ4_E_NULL, TQ4_E_SHAPE
 * (t < 0, topk < 1, n_experts < 1 or > 512), TQ4_E_DEVICE. */
int tq4_moe_route(const int32_t *topk_ids, int64_t t, int32_t topk, int32_t n_experts,
                  int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                  void *stream);

/* Workspace bytes tq4_moe_grouped needs (0 if the sizes are invalid). */
size_t tq4_moe_workspace_size(int64_t t, int32_t topk, int32_t n_experts,
                              int64_t n1, int64_t k);

/* The MoE layer on TQ4_1S experts, without host synchronization (model card,
 * Running it: "sync-free MoE"; The model underneath: 128 experts, top-6):
 *   out[t, :] = sum_j topk_w[t, j] * relu(x[t, :] . W1_e^T)^2 . W2_e^T,
 *   e = topk_ids[t, j]; ids outside [0, n_experts) contribute nothing.
 *   x_bf16    : [t, k] bf16 bit patterns, device, 16-byte aligned
 *   topk_ids  : [t, topk] int32, device;  topk_w : [t, topk] fp32, device
 *   w1_packed : [n_experts][n1][k/32][20] (up projections), device
 *   w2_packed : [n_experts][k][n1/32][20] (down projections), device
 *   out       : [t, k] fp32, device, overwritten
 *   workspace : at least tq4_moe_workspace_size(...) bytes, device,
 *               256-byte aligned; no initial contents required
 * Steps: bucketing (tq4_moe_route), activation rotation, grouped up
 * projection with relu^2, rotation of the hidden rows, grouped down
 * projection, and a per-token weighted sum over the top-k slots in slot
 * order (deterministic).  Errors: TQ4_E_NULL, TQ4_E_SHAPE (k or n1 not a
 * multiple of 32, topk > n_experts, ...), TQ4_E_ALIGN, TQ4_E_WORKSPACE,
 * TQ4_E_DEVICE.  t == 0 is a no-op. */
int tq4_moe_grouped(const uint16_t *x_bf16, int64_t t, int64_t k,
                    const int32_t *topk_ids, const float *topk_w, int32_t topk,
                    int32_t n_experts, const uint8_t *w1_packed, int64_t n1,
                    const uint8_t *w2_packed, uint32_t sign_bits, float *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* The router in front of the MoE layer (model card, The model underneath:
 * 128 experts, top-6), on the device so that a layer goes from router logits
 * to its output without the host:
 *   per token t: p = softmax(logits[t, :]) over all n_experts;
 *   topk_ids[t, :] = the topk experts with the largest logits, in decreasing
 *                    order, ties to the lower expert id;
 *   topk_w[t, j]   = p[topk_ids[t, j]] (not renormalized over the k).
 *   logits   : [t, n_experts] fp32, device, finite values
 *   topk_ids : [t, topk] int32, device, overwritten
 *   topk_w   : [t, topk] fp32, device, overwritten
 * Ids are decided on the fp32 logits exactly; gates are fp32 (expf).
 * Errors: TQ4_E_SHAPE (t < 0 or t > 2^33, n_experts outside 1..512, topk
 * outside 1..n_experts), TQ4_E_NULL, TQ4_E_ALIGN (4-byte), TQ4_E_DEVICE.
 * t == 0 is a no-op. */
int tq4_moe_router(const float *logits, int64_t t, int32_t n_experts, int32_t topk,
                   int32_t *topk_ids, float *topk_w, void *stream);

/* Workspace bytes tq4_moe_block needs (0 if the sizes are invalid). */
size_t tq4_moe_block_workspace_size(int64_t t, int32_t topk, int32_t n_experts,
                                    int64_t n1, int64_t k);

/* The whole MoE block of a denoiser step, from router logits to the layer's
 * output, on one stream and without the host (model card, Running it:
 * "sync-free MoE"; The model underneath: 128 experts, top-6):
 * tq4_moe_router into the workspace, then tq4_moe_grouped with those ids and
 * gates.  Graph-capturable like every call here.  Results equal those of
 * the two calls made separately, bit for bit.
 *   logits : [t, n_experts] fp32, device, 4-byte aligned, finite
 *   other arguments as tq4_moe_grouped; workspace of at least
 *   tq4_moe_block_workspace_size(...) bytes, 256-byte aligned.
 * Errors as tq4_moe_grouped. */
int tq4_moe_block(const uint16_t *x_bf16, int64_t t, int64_t k, const float *logits,
                  int32_t n_experts, int32_t topk, const uint8_t *w1_packed, int64_t n1,
                  const uint8_t *w2_packed, uint32_t sign_bits, float *out, void *workspace,
                  size_t workspace_bytes, void *stream);

/* Workspace bytes tq4_moe_block_persistent needs (0 if the sizes are
 * invalid or outside its range). */
size_t tq4_moe_block_persistent_workspace_size(int64_t t, int32_t topk, int32_t n_experts,
                                               int64_t n1, int64_t k);

/* tq4_moe_block as one persistent kernel (model card, Running it: sync-free
 * MoE; the help-wanted list asks for fused kernels): a small launch that
 * clears the grid barrier's counters, then one cooperative launch of as many
 * workgroups as the device holds at once, which runs the router, the
 * activation rotation, the bucketing, the up product with ReLU^2, the down
 * product and the weighted combine in that order, with a grid-wide barrier
 * between them.  Results equal tq4_moe_block's bit for bit.  Only for
 * layers whose tiles are 16 rows: t * topk <= 16 * n_experts (a denoiser
 * block of 16 tokens is 96 pairs).  Not graph-capturable (a cooperative
 * launch).  Arguments as tq4_moe_block; workspace of at least
 * tq4_moe_block_persistent_workspace_size(...) bytes, 256-byte aligned.
 * Errors as tq4_moe_block; TQ4_E_SHAPE also for t * topk > 16 * n_experts. */
int tq4_moe_block_persistent(const uint16_t *x_bf16, int64_t t, int64_t k, const float *logits,
                             int32_t n_experts, int32_t topk, const uint8_t *w1_packed,
                             int64_t n1, const uint8_t *w2_packed, uint32_t sign_bits,
                             float *out, void *workspace, size_t workspace_bytes, void *stream);

/* Measurement aid: the same layer computed with another placement of the
 * rotation or another arithmetic for the product, so that the library's
 * choice can be measured against the alternatives the format admits (model
 * card, What "Config-I" means: the rotation belongs to every weight block;
 * it may equally be applied to the activations, since it is orthogonal).
 *   TQ4_VARIANT_DEFAULT          tq4_linear itself
 *   TQ4_VARIANT_WEIGHT_ROTATION  the rotation undone on the decoded weight
 *       tiles by a butterfly across the wavefront (w = s .* H z / sqrt(32)),
 *       the activations entering the products unrotated (as s .* x, fp16);
 *       m <= 16 with k a multiple of 128 up to 2944 and 16-byte aligned x
 *       and packed, or the 256 x 256 tile shapes of large m (workspace of
 *       m * k * 2 bytes, 256-byte aligned)
 *   TQ4_VARIANT_VALU_PRODUCT     the activation rotation and the products on
 *       the vector ALU (fp16 pairs, fp32 sums) instead of MFMA; the m <= 16
 *       shapes above only
 * Arguments as tq4_linear; results meet the same error bar (the large-m
 * weight-side butterfly runs in fp16 and adds up to about 5e-4 relative
 * error).  Errors as tq4_linear, and TQ4_E_SHAPE for an unknown variant or
 * a shape the variant does not cover. */
#define TQ4_VARIANT_DEFAULT 0
#define TQ4_VARIANT_WEIGHT_ROTATION 1
#define TQ4_VARIANT_VALU_PRODUCT 2
int tq4_linear_variant(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *packed,
                       int64_t n, uint32_t sign_bits, float *y, void *workspace,
                       size_t workspace_bytes, int variant, void *stream);

/* Measurement aid, not a step of the method: reads `bytes` bytes of device
 * memory at `src` once (16 bytes per thread, one launch) and discards them.
 * Timing one call over the footprint of a packed matrix gives the read
 * ceiling that a single kernel streaming those bytes can reach.
 *   src  : device, 16-byte aligned; bytes a non-negative multiple of 16
 *   sink : device fp32[256]; never written for data the library produces
 * Errors: TQ4_E_NULL, TQ4_E_SHAPE (bytes < 0 or not a multiple of 16),
 * TQ4_E_ALIGN, TQ4_E_DEVICE.  bytes == 0 is a no-op. */
int tq4_read_probe(const void *src, int64_t bytes, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ4_H */
