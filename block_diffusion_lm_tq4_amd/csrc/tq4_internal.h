// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq4 {

// The 16 stored levels (fp32, ascending); passed to kernels by value.
struct Codebook {
  float c[16];
};

// Lloyd-Max levels of N(0,1) rounded to fp32, computed once on the host.
const Codebook &codebook();

// fp16 operand range.  The products take 16-bit operands (fp16 keeps 11
// significant bits, which the error bar needs; its exponent spans only
// 2^-14 .. 65504), so the values entering them are shifted by exact powers
// of two and the shifts are undone on the fp32 results:
//  * weight operand: S * c * 2^kWeightShift.  Half-block scales S from about
//    2e-6 to 93.6 then give normal fp16 values (a bf16 scale is exact in fp16
//    there), instead of 5e-4 to 2.4e4 unshifted: weights down to an rms of
//    about 1e-6 keep full precision, and blocks whose rotated values stay
//    below 255 cannot overflow;
//  * MoE hidden rows: R relu(u)^2 * 2^-kHiddenShift, so that |u| up to about
//    430 fits (the square doubles the exponent range of u);
//  * the M <= 16 kernels rotate with +-2^-3 entries (exact in bf16) and fold
//    the 8 into the final 1/sqrt(32): a 32-block sum reaches fp16's limit
//    only at |sum of +-x| = 8 * 65504.
constexpr int kWeightShift = 8;
constexpr float kWeightScale = 256.0f;         // 2^kWeightShift
constexpr float kWeightUnscale = 0x1p-8f;      // 2^-kWeightShift
constexpr int kHiddenShift = 4;
// 1/sqrt(32) * 2^-kHiddenShift (fp32; the power of two is exact)
constexpr float kHiddenRotScale = 0x1.6a09e6p-7f;
// the down product's result: 2^(kHiddenShift - kWeightShift)
constexpr float kHiddenUnscale = 0x1p-4f;
// M <= 16 kernels: sum * 8 / sqrt(32) * 2^-kWeightShift = sum * fp32(sqrt 2) * 2^-8
constexpr float kSkinnyUnscale = 0x1.6a09e6p-8f;
// bf16 bits of +-2^-3, the entries of the M <= 16 kernels' rotation operand
constexpr uint16_t kRotEntryBF16 = 0x3E00u;

// Register decode of the codebook (no memory access): the 16 levels are
// symmetric, c_{15-j} = -c_j, so the fp16 bit patterns of the 8 positive
// levels c_8 .. c_15 fit in four 32-bit byte tables (low bytes of levels
// 0-3 and 4-7, high bytes of levels 0-3 and 4-7), and v_perm_b32 turns four
// 3-bit magnitude indices into four table bytes at once.  A code q >= 8 is
// +level q - 8; q < 8 is -level 7 - q, i.e. magnitude index q ^ 7 with the
// sign bit set.
struct PermTable {
  uint32_t lo03, lo47, hi03, hi47;
};

__device__ inline PermTable make_perm_table(const Codebook &cb) {
  uint32_t b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(cb.c[8 + j]));
  PermTable t;
  t.lo03 = (b[0] & 0xFFu) | (b[1] & 0xFFu) << 8 | (b[2] & 0xFFu) << 16 | (b[3] & 0xFFu) << 24;
  t.lo47 = (b[4] & 0xFFu) | (b[5] & 0xFFu) << 8 | (b[6] & 0xFFu) << 16 | (b[7] & 0xFFu) << 24;
  t.hi03 = (b[0] >> 8) | (b[1] >> 8) << 8 | (b[2] >> 8) << 16 | (b[3] >> 8) << 24;
  t.hi47 = (b[4] >> 8) | (b[5] >> 8) << 8 | (b[6] >> 8) << 16 | (b[7] >> 8) << 24;
  return t;
}

// The 8 fp16 levels of one code word (nibble i = code of element i), as four
// packed pairs in the order of elements (0,2), (4,6), (1,3), (5,7): each
// pair is the low and high byte of two table lookups, merged by one
// v_perm_b32.  Callers pair them with activations in that element order.
__device__ inline void decode8_perm(uint32_t w, const PermTable &t, uint32_t (&d)[4]) {
  const uint32_t neg = ~w & 0x88888888u;            // bit 3 of every code below 8
  const uint32_t j = w ^ (neg - (neg >> 3));        // magnitude index in bits 0-2
  const uint32_t ev = j & 0x07070707u;              // elements 0, 2, 4, 6
  const uint32_t od = (j >> 4) & 0x07070707u;       // elements 1, 3, 5, 7
  const uint32_t ev_lo = __builtin_amdgcn_perm(t.lo47, t.lo03, ev);
  const uint32_t ev_hi = __builtin_amdgcn_perm(t.hi47, t.hi03, ev) | ((neg << 4) & 0x80808080u);
  const uint32_t od_lo = __builtin_amdgcn_perm(t.lo47, t.lo03, od);
  const uint32_t od_hi = __builtin_amdgcn_perm(t.hi47, t.hi03, od) | (neg & 0x80808080u);
  d[0] = __builtin_amdgcn_perm(ev_hi, ev_lo, 0x05010400u);  // elements 0, 2
  d[1] = __builtin_amdgcn_perm(ev_hi, ev_lo, 0x07030602u);  // elements 4, 6
  d[2] = __builtin_amdgcn_perm(od_hi, od_lo, 0x05010400u);  // elements 1, 3
  d[3] = __builtin_amdgcn_perm(od_hi, od_lo, 0x07030602u);  // elements 5, 7
}

// The values of lanes l and l ^ 16 (lower, upper) for every lane, by one
// v_permlane16_swap of two copies of v; with 32 the same for lanes l and
// l ^ 32.  The copy is opaque to the compiler: given the same register for
// both operands it has been seen to treat the two results as one value.
__device__ inline void lane_pair16(uint32_t v, uint32_t &lower, uint32_t &upper) {
  uint32_t c;
  asm volatile("v_mov_b32 %0, %1" : "=v"(c) : "v"(v));
  auto p = __builtin_amdgcn_permlane16_swap(v, c, false, false);
  lower = p[0];
  upper = p[1];
}
__device__ inline void lane_pair32(uint32_t v, uint32_t &lower, uint32_t &upper) {
  uint32_t c;
  asm volatile("v_mov_b32 %0, %1" : "=v"(c) : "v"(v));
  auto p = __builtin_amdgcn_permlane32_swap(v, c, false, false);
  lower = p[0];
  upper = p[1];
}

// xt = H32 diag(s) x / sqrt(32) of one 32-element block: bf16 in (16-byte
// aligned), fp32 butterfly in natural (Sylvester) order, fp16 out.  The format
// rotates every weight block by this orthogonal matrix (Nemotron-TheHobbit-
// 30B-A3B model card, What "Config-I" means), so rotating the activations
// instead leaves the weight side of a product as lookups times scales.
__device__ inline void rotate_block_bf16(const uint16_t *x, uint32_t sign_bits, uint16_t *xt) {
  float v[32];
  const uint4 *q = reinterpret_cast<const uint4 *>(x);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 d = q[i];
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if ((sign_bits >> i) & 1u) v[i] = -v[i];
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  const float rs32 = 0x1.6a09e6p-3f;  // 1/sqrt(32) rounded to fp32
  uint4 *dst = reinterpret_cast<uint4 *>(xt);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = static_cast<_Float16>(v[8 * i + 2 * j] * rs32);
      const _Float16 hi = static_cast<_Float16>(v[8 * i + 2 * j + 1] * rs32);
      w[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    dst[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The linear layer's additive tail: y[m, n] = acc + bias[n] + residual[m, n],
// either term optional, summed in fp32 in that order.  With bf16 set, the
// residual and the output are bf16 and the fp32 sum is rounded once, to
// nearest even.  The residual may be the output itself: every element is read
// and then written by one thread.
struct Tail {
  const float *bias;     // [n] fp32, or null
  const void *residual;  // [m, n], or null
  int32_t bf16;          // 0: residual and output fp32; 1: both bf16
};

template <bool kBF16>
__device__ inline float tail_residual_as(const void *residual, int64_t i) {
  if constexpr (kBF16)
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(residual)[i]) << 16);
  else
    return static_cast<const float *>(residual)[i];
}

template <bool kBF16>
__device__ inline void tail_store_as(float *out, int64_t i, float v) {
  if constexpr (kBF16)
    reinterpret_cast<uint16_t *>(out)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  else
    out[i] = v;
}

__device__ inline float tail_residual(const Tail &t, int64_t i) {
  return t.bf16 ? tail_residual_as<true>(t.residual, i) : tail_residual_as<false>(t.residual, i);
}

// acc plus the tail's terms for column n, given the residual value (ignored
// without a residual).  No contraction: the first add is never fused with the
// product's last multiply, so the result is the rounded product plus the
// tail, as separate adds.
__device__ inline float tail_sum(const Tail &t, float acc, int64_t n, float res) {
#pragma clang fp contract(off)
  if (t.bias != nullptr) acc += t.bias[n];
  if (t.residual != nullptr) acc += res;
  return acc;
}

// Stores one output element (fp32, or bf16 rounded to nearest even).
__device__ inline void tail_store(const Tail &t, float *out, int64_t i, float v) {
  if (t.bf16)
    tail_store_as<true>(out, i, v);
  else
    tail_store_as<false>(out, i, v);
}

// The whole tail of element (m, n) of an output with row stride ldn.
__device__ inline void tail_apply(const Tail &t, float *out, int64_t m, int64_t n, int64_t ldn,
                                  float acc) {
  const int64_t i = m * ldn + n;
  const float res = t.residual != nullptr ? tail_residual(t, i) : 0.f;
  tail_store(t, out, i, tail_sum(t, acc, n, res));
}

// ---- launchers (return hipSuccess or the launch error) --------------------
hipError_t launch_pack(const float *w, int64_t n_blocks, uint32_t sign_bits,
                       uint8_t *packed, int32_t *nonfinite, hipStream_t s);
hipError_t launch_pack_bf16(const uint16_t *w, int64_t n_blocks, uint32_t sign_bits,
                            uint8_t *packed, int32_t *nonfinite, hipStream_t s);

// Rotate [m, k] bf16 rows to fp16.
hipError_t launch_act_rht_bf16(const uint16_t *x, int64_t m, int64_t k, uint32_t sign_bits,
                               uint16_t *xt, hipStream_t s);

hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t s);

// y[i] = bias[i % n] + residual[i] over an [m, n] output (k == 0 products).
hipError_t launch_tail_only(const Tail &t, int64_t m, int64_t n, float *y, hipStream_t s);

// Dense product y[m, n] = xt[m, :] . Zhat[n, :]^T with xt already rotated.
struct DensePlan {
  int msub;       // 16-row MFMA tiles per wave along m
  int nsub;       // 16-row MFMA tiles per wave along n
  int waves_m;    // waves per workgroup along m
  int waves_n;    // waves per workgroup along n
  int ksplit;     // workgroups along k (partial sums reduced in fixed order)
  int64_t m_tiles, n_tiles, chunks;
  size_t partial_bytes;  // split-K partial sums (workspace, beyond xt)
};
DensePlan plan_dense(int64_t m, int64_t k, int64_t n);
hipError_t launch_dense(const DensePlan &p, const uint16_t *xt, int64_t m, int64_t k,
                        const uint8_t *packed, int64_t n, float *y, float *partial,
                        hipStream_t s, const Tail &tail = Tail{});

// Single-kernel path for m <= 16 (rotation fused, no workspace).
bool skinny_fits(int64_t m, int64_t k, int64_t n);
hipError_t launch_skinny(const uint16_t *x, int64_t m, int64_t k, const uint8_t *packed,
                         int64_t n, uint32_t sign_bits, float *y, hipStream_t s,
                         const Tail &tail = Tail{});

// Measurement variants of the M <= 16 streaming kernel (tq4_linear_variant):
// arith 0 the library's product, 1 the rotation undone on the weight tiles,
// 2 the products on the VALU.  Only for shapes skinny_dma_fits accepts.
bool skinny_dma_fits(int64_t m, int64_t k, int64_t n, const void *x, const void *packed);
hipError_t launch_skinny_variant(int arith, const uint16_t *x, int64_t m, int64_t k,
                                 const uint8_t *packed, int64_t n, uint32_t sign_bits, float *y,
                                 hipStream_t s);

// Weight-side measurement variant of the large-M product: xs = s .* x in
// fp16, then the 256 x 256 tile kernel rotating its decoded weights back.
hipError_t launch_act_sign_f16(const uint16_t *x, int64_t m, int64_t k, uint32_t sign_bits,
                               uint16_t *xs, hipStream_t s);
bool dense_huge_fits(int64_t m, int64_t k, int64_t n);
hipError_t launch_dense_weight_side(const uint16_t *xs, int64_t m, int64_t k,
                                    const uint8_t *packed, int64_t n, float *y, hipStream_t s);

// MoE pieces.
struct MoETile {  // one m-tile of one expert's segment in bucket order
  int32_t expert;
  int32_t row0;   // first row (bucket position) of the tile
  int32_t rows;   // rows in this tile (<= tile height)
  int32_t pad;
};
// Bucketing (one workgroup up to 8191 pairs, else three launches whose first
// counts chunks of pairs).  With x != nullptr the first launch also rotates
// the [t, k] bf16 activation rows into xt (extra workgroups, one thread per
// 32-block).  With logits != nullptr the bucketing workgroup first routes the
// pairs / topk tokens itself (the router's arithmetic, bit for bit), writing
// ids (then writable device memory) and gates.
hipError_t launch_route(const int32_t *ids, int64_t pairs, int32_t topk, int32_t n_experts,
                        int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                        MoETile *tiles, int32_t *n_tiles, int32_t tile_rows,
                        int32_t *status, hipStream_t s, const uint16_t *x = nullptr,
                        int64_t x_blocks = 0, uint32_t sign_bits = 0, uint16_t *xt = nullptr,
                        const float *logits = nullptr, float *gates = nullptr);

struct MoEPlan {
  int msub, nsub, waves_m, waves_n;
  int tile_rows;       // rows per MoE tile = 16 * msub * waves_m
  int64_t max_tiles;   // upper bound on tiles over all experts
};
MoEPlan plan_moe(int64_t pairs, int32_t n_experts);

// Grouped product over MoE tiles.  mode 0 (up): A rows gathered through
// perm[]/topk from xt [t, k]; output out16[row, n] = the rotation (sign_bits,
// per 32-block, fp16) of relu(acc)^2, n % 32 == 0.  mode 1 (down): A rows are
// the bucket rows of ht [pairs, k]; output out[row, n] = acc (fp32).
hipError_t launch_moe_gemm(const MoEPlan &p, int mode, const uint16_t *a, int64_t k,
                           const int32_t *perm, int32_t topk, const uint8_t *w_packed,
                           int64_t n, const MoETile *tiles, const int32_t *n_tiles,
                           float *out, uint16_t *out16, uint32_t sign_bits, hipStream_t s);

// fp8 weight cache (MXFP8: e4m3 codes, one E8M0 scale per 32 k), rows
// padded to fp8_padded_k(k) (a multiple of 128) with zero codes and scales.
int64_t fp8_padded_k(int64_t k);
hipError_t launch_fp8_cache(const uint8_t *packed, int64_t n, int64_t k, uint32_t sign_bits,
                            uint8_t *codes, uint8_t *scales, hipStream_t s);
hipError_t launch_act_mxfp8(const uint16_t *x, int64_t m, int64_t k, uint8_t *codes,
                            uint8_t *scales, hipStream_t s);
bool fp8_shape_fits(int64_t m, int64_t k, int64_t n);
// y = dequant(xq, xs) . dequant(wq, ws)^T, fp32.
hipError_t launch_linear_fp8(const uint8_t *xq, const uint8_t *xs, int64_t m, int64_t k,
                             const uint8_t *wq, const uint8_t *ws, int64_t n, float *y,
                             hipStream_t s);

hipError_t launch_act_mxfp8_f32(const float *x, int64_t m, int64_t k, uint8_t *codes,
                                uint8_t *scales, hipStream_t s);
// Grouped MoE products over fp8 expert caches (expert e's rows at e * n of
// the stacked [E * n, k] cache).  mode 0 (up): activation rows gathered as
// perm[row] / topk from aq [a_rows][kp]; writes MXFP8 codes and scale bytes of
// relu(acc)^2 into hq [pairs][n_store], hs [pairs][n_store / 32] (n_store =
// hidden width padded to 128).  mode 1 (down): activation rows are the bucket
// rows of aq; out[row][n] = acc (fp32).  tile_rows: 16 or 64 (as given to
// launch_route).
int fp8_moe_tile_rows(int64_t pairs, int32_t n_experts);
bool fp8_moe_shape_fits(int64_t a_rows, int64_t k, int64_t n);
hipError_t launch_moe_fp8(int mode, int tile_rows, const uint8_t *aq, const uint8_t *as,
                          int64_t a_rows, int64_t k, const int32_t *perm, int32_t topk,
                          const uint8_t *wq, const uint8_t *ws, int64_t n, int64_t n_store,
                          const MoETile *tiles, const int32_t *n_tiles, int64_t max_tiles,
                          float *out, uint8_t *hq, uint8_t *hs, hipStream_t s);

// Streaming read of `bytes` (a multiple of 16) from a 16-byte aligned buffer.
hipError_t launch_read_probe(const void *src, int64_t bytes, float *sink, hipStream_t s);

// Router: per token, softmax over the n_experts logits, ids of the topk
// largest (ties to the lower id), gates = their probabilities.
hipError_t launch_router(const float *logits, int64_t t, int32_t n_experts, int32_t topk,
                         int32_t *ids, float *gates, hipStream_t s);

hipError_t launch_combine(const float *o, const int32_t *inv, const float *topk_w,
                          int64_t t, int32_t topk, int64_t k, float *out, hipStream_t s);

}  // namespace tq4
