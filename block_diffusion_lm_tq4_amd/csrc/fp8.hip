// fp8 weight-cache variant of the linear layer (Nemotron-TheHobbit-30B-A3B
// model card, Help wanted: decode the weights once into a resident fp8 copy,
// about 63 GB for both towers, so that no forward pass decodes).
//
// Storage (MXFP8): OCP e4m3 codes, one power-of-two scale 2^e per 32
// consecutive k of a row, kept as the E8M0 byte e + 127; e is the smallest
// integer in [-127, 127] with the block's largest magnitude <= 448 * 2^e.
// Rows are padded to kp = k rounded up to a multiple of 128 (zero codes, zero
// scale bytes), so every 128-k step is whole and every row of scales is
// 4-byte aligned.  The cache holds the decoded weights W_hat (rotation undone); activations
// are quantized the same way per call, and the product runs on the
// block-scaled fp8 MFMA of gfx950 (v_mfma_scale_f32_16x16x128_f8f6f4), whose
// per-32 scales are exactly these blocks.
//
// Operand layout of that instruction with 8-bit data (measured on the
// device): lane l = i + 16 g holds 32 bytes of row i: bytes 0-15 are
// k = 16 g .. 16 g + 15 and bytes 16-31 are k = 64 + 16 g .. 64 + 16 g + 15
// of the 128-k step; the B operand is laid out the same way per column.  The
// scale operand of lane i + 16 b (its low byte) scales k = 32 b .. 32 b + 31
// of row i.  The accumulator layout is that of the 16x16 f16 MFMAs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq4_internal.h"

namespace tq4 {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------
// Encoding

// Nearest e4m3 code to v (|v| <= 448), ties to the even code, from fp64 with
// one rounding: |v| = mant * 2^E with mant in [1, 2) gives the 3-bit mantissa
// rint((mant - 1) * 8), exact in fp64; below 2^-6 the grid is 2^-9 apart.
__device__ inline uint32_t e4m3_from_f64(double v) {
  const uint32_t sign = __builtin_signbit(v) ? 0x80u : 0u;
  const double a = __builtin_fabs(v);
  if (a < 0x1p-6) return sign | static_cast<uint32_t>(__builtin_rint(a * 512.0));  // 8 = 2^-6
  int p;
  const double f = __builtin_frexp(a, &p);  // a = f * 2^p, f in [0.5, 1)
  int e = p - 1;
  double r = __builtin_rint((2.0 * f - 1.0) * 8.0);
  if (r == 8.0) {
    r = 0.0;
    ++e;
  }
  return sign | (static_cast<uint32_t>(e + 7) << 3) | static_cast<uint32_t>(r);
}

// The block exponent for a largest magnitude amax: 448 = 0.875 * 2^9, so with
// amax = f * 2^p (f in [0.5, 1)) it is p - 9, plus one when f > 0.875.
__device__ inline int block_exponent(double amax) {
  if (amax == 0.0) return -127;
  int p;
  const double f = __builtin_frexp(amax, &p);
  int e = p - 9 + (f > 0.875 ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ inline int block_exponent_f32(float amax) {
  if (amax == 0.f) return -127;
  int p;
  const float f = __builtin_frexpf(amax, &p);
  int e = p - 9 + (f > 0.875f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// One thread per 32-weight block: z_hat = S_h * c_q, w_hat = s * H32 z_hat
// * (1/sqrt 32) in fp64 (the butterfly's sums are exact while the two
// half-block scales are within 2^12 of each other), then the block exponent
// and the e4m3 codes of w_hat / 2^e.
// Thread t covers block t % kpb of row t / kpb (kpb = kp / 32 blocks per
// padded row); padding blocks are written as zeros.
__global__ __launch_bounds__(256) void fp8_cache_kernel(const uint8_t *__restrict__ packed,
                                                        int64_t n, int32_t kb, int32_t kpb,
                                                        uint32_t sign_bits, Codebook cb,
                                                        uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ scales) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n * kpb) return;
  const int64_t row = t / kpb;
  const int32_t col = static_cast<int32_t>(t % kpb);
  uint4 *dst = reinterpret_cast<uint4 *>(codes + t * 32);
  if (col >= kb) {
    dst[0] = make_uint4(0u, 0u, 0u, 0u);
    dst[1] = make_uint4(0u, 0u, 0u, 0u);
    scales[t] = 0;
    return;
  }
  const uint32_t *p = reinterpret_cast<const uint32_t *>(packed + (row * kb + col) * 20);
  uint32_t wd[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) wd[i] = p[i];
  const double s0 = static_cast<double>(__uint_as_float((wd[4] & 0xFFFFu) << 16));
  const double s1 = static_cast<double>(__uint_as_float(wd[4] & 0xFFFF0000u));
  double v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t byte = (wd[i / 8] >> (8 * ((i / 2) % 4))) & 0xFFu;
    const uint32_t q = (i % 2 == 0) ? (byte & 15u) : (byte >> 4);
    v[i] = (i < 16 ? s0 : s1) * static_cast<double>(cb.c[q]);
  }
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const double a = v[i], c = v[i + h];
        v[i] = a + c;
        v[i + h] = a - c;
      }
    }
  }
  const double rs32 = 0x1.6a09e667f3bcdp-3;  // 1/sqrt(32) rounded to fp64
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] *= rs32;
    if ((sign_bits >> i) & 1u) v[i] = -v[i];
    amax = __builtin_fmax(amax, __builtin_fabs(v[i]));
  }
  const int e = block_exponent(amax);
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      word |= e4m3_from_f64(__builtin_ldexp(v[4 * w + t], -e)) << (8 * t);
    out[w] = word;
  }
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[t] = static_cast<uint8_t>(e + 127);
}

// One thread per 32-element activation block: bf16 -> fp32 (exact) or fp32
// as is, block exponent, codes of x / 2^e (exact scaling, then one hardware
// rounding to nearest even).
template <typename In>
__device__ inline void load_block32(const In *src, float (&v)[32]);

template <>
__device__ inline void load_block32<uint16_t>(const uint16_t *src, float (&v)[32]) {
  const uint4 *q = reinterpret_cast<const uint4 *>(src);
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
}

template <>
__device__ inline void load_block32<float>(const float *src, float (&v)[32]) {
  const float4 *q = reinterpret_cast<const float4 *>(src);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 d = q[i];
    v[4 * i] = d.x;
    v[4 * i + 1] = d.y;
    v[4 * i + 2] = d.z;
    v[4 * i + 3] = d.w;
  }
}

template <typename In>
__global__ __launch_bounds__(256) void act_mxfp8_kernel(const In *__restrict__ x, int64_t m,
                                                        int32_t kb, int32_t kpb,
                                                        uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ scales) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= m * kpb) return;
  const int64_t row = t / kpb;
  const int32_t col = static_cast<int32_t>(t % kpb);
  uint4 *dst = reinterpret_cast<uint4 *>(codes + t * 32);
  if (col >= kb) {
    dst[0] = make_uint4(0u, 0u, 0u, 0u);
    dst[1] = make_uint4(0u, 0u, 0u, 0u);
    scales[t] = 0;
    return;
  }
  float v[32];
  load_block32<In>(x + (row * kb + col) * 32, v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  const int e = block_exponent_f32(amax);
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(v[4 * w], -e),
                                              __builtin_ldexpf(v[4 * w + 1], -e), 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(v[4 * w + 2], -e),
                                          __builtin_ldexpf(v[4 * w + 3], -e), word, true);
    out[w] = static_cast<uint32_t>(word);
  }
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[t] = static_cast<uint8_t>(e + 127);
}

// ---------------------------------------------------------------------------
// Products

struct F8Args {
  const uint8_t *xq;  // activation codes [m][kp]
  const uint8_t *xs;  // activation scales [m][kp/32]
  const uint8_t *wq;  // weight codes [n][kp]
  const uint8_t *ws;  // weight scales [n][kp/32]
  float *y;           // [m][n]
  int64_t m, n;
  int64_t kp;         // padded k, a multiple of 128
  int32_t kpb;        // kp / 32
  int32_t chunks;     // kp / 128
  int32_t tiles_m, tiles_n;
};

__device__ inline intx8 join(uint4 lo, uint4 hi) {
  intx8 r;
  r[0] = static_cast<int>(lo.x); r[1] = static_cast<int>(lo.y);
  r[2] = static_cast<int>(lo.z); r[3] = static_cast<int>(lo.w);
  r[4] = static_cast<int>(hi.x); r[5] = static_cast<int>(hi.y);
  r[6] = static_cast<int>(hi.z); r[7] = static_cast<int>(hi.w);
  return r;
}

// Small M (<= 16 * MT): one workgroup of four waves per 16 output columns;
// wave w takes the 128-k steps w, w + 4, ...; within a batch of CB steps every
// load is issued before the first product.  Partial sums meet in LDS and are
// added in wave order.
constexpr int kF8SkWaves = 4;

template <int MT>
constexpr int f8_batch() {
  return MT == 1 ? 6 : (MT == 2 ? 4 : 2);
}

template <int MT>
__global__ __launch_bounds__(64 * kF8SkWaves) void fp8_skinny_kernel(F8Args g) {
  constexpr int CB = f8_batch<MT>();
  __shared__ floatx4 red[kF8SkWaves][MT][64];
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t nl = n0 + r < g.n ? n0 + r : g.n - 1;  // rows past n read row n - 1
  const uint8_t *wrow = g.wq + nl * g.kp + 16 * grp;
  const uint8_t *wsrow = g.ws + nl * g.kpb + grp;
  const uint8_t *xrow[MT];
  const uint8_t *xsrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t ml = 16 * t + r < g.m ? 16 * t + r : g.m - 1;
    xrow[t] = g.xq + ml * g.kp + 16 * grp;
    xsrow[t] = g.xs + ml * g.kpb + grp;
  }
  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = wave; c0 < g.chunks; c0 += CB * kF8SkWaves) {
    uint4 b[CB][2];
    uint4 a[CB][MT][2];
    int sb[CB];
    int sa[CB][MT];
#pragma unroll
    for (int s = 0; s < CB; ++s) {
      // A step past the end reloads the last one with both scale bytes 0
      // (2^-127 each): its products, at most 448^2 * 128 * 2^-254, round to
      // zero in fp32, so it adds exactly nothing.  Every load and product
      // stays unconditional, so all loads of the batch are in flight at once.
      const int c_raw = c0 + s * kF8SkWaves;
      const bool live = c_raw < g.chunks;
      const int c = live ? c_raw : g.chunks - 1;
      const int64_t k0 = 128 * static_cast<int64_t>(c);
      b[s][0] = *reinterpret_cast<const uint4 *>(wrow + k0);
      b[s][1] = *reinterpret_cast<const uint4 *>(wrow + k0 + 64);
      const int wsc = wsrow[4 * c];
      sb[s] = live ? wsc : 0;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        a[s][t][0] = *reinterpret_cast<const uint4 *>(xrow[t] + k0);
        a[s][t][1] = *reinterpret_cast<const uint4 *>(xrow[t] + k0 + 64);
        const int xsc = xsrow[t][4 * c];
        sa[s][t] = live ? xsc : 0;
      }
    }
#pragma unroll
    for (int s = 0; s < CB; ++s) {
      const intx8 bv = join(b[s][0], b[s][1]);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            join(a[s][t][0], a[s][t][1]), bv, acc[t], 0, 0, 0, sa[s][t], 0, sb[s]);
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave < MT) {
    floatx4 s = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kF8SkWaves; ++w) s += red[w][wave][lane];
    const int64_t n = n0 + r;
    if (n < g.n) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = 16 * wave + 4 * grp + v;
        if (m < g.m) g.y[m * g.n + n] = s[v];
      }
    }
  }
}

// M <= 16, kp <= 3072: one workgroup of 8 waves per 32 output columns.  The
// 16 quantized activation rows (codes and scale words) go to LDS once, and
// wave w streams the weights of column tile w / 4 for the 128-k steps
// c = w % 4, w % 4 + 4, ... (at most six): every load -- coalesced 1 KB
// LDS-direct pieces of 8 rows x 128 bytes -- is issued before the first
// product, so the whole workgroup's share (about 100 KB) is in flight at
// once.  LDS rows of 128 bytes use the XOR swizzle of the large kernel; the
// four partial sums of a column tile are added in wave order.
constexpr int kF8BufferFlags = 0x00020000;
constexpr int kF8StWaves = 8;
constexpr int kF8StSteps = 6;                    // 128-k steps per wave at most
constexpr int kF8StMaxKp = 4 * kF8StSteps * 128;  // 3072
constexpr int kF8StX = 16 * kF8StMaxKp;           // activation codes, [step][row][128]
constexpr int kF8StXs = 16 * (kF8StMaxKp / 32);   // activation scale bytes, [row][kpb]
constexpr int kF8StW = kF8StSteps * 16 * 128;     // one wave's weight steps, [step][row][128]

__global__ __launch_bounds__(64 * kF8StWaves) void fp8_stream_kernel(F8Args g) {
  __shared__ __attribute__((aligned(16))) uint8_t xbuf[kF8StX];
  __shared__ __attribute__((aligned(16))) uint8_t xsbuf[kF8StXs];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf[kF8StWaves][kF8StW];
  // two 64-lane scale loads per wave: 512 bytes, of which steps 0..5 use 384
  __shared__ __attribute__((aligned(16))) uint8_t wsbuf[kF8StWaves][512];
  __shared__ floatx4 red[kF8StWaves][64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int kp = static_cast<int>(g.kp);
  const int kpb = g.kpb;
  const int chunks = g.chunks;
  const int ntile = wave / 4;
  const int ks = wave % 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 32 + 16 * ntile;

  // rows past m and past n read zeros through the buffer ranges
  const int64_t m_rows = g.m < 16 ? g.m : 16;
  const int64_t n_rows = g.n - n0 < 16 ? (g.n - n0 > 0 ? g.n - n0 : 0) : 16;
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.xq), static_cast<short>(0), static_cast<int>(m_rows * kp),
      kF8BufferFlags);
  const __amdgpu_buffer_rsrc_t xs_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.xs), static_cast<short>(0), static_cast<int>(m_rows * kpb),
      kF8BufferFlags);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.wq + n0 * g.kp), static_cast<short>(0),
      static_cast<int>(n_rows * kp), kF8BufferFlags);
  const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.ws + n0 * kpb), static_cast<short>(0),
      static_cast<int>(n_rows * kpb), kF8BufferFlags);
  // piece = 8 rows x 128 bytes of one step; key of row (8 h + l / 8) is
  // (l / 16) ^ 4 h for h = 0, 1
  const int key0 = (lane % 8) ^ (lane / 16);
  const uint32_t voff0 = static_cast<uint32_t>((lane / 8) * kp + 16 * key0);
  const uint32_t voff1 = static_cast<uint32_t>((lane / 8 + 8) * kp + 16 * (key0 ^ 4));

  // activations: 2 pieces per step, spread over the waves
  for (int piece = wave; piece < 2 * chunks; piece += kF8StWaves) {
    const int c = piece / 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (lds_void *)(xbuf + piece * 1024), 16,
                                             piece % 2 ? voff1 : voff0, 128 * c, 0, 0);
  }
  // activation scale bytes: 16 rows x kpb, 64 words per load
  for (int wd = 64 * wave; wd < 16 * kpb / 4; wd += 64 * kF8StWaves) {
    const int w = wd + lane;
    const int row = (4 * w) / kpb;
    const int col = (4 * w) % kpb;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xs_rsrc, (lds_void *)(xsbuf + 4 * wd), 4,
                                             static_cast<uint32_t>(row * kpb + col), 0, 0, 0);
  }
  // this wave's weight steps and their scale words (lane l: row l % 16 of
  // step ks + 4 (l / 16); two loads cover six steps)
  int nsteps = 0;
#pragma unroll
  for (int s = 0; s < kF8StSteps; ++s) {
    const int c = ks + 4 * s;
    if (c < chunks) {
      nsteps = s + 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void *)(wbuf[wave] + s * 2048), 16,
                                               voff0, 128 * c, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void *)(wbuf[wave] + s * 2048 + 1024),
                                               16, voff1, 128 * c, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (ks + 16 * t < chunks)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ws_rsrc, (lds_void *)(wsbuf[wave] + 256 * t), 4,
          static_cast<uint32_t>(r * kpb + 16 * grp), 4 * (ks + 16 * t), 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  const int key = (r >> 1) % 8;
  for (int s = 0; s < nsteps; ++s) {
    const int c = ks + 4 * s;
    const uint8_t *xr = xbuf + c * 2048 + r * 128;
    const uint8_t *wr = wbuf[wave] + s * 2048 + r * 128;
    const intx8 aq = join(*reinterpret_cast<const uint4 *>(xr + 16 * (grp ^ key)),
                          *reinterpret_cast<const uint4 *>(xr + 16 * ((4 + grp) ^ key)));
    const intx8 bq = join(*reinterpret_cast<const uint4 *>(wr + 16 * (grp ^ key)),
                          *reinterpret_cast<const uint4 *>(wr + 16 * ((4 + grp) ^ key)));
    const int sa = xsbuf[r * kpb + 4 * c + grp];
    const int sb = wsbuf[wave][256 * (s / 4) + 64 * (s % 4) + 4 * r + grp];
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq, bq, acc, 0, 0, 0, sa, 0, sb);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave % 4 == 0) {
    floatx4 sum = red[wave][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) sum += red[wave + w][lane];
    const int64_t n = n0 + r;
    if (n < g.n) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = 4 * grp + v;
        if (m < g.m) g.y[m * g.n + n] = sum[v];
      }
    }
  }
}

// Large M: 256 x 128 output tile per workgroup of 8 waves (4 along m, 2
// along n; each 64 x 64 as 4 x 4 tiles of 16 x 16), two waves per SIMD.  Per
// 128-k step the tile's activation rows (256 x 128 bytes), weight rows
// (128 x 128 bytes) and their scale words (4 bytes per row) go to LDS by
// LDS-direct buffer loads into three stages, two steps ahead.  Piece p of an
// operand's stage (1 KB) holds rows 8p .. 8p + 7: lane l fills row 8p + l / 8
// at 16-byte slot l % 8 with global piece slot ^ ((row / 2) % 8), so the 16
// rows of a fragment read hit distinct bank groups.
constexpr int kF8Waves = 8;
constexpr int kF8MSub = 4;
constexpr int kF8NSub = 4;
constexpr int kF8TM = 256;
constexpr int kF8TN = 128;
constexpr int kF8Row = 128;
constexpr int kF8ALoads = kF8TM * kF8Row / 1024 / kF8Waves;  // 4
constexpr int kF8WLoads = kF8TN * kF8Row / 1024 / kF8Waves;  // 2
constexpr int kF8Loads = kF8ALoads + kF8WLoads + 1;           // + one scale load
constexpr int kF8Stage = (kF8TM + kF8TN) * kF8Row + 512 * 4;  // data, then 512 scale words

__global__ __launch_bounds__(64 * kF8Waves) void fp8_gemm_kernel(F8Args g) {
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kF8Stage];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kF8Stage];
  __shared__ __attribute__((aligned(16))) uint8_t stage2[kF8Stage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int wm = wave / 2;
  const int wn = wave % 2;

  // XCD-banded tile order: consecutive workgroups go to different XCDs, so
  // each XCD keeps one band of activation rows in its L2
  int mt, nt;
  {
    const int id = static_cast<int>(blockIdx.x);
    if (g.tiles_m % 8 == 0) {
      const int band = g.tiles_m / 8;
      const int j = id / 8;
      mt = (id % 8) * band + j % band;
      nt = j / band;
    } else {
      mt = id / g.tiles_n;
      nt = id % g.tiles_n;
    }
  }
  const int64_t m_base = static_cast<int64_t>(mt) * kF8TM;
  const int64_t n_base = static_cast<int64_t>(nt) * kF8TN;
  const int64_t rows_valid = g.m - m_base;
  const int64_t cols_valid = g.n - n_base;
  const int kp = static_cast<int>(g.kp);
  const int kpb = g.kpb;

  // Each buffer's range ends at the matrix's last row, so a load of a row
  // past it reads zeros without touching memory (those rows are not stored).
  // Piece p holds rows 8p .. 8p + 7; its key (row / 2) % 8 is (lane / 16) ^
  // (4 * (p % 2)), so a lane needs one offset for even and one for odd
  // pieces; 8p rows and the step go in the scalar offset.
  const int64_t a_rows = rows_valid < kF8TM ? rows_valid : kF8TM;
  const int64_t w_rows = cols_valid < kF8TN ? cols_valid : kF8TN;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.xq + m_base * g.kp), static_cast<short>(0),
      static_cast<int>(a_rows * kp), kF8BufferFlags);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.wq + n_base * g.kp), static_cast<short>(0),
      static_cast<int>(w_rows * kp), kF8BufferFlags);
  const int key0 = (lane % 8) ^ (lane / 16);
  const uint32_t voff_even = static_cast<uint32_t>((lane / 8) * kp + 16 * key0);
  const uint32_t voff_odd = static_cast<uint32_t>((lane / 8) * kp + 16 * (key0 ^ 4));
  // scales: one 64-row load per wave; waves 0-3 take the 256 activation rows
  // (words 0-255 of the stage's scale area), waves 4-5 the 128 weight rows
  // (words 256-383), waves 6-7 repeat the weight rows into words 384-511,
  // which nothing reads, so that every wave waits on the same load count
  const bool s_act = wave < 4;
  const int s_row0 = s_act ? 64 * wave : 64 * (wave % 2);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(s_act ? g.xs + m_base * kpb : g.ws + n_base * kpb),
      static_cast<short>(0), static_cast<int>((s_act ? a_rows : w_rows) * kpb), kF8BufferFlags);
  const uint32_t soff = static_cast<uint32_t>(lane * kpb);
  const int sdst = (kF8TM + kF8TN) * kF8Row + 256 * wave;
  constexpr int kWBase = kF8TM * kF8Row;                 // weight rows after the activations
  constexpr int kSBase = (kF8TM + kF8TN) * kF8Row;       // scale words after the data

  const int chunks = g.chunks;
  auto issue = [&](int c, uint8_t *st) __attribute__((always_inline)) {
    const int cc = c < chunks ? c : chunks - 1;  // padding steps reload the last one
#pragma unroll
    for (int i = 0; i < kF8ALoads; ++i) {
      const int piece = kF8ALoads * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (lds_void *)(st + piece * 1024), 16, piece % 2 ? voff_odd : voff_even,
          8 * piece * kp + kF8Row * cc, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kF8WLoads; ++i) {
      const int piece = kF8WLoads * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_rsrc, (lds_void *)(st + kWBase + piece * 1024), 16, piece % 2 ? voff_odd : voff_even,
          8 * piece * kp + kF8Row * cc, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_void *)(st + sdst), 4, soff,
                                             s_row0 * kpb + 4 * cc, 0, 0);
  };

  floatx4 acc[kF8MSub][kF8NSub];
#pragma unroll
  for (int i = 0; i < kF8MSub; ++i)
#pragma unroll
    for (int j = 0; j < kF8NSub; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t *st) __attribute__((always_inline)) {
    intx8 bq[kF8NSub];
    int sb[kF8NSub];
#pragma unroll
    for (int j = 0; j < kF8NSub; ++j) {
      const int row = wn * (16 * kF8NSub) + 16 * j + r;
      const int key = (row >> 1) % 8;
      const uint8_t *base = st + kWBase + row * kF8Row;
      bq[j] = join(*reinterpret_cast<const uint4 *>(base + 16 * (grp ^ key)),
                   *reinterpret_cast<const uint4 *>(base + 16 * ((4 + grp) ^ key)));
      sb[j] = st[kSBase + 4 * (kF8TM + row) + grp];
    }
#pragma unroll
    for (int i = 0; i < kF8MSub; ++i) {
      const int row = wm * (16 * kF8MSub) + 16 * i + r;
      const int key = (row >> 1) % 8;
      const uint8_t *base = st + row * kF8Row;
      const intx8 aq = join(*reinterpret_cast<const uint4 *>(base + 16 * (grp ^ key)),
                            *reinterpret_cast<const uint4 *>(base + 16 * ((4 + grp) ^ key)));
      const int sa = st[kSBase + 4 * row + grp];
#pragma unroll
      for (int j = 0; j < kF8NSub; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq, bq[j], acc[i][j], 0, 0,
                                                                     0, sa, 0, sb[j]);
    }
  };

  // Step c: wait until only step c + 1's loads are outstanding (loads retire
  // in issue order), wait for this wave's LDS reads, barrier (step c is in LDS
  // for every wave, and every wave is done with step c - 1's stage), refill
  // that stage with step c + 2, multiply step c.  The step count is padded to
  // a multiple of three; padding steps reload the last step and are not
  // multiplied, which keeps every wait exact.
  constexpr int kWait = 0x0F70 | (kF8Loads & 15) | ((kF8Loads >> 4) << 14);
  auto step = [&](int c, const uint8_t *cur, uint8_t *far) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWait);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    issue(c + 2, far);
    if (c < chunks) compute(cur);
  };
  issue(0, stage0);
  issue(1, stage1);
  for (int c = 0; c < chunks; c += 3) {
    step(c, stage0, stage2);
    step(c + 1, stage1, stage0);
    step(c + 2, stage2, stage1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the padding steps' loads

  const bool full = rows_valid >= kF8TM && cols_valid >= kF8TN;
#pragma unroll
  for (int i = 0; i < kF8MSub; ++i)
#pragma unroll
    for (int j = 0; j < kF8NSub; ++j) {
      const int64_t n = n_base + wn * (16 * kF8NSub) + 16 * j + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m_base + wm * (16 * kF8MSub) + 16 * i + 4 * grp + v;
        if (full || (m < g.m && n < g.n)) g.y[m * g.n + n] = acc[i][j][v];
      }
    }
}

// Grouped MoE product over the fp8 expert caches.  One workgroup of 8 waves
// per (MoE tile, 256 output columns): the tile's activation rows (16 * MT of
// them, gathered through the bucket permutation for the up projection) and
// the expert's 256 weight rows stream through S LDS stages of one 128-k step
// each, S - 1 steps ahead, as in fp8_gemm_kernel (same XOR swizzle, same
// exact load-count waits).  Wave w owns output columns 32 w .. 32 w + 31 of
// the slab: two 16-column tiles against all MT row tiles.
//   up (MODE 0):   h = relu(acc)^2 in fp32, then MXFP8 of h per row and
//                  32-block -- a wave's 32 columns are exactly one block --
//                  stored as codes hq[row][np] and scale bytes hs[row][np/32]
//                  (np = hidden width padded to 128: the padding blocks have
//                  zero weights, so they come out as zero codes and scale 0).
//   down (MODE 1): out[row][n] = acc (fp32), rows in bucket order.
// Rows past the tile's end load the tile's first row (not stored); weight
// rows past n read zeros through the buffer range.
constexpr int kF8MoeWaves = 8;
constexpr int kF8MoeTN = 32 * kF8MoeWaves;  // 256 output columns per workgroup

struct F8MoeArgs {
  const uint8_t *aq;  // activation codes: up [t][kp] (gathered), down [pairs][kp]
  const uint8_t *as;  // their scale bytes [.][kpb]
  const uint8_t *wq;  // expert codes [E * n][kp]
  const uint8_t *ws;  // expert scale bytes [E * n][kpb]
  const int32_t *perm;
  const MoETile *tiles;
  const int32_t *n_tiles;
  float *out;         // down: [pairs][n]
  uint8_t *hq;        // up: [pairs][n_store]
  uint8_t *hs;        // up: [pairs][n_store / 32]
  int64_t n;          // weight rows per expert
  int64_t n_store;    // up: hidden width padded to 128; down: n
  int64_t a_rows;     // rows of aq
  int32_t kp, kpb, chunks, topk;
};

template <int MT>
constexpr int f8_moe_stages() {
  return MT == 1 ? 4 : 3;
}

template <int MT, int MODE>
__global__ __launch_bounds__(64 * kF8MoeWaves) void fp8_moe_kernel(F8MoeArgs g) {
  constexpr int TM = 16 * MT;
  constexpr int S = f8_moe_stages<MT>();
  constexpr int kA = TM * kF8Row;                 // activation rows of a stage
  constexpr int kB = kF8MoeTN * kF8Row;           // weight rows of a stage
  constexpr int kStage = kA + kB + 512 * 4;       // then 512 scale words
  constexpr int kSc = kA + kB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S * kStage];

  if (static_cast<int32_t>(blockIdx.y) >= *g.n_tiles) return;
  const MoETile tile = g.tiles[blockIdx.y];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int kp = g.kp;
  const int kpb = g.kpb;
  const int rows = tile.rows;
  const int64_t m_base = tile.row0;
  const int64_t n_base = static_cast<int64_t>(blockIdx.x) * kF8MoeTN;
  const int64_t w_valid = g.n - n_base < kF8MoeTN ? (g.n - n_base > 0 ? g.n - n_base : 0)
                                                  : kF8MoeTN;

  // source row of local activation row i (rows past the tile's end: row 0)
  auto src_row = [&](int i) __attribute__((always_inline)) -> int64_t {
    const int64_t local = i < rows ? i : 0;
    if constexpr (MODE == 0) return g.perm[m_base + local] / g.topk;
    return m_base + local;
  };

  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.aq), static_cast<short>(0), static_cast<int>(g.a_rows * kp),
      kF8BufferFlags);
  const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.as), static_cast<short>(0), static_cast<int>(g.a_rows * kpb),
      kF8BufferFlags);
  const int64_t w_row0 = static_cast<int64_t>(tile.expert) * g.n + n_base;
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.wq + w_row0 * kp), static_cast<short>(0),
      static_cast<int>(w_valid * kp), kF8BufferFlags);
  const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.ws + w_row0 * kpb), static_cast<short>(0),
      static_cast<int>(w_valid * kpb), kF8BufferFlags);

  // Activation loads.  MT == 1: 16 rows x 128 bytes = one dword per lane of
  // the workgroup; lane l of wave w fills LDS bytes 256 w + 4 l, i.e. row
  // 2 w + l / 32, stored slot (l % 32) / 4, dword l % 4, whose key
  // (row / 2) % 8 is w.  MT >= 4: 1 KB pieces of 8 rows, MT / 4 per wave;
  // lane l fills row 8 p + l / 8 at stored slot l % 8.
  constexpr int kAPieces = MT == 1 ? 1 : MT / 4;
  static_assert(kAPieces <= 2, "at most two activation pieces per wave");
  // (a bound that depends on MT here made the host pass drop launch stubs)
  uint32_t a_voff[2];
  if constexpr (MT == 1) {
    const int row = 2 * wave + lane / 32;
    a_voff[0] = static_cast<uint32_t>(src_row(row) * kp + 16 * (((lane % 32) / 4) ^ wave) +
                                      4 * (lane % 4));
  } else {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i) {
      const int piece = kAPieces * wave + i;
      const int row = 8 * piece + lane / 8;
      a_voff[i] = static_cast<uint32_t>(src_row(row) * kp + 16 * ((lane % 8) ^ ((row >> 1) % 8)));
    }
  }
  // Weight loads: wave w takes pieces 4 w .. 4 w + 3, i.e. exactly the rows of
  // its own 32 columns; the key of piece p is (l / 16) ^ 4 (p % 2).
  const int key0 = (lane % 8) ^ (lane / 16);
  const uint32_t w_voff_even = static_cast<uint32_t>((lane / 8) * kp + 16 * key0);
  const uint32_t w_voff_odd = static_cast<uint32_t>((lane / 8) * kp + 16 * (key0 ^ 4));
  // Scale words (4 bytes per row and step): waves 0-3 load weight rows
  // 64 w + l into words 64 w + l; waves 4-7 load activation rows
  // min(64 (w - 4) + l, TM - 1) into words 64 w + l, so activation row i sits
  // at word 256 + i and the clamped repeats land in words nothing reads.
  const bool s_w = wave < 4;
  uint32_t s_voff;
  if (s_w) {
    s_voff = static_cast<uint32_t>((64 * wave + lane) * kpb);
  } else {
    const int arow = 64 * (wave - 4) + lane < TM ? 64 * (wave - 4) + lane : TM - 1;
    s_voff = static_cast<uint32_t>(src_row(arow) * kpb);
  }

  const int chunks = g.chunks;
  auto issue = [&](int c, uint8_t *st) __attribute__((always_inline)) {
    const int cc = c < chunks ? c : chunks - 1;  // padding steps reload the last one
    if constexpr (MT == 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void *)(st + 256 * wave), 4,
                                               a_voff[0], kF8Row * cc, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < kAPieces; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (lds_void *)(st + (kAPieces * wave + i) * 1024), 16, a_voff[i],
            kF8Row * cc, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = 4 * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_rsrc, (lds_void *)(st + kA + piece * 1024), 16, i % 2 ? w_voff_odd : w_voff_even,
          8 * piece * kp + kF8Row * cc, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_w ? ws_rsrc : as_rsrc,
                                             (lds_void *)(st + kSc + 256 * wave), 4, s_voff,
                                             4 * cc, 0, 0);
  };

  floatx4 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t *st) __attribute__((always_inline)) {
    intx8 bq[2];
    int sb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 32 * wave + 16 * j + r;
      const int key = (row >> 1) % 8;
      const uint8_t *base = st + kA + row * kF8Row;
      bq[j] = join(*reinterpret_cast<const uint4 *>(base + 16 * (grp ^ key)),
                   *reinterpret_cast<const uint4 *>(base + 16 * ((4 + grp) ^ key)));
      sb[j] = st[kSc + 4 * row + grp];
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = 16 * i + r;
      const int key = (row >> 1) % 8;
      const uint8_t *base = st + row * kF8Row;
      const intx8 aq = join(*reinterpret_cast<const uint4 *>(base + 16 * (grp ^ key)),
                            *reinterpret_cast<const uint4 *>(base + 16 * ((4 + grp) ^ key)));
      const int sa = st[kSc + 4 * (256 + row) + grp];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq, bq[j], acc[i][j], 0, 0,
                                                                     0, sa, 0, sb[j]);
    }
  };

  // Step c: wait until only steps c + 1 .. c + S - 2 are outstanding, barrier
  // (step c is in LDS for every wave; every wave is done with step c - 1's
  // stage), refill that stage with step c + S - 1, multiply step c.
  constexpr int kLoads = kAPieces + 4 + 1;
  constexpr int kAhead = (S - 2) * kLoads;
  constexpr int kWait = 0x0F70 | (kAhead & 15) | ((kAhead >> 4) << 14);
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s, smem + s * kStage);
  for (int c = 0; c < chunks; c += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      __builtin_amdgcn_s_waitcnt(kWait);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      issue(c + s + S - 1, smem + ((s + S - 1) % S) * kStage);
      if (c + s < chunks) compute(smem + s * kStage);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the padding steps' loads

  const int64_t col0 = n_base + 32 * wave;
  if constexpr (MODE == 0) {
    const bool col_ok = col0 < g.n_store;
    const int64_t npb = g.n_store / 32;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float u0 = acc[i][0][v];
        const float u1 = acc[i][1][v];
        const float h0 = u0 > 0.f ? u0 * u0 : 0.f;
        const float h1 = u1 > 0.f ? u1 * u1 : 0.f;
        float amax = __builtin_fmaxf(h0, h1);
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, d));
        const int e = block_exponent_f32(amax);
        const int pair = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(h0, -e),
                                                         __builtin_ldexpf(h1, -e), 0, false);
        const int local = 16 * i + 4 * grp + v;
        if (col_ok && local < rows) {
          uint8_t *dst = g.hq + (m_base + local) * g.n_store + col0;
          dst[r] = static_cast<uint8_t>(pair & 0xFF);
          dst[16 + r] = static_cast<uint8_t>((pair >> 8) & 0xFF);
          if (r == 0) g.hs[(m_base + local) * npb + col0 / 32] = static_cast<uint8_t>(e + 127);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = col0 + 16 * j + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int local = 16 * i + 4 * grp + v;
          if (local < rows && n < g.n) g.out[(m_base + local) * g.n + n] = acc[i][j][v];
        }
      }
  }
}

}  // namespace

int64_t fp8_padded_k(int64_t k) { return (k + 127) / 128 * 128; }

hipError_t launch_fp8_cache(const uint8_t *packed, int64_t n, int64_t k, uint32_t sign_bits,
                            uint8_t *codes, uint8_t *scales, hipStream_t s) {
  const int32_t kpb = static_cast<int32_t>(fp8_padded_k(k) / 32);
  const int64_t threads = n * kpb;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_cache_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)),
                     dim3(256), 0, s, packed, n, static_cast<int32_t>(k / 32), kpb, sign_bits,
                     codebook(), codes, scales);
  return hipGetLastError();
}

hipError_t launch_act_mxfp8(const uint16_t *x, int64_t m, int64_t k, uint8_t *codes,
                            uint8_t *scales, hipStream_t s) {
  const int32_t kpb = static_cast<int32_t>(fp8_padded_k(k) / 32);
  const int64_t threads = m * kpb;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(act_mxfp8_kernel<uint16_t>, dim3(static_cast<unsigned>((threads + 255) / 256)),
                     dim3(256), 0, s, x, m, static_cast<int32_t>(k / 32), kpb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_act_mxfp8_f32(const float *x, int64_t m, int64_t k, uint8_t *codes,
                                uint8_t *scales, hipStream_t s) {
  const int32_t kpb = static_cast<int32_t>(fp8_padded_k(k) / 32);
  const int64_t threads = m * kpb;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(act_mxfp8_kernel<float>, dim3(static_cast<unsigned>((threads + 255) / 256)),
                     dim3(256), 0, s, x, m, static_cast<int32_t>(k / 32), kpb, codes, scales);
  return hipGetLastError();
}

bool fp8_shape_fits(int64_t m, int64_t k, int64_t n) {
  // 32-bit buffer offsets over one tile's 256 padded rows
  return m >= 1 && n >= 1 && k >= 32 && fp8_padded_k(k) * kF8TM < (int64_t{1} << 31);
}

hipError_t launch_linear_fp8(const uint8_t *xq, const uint8_t *xs, int64_t m, int64_t k,
                             const uint8_t *wq, const uint8_t *ws, int64_t n, float *y,
                             hipStream_t s) {
  if (!fp8_shape_fits(m, k, n)) return hipErrorInvalidValue;
  F8Args g{};
  g.xq = xq;
  g.xs = xs;
  g.wq = wq;
  g.ws = ws;
  g.y = y;
  g.m = m;
  g.n = n;
  g.kp = fp8_padded_k(k);
  g.kpb = static_cast<int32_t>(g.kp / 32);
  g.chunks = static_cast<int32_t>(g.kp / 128);
  if (m <= 16 && g.kp <= kF8StMaxKp) {
    hipLaunchKernelGGL(fp8_stream_kernel, dim3(static_cast<unsigned>((n + 31) / 32)),
                       dim3(64 * kF8StWaves), 0, s, g);
    return hipGetLastError();
  }
  if (m <= 64) {
    const dim3 grid(static_cast<unsigned>((n + 15) / 16));
    const dim3 block(64 * kF8SkWaves);
    switch ((m + 15) / 16) {
      case 1: hipLaunchKernelGGL(fp8_skinny_kernel<1>, grid, block, 0, s, g); break;
      case 2: hipLaunchKernelGGL(fp8_skinny_kernel<2>, grid, block, 0, s, g); break;
      case 3: hipLaunchKernelGGL(fp8_skinny_kernel<3>, grid, block, 0, s, g); break;
      default: hipLaunchKernelGGL(fp8_skinny_kernel<4>, grid, block, 0, s, g); break;
    }
    return hipGetLastError();
  }
  g.tiles_m = static_cast<int32_t>((m + kF8TM - 1) / kF8TM);
  g.tiles_n = static_cast<int32_t>((n + kF8TN - 1) / kF8TN);
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(g.tiles_m) * g.tiles_n));
  hipLaunchKernelGGL(fp8_gemm_kernel, grid, dim3(64 * kF8Waves), 0, s, g);
  return hipGetLastError();
}

int fp8_moe_tile_rows(int64_t pairs, int32_t n_experts) {
  // about one row per expert: 16-row tiles; otherwise 64 rows (measured
  // 3 % faster than 128-row tiles at 1024 tokens with uniform routing, equal
  // under Zipf routing, where 128-row tiles would stream a popular expert's
  // weights half as often)
  return pairs <= 16 * static_cast<int64_t>(n_experts) ? 16 : 64;
}

bool fp8_moe_shape_fits(int64_t a_rows, int64_t k, int64_t n) {
  const int64_t kp = fp8_padded_k(k);
  return a_rows * kp < (int64_t{1} << 31) && kF8MoeTN * kp < (int64_t{1} << 31) && n >= 1;
}

hipError_t launch_moe_fp8(int mode, int tile_rows, const uint8_t *aq, const uint8_t *as,
                          int64_t a_rows, int64_t k, const int32_t *perm, int32_t topk,
                          const uint8_t *wq, const uint8_t *ws, int64_t n, int64_t n_store,
                          const MoETile *tiles, const int32_t *n_tiles, int64_t max_tiles,
                          float *out, uint8_t *hq, uint8_t *hs, hipStream_t s) {
  if (!fp8_moe_shape_fits(a_rows, k, n) || max_tiles > 65535) return hipErrorInvalidValue;
  if (mode == 0 && n_store % 128 != 0) return hipErrorInvalidValue;
  if (max_tiles == 0) return hipSuccess;
  F8MoeArgs g{};
  g.aq = aq;
  g.as = as;
  g.wq = wq;
  g.ws = ws;
  g.perm = perm;
  g.tiles = tiles;
  g.n_tiles = n_tiles;
  g.out = out;
  g.hq = hq;
  g.hs = hs;
  g.n = n;
  g.n_store = n_store;
  g.a_rows = a_rows;
  g.kp = static_cast<int32_t>(fp8_padded_k(k));
  g.kpb = g.kp / 32;
  g.chunks = g.kp / 128;
  g.topk = topk;
  const dim3 grid(static_cast<unsigned>((n_store + kF8MoeTN - 1) / kF8MoeTN),
                  static_cast<unsigned>(max_tiles));
  const dim3 block(64 * kF8MoeWaves);
  if (mode == 0) {
    switch (tile_rows) {
      case 16: hipLaunchKernelGGL((fp8_moe_kernel<1, 0>), grid, block, 0, s, g); break;
      case 64: hipLaunchKernelGGL((fp8_moe_kernel<4, 0>), grid, block, 0, s, g); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (tile_rows) {
      case 16: hipLaunchKernelGGL((fp8_moe_kernel<1, 1>), grid, block, 0, s, g); break;
      case 64: hipLaunchKernelGGL((fp8_moe_kernel<4, 1>), grid, block, 0, s, g); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace tq4
