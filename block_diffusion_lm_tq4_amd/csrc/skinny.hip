// Decode-shaped TQ4_1S linear layer: up to 16 activation rows (one 16-token
// diffusion block, the shape every denoiser projection sees on each step;
// Nemotron-TheHobbit-30B-A3B model card, sections Running it and Performance
// & why it's slow) in a single kernel launch.
//
// The weight stream is the whole cost here, so the kernel is built around it:
//
//  1. Each lane issues the loads of all its 20-byte weight blocks at once
//     (they stay in registers), before anything else, so the whole weight
//     tile of the workgroup is in flight from HBM while the rest happens.
//  2. The activations are rotated in the meantime, straight into LDS:
//     xt_b = H32 diag(s) x_b / sqrt(32) is itself a product with a +-1 matrix,
//     so two v_mfma_f32_16x16x32_bf16 per 32-block compute it exactly from the
//     bf16 input (products by +-1 are exact, sums are fp32), and the fp32
//     result is scaled and rounded to fp16.
//  3. The decode + MFMA loop then reads activation fragments from LDS and
//     decodes weights from registers (see gemm.hip for the operand mapping).
//
// Workgroup = 8 waves over 32 weight rows.  Waves 0-3 hold the weights: wave
// w takes rows (w & 1) * 16 .. +15 and the K half (w >> 1).  Waves 4-7 build
// the codebook table and the rotated activations.  The split matters because
// a wave's vector-memory counter retires in issue order: a wave that waited
// for an activation load would also wait for every weight load it issued
// before it.  The two K halves are added through LDS in a fixed order, so
// results are deterministic and no workgroup ever waits on another one.
#include "tq4_internal.h"

namespace tq4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWG = 32;
constexpr size_t kSkinnyMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kLutBytes = 1024;
constexpr int kRedBytes = 2 * 64 * 16;  // two waves' accumulators

struct SkinnyArgs {
  const uint16_t *x;      // bf16 [m][k]
  const uint8_t *w;       // packed [n][k/32][20]
  float *y;               // [m][n]
  int64_t m, n, k;
  int32_t xt_stride;      // LDS row stride of the rotated activations, halves
  uint32_t sign_bits;
  Codebook cb;
};

__device__ inline uint32_t f16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(f)));
}

__device__ inline half8 dequant8(uint32_t codes, half2v scale, const uint32_t *lut) {
  const half2v p0 = __builtin_bit_cast(half2v, lut[codes & 0xFFu]) * scale;
  const half2v p1 = __builtin_bit_cast(half2v, lut[(codes >> 8) & 0xFFu]) * scale;
  const half2v p2 = __builtin_bit_cast(half2v, lut[(codes >> 16) & 0xFFu]) * scale;
  const half2v p3 = __builtin_bit_cast(half2v, lut[codes >> 24]) * scale;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ inline half2v scale_pair(uint32_t bf16_bits) {
  const _Float16 h = static_cast<_Float16>(__uint_as_float(bf16_bits << 16));
  half2v r;
  r[0] = h;
  r[1] = h;
  return r;
}

struct WRaw {
  uint32_t v[5];
};

template <int CH>
__global__ __launch_bounds__(512) void skinny_kernel(SkinnyArgs g) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t *lut = reinterpret_cast<uint32_t *>(smem);
  floatx4 *red = reinterpret_cast<floatx4 *>(smem + kLutBytes);
  _Float16 *xts = reinterpret_cast<_Float16 *>(smem + kLutBytes + kRedBytes);

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int64_t kb = g.k / 32;

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  WRaw wr[CH];
  uint32_t ok_mask = 0;  // bit i: chunk c0 + i holds a real block for this lane
  int c0 = 0, c1 = 0;
  int64_t n = 0;
  bool n_ok = false;
  const int rg = wave & 1;        // consumer: 16-row group
  const int kh = (wave >> 1) & 1; // consumer: K half

  if (wave < 4) {
    // consumers: put this lane's whole weight share in flight first.  The
    // loads are unconditional (a lane with no block here re-reads block 0 of
    // row 0 and later zeroes its scales), so the compiler can retire them one
    // chunk at a time instead of waiting for all of them before the first use.
    const int chunks = static_cast<int>((kb + 3) / 4);
    const int half = (chunks + 1) / 2;
    c0 = kh ? half : 0;
    c1 = kh ? chunks : half;
    n = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + rg * 16 + r;
    n_ok = n < g.n;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = c0 + i;
      const int64_t b = 4 * static_cast<int64_t>(c) + grp;
      const bool ok = c < c1 && b < kb && n_ok;
      ok_mask |= static_cast<uint32_t>(ok) << i;
      const uint32_t *p = reinterpret_cast<const uint32_t *>(g.w + (ok ? (n * kb + b) * 20 : 0));
#pragma unroll
      for (int q = 0; q < 5; ++q) wr[i].v[q] = p[q];
    }
  } else {
    // producers: codebook pair table, then the rotated activations in LDS.
    const int ptid = tid - 256;
    const int pw = wave - 4;
    lut[ptid] = f16_bits(g.cb.c[ptid & 15]) | (f16_bits(g.cb.c[ptid >> 4]) << 16);
    // MFMA rows are output elements j of the block, columns are activation
    // rows m:  C[j][m] = sum_k H[j][k] s_k x[m][k].  Lane (r, grp) supplies
    // H[j = r (+16)][8 grp + i] s_{8 grp + i} and x[m = r][8 grp + i]; it
    // receives C[4 grp + v][r] = xt[r][4 grp + v (+16)].
    bf16x8 h_lo, h_hi;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * grp + i;
      const bool neg = ((__builtin_popcount(r & k) & 1) != 0) ^ (((g.sign_bits >> k) & 1u) != 0);
      const uint16_t one = neg ? 0xBF80u : 0x3F80u;
      h_lo[i] = __builtin_bit_cast(__bf16, one);
      h_hi[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(k >= 16 ? one ^ 0x8000u : one));
    }
    const float rs32 = 0x1.6a09e6p-3f;
    const bool m_ok = r < g.m;
    const uint16_t *xrow = g.x + (m_ok ? r : 0) * g.k;
    _Float16 *xts_row = xts + r * g.xt_stride;
    for (int64_t b = pw; b < kb; b += 4) {
      uint4 xv = make_uint4(0u, 0u, 0u, 0u);
      if (m_ok) xv = *reinterpret_cast<const uint4 *>(xrow + b * 32 + 8 * grp);
      const bf16x8 xb = __builtin_bit_cast(bf16x8, xv);
      const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
      const floatx4 lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h_lo, xb, zero, 0, 0, 0);
      const floatx4 hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h_hi, xb, zero, 0, 0, 0);
      uint2 plo, phi;
      plo.x = f16_bits(lo[0] * rs32) | (f16_bits(lo[1] * rs32) << 16);
      plo.y = f16_bits(lo[2] * rs32) | (f16_bits(lo[3] * rs32) << 16);
      phi.x = f16_bits(hi[0] * rs32) | (f16_bits(hi[1] * rs32) << 16);
      phi.y = f16_bits(hi[2] * rs32) | (f16_bits(hi[3] * rs32) << 16);
      *reinterpret_cast<uint2 *>(xts_row + b * 32 + 4 * grp) = plo;
      *reinterpret_cast<uint2 *>(xts_row + b * 32 + 16 + 4 * grp) = phi;
    }
  }
  __syncthreads();

  if (wave < 4) {
    // decode + MFMA over this wave's K half, weights consumed as they land
    const _Float16 *xts_row = xts + r * g.xt_stride;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = c0 + i;
      if (c < c1) {
        // a lane without a block reads block 0's (finite) activations and a
        // zero scale, so it adds exact zeros
        const bool ok = (ok_mask >> i) & 1u;
        const uint32_t sw = ok ? wr[i].v[4] : 0u;
        const half2v s0 = scale_pair(sw & 0xFFFFu);
        const half2v s1 = scale_pair(sw >> 16);
        const int64_t b = 4 * static_cast<int64_t>(c) + grp;
        const _Float16 *arow = xts_row + (b < kb ? b : 0) * 32;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const half8 aq =
              __builtin_bit_cast(half8, *reinterpret_cast<const uint4 *>(arow + 8 * t));
          const half8 bq = dequant8(wr[i].v[t], t < 2 ? s0 : s1, lut);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bq, acc, 0, 0, 0);
        }
      }
    }
    if (kh == 1) red[rg * 64 + lane] = acc;
  }
  __syncthreads();

  // add the two K halves in a fixed order and store: lane holds C[4grp+v][r]
  if (wave < 2 && n_ok) {
    const floatx4 other = red[rg * 64 + lane];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 4 * grp + v;
      if (m < g.m) g.y[m * g.n + n] = acc[v] + other[v];
    }
  }
}

template <int CH>
hipError_t launch_ch(const SkinnyArgs &a, hipStream_t s) {
  const size_t lds = kLutBytes + kRedBytes + static_cast<size_t>(16) * a.xt_stride * 2;
  static bool attr_set = false;  // raising the limit is idempotent; races are harmless
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&skinny_kernel<CH>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(kSkinnyMaxLds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = static_cast<unsigned>((a.n + kRowsPerWG - 1) / kRowsPerWG);
  hipLaunchKernelGGL(skinny_kernel<CH>, dim3(grid), dim3(512), lds, s, a);
  return hipGetLastError();
}

}  // namespace

// LDS row stride (halves) of the rotated activations: the row length padded
// so that consecutive rows start 4 banks apart (16-lane 128-bit reads of 16
// different rows then touch 64 distinct banks).
int32_t skinny_xt_stride(int64_t k) {
  const int64_t dwords = ((k / 2 + 63) / 64) * 64 + 4;
  return static_cast<int32_t>(2 * dwords);
}

bool skinny_fits(int64_t m, int64_t k) {
  if (m < 1 || m > 16 || k < 32 || k > 4096) return false;
  const size_t lds = kLutBytes + kRedBytes + static_cast<size_t>(16) * skinny_xt_stride(k) * 2;
  return lds <= kSkinnyMaxLds;
}

hipError_t launch_skinny(const uint16_t *x, int64_t m, int64_t k, const uint8_t *packed,
                         int64_t n, uint32_t sign_bits, float *y, hipStream_t s) {
  SkinnyArgs a{};
  a.x = x;
  a.w = packed;
  a.y = y;
  a.m = m;
  a.n = n;
  a.k = k;
  a.xt_stride = skinny_xt_stride(k);
  a.sign_bits = sign_bits;
  a.cb = codebook();
  const int64_t chunks = (k / 32 + 3) / 4;
  const int64_t half = (chunks + 1) / 2;
  switch (half) {
    case 1: return launch_ch<1>(a, s);
    case 2: return launch_ch<2>(a, s);
    case 3: return launch_ch<3>(a, s);
    case 4: return launch_ch<4>(a, s);
    case 5: return launch_ch<5>(a, s);
    case 6: return launch_ch<6>(a, s);
    case 7: return launch_ch<7>(a, s);
    case 8: return launch_ch<8>(a, s);
    case 9: return launch_ch<9>(a, s);
    case 10: return launch_ch<10>(a, s);
    case 11: return launch_ch<11>(a, s);
    case 12: return launch_ch<12>(a, s);
    case 13: return launch_ch<13>(a, s);
    case 14: return launch_ch<14>(a, s);
    case 15: return launch_ch<15>(a, s);
    case 16: return launch_ch<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq4
