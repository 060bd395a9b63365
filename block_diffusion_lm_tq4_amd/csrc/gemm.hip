// TQ4_1S dequantize-and-multiply on MFMA (gfx950).
//
// Nemotron-TheHobbit-30B-A3B model card, section Running it: every quantized
// Linear becomes a layer that decodes its 4-bit weights on each forward;
// section Performance & why it's slow names this per-forward decode as the
// cost to remove.  Here the decode happens in registers on the way into the
// matrix cores and never touches memory:
//
//   y[m, n] = sum_b sum_j xt[m, 32b + j] * S_{n,b,h(j)} * c[q_{n,b,j}]
//
// with xt = R x the rotated activations (see rht.hip) and S, q the block's
// scales and codes.  The weight operand of each v_mfma_f32_16x16x32_f16 is
// built from one 32-bit word of codes (8 nibbles): four byte-indexed lookups
// in an LDS table of fp16 level pairs, then one packed fp16 multiply by the
// half-block scale per pair.
//
// Mapping.  A wave owns MSUB x NSUB tiles of 16 x 16 outputs.  Lane l has
// r = l % 16 (row inside a tile) and g = l / 16 (k-group).  The MFMA sums over
// 32 k-slots, 8 per lane group; the k-slots may be assigned to the K axis in
// any order as long as both operands agree.  Per chunk of 4 blocks, lane
// group g owns block 4c+g and MFMA step t in 0..3 takes elements 8t..8t+7 of
// it: each lane then loads one whole 20-byte block per weight tile (codes
// word t for step t, scales word 4) and 64 contiguous bytes of xt per
// activation tile.
//
// Split-K.  When there are too few output tiles to fill the chip, the K axis
// is cut into `ksplit` ranges; each workgroup writes an fp32 partial tile and
// a second kernel adds the partials in split order (deterministic, and the
// kernel boundary is the only synchronization needed).
//
// MoE.  The same core runs over a device-built list of (expert, first row,
// rows) tiles.  Mode up gathers activation rows through the bucket
// permutation and stores relu(acc)^2; mode down reads the bucketed hidden
// rows and stores acc.  Tiles past the device-side count exit at once, so the
// grid is sized on the host from t*topk without a sync.
#include "tq4_internal.h"

namespace tq4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

enum Mode { kDense = 0, kMoEUp = 1, kMoEDown = 2 };

struct GemmArgs {
  const uint16_t *a;         // rotated activations (fp16 bits), row stride k
  const uint8_t *w;          // packed weights [n][k/32][20] (per expert for MoE)
  float *out;                // output rows, stride n
  float *partial;            // [ksplit][m][n] (dense split-K)
  const int32_t *perm;       // MoE: bucket position -> pair
  const MoETile *tiles;      // MoE tile list
  const int32_t *n_tiles;    // MoE tile count (device)
  int64_t m, n, k;
  int64_t expert_stride;     // bytes between experts' packed matrices
  int32_t topk;
  int32_t ksplit;
  int32_t chunks;            // ceil(k / 128)
  Codebook cb;
};

__device__ inline uint32_t f16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(f)));
}

// 8 dequantized weights (one codes word) times the half-block scale pair.
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
struct ARaw {
  uint4 v[4];
};

template <int MSUB, int NSUB, int WM, int WN, int MODE>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs g) {
  constexpr int WG_M = 16 * MSUB * WM;
  constexpr int WG_N = 16 * NSUB * WN;

  __shared__ uint32_t lut[256];

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int wave_m = wave / WN;
  const int wave_n = wave % WN;

  // ---- which tile -------------------------------------------------------
  int64_t m_base = 0;        // first output row of the workgroup tile
  int64_t rows_valid = g.m;  // rows of this tile that exist (relative to m_base)
  const uint8_t *wmat = g.w;
  int split = 0;
  if constexpr (MODE == kDense) {
    m_base = static_cast<int64_t>(blockIdx.y) * WG_M;
    rows_valid = g.m - m_base;
    split = blockIdx.z;
  } else {
    if (static_cast<int32_t>(blockIdx.y) >= *g.n_tiles) return;
    const MoETile t = g.tiles[blockIdx.y];
    m_base = t.row0;
    rows_valid = t.rows;
    wmat = g.w + static_cast<int64_t>(t.expert) * g.expert_stride;
  }
  const int64_t n_base = static_cast<int64_t>(blockIdx.x) * WG_N;

  // ---- codebook pair table ------------------------------------------------
  for (int i = tid; i < 256; i += 64 * WM * WN)
    lut[i] = f16_bits(g.cb.c[i & 15]) | (f16_bits(g.cb.c[i >> 4]) << 16);
  __syncthreads();

  const int64_t kb = g.k / 32;
  const int c_begin = static_cast<int>((static_cast<int64_t>(g.chunks) * split) / g.ksplit);
  const int c_end = static_cast<int>((static_cast<int64_t>(g.chunks) * (split + 1)) / g.ksplit);

  // activation row pointers and weight row pointers for this lane
  const uint16_t *arow[MSUB];
  bool a_ok[MSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i) {
    const int64_t local = wave_m * (16 * MSUB) + 16 * i + r;
    a_ok[i] = local < rows_valid;
    int64_t src_row = 0;
    if (a_ok[i]) {
      if constexpr (MODE == kDense) {
        src_row = m_base + local;
      } else if constexpr (MODE == kMoEUp) {
        src_row = g.perm[m_base + local] / g.topk;
      } else {
        src_row = m_base + local;
      }
    }
    arow[i] = g.a + src_row * g.k;
  }
  const uint8_t *wrow[NSUB];
  bool w_ok[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int64_t n = n_base + wave_n * (16 * NSUB) + 16 * j + r;
    w_ok[j] = n < g.n;
    wrow[j] = wmat + (w_ok[j] ? n : 0) * kb * 20;
  }

  floatx4 acc[MSUB][NSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto load_chunk = [&](int c, WRaw (&wr)[NSUB], ARaw (&ar)[MSUB]) {
    const int64_t b = 4 * static_cast<int64_t>(c) + grp;
    const bool b_ok = b < kb;
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      if (b_ok && w_ok[j]) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(wrow[j] + b * 20);
#pragma unroll
        for (int q = 0; q < 5; ++q) wr[j].v[q] = p[q];
      } else {
#pragma unroll
        for (int q = 0; q < 5; ++q) wr[j].v[q] = 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < MSUB; ++i) {
      if (b_ok && a_ok[i]) {
        const uint4 *p = reinterpret_cast<const uint4 *>(arow[i] + b * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) ar[i].v[q] = p[q];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) ar[i].v[q] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  auto compute_chunk = [&](const WRaw (&wr)[NSUB], const ARaw (&ar)[MSUB]) {
    half2v sc[NSUB][2];
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      sc[j][0] = scale_pair(wr[j].v[4] & 0xFFFFu);
      sc[j][1] = scale_pair(wr[j].v[4] >> 16);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      half8 bq[NSUB];
#pragma unroll
      for (int j = 0; j < NSUB; ++j) bq[j] = dequant8(wr[j].v[t], sc[j][t >> 1], lut);
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
        const half8 aq = __builtin_bit_cast(half8, ar[i].v[t]);
#pragma unroll
        for (int j = 0; j < NSUB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bq[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  if (c_begin < c_end) {
    WRaw wr_next[NSUB];
    ARaw ar_next[MSUB];
    load_chunk(c_begin, wr_next, ar_next);
    for (int c = c_begin; c < c_end; ++c) {
      WRaw wr[NSUB];
      ARaw ar[MSUB];
#pragma unroll
      for (int j = 0; j < NSUB; ++j) wr[j] = wr_next[j];
#pragma unroll
      for (int i = 0; i < MSUB; ++i) ar[i] = ar_next[i];
      if (c + 1 < c_end) load_chunk(c + 1, wr_next, ar_next);
      compute_chunk(wr, ar);
    }
  }

  // ---- epilogue: lane holds C[4*grp + v][r] of every 16x16 tile ----------
  if constexpr (MODE == kDense) {
    float *dst = g.ksplit > 1 ? g.partial + static_cast<int64_t>(split) * g.m * g.n : g.out;
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        const int64_t n = n_base + wave_n * (16 * NSUB) + 16 * j + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t m = m_base + wave_m * (16 * MSUB) + 16 * i + 4 * grp + v;
          if (m < g.m && n < g.n) dst[m * g.n + n] = acc[i][j][v];
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        const int64_t n = n_base + wave_n * (16 * NSUB) + 16 * j + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t local = wave_m * (16 * MSUB) + 16 * i + 4 * grp + v;
          if (local < rows_valid && n < g.n) {
            float val = acc[i][j][v];
            if constexpr (MODE == kMoEUp) {
              val = val > 0.f ? val * val : 0.f;
            }
            g.out[(m_base + local) * g.n + n] = val;
          }
        }
      }
  }
}

// y[i] = sum over splits of partial[s][i], in split order.
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float *__restrict__ partial,
                                                              int32_t ksplit, int64_t mn,
                                                              float *__restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= mn) return;
  float s = partial[i];
  for (int q = 1; q < ksplit; ++q) s += partial[q * mn + i];
  y[i] = s;
}

template <int MSUB, int NSUB, int WM, int WN, int MODE>
hipError_t launch_cfg(const GemmArgs &g, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<MSUB, NSUB, WM, WN, MODE>), grid, dim3(64 * WM * WN), 0, s, g);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(int msub, int nsub, int wm, int wn, const GemmArgs &g, dim3 grid,
                    hipStream_t s) {
  if (wm == 1 && wn == 4 && nsub == 2) {
    switch (msub) {
      case 1: return launch_cfg<1, 2, 1, 4, MODE>(g, grid, s);
      case 2: return launch_cfg<2, 2, 1, 4, MODE>(g, grid, s);
      case 3: return launch_cfg<3, 2, 1, 4, MODE>(g, grid, s);
      case 4: return launch_cfg<4, 2, 1, 4, MODE>(g, grid, s);
      default: break;
    }
  }
  if (wm == 2 && wn == 2 && msub == 4 && nsub == 4) return launch_cfg<4, 4, 2, 2, MODE>(g, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

DensePlan plan_dense(int64_t m, int64_t k, int64_t n) {
  DensePlan p{};
  p.chunks = (k / 32 + 3) / 4;
  if (m <= 64) {
    p.msub = static_cast<int>((m + 15) / 16);
    if (p.msub < 1) p.msub = 1;
    p.nsub = 2;
    p.waves_m = 1;
    p.waves_n = 4;
  } else {
    p.msub = 4;
    p.nsub = 4;
    p.waves_m = 2;
    p.waves_n = 2;
  }
  const int64_t wg_m = 16 * p.msub * p.waves_m;
  const int64_t wg_n = 16 * p.nsub * p.waves_n;
  p.m_tiles = (m + wg_m - 1) / wg_m;
  p.n_tiles = (n + wg_n - 1) / wg_n;
  const int64_t tiles = p.m_tiles * p.n_tiles;
  int64_t ks = 1;
  const int64_t target = 256;  // one workgroup per compute unit
  if (tiles < target && p.chunks > 1) {
    ks = (target + tiles - 1) / tiles;
    if (ks > p.chunks) ks = p.chunks;
    if (ks > 16) ks = 16;
  }
  p.ksplit = static_cast<int>(ks);
  p.partial_bytes = ks > 1 ? static_cast<size_t>(ks) * m * n * sizeof(float) : 0;
  return p;
}

hipError_t launch_dense(const DensePlan &p, const uint16_t *xt, int64_t m, int64_t k,
                        const uint8_t *packed, int64_t n, float *y, float *partial,
                        hipStream_t s) {
  GemmArgs g{};
  g.a = xt;
  g.w = packed;
  g.out = y;
  g.partial = partial;
  g.m = m;
  g.n = n;
  g.k = k;
  g.ksplit = p.ksplit;
  g.chunks = static_cast<int32_t>(p.chunks);
  g.cb = codebook();
  const dim3 grid(static_cast<unsigned>(p.n_tiles), static_cast<unsigned>(p.m_tiles),
                  static_cast<unsigned>(p.ksplit));
  hipError_t e = dispatch<kDense>(p.msub, p.nsub, p.waves_m, p.waves_n, g, grid, s);
  if (e != hipSuccess || p.ksplit == 1) return e;
  const int64_t mn = m * n;
  hipLaunchKernelGGL(reduce_partials_kernel, dim3(static_cast<unsigned>((mn + 255) / 256)),
                     dim3(256), 0, s, partial, p.ksplit, mn, y);
  return hipGetLastError();
}

MoEPlan plan_moe(int64_t pairs, int32_t n_experts) {
  MoEPlan p{};
  p.nsub = 2;
  p.waves_m = 1;
  p.waves_n = 4;
  p.msub = (pairs <= 16 * static_cast<int64_t>(n_experts)) ? 1 : 4;
  p.tile_rows = 16 * p.msub * p.waves_m;
  const int64_t busy = pairs < n_experts ? pairs : n_experts;
  p.max_tiles = pairs / p.tile_rows + busy + 1;
  return p;
}

hipError_t launch_moe_gemm(const MoEPlan &p, int mode, const uint16_t *a, int64_t k,
                           const int32_t *perm, int32_t topk, const uint8_t *w_packed, int64_t n,
                           const MoETile *tiles, const int32_t *n_tiles, float *out,
                           hipStream_t s) {
  GemmArgs g{};
  g.a = a;
  g.w = w_packed;
  g.out = out;
  g.perm = perm;
  g.tiles = tiles;
  g.n_tiles = n_tiles;
  g.m = 0;
  g.n = n;
  g.k = k;
  g.expert_stride = n * (k / 32) * 20;
  g.topk = topk;
  g.ksplit = 1;
  g.chunks = static_cast<int32_t>((k / 32 + 3) / 4);
  g.cb = codebook();
  const int64_t wg_n = 16 * p.nsub * p.waves_n;
  const dim3 grid(static_cast<unsigned>((n + wg_n - 1) / wg_n), static_cast<unsigned>(p.max_tiles),
                  1);
  if (mode == 0) return dispatch<kMoEUp>(p.msub, p.nsub, p.waves_m, p.waves_n, g, grid, s);
  return dispatch<kMoEDown>(p.msub, p.nsub, p.waves_m, p.waves_n, g, grid, s);
}

}  // namespace tq4
