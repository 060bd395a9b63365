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
// permutation and stores relu(acc)^2 already rotated for the down
// projection (fp16, one 32-block per wave, scaled by 2^-kHiddenShift to keep
// large hidden values in fp16's range); mode down reads the bucketed hidden
// rows and stores acc with both shifts undone.  Tiles past the device-side count exit at once, so the
// grid is sized on the host from t*topk without a sync.
#include "tq4_internal.h"
#include "moe_block.h"

#include <atomic>

namespace tq4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

#include "moe_route.h"

enum Mode { kDense = 0, kMoEUp = 1, kMoEDown = 2 };

struct GemmArgs {
  const uint16_t *a;         // rotated activations (fp16 bits), row stride k
  const uint8_t *w;          // packed weights [n][k/32][20] (per expert for MoE)
  float *out;                // output rows, stride n
  uint16_t *out16;           // MoE up: rotated hidden rows (fp16 bits), stride n
  float *partial;            // [ksplit][m][n] (dense split-K)
  Tail tail;                 // dense: bias / residual / bf16 output
  const int32_t *perm;       // MoE: bucket position -> pair
  const MoETile *tiles;      // MoE tile list
  const int32_t *n_tiles;    // MoE tile count (device)
  int64_t m, n, k;
  int64_t expert_stride;     // bytes between experts' packed matrices
  int32_t topk;
  int32_t ksplit;
  int32_t chunks;            // ceil(k / 128)
  int32_t tiles_m, tiles_n;  // workgroup tiles along m and n (MoE: column blocks in tiles_n)
  uint32_t sign_bits;        // MoE up: rotation signs of the hidden rows
  Codebook cb;
};

constexpr int kWaves = 4;          // waves per workgroup, side by side along n
constexpr int kUpWaves16 = 1;      // the same for the MoE up product on 16-row tiles
constexpr int kChunkBytes = 256;   // one fp16 activation row over one chunk (128 k)

__device__ inline uint32_t f16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(f)));
}

// 8 dequantized weights (one codes word) times the half-block scale pair.
// `lut` points at this lane's copy of the pair table: entry e is lut[e * LUTC].
template <int LUTC>
__device__ inline half8 dequant8(uint32_t codes, half2v scale, const uint32_t *lut) {
  const half2v p0 = __builtin_bit_cast(half2v, lut[(codes & 0xFFu) * LUTC]) * scale;
  const half2v p1 = __builtin_bit_cast(half2v, lut[((codes >> 8) & 0xFFu) * LUTC]) * scale;
  const half2v p2 = __builtin_bit_cast(half2v, lut[((codes >> 16) & 0xFFu) * LUTC]) * scale;
  const half2v p3 = __builtin_bit_cast(half2v, lut[(codes >> 24) * LUTC]) * scale;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Stores a wave's MS x NS grid of 16x16 fp32 accumulator tiles of a dense
// product, plus the tail: lane (grp, r) holds, in tile (i, j), the rows
// m0 + 16 i + 4 grp + v (v = 0..3) of column n0 + 16 j + r; out has row
// stride nlim.  Per batch of two row tiles, every residual value is loaded and
// every sum formed before the first store, so the loads overlap and no store
// waits on memory.  The residual may be the output itself, which keeps the
// compiler from moving a load above an earlier store; reordering by hand is
// sound because each element is read and written by its own lane only.
// kCheck = false: the whole grid lies inside the output (no bounds tests).
// kBF16: the residual and output are bf16 (the tail's flag, as a constant).
template <bool kCheck, bool kBF16, int MS, int NS>
__device__ inline void store_tiles_impl(const floatx4 (&acc)[MS][NS], float *out, const Tail &t,
                                        int64_t m0, int64_t n0, int64_t mlim, int64_t nlim,
                                        int grp, int r, float unscale) {
  // Loads use indices clamped into the output, so they need no branches;
  // what they read for an element outside it is never stored.
  const auto clamp_m = [&](int64_t m) { return kCheck && m >= mlim ? mlim - 1 : m; };
  const auto clamp_n = [&](int64_t n) { return kCheck && n >= nlim ? nlim - 1 : n; };
  float bv[NS];  // the bias of this lane's columns, loaded once
#pragma unroll
  for (int j = 0; j < NS; ++j) bv[j] = t.bias != nullptr ? t.bias[clamp_n(n0 + 16 * j + r)] : 0.f;
  constexpr int kIB = 2;  // row tiles per batch
#pragma unroll
  for (int i0 = 0; i0 < MS; i0 += kIB) {
    float y[kIB][NS][4];
    if (t.residual != nullptr) {
#pragma unroll
      for (int ii = 0; ii < kIB; ++ii) {
        if (i0 + ii >= MS) break;
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int64_t m = clamp_m(m0 + 16 * (i0 + ii) + 4 * grp + v);
            const int64_t n = clamp_n(n0 + 16 * j + r);
            y[ii][j][v] = tail_residual_as<kBF16>(t.residual, m * nlim + n);
          }
      }
    }
#pragma unroll
    for (int ii = 0; ii < kIB; ++ii) {
      if (i0 + ii >= MS) break;
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // the weight shift undone (exact for the library's products),
          // then the same two adds, in order, as tail_sum
          float a = acc[i0 + ii][j][v] * unscale;
          if (t.bias != nullptr) a += bv[j];
          if (t.residual != nullptr) a += y[ii][j][v];
          y[ii][j][v] = a;
        }
    }
#pragma unroll
    for (int ii = 0; ii < kIB; ++ii) {
      if (i0 + ii >= MS) break;
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t m = m0 + 16 * (i0 + ii) + 4 * grp + v;
          const int64_t n = n0 + 16 * j + r;
          if (!kCheck || (m < mlim && n < nlim))
            tail_store_as<kBF16>(out, m * nlim + n, y[ii][j][v]);
        }
    }
  }
}

template <int MS, int NS>
__device__ inline void store_tiles(const floatx4 (&acc)[MS][NS], float *out, const Tail &t,
                                   int64_t m0, int64_t n0, int64_t mlim, int64_t nlim, int grp,
                                   int r, float unscale = kWeightUnscale) {
  const bool full = m0 + 16 * MS <= mlim && n0 + 16 * NS <= nlim;
  if (t.bf16) {
    if (full)
      store_tiles_impl<false, true>(acc, out, t, m0, n0, mlim, nlim, grp, r, unscale);
    else
      store_tiles_impl<true, true>(acc, out, t, m0, n0, mlim, nlim, grp, r, unscale);
  } else {
    if (full)
      store_tiles_impl<false, false>(acc, out, t, m0, n0, mlim, nlim, grp, r, unscale);
    else
      store_tiles_impl<true, false>(acc, out, t, m0, n0, mlim, nlim, grp, r, unscale);
  }
}

// The half-block scale as an fp16 pair, shifted by 2^kWeightShift (exact;
// the shift is undone on the fp32 results, see tq4_internal.h).
__device__ inline half2v scale_pair(uint32_t bf16_bits) {
  const _Float16 h = static_cast<_Float16>(__uint_as_float(bf16_bits << 16) * kWeightScale);
  half2v r;
  r[0] = h;
  r[1] = h;
  return r;
}

struct WRaw {
  uint32_t v[5];
};

// The (tile, column block) pair of a grouped-kernel workgroup.  The grid is
// one-dimensional, 8 * ceil(max tiles / 8) * cols long.  Workgroup ids go
// round robin over the 8 XCDs: XCD x takes tiles x, x + 8, x + 16, ..., each
// with all of its column blocks in a row (ids 8 j + x, j = 0, 1, ...).  So
// the workgroups in flight on one L2 share each tile's gathered activation
// rows, and a popular expert, whose tiles are consecutive, is spread evenly
// over the XCDs and read about once by each of them.  Returns false for
// workgroups past the device-side tile count.
__device__ inline bool moe_item(const GemmArgs &g, int lin, int &tile, int64_t &col_block) {
  const int cols = g.tiles_n;
  const int j = lin / 8;
  tile = 8 * (j / cols) + lin % 8;
  col_block = j % cols;
  return tile < *g.n_tiles;
}

// MoE epilogues.  Lane (grp, r) of wave `wave` holds acc[i][j][v] =
// C[16 i + 4 grp + v][16 NSUB wave + 16 j + r] of the workgroup tile (rows
// from m_base, columns from n_base); abuf0 and abuf1 are two LDS buffers of
// at least kWaves * 8 * MSUB * 32 floats that every wave is done with once
// the up epilogue's leading barrier has passed.
template <int MSUB, int NSUB, int MODE>
__device__ inline void moe_store(const floatx4 (&acc)[MSUB][NSUB], const GemmArgs &g,
                                 int64_t m_base, int64_t rows_valid, int64_t n_base, int wave,
                                 int lane, uint8_t *abuf0, uint8_t *abuf1) {
  const int r = lane % 16;
  const int grp = lane / 16;
  if constexpr (MODE == kMoEUp) {
    // h = relu(u)^2, then its rotation ht = H32 diag(s) h / sqrt(32), stored
    // as fp16: a wave's 32 output columns are one 32-block of h.  The wave
    // parks its rows of h in LDS (rows 0-7 of every 16-row tile in abuf0,
    // rows 8-15 in abuf1; 8 * MSUB staged rows x 32 per wave and buffer,
    // 16-byte column groups XOR-swizzled by (row / 2) % 8); then two lanes
    // per staged row rotate it in registers: lane parity p holds elements
    // 16p .. 16p + 15, rotated in-lane over bits 0-3 of the element index,
    // and bit 4 pairs the two lanes (a quad-permute exchange).  Each lane
    // writes 32 contiguous bytes.  The stored values carry the factor
    // 2^-kHiddenShift, which the down product's result undoes.
    static_assert(NSUB == 2, "one 32-block of hidden units per wave");
    __syncthreads();  // every wave is done with the activation stages
    float *const hs0 = reinterpret_cast<float *>(abuf0) + wave * (8 * MSUB * 32);
    float *const hs1 = reinterpret_cast<float *>(abuf1) + wave * (8 * MSUB * 32);
    const float rs32 = kHiddenRotScale;  // 1/sqrt(32) and the hidden shift
    const int p = lane & 1;
    const int srow = (lane >> 1) < 8 * MSUB ? (lane >> 1) : 0;
    const int key = 4 * ((srow >> 1) & 7);
#pragma unroll
    for (int jp = 0; jp < NSUB / 2; ++jp) {
      {
        float *const hw = (grp >> 1) ? hs1 : hs0;
#pragma unroll
        for (int i = 0; i < MSUB; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float u = acc[i][2 * jp + j][v] * kWeightUnscale;
              const int sr = 8 * i + 4 * (grp & 1) + v;
              hw[sr * 32 + ((16 * j + r) ^ (4 * ((sr >> 1) & 7)))] = u > 0.f ? u * u : 0.f;
            }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's own writes are visible
      const int64_t col0 = n_base + wave * (16 * NSUB) + 32 * jp;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float *hs = half ? hs1 : hs0;
        const int64_t local = 16 * (srow / 8) + 8 * half + srow % 8;
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f =
              *reinterpret_cast<const float4 *>(hs + srow * 32 + ((16 * p + 4 * q) ^ key));
          v[4 * q] = f.x;
          v[4 * q + 1] = f.y;
          v[4 * q + 2] = f.z;
          v[4 * q + 3] = f.w;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((g.sign_bits >> (16 * p + e)) & 1u) v[e] = -v[e];
#pragma unroll
        for (int hstep = 1; hstep < 16; hstep <<= 1)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if ((e & hstep) == 0) {
              const float a = v[e], b = v[e + hstep];
              v[e] = a + b;
              v[e + hstep] = a - b;
            }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float o = __builtin_bit_cast(
              float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[e]), 0xB1, 0xF, 0xF, false));
          v[e] = p ? o - v[e] : v[e] + o;
        }
        if ((lane >> 1) < 8 * MSUB && local < rows_valid && col0 < g.n) {
          uint4 *dst = reinterpret_cast<uint4 *>(g.out16 + (m_base + local) * g.n + col0 + 16 * p);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            uint32_t w[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t lo =
                  __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[8 * q + 2 * t] * rs32));
              const uint32_t hi =
                  __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[8 * q + 2 * t + 1] * rs32));
              w[t] = lo | (hi << 16);
            }
            dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        const int64_t n = n_base + wave * (16 * NSUB) + 16 * j + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t local = 16 * i + 4 * grp + v;
          if (local < rows_valid && n < g.n)
            g.out[(m_base + local) * g.n + n] = acc[i][j][v] * kHiddenUnscale;
        }
      }
  }
}

// LUTC copies of the pair table are interleaved (entry e of copy q at
// e * LUTC + q; lane L uses copy L % LUTC), so that random lookups by the
// lanes of a wave spread over the LDS banks.  The small-tile configurations
// use one copy: the lookup address is then the code byte times 4, one
// byte-select shift per lookup (SDWA) instead of an extract and a shift-or,
// and on this table a single copy measured no slower than eight.
// Occupancy targets (waves per SIMD) for the tile heights the MoE layer
// uses: more resident workgroups hide the per-chunk load latency better than
// the registers the compiler would otherwise spend (measured on the MoE
// layer at 16 and 1024 tokens).
constexpr int waves_per_eu_for(int msub) { return msub == 1 ? 6 : (msub == 4 ? 4 : 1); }

// One workgroup tile of the product: `lin` is the tile's linear index (the
// workgroup id of gemm_kernel), `split_z` its K range (dense split-K); abuf0
// and abuf1 are the activation stages (16 * MSUB * kChunkBytes bytes each,
// 16-byte aligned) and lut the pair table (256 * LUTC words), all LDS; tid
// is the thread's index in the workgroup.  Every thread of the workgroup
// calls it (it holds workgroup barriers).
template <int MSUB, int NSUB, int LUTC, int MODE, int WV>
__device__ inline void gemm_tile(const GemmArgs &g, int lin, int split_z, uint8_t *abuf0,
                                 uint8_t *abuf1, uint32_t *lut, int tid) {
  constexpr int TM = 16 * MSUB;           // activation rows per workgroup
  constexpr int TN = 16 * NSUB * WV;      // weight rows per workgroup
  constexpr int LPW = 4 * MSUB / WV;      // activation loads per wave per chunk
  static_assert(LPW * WV == 4 * MSUB, "activation loads split evenly");

  const int wave = tid / 64;
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;

  // ---- which tile -------------------------------------------------------
  int64_t m_base = 0;        // first activation row of the workgroup tile
  int64_t rows_valid = g.m;  // rows of this tile that exist (relative to m_base)
  int64_t n_base = 0;
  const uint8_t *wmat = g.w;
  int split = 0;
  if constexpr (MODE == kDense) {
    // Consecutive workgroup ids go to different XCDs (round robin over 8);
    // renumber so that each XCD works on a contiguous range of tiles (a band
    // of activation rows against all weight rows), which its own L2 serves.
    const int tiles = g.tiles_m * g.tiles_n;
    int t = lin;
    if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
    m_base = static_cast<int64_t>(t / g.tiles_n) * TM;
    n_base = static_cast<int64_t>(t % g.tiles_n) * TN;
    rows_valid = g.m - m_base;
    split = split_z;
  } else {
    int ti;
    int64_t cb;
    if (!moe_item(g, lin, ti, cb)) return;
    const MoETile t = g.tiles[ti];
    m_base = t.row0;
    rows_valid = t.rows;
    wmat = g.w + static_cast<int64_t>(t.expert) * g.expert_stride;
    n_base = cb * TN;
  }

  // ---- codebook pair table, LUTC interleaved copies -----------------------
  for (int i = tid; i < 256 * LUTC; i += 64 * WV) {
    const int e = i / LUTC;
    lut[i] = f16_bits(g.cb.c[e & 15]) | (f16_bits(g.cb.c[e >> 4]) << 16);
  }
  const uint32_t *lutp = lut + (lane % LUTC);

  const int kb = static_cast<int>(g.k / 32);
  const int c_begin = static_cast<int>((static_cast<int64_t>(g.chunks) * split) / g.ksplit);
  const int c_end = static_cast<int>((static_cast<int64_t>(g.chunks) * (split + 1)) / g.ksplit);

  // ---- activation rows this lane copies into LDS ---------------------------
  // A tile is TM rows x 256 bytes = 4*MSUB loads of 1 KB (4 rows each); wave
  // w issues loads w*MSUB .. w*MSUB+MSUB-1.  Lane L of load q fills LDS row
  // 4q + L/16, slot L%16, i.e. global slot (L%16) ^ (row%16) of that row.
  // Rows past the tile's end copy a valid row (their outputs are not stored).
  const uint16_t *asrc[LPW];
  int aslot[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = 4 * (wave * LPW + i) + lane / 16;
    const int64_t local = row < rows_valid ? row : 0;
    int64_t src_row;
    if constexpr (MODE == kMoEUp) {
      src_row = g.perm[m_base + local] / g.topk;
    } else {
      src_row = m_base + local;
    }
    asrc[i] = g.a + src_row * g.k;
    aslot[i] = (lane % 16) ^ (row % 16);
  }
  auto issue_a = [&](int c, uint8_t *buf) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      // MoE: 4-row groups past the tile's rows are not loaded; their LDS rows
      // keep earlier values, which reach only outputs that are not stored
      if (MODE != kDense && i + wave > 0 && 4 * (wave * LPW + i) >= rows_valid) break;
      const int blk = 4 * c + aslot[i] / 4;
      const uint16_t *src = asrc[i] + (blk < kb ? 128 * c + 8 * aslot[i] : 0);
      __builtin_amdgcn_global_load_lds((const global_void *)src,
                                       (lds_void *)(buf + (wave * LPW + i) * 4 * kChunkBytes),
                                       16, 0, 0);
    }
  };

  // ---- weight rows of this lane: 16*NSUB rows per wave ----------------------
  const uint8_t *wrow[NSUB];
  bool w_ok[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int64_t n = n_base + wave * (16 * NSUB) + 16 * j + r;
    w_ok[j] = n < g.n;
    wrow[j] = wmat + (w_ok[j] ? n : 0) * kb * 20;
  }
  // Lane group g takes block 4c+g of each row.  Blocks past k and rows past n
  // read block 0 of a valid row and get a zero scale word, so they add 0.
  auto load_w = [&](int c, WRaw (&wr)[NSUB]) {
    const int b = 4 * c + grp;
    const bool b_ok = b < kb;
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      const uint32_t *p = reinterpret_cast<const uint32_t *>(wrow[j] + (b_ok ? b : 0) * 20);
#pragma unroll
      for (int q = 0; q < 5; ++q) wr[j].v[q] = p[q];
    }
  };

  // For large tiles, an (empty) use of an accumulation register lets the
  // compiler keep the accumulators in them for the whole loop instead of
  // copying them in and out of ordinary vector registers around every MFMA.
  if constexpr (MSUB * NSUB >= 32) asm volatile("" ::"a"(0));
  floatx4 acc[MSUB][NSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute_chunk = [&](const WRaw (&wr)[NSUB], const uint8_t *abase, int c) {
    const bool b_ok = 4 * c + grp < kb;
    half2v sc[NSUB][2];
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      const uint32_t sw = (b_ok && w_ok[j]) ? wr[j].v[4] : 0u;
      sc[j][0] = scale_pair(sw & 0xFFFFu);
      sc[j][1] = scale_pair(sw >> 16);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      half8 bq[NSUB];
#pragma unroll
      for (int j = 0; j < NSUB; ++j) bq[j] = dequant8<LUTC>(wr[j].v[t], sc[j][t >> 1], lutp);
      const int slot = (4 * grp + t) ^ r;
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
        // an MoE tile holds as many rows as its expert has left: 16-row
        // sub-tiles past them (uniform per workgroup) are skipped
        if (MODE != kDense && i > 0 && 16 * i >= rows_valid) break;
        const half8 aq =
            *reinterpret_cast<const half8 *>(abase + (16 * i + r) * kChunkBytes + 16 * slot);
#pragma unroll
        for (int j = 0; j < NSUB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bq[j], acc[i][j], 0, 0, 0);
      }
      // with large tiles, keep one step's operands live at a time
      if constexpr (MSUB * NSUB >= 64) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Two-stage pipeline: while chunk c is multiplied out of one buffer, chunk
  // c+1 streams into the other (the loop is unrolled by two so that each
  // step names its buffers statically).
  auto step = [&](int c, WRaw (&wr)[NSUB], WRaw (&wn)[NSUB], const uint8_t *cur, uint8_t *nxt) {
    if (c + 1 < c_end) {
      issue_a(c + 1, nxt);
      load_w(c + 1, wn);
    }
    compute_chunk(wr, cur, c);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // next chunk landed; this buffer is free again
  };
  if (c_begin < c_end) {
    WRaw w0[NSUB], w1[NSUB];
    issue_a(c_begin, abuf0);
    load_w(c_begin, w0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // pair table and first activation chunk in LDS
    int c = c_begin;
    for (; c + 1 < c_end; c += 2) {
      step(c, w0, w1, abuf0, abuf1);
      step(c + 1, w1, w0, abuf1, abuf0);
    }
    if (c < c_end) step(c, w0, w1, abuf0, abuf1);
  }

  // ---- epilogue: lane holds C[4*grp + v][r] of every 16x16 tile ----------
  if constexpr (MODE == kDense) {
    // split-K partial sums take the tail in the reduction
    const bool split_k = g.ksplit > 1;
    float *dst = split_k ? g.partial + static_cast<int64_t>(split) * g.m * g.n : g.out;
    store_tiles(acc, dst, split_k ? Tail{} : g.tail, m_base, n_base + wave * (16 * NSUB), g.m,
                g.n, grp, r);
  } else {
    static_assert(WV * 8 * MSUB * 32 * 4 <= TM * kChunkBytes, "staging fits");
    moe_store<MSUB, NSUB, MODE>(acc, g, m_base, rows_valid, n_base, wave, lane, abuf0, abuf1);
  }
}

template <int MSUB, int NSUB, int LUTC, int MODE, int WV = kWaves>
__global__ __launch_bounds__(64 * WV)
__attribute__((amdgpu_waves_per_eu(waves_per_eu_for(MSUB)))) void gemm_kernel(GemmArgs g) {
  // Activation tile of one chunk, double buffered.  Row r occupies 256 bytes
  // (16 slots of 8 halves); global slot s of row r is stored in slot
  // s ^ (r % 16), so the fragment reads (16 rows, one slot each) fall on 16
  // distinct 16-byte bank groups.
  __shared__ __attribute__((aligned(16))) uint8_t abuf0[16 * MSUB * kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t abuf1[16 * MSUB * kChunkBytes];
  __shared__ uint32_t lut[256 * LUTC];
  gemm_tile<MSUB, NSUB, LUTC, MODE, WV>(g, static_cast<int>(blockIdx.x),
                                        static_cast<int>(blockIdx.z), abuf0, abuf1, lut,
                                        static_cast<int>(threadIdx.x));
}

// Dense large-M variant of the same product, software-pipelined by k-step.
// Tile: 128 activation rows x 256 weight rows per workgroup, 4 waves of
// 128 x 64 (8 x 4 MFMA tiles, 128 accumulators held in AGPRs for the whole
// loop).  Within a chunk, while the 32 MFMAs of step t issue, the wave
// decodes the weight fragments of step t+1 and reads its activation
// fragments; the last step of a chunk prefetches the first step of the next
// one, with the chunk's barrier placed after that step's MFMAs are issued.
//
// What bounds this shape is how fast a compute unit takes in its tiles, so
// both operands stream in with LDS-direct loads (1 KB of consecutive memory
// per instruction), two chunks ahead of the multiply, into three stages:
// activation chunks (128 rows x 256 bytes, XOR-swizzled) and weight chunks
// (each wave's 64 rows x 80 bytes).  A wave reads its lanes' 20-byte blocks
// back from LDS at the start of each chunk.  Requires K to be a multiple of
// 128 (weight rows 16-byte aligned); other K use gemm_kernel.
constexpr int kBigMSub = 8;
constexpr int kBigNSub = 4;
constexpr int kBigLut = 4;
constexpr int kBigTM = 16 * kBigMSub;                 // 128
constexpr int kBigTN = 16 * kBigNSub * kWaves;        // 256
constexpr int kBigWWave = 16 * kBigNSub * 80;         // 5120: a wave's weight chunk
constexpr int kBigLoads = kBigMSub + kBigWWave / 1024;  // 13 per chunk per wave

__global__ __launch_bounds__(64 * kWaves) void gemm_big_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t abuf0[kBigTM * kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t abuf1[kBigTM * kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t abuf2[kBigTM * kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf0[kWaves * kBigWWave];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf1[kWaves * kBigWWave];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf2[kWaves * kBigWWave];
  __shared__ uint32_t lut[256 * kBigLut];

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;

  // Workgroup ids go round robin over the 8 XCDs.  XCD x takes a band of
  // tiles_m / 8 activation tiles and, within it, runs the activation tiles
  // fastest: the workgroups in flight on one XCD then share a few weight
  // tiles and a few activation tiles, which its L2 keeps.
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
  const int64_t m_base = static_cast<int64_t>(mt) * kBigTM;
  const int64_t n_base = static_cast<int64_t>(nt) * kBigTN;
  const int64_t rows_valid = g.m - m_base;

  for (int i = tid; i < 256 * kBigLut; i += 64 * kWaves) {
    const int e = i / kBigLut;
    lut[i] = f16_bits(g.cb.c[e & 15]) | (f16_bits(g.cb.c[e >> 4]) << 16);
  }
  const uint32_t *lutp = lut + (lane % kBigLut);

  const int kb = static_cast<int>(g.k / 32);
  const int chunks = g.chunks;  // kb / 4

  // activation rows this lane copies: load i of wave w fills LDS rows
  // 4 (w kBigMSub + i) + lane / 16, slot lane % 16 = global slot ^ (row % 16)
  const uint16_t *asrc[kBigMSub];
  int aslot[kBigMSub];
#pragma unroll
  for (int i = 0; i < kBigMSub; ++i) {
    const int row = 4 * (wave * kBigMSub + i) + lane / 16;
    asrc[i] = g.a + (m_base + (row < rows_valid ? row : 0)) * g.k;
    aslot[i] = (lane % 16) ^ (row % 16);
  }
  // weight pieces this lane copies: load s of the wave takes piece
  // q = 64 s + lane of its 64 rows x 80 bytes (row q / 5, part q % 5); rows
  // past n copy row n - 1 and get zero scales
  const uint8_t *wsrc[kBigWWave / 1024];
#pragma unroll
  for (int s = 0; s < kBigWWave / 1024; ++s) {
    const int q = 64 * s + lane;
    const int row = q / 5;
    const int64_t n = n_base + wave * (16 * kBigNSub) + row;
    wsrc[s] = g.w + (n < g.n ? n : g.n - 1) * kb * 20 + 16 * (q - 5 * row);
  }
  uint32_t w_okm = 0;
#pragma unroll
  for (int j = 0; j < kBigNSub; ++j)
    w_okm |= static_cast<uint32_t>(n_base + wave * (16 * kBigNSub) + 16 * j + r < g.n) << j;
  // chunk c into stage (abuf, wbuf); chunks past the end (padding, see
  // below) load the last chunk again and get zero scales
  auto issue = [&](int c, uint8_t *abuf, uint8_t *wbuf) {
    const int cc = c < chunks ? c : chunks - 1;
#pragma unroll
    for (int i = 0; i < kBigMSub; ++i)
      __builtin_amdgcn_global_load_lds((const global_void *)(asrc[i] + 128 * cc + 8 * aslot[i]),
                                       (lds_void *)(abuf + (wave * kBigMSub + i) * 4 * kChunkBytes),
                                       16, 0, 0);
#pragma unroll
    for (int s = 0; s < kBigWWave / 1024; ++s)
      __builtin_amdgcn_global_load_lds((const global_void *)(wsrc[s] + 80 * cc),
                                       (lds_void *)(wbuf + wave * kBigWWave + 1024 * s), 16, 0, 0);
  };
  // this lane's block 4c + grp of each of its weight rows, from LDS
  auto read_w = [&](const uint8_t *wbuf, WRaw (&wr)[kBigNSub]) {
#pragma unroll
    for (int j = 0; j < kBigNSub; ++j) {
      const uint32_t *p =
          reinterpret_cast<const uint32_t *>(wbuf + wave * kBigWWave + (16 * j + r) * 80 + 20 * grp);
#pragma unroll
      for (int q = 0; q < 5; ++q) wr[j].v[q] = p[q];
    }
  };
  auto scales = [&](const WRaw (&wr)[kBigNSub], int c, half2v (&sc)[kBigNSub][2]) {
#pragma unroll
    for (int j = 0; j < kBigNSub; ++j) {
      const uint32_t sw = (c < chunks && ((w_okm >> j) & 1u)) ? wr[j].v[4] : 0u;
      sc[j][0] = scale_pair(sw & 0xFFFFu);
      sc[j][1] = scale_pair(sw >> 16);
    }
  };
  auto decode = [&](const WRaw (&wr)[kBigNSub], const half2v (&sc)[kBigNSub][2], int t,
                    half8 (&bq)[kBigNSub]) {
#pragma unroll
    for (int j = 0; j < kBigNSub; ++j) bq[j] = dequant8<kBigLut>(wr[j].v[t], sc[j][t >> 1], lutp);
  };
  auto read_a = [&](const uint8_t *abase, int t, half8 (&aq)[kBigMSub]) {
    const int slot = (4 * grp + t) ^ r;
#pragma unroll
    for (int i = 0; i < kBigMSub; ++i)
      aq[i] = *reinterpret_cast<const half8 *>(abase + (16 * i + r) * kChunkBytes + 16 * slot);
  };

  asm volatile("" ::"a"(0));
  floatx4 acc[kBigMSub][kBigNSub];
#pragma unroll
  for (int i = 0; i < kBigMSub; ++i)
#pragma unroll
    for (int j = 0; j < kBigNSub; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto mfmas = [&](const half8 (&aq)[kBigMSub], const half8 (&bq)[kBigNSub]) {
#pragma unroll
    for (int i = 0; i < kBigMSub; ++i)
#pragma unroll
      for (int j = 0; j < kBigNSub; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[i], bq[j], acc[i][j], 0, 0, 0);
  };

  constexpr int kWaitNext = 0x0F70 | (kBigLoads & 15) | ((kBigLoads >> 4) << 14);  // vmcnt(13)
  // One chunk: steps t = 0..3 on (cur, wr); step 0's operands (aq, bq) are
  // ready on entry, and on exit hold step 0 of the next chunk.  Chunk c + 2
  // is requested into the far stage on entry; chunk c + 1 is waited for at
  // the end.  The chunk count is padded to a multiple of three so that every
  // chunk issues and waits for the same loads and the waits are exact.
  auto chunk = [&](int c, const uint8_t *acur, const uint8_t *anxt, uint8_t *afar,
                   const uint8_t *wnxt, uint8_t *wfar, WRaw (&wr)[kBigNSub],
                   half8 (&aq)[kBigMSub], half8 (&bq)[kBigNSub]) {
    issue(c + 2, afar, wfar);
    half2v sc[kBigNSub][2];
    scales(wr, c, sc);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      half8 aq2[kBigMSub], bq2[kBigNSub];
      decode(wr, sc, t + 1, bq2);
      read_a(acur, t + 1, aq2);
      mfmas(aq, bq);
#pragma unroll
      for (int i = 0; i < kBigMSub; ++i) aq[i] = aq2[i];
#pragma unroll
      for (int j = 0; j < kBigNSub; ++j) bq[j] = bq2[j];
    }
    // step 3; chunk c + 1 is in once only chunk c + 2's loads are
    // outstanding (loads retire in issue order)
    __builtin_amdgcn_s_waitcnt(kWaitNext);
    mfmas(aq, bq);
    // chunk c + 1 visible to all waves; the current stage free again.  A bare
    // barrier: __syncthreads would also wait for the loads of chunk c + 2.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    read_w(wnxt, wr);
    half2v sn[kBigNSub][2];
    scales(wr, c + 1, sn);
    decode(wr, sn, 0, bq);
    read_a(anxt, 0, aq);
  };

  WRaw wr[kBigNSub];
  half8 aq[kBigMSub], bq[kBigNSub];
  issue(0, abuf0, wbuf0);
  issue(1, abuf1, wbuf1);
  __builtin_amdgcn_s_waitcnt(kWaitNext);  // chunk 0 is in
  __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): pair table written
  __builtin_amdgcn_s_barrier();
  {
    read_w(wbuf0, wr);
    half2v sc[kBigNSub][2];
    scales(wr, 0, sc);
    decode(wr, sc, 0, bq);
    read_a(abuf0, 0, aq);
  }
  for (int c = 0; c < chunks; c += 3) {
    chunk(c, abuf0, abuf1, abuf2, wbuf1, wbuf2, wr, aq, bq);
    chunk(c + 1, abuf1, abuf2, abuf0, wbuf2, wbuf0, wr, aq, bq);
    chunk(c + 2, abuf2, abuf0, abuf1, wbuf0, wbuf1, wr, aq, bq);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the padding chunks' loads

  store_tiles(acc, g.out, g.tail, m_base, n_base + wave * (16 * kBigNSub), g.m, g.n, grp, r);
}

// Dense large-M variant with two waves on every SIMD.  Tile: 256 activation
// rows x 256 weight rows per workgroup, 8 waves of 128 x 64 (2 along m, 4
// along n; 8 x 4 MFMA tiles, 128 accumulators each, so a wave fits in half a
// SIMD's registers and the other wave's decode and LDS reads overlap its
// MFMAs).  Chunks are 64 k (2 blocks): activation chunks are 256 rows x 128
// bytes (16-byte pieces XOR-swizzled by (row / 2) % 8), weight chunks 256 rows x
// 40 bytes, both streamed in with LDS-direct loads two chunks ahead into
// three stages.  Activation pieces move 16 bytes per lane; weight rows of 40
// bytes move as dwords, so packed weights need only 4-byte alignment.
//
// k-slots: lane group g = 2b + h takes block b of the chunk, elements
// 16h + 8t .. 16h + 8t + 7 at step t in 0..1 (codes word 2h + t, half-block
// scale h); the activation side reads k = 16g + 8t of the chunk to match.
// Requires K to be a multiple of 64.
constexpr int kHugeWaves = 8;
constexpr int kHugeMSub = 8;
constexpr int kHugeNSub = 4;
constexpr int kHugeLut = 32;
constexpr int kHugeTM = 2 * 16 * kHugeMSub;                    // 256
constexpr int kHugeTN = (kHugeWaves / 2) * 16 * kHugeNSub;     // 256
constexpr int kHugeRowA = 128;                                 // 64 k of fp16
constexpr int kHugeRowW = 40;                                  // 2 blocks
constexpr int kHugeALoads = kHugeTM * kHugeRowA / 1024 / kHugeWaves;  // 4
constexpr int kHugeWLoads = kHugeTN * kHugeRowW / 256 / kHugeWaves;   // 5
constexpr int kHugeLoads = kHugeALoads + kHugeWLoads;                 // 9
// buffer resource word 3 for raw (untyped) dword loads on gfx9-family parts
constexpr int kBufferFlags = 0x00020000;

// WSIDE (measurement variant, tq4_linear_variant): the rotation undone on the
// decoded weight tiles instead of applied to the activations.  The
// activations are then s .* x in fp16 (act_sign_kernel), and each lane's two
// k-steps of a block half (elements 16 h + 8 t + e) are rotated back by a
// butterfly over e and t in-lane and over h between lane groups 2 b and
// 2 b + 1 (lanes l and l ^ 16).
template <bool WSIDE>
__global__ __launch_bounds__(64 * kHugeWaves) void gemm_huge_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t abuf0[kHugeTM * kHugeRowA];
  __shared__ __attribute__((aligned(16))) uint8_t abuf1[kHugeTM * kHugeRowA];
  __shared__ __attribute__((aligned(16))) uint8_t abuf2[kHugeTM * kHugeRowA];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf0[kHugeTN * kHugeRowW];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf1[kHugeTN * kHugeRowW];
  __shared__ __attribute__((aligned(16))) uint8_t wbuf2[kHugeTN * kHugeRowW];
  __shared__ uint32_t lut[256 * kHugeLut];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int wm = wave / (kHugeWaves / 2);
  const int wn = wave % (kHugeWaves / 2);

  // XCD-banded tile order, as in gemm_big_kernel
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
  const int64_t m_base = static_cast<int64_t>(mt) * kHugeTM;
  const int64_t n_base = static_cast<int64_t>(nt) * kHugeTN;
  const int64_t rows_valid = g.m - m_base;

  for (int i = tid; i < 256 * kHugeLut; i += 64 * kHugeWaves) {
    const int e = i / kHugeLut;
    lut[i] = f16_bits(g.cb.c[e & 15]) | (f16_bits(g.cb.c[e >> 4]) << 16);
  }
  const uint32_t *lutp = lut + (lane % kHugeLut);

  const int kb = static_cast<int>(g.k / 32);
  const int chunks = kb / 2;

  // Loads go through buffer resources over the workgroup's activation and
  // weight rows: the per-lane source offsets (bytes, 32-bit) are loop
  // invariant and the chunk's offset is a scalar.  Activation piece
  // p = kHugeALoads * wave + i holds rows 8p .. 8p + 7: lane l fills row
  // 8p + l / 8, slot l % 8 with global piece slot ^ ((row / 2) % 8).  The LDS
  // has 64 four-byte banks, so a 128-byte row covers half of them: the 16
  // rows of a fragment read hit distinct 16-byte bank groups when the key
  // differs between rows of equal parity.
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(g.a + m_base * g.k), static_cast<short>(0),
      static_cast<int>(kHugeTM * g.k * 2), kBufferFlags);
  uint32_t aoff[kHugeALoads];
#pragma unroll
  for (int i = 0; i < kHugeALoads; ++i) {
    const int row = 8 * (kHugeALoads * wave + i) + lane / 8;
    aoff[i] = static_cast<uint32_t>((row < rows_valid ? row : 0) * g.k * 2) +
              16u * static_cast<uint32_t>((lane % 8) ^ ((row >> 1) % 8));
  }
  // Weight piece p = kHugeWLoads * wave + s is bytes 256p .. 256p + 255 of
  // the chunk's 256 rows x 40 bytes; rows past n copy row n - 1 and get zero
  // scales.
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(g.w + n_base * kb * 20), static_cast<short>(0),
      static_cast<int>(kHugeTN * kb * 20), kBufferFlags);
  uint32_t woff[kHugeWLoads];
#pragma unroll
  for (int s = 0; s < kHugeWLoads; ++s) {
    const int o = 256 * (kHugeWLoads * wave + s) + 4 * lane;
    const int row = o / kHugeRowW;
    const int64_t nrow = n_base + row < g.n ? row : g.n - 1 - n_base;
    woff[s] = static_cast<uint32_t>(nrow * kb * 20 + (o - kHugeRowW * row));
  }
  uint32_t w_okm = 0;
#pragma unroll
  for (int j = 0; j < kHugeNSub; ++j)
    w_okm |= static_cast<uint32_t>(n_base + wn * (16 * kHugeNSub) + 16 * j + r < g.n) << j;
  auto issue = [&](int c, uint8_t *abuf, uint8_t *wbuf) __attribute__((always_inline)) {
    const int cc = c < chunks ? c : chunks - 1;
#pragma unroll
    for (int i = 0; i < kHugeALoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (lds_void *)(abuf + (kHugeALoads * wave + i) * 1024), 16, aoff[i],
          kHugeRowA * cc, 0, 0);
#pragma unroll
    for (int s = 0; s < kHugeWLoads; ++s)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_rsrc, (lds_void *)(wbuf + (kHugeWLoads * wave + s) * 256), 4, woff[s],
          kHugeRowW * cc, 0, 0);
  };

  floatx4 acc[kHugeMSub][kHugeNSub];
#pragma unroll
  for (int i = 0; i < kHugeMSub; ++i)
#pragma unroll
    for (int j = 0; j < kHugeNSub; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int blk = grp >> 1;
  const int half = grp & 1;
  auto compute = [&](int c, const uint8_t *abuf, const uint8_t *wbuf)
                     __attribute__((always_inline)) {
    uint32_t cw[kHugeNSub][2];
    half2v sc[kHugeNSub];
#pragma unroll
    for (int j = 0; j < kHugeNSub; ++j) {
      const uint32_t *p = reinterpret_cast<const uint32_t *>(
          wbuf + (wn * (16 * kHugeNSub) + 16 * j + r) * kHugeRowW + 20 * blk);
      cw[j][0] = p[2 * half];
      cw[j][1] = p[2 * half + 1];
      const uint32_t sw = (c < chunks && ((w_okm >> j) & 1u)) ? p[4] : 0u;
      if constexpr (WSIDE) {
        // z_hat * 2^3: the butterfly's sums grow by up to 32
        const _Float16 h = static_cast<_Float16>(
            __uint_as_float((half ? (sw >> 16) : (sw & 0xFFFFu)) << 16) * 8.0f);
        sc[j][0] = h;
        sc[j][1] = h;
      } else {
        sc[j] = scale_pair(half ? (sw >> 16) : (sw & 0xFFFFu));
      }
    }
    half8 bws[kHugeNSub];  // WSIDE: the second step's rotated weights
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      half8 bq[kHugeNSub];
#pragma unroll
      for (int j = 0; j < kHugeNSub; ++j) {
        if constexpr (WSIDE) {
          if (t == 0) {
            // vp[e] = (element 16 half + e, element 16 half + 8 + e): the
            // butterfly in packed fp16, stages over e in-lane, the stage over
            // the pair within each register, the stage over half across lanes
            half2v vp[8];
            {
              const half8 q0 = dequant8<kHugeLut>(cw[j][0], sc[j], lutp);
              const half8 q1 = dequant8<kHugeLut>(cw[j][1], sc[j], lutp);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                vp[e][0] = q0[e];
                vp[e][1] = q1[e];
              }
            }
#pragma unroll
            for (int hb = 1; hb < 8; hb <<= 1)
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if ((e & hb) == 0) {
                  const half2v lo = vp[e], hi = vp[e + hb];
                  vp[e] = lo + hi;
                  vp[e + hb] = lo - hi;
                }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const _Float16 a0 = vp[e][0], a1 = vp[e][1];
              vp[e][0] = a0 + a1;
              vp[e][1] = a0 - a1;
            }
            const half2v sg = half ? half2v{-1.f16, -1.f16} : half2v{1.f16, 1.f16};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              uint32_t lo, hi;
              lane_pair16(__builtin_bit_cast(uint32_t, vp[e]), lo, hi);
              vp[e] = __builtin_bit_cast(half2v, hi) * sg + __builtin_bit_cast(half2v, lo);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              bq[j][e] = vp[e][0];
              bws[j][e] = vp[e][1];
            }
          } else {
            bq[j] = bws[j];
          }
        } else {
          bq[j] = dequant8<kHugeLut>(cw[j][t], sc[j], lutp);
        }
      }
      const int slot = (2 * grp + t) ^ ((r >> 1) % 8);
#pragma unroll
      for (int i = 0; i < kHugeMSub; ++i) {
        const half8 aq = *reinterpret_cast<const half8 *>(
            abuf + (wm * (16 * kHugeMSub) + 16 * i + r) * kHugeRowA + 16 * slot);
#pragma unroll
        for (int j = 0; j < kHugeNSub; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bq[j], acc[i][j], 0, 0, 0);
      }
    }
  };
  // Chunk c: wait until only chunk c + 1's loads are outstanding (loads
  // retire in issue order), publish chunk c with a bare barrier (which also
  // shows that every wave is done with chunk c - 1's stage), refill that
  // stage with chunk c + 2, multiply chunk c.  The chunk count is padded to
  // a multiple of three; padding chunks reload the last chunk, get zero
  // scales, and keep every wait exact.
  constexpr int kWait = 0x0F70 | (kHugeLoads & 15) | ((kHugeLoads >> 4) << 14);
  auto step = [&](int c, const uint8_t *acur, const uint8_t *wcur, uint8_t *afar, uint8_t *wfar)
                  __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWait);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    issue(c + 2, afar, wfar);
    compute(c, acur, wcur);
  };
  issue(0, abuf0, wbuf0);
  issue(1, abuf1, wbuf1);
  for (int c = 0; c < chunks; c += 3) {
    step(c, abuf0, wbuf0, abuf2, wbuf2);
    step(c + 1, abuf1, wbuf1, abuf0, wbuf0);
    step(c + 2, abuf2, wbuf2, abuf1, wbuf1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the padding chunks' loads

  // WSIDE: sum * 2^-3 / sqrt(32) (the 2^3 shift of its weight operand)
  store_tiles(acc, g.out, g.tail, m_base + wm * (16 * kHugeMSub), n_base + wn * (16 * kHugeNSub),
              g.m, g.n, grp, r, WSIDE ? 0x1.6a09e6p-6f : kWeightUnscale);
}

// y[i] = sum over splits of partial[s][i], in split order, then the tail.
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float *__restrict__ partial,
                                                              int32_t ksplit, int64_t m, int64_t n,
                                                              Tail tail, float *y) {
  const int64_t mn = m * n;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= mn) return;
  float s = partial[i];
  for (int q = 1; q < ksplit; ++q) s += partial[q * mn + i];
  const int64_t col = tail.bias != nullptr ? i % n : 0;  // the column only feeds the bias
  const float res = tail.residual != nullptr ? tail_residual(tail, i) : 0.f;
  tail_store(tail, y, i, tail_sum(tail, s, col, res));
}

template <int MSUB, int NSUB, int LUTC, int MODE, int WV = kWaves>
hipError_t launch_cfg(const GemmArgs &g, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<MSUB, NSUB, LUTC, MODE, WV>), grid, dim3(64 * WV), 0, s, g);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(int msub, int nsub, int waves_m, const GemmArgs &g, dim3 grid,
                    hipStream_t s) {
  if (nsub == 2 && waves_m == 1) {
    switch (msub) {
      case 1:
        // the 16-row up product: one wave (32 columns) per workgroup, so that
        // the few (tile, column block) pairs of a small-token layer become
        // four times as many workgroups (measured per 16-token layer: 4
        // waves 140-142 us, 2 waves 139-140, 1 wave 136-138; 2 waves for
        // the down product were 4 us slower)
        if (MODE == kMoEUp) return launch_cfg<1, 2, 1, MODE, kUpWaves16>(g, grid, s);
        return launch_cfg<1, 2, 1, MODE>(g, grid, s);
      case 2: return launch_cfg<2, 2, 1, MODE>(g, grid, s);
      case 3: return launch_cfg<3, 2, 1, MODE>(g, grid, s);
      case 4: return launch_cfg<4, 2, 1, MODE>(g, grid, s);
      default: break;
    }
  }
  if constexpr (MODE == kDense) {
    if (waves_m == 2 && nsub == 4 && msub == 8 && g.ksplit == 1 && g.k % 64 == 0) {
      hipLaunchKernelGGL(gemm_huge_kernel<false>, grid, dim3(64 * kHugeWaves), 0, s, g);
      return hipGetLastError();
    }
    if (waves_m != 1) return hipErrorInvalidValue;
    if (nsub == 4 && msub == 8 && g.ksplit == 1 && g.k % 128 == 0 &&
        reinterpret_cast<uintptr_t>(g.w) % 16 == 0) {
      hipLaunchKernelGGL(gemm_big_kernel, grid, dim3(64 * kWaves), 0, s, g);
      return hipGetLastError();
    }
    if (nsub == 4 && msub == 8) return launch_cfg<8, 4, 32, MODE>(g, grid, s);
  }
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------
// The MoE block in one persistent launch (Nemotron-TheHobbit-30B-A3B model
// card: section Running it, "sync-free MoE", and the help-wanted list's
// fused kernels).  A cooperative launch of as many 4-wave workgroups as the
// device holds at once (4 per compute unit) runs the block's steps in order,
// with a grid-wide barrier between steps:
//   1. workgroup 0 routes every token (route_one_token, one wave per token)
//      and buckets the pairs (bucket_group), as the bucketing launch of
//      tq4_moe_block does; the other workgroups rotate the activation rows
//      (one thread per 32-block);
//   2. the up product, ReLU^2 and the rotation of the hidden rows, one
//      (16-row tile, 128-column block) per workgroup and item (gemm_tile);
//   3. the down product, likewise;
//   4. the weighted combine (combine_quad), four outputs per thread.
// Each step is the code of the launch that does it in tq4_moe_block, on
// the same data in the same order, so the results are the same bit for bit.
// Items are dealt as gemm_kernel's grid deals its workgroups (moe_item), the
// grid being a multiple of 8 workgroups, so an item runs on the XCD that
// workgroup would have.  The 16-token layer's items (about 1100 and 1500)
// take two rounds each on the 1024 workgroups; 6 workgroups per compute unit
// (one round) measured slower: a compute unit's items do not finish sooner
// when more of them share it.
//
// The barrier: after a workgroup barrier one thread of each workgroup
// releases the workgroup's writes (an agent-scope fence) and counts itself
// in one of kBarStripes counters, 128-byte lines apart; the last of a
// stripe acquires and re-releases (fence to fence through the counter's
// chain of adds) and counts the stripe in a top counter, and the last
// stripe does the same and writes the round into kBarFlags flag words.  The
// waiting workgroups poll one flag each (one lane, spread over the flags),
// then acquire.  Counters only grow within a launch (round r
// completes at r arrivals per workgroup); a small kernel zeroes them before
// it.  A poll gives up after kBarSpinLimit rounds, so a grid that could not
// be co-resident ends with wrong results instead of hanging (the
// cooperative launch refuses such grids anyway).
constexpr int kBlockWaves = 4;
constexpr int kBlockThreads = 64 * kBlockWaves;
constexpr int kBarStripes = 16;
constexpr int kBarFlags = 32;
constexpr int kBarStride = 32;  // words: one counter or flag per 128-byte line
constexpr int kBarWords = (kBarStripes + 1 + kBarFlags) * kBarStride;
constexpr uint32_t kBarSpinLimit = 1u << 20;

struct BlockArgs {
  GemmArgs up, down;  // the grouped products; tiles_n = 128-column blocks
  const float *logits;
  const uint16_t *x;
  int64_t t, k, x_blocks;
  int32_t n_experts, topk, tile_rows;
  uint32_t sign_bits;
  int32_t *ids;
  float *gates;
  int32_t *counts, *offsets, *perm, *inv;
  MoETile *tiles;
  int32_t *n_tiles;
  uint16_t *xt;
  float *o, *out;
  uint32_t *bar;  // kBarWords words, zero at the start
};

__device__ inline void grid_barrier(uint32_t *bar, uint32_t round) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t nblk = gridDim.x;
    const uint32_t s = blockIdx.x % kBarStripes;
    const uint32_t stripes = nblk < kBarStripes ? nblk : kBarStripes;
    const uint32_t per = (nblk - s + kBarStripes - 1) / kBarStripes;  // workgroups of stripe s
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = __hip_atomic_fetch_add(bar + s * kBarStride, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == round * per) {
      // the last of the stripe acquires the stripe's releases (its add read
      // the end of their chain of adds) and passes them on
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
      const uint32_t top = __hip_atomic_fetch_add(bar + kBarStripes * kBarStride, 1u,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (top + 1 == round * stripes) {
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
        for (int c = 0; c < kBarFlags; ++c)
          __hip_atomic_store(bar + (kBarStripes + 1 + c) * kBarStride, round, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    const uint32_t *flag = bar + (kBarStripes + 1 + blockIdx.x % kBarFlags) * kBarStride;
    for (uint32_t spin = 0; spin < kBarSpinLimit; ++spin) {
      if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= round) break;
      __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

__global__ __launch_bounds__(kBlockThreads) void moe_block_kernel(BlockArgs b) {
  __shared__ __attribute__((aligned(16))) uint8_t abuf0[16 * kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t abuf1[16 * kChunkBytes];
  __shared__ uint32_t lut[256];
  __shared__ int32_t hist[kBlockWaves][kMaxExperts];
  __shared__ int32_t base[kMaxExperts + 1];
  __shared__ int32_t tile_base[kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int64_t nblk = gridDim.x;
  const int64_t blk = blockIdx.x;

  // 1. routing and bucketing (workgroup 0), activation rotation (the rest)
  if (blk == 0) {
    for (int64_t tok = wave; tok < b.t; tok += kBlockWaves)
      route_one_token(b.logits + tok * b.n_experts, b.n_experts, b.topk, lane,
                      b.ids + tok * b.topk, b.gates + tok * b.topk);
    // the ids are read back by this workgroup only
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __syncthreads();
    bucket_group<kBlockWaves>(hist, base, tile_base, b.ids, b.t * b.topk, b.n_experts, b.counts,
                              b.offsets, b.perm, b.inv, b.tiles, b.n_tiles, b.tile_rows,
                              nullptr);
  } else {
    for (int64_t i = (blk - 1) * kBlockThreads + tid; i < b.x_blocks;
         i += (nblk - 1) * kBlockThreads)
      rotate_block_bf16(b.x + i * 32, b.sign_bits, b.xt + i * 32);
  }
  grid_barrier(b.bar, 1);

  // 2, 3. the grouped products; a workgroup barrier after each item, since
  // the next one's loads refill stages the up epilogue may still be reading
  const int64_t tiles8 = (static_cast<int64_t>(*b.n_tiles) + 7) / 8 * 8;
  for (int64_t it = blk; it < tiles8 * b.up.tiles_n; it += nblk) {
    gemm_tile<1, 2, 1, kMoEUp, kBlockWaves>(b.up, static_cast<int>(it), 0, abuf0, abuf1, lut,
                                            tid);
    __syncthreads();
  }
  grid_barrier(b.bar, 2);
  for (int64_t it = blk; it < tiles8 * b.down.tiles_n; it += nblk) {
    gemm_tile<1, 2, 1, kMoEDown, kBlockWaves>(b.down, static_cast<int>(it), 0, abuf0, abuf1,
                                              lut, tid);
    __syncthreads();
  }
  grid_barrier(b.bar, 3);

  // 4. combine
  const int64_t q = b.k / 4;
  for (int64_t i = blk * kBlockThreads + tid; i < b.t * q; i += nblk * kBlockThreads)
    combine_quad(b.o, b.inv, b.gates, i / q, i % q, b.topk, b.k, b.out);
}

__global__ __launch_bounds__(256) void bar_reset_kernel(uint32_t *bar) {
  for (int i = threadIdx.x; i < kBarWords; i += 256) bar[i] = 0u;
}

}  // namespace

DensePlan plan_dense(int64_t m, int64_t k, int64_t n) {
  DensePlan p{};
  p.chunks = (k / 32 + 3) / 4;
  p.waves_m = 1;
  p.waves_n = 4;
  if (m <= 64) {
    p.msub = static_cast<int>((m + 15) / 16);
    if (p.msub < 1) p.msub = 1;
    p.nsub = 2;
  } else {
    p.msub = 8;
    p.nsub = 4;
    // 256 x 256 tiles (two waves per SIMD) once there are enough of them to
    // give every compute unit one; else 128 x 256
    const int64_t tiles256 = ((m + 255) / 256) * ((n + 255) / 256);
    if (k % 64 == 0 && tiles256 >= 256 && 256 * k * 2 < (int64_t{1} << 31) &&
        n * (k / 32) * 20 < (int64_t{1} << 31))
      p.waves_m = 2;
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
                        hipStream_t s, const Tail &tail) {
  GemmArgs g{};
  g.a = xt;
  g.w = packed;
  g.out = y;
  g.partial = partial;
  g.tail = tail;
  g.m = m;
  g.n = n;
  g.k = k;
  g.ksplit = p.ksplit;
  g.chunks = static_cast<int32_t>(p.chunks);
  g.tiles_m = static_cast<int32_t>(p.m_tiles);
  g.tiles_n = static_cast<int32_t>(p.n_tiles);
  g.cb = codebook();
  const dim3 grid(static_cast<unsigned>(p.n_tiles * p.m_tiles), 1, static_cast<unsigned>(p.ksplit));
  hipError_t e = dispatch<kDense>(p.msub, p.nsub, p.waves_m, g, grid, s);
  if (e != hipSuccess || p.ksplit == 1) return e;
  const int64_t mn = m * n;
  hipLaunchKernelGGL(reduce_partials_kernel, dim3(static_cast<unsigned>((mn + 255) / 256)),
                     dim3(256), 0, s, partial, p.ksplit, m, n, tail, y);
  return hipGetLastError();
}

bool dense_huge_fits(int64_t m, int64_t k, int64_t n) {
  const DensePlan p = plan_dense(m, k, n);
  return p.waves_m == 2 && p.ksplit == 1 && k % 64 == 0;
}

hipError_t launch_dense_weight_side(const uint16_t *xs, int64_t m, int64_t k,
                                    const uint8_t *packed, int64_t n, float *y, hipStream_t s) {
  if (!dense_huge_fits(m, k, n)) return hipErrorInvalidValue;
  const DensePlan p = plan_dense(m, k, n);
  GemmArgs g{};
  g.a = xs;
  g.w = packed;
  g.out = y;
  g.m = m;
  g.n = n;
  g.k = k;
  g.ksplit = 1;
  g.chunks = static_cast<int32_t>(p.chunks);
  g.tiles_m = static_cast<int32_t>(p.m_tiles);
  g.tiles_n = static_cast<int32_t>(p.n_tiles);
  g.cb = codebook();
  const dim3 grid(static_cast<unsigned>(p.n_tiles * p.m_tiles), 1, 1);
  hipLaunchKernelGGL(gemm_huge_kernel<true>, grid, dim3(64 * kHugeWaves), 0, s, g);
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

namespace {

// Arguments of a grouped product over the MoE tile list; tiles_n (the column
// blocks) is set by the caller from its workgroup width.
GemmArgs moe_gemm_args(const uint16_t *a, int64_t k, const int32_t *perm, int32_t topk,
                       const uint8_t *w_packed, int64_t n, const MoETile *tiles,
                       const int32_t *n_tiles, float *out, uint16_t *out16, uint32_t sign_bits) {
  GemmArgs g{};
  g.a = a;
  g.w = w_packed;
  g.out = out;
  g.out16 = out16;
  g.sign_bits = sign_bits;
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
  return g;
}

}  // namespace

hipError_t launch_moe_gemm(const MoEPlan &p, int mode, const uint16_t *a, int64_t k,
                           const int32_t *perm, int32_t topk, const uint8_t *w_packed, int64_t n,
                           const MoETile *tiles, const int32_t *n_tiles, float *out,
                           uint16_t *out16, uint32_t sign_bits, hipStream_t s) {
  if (mode == 0 && n % 32 != 0) return hipErrorInvalidValue;
  GemmArgs g = moe_gemm_args(a, k, perm, topk, w_packed, n, tiles, n_tiles, out, out16, sign_bits);
  // one workgroup per (tile, column block) pair that can exist, the tile
  // count rounded up to a multiple of 8 (see moe_item)
  const int64_t wg_n = 16 * p.nsub * (mode == 0 && p.msub == 1 ? kUpWaves16 : p.waves_n);
  const int64_t cols = (n + wg_n - 1) / wg_n;
  g.tiles_n = static_cast<int32_t>(cols);
  const dim3 grid(static_cast<unsigned>((p.max_tiles + 7) / 8 * 8 * cols), 1, 1);
  if (mode == 0) return dispatch<kMoEUp>(p.msub, p.nsub, p.waves_m, g, grid, s);
  return dispatch<kMoEDown>(p.msub, p.nsub, p.waves_m, g, grid, s);
}


size_t moe_block_persistent_scratch_bytes() { return kBarWords * sizeof(uint32_t); }

hipError_t launch_moe_block_persistent(const uint16_t *x, int64_t t, int64_t k,
                                       const float *logits, int32_t n_experts, int32_t topk,
                                       const uint8_t *w1, int64_t n1, const uint8_t *w2,
                                       uint32_t sign_bits, float *out, const MoEScratch &sc,
                                       hipStream_t s) {
  const MoEPlan p = plan_moe(t * topk, n_experts);
  if (p.msub != 1 || n1 % 32 != 0 || k % 4 != 0 || n_experts > kMaxExperts)
    return hipErrorInvalidValue;
  // co-resident workgroups of this device, a multiple of 8 (cached per
  // device; concurrent first calls compute the same value)
  static std::atomic<int> grid_of[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int grid = grid_of[dev].load(std::memory_order_relaxed);
  if (grid == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_block_kernel, kBlockThreads, 0);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    grid = per_cu * cus / 8 * 8;
    if (grid < 8) return hipErrorInvalidConfiguration;
    grid_of[dev].store(grid, std::memory_order_relaxed);
  }
  BlockArgs b{};
  b.up = moe_gemm_args(sc.xt, k, sc.perm, topk, w1, n1, sc.tiles, sc.n_tiles, nullptr, sc.ht,
                       sign_bits);
  b.down = moe_gemm_args(sc.ht, n1, sc.perm, topk, w2, k, sc.tiles, sc.n_tiles, sc.o, nullptr,
                         sign_bits);
  const int64_t wg_n = 16 * 2 * kBlockWaves;
  b.up.tiles_n = static_cast<int32_t>((n1 + wg_n - 1) / wg_n);
  b.down.tiles_n = static_cast<int32_t>((k + wg_n - 1) / wg_n);
  b.logits = logits;
  b.x = x;
  b.t = t;
  b.k = k;
  b.x_blocks = t * (k / 32);
  b.n_experts = n_experts;
  b.topk = topk;
  b.tile_rows = p.tile_rows;
  b.sign_bits = sign_bits;
  b.ids = sc.ids;
  b.gates = sc.gates;
  b.counts = sc.counts;
  b.offsets = sc.offsets;
  b.perm = sc.perm;
  b.inv = sc.inv;
  b.tiles = sc.tiles;
  b.n_tiles = sc.n_tiles;
  b.xt = sc.xt;
  b.o = sc.o;
  b.out = out;
  b.bar = sc.bar;
  hipLaunchKernelGGL(bar_reset_kernel, dim3(1), dim3(256), 0, s, sc.bar);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  void *args[] = {&b};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(moe_block_kernel),
                                    dim3(static_cast<unsigned>(grid)),
                                    dim3(kBlockThreads), args, 0, s);
}

}  // namespace tq4
