// Decode-shaped TQ4_1S linear layer: up to 16 activation rows (one 16-token
// diffusion block, the shape every denoiser projection sees on each step;
// Nemotron-TheHobbit-30B-A3B model card, sections Running it and Performance
// & why it's slow) in a single kernel launch, rotation included.
//
// The weight stream is the whole cost, so the kernel is arranged to start
// consuming weights as early as possible and to keep everything else off that
// path.  A workgroup owns 32 weight rows (two 16-row MFMA tiles) and all of
// K, with two kinds of waves:
//
//  * 4 producer waves bring x (16 rows of 2k bytes) into LDS with whole-row
//    LDS-direct loads (1 KB per load instruction, every cache line fully
//    used) and build the codebook pair table.  Their loads are issued before any weight load
//    (a workgroup barrier orders the two), so x arrives first.
//  * 8 consumer waves split K by chunks of 4 blocks (128 inputs).  Each
//    issues every weight load it will need at once (its 20-byte block of each
//    row tile, chunk by chunk) and then consumes the chunks in issue order: a
//    wave's vector-memory counter retires in that order, so chunk i is used
//    as soon as its own blocks are in while later chunks still stream.  (The
//    two roles live in different waves for the same reason: a wave that both
//    streamed weights and waited for x would wait for its weights too.)
//
// Per chunk, a consumer
//  1. rotates the chunk's 4 activation blocks from LDS:
//     xt_b = H32 diag(s) x_b / sqrt(32) is a product with a +-1 matrix, so two
//     v_mfma_f32_16x16x32_bf16 per block compute it from the bf16 input
//     against entries +-2^-3 (exact in bf16; products exact, sums fp32).  The
//     MFMA rows are permuted so that lane group g receives xt elements
//     8g..8g+7 of the block: that is directly the activation operand of the
//     block's product MFMA.  The remaining 8/sqrt(32) is applied once to y
//     (with the weight operand's 2^-8, see tq4_internal.h);
//  2. transposes its weight words across the 4 lane groups (lane group g
//     loaded block 4c+g; after two v_permlane32_swap and two
//     v_permlane16_swap per 4 words it holds word g of every block), so that
//     the product of block 4c+t takes elements 8g..8g+7 from lane group g;
//  3. decodes in registers (four byte-indexed lookups of fp16 level pairs in
//     an LDS table, one copy per lane % 8 to spread random lookups over the
//     banks; one packed fp16 multiply by the half-block scale per pair) and
//     accumulates with v_mfma_f32_16x16x32_f16.
// The consumers' partial sums are added at the end in wave order, so results
// are deterministic.
#include "tq4_internal.h"

namespace tq4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kConsumers = 8;
constexpr int kProducers = 4;
constexpr int kThreads = 64 * (kConsumers + kProducers);
constexpr int kRowTiles = 2;                 // 16-row MFMA tiles per workgroup
constexpr int kRowsPerWG = 16 * kRowTiles;   // 32
constexpr int kLutCopies = 8;
constexpr int kMaxK = 4096;
constexpr int kXStrideMax = kMaxK + 8;  // halves per x row slot in LDS

struct SkinnyArgs {
  const uint16_t *x;  // bf16 [m][k]
  const uint8_t *w;   // packed [n][k/32][20]
  float *y;           // [m][n]
  Tail tail;          // bias / residual / bf16 output
  int32_t m, n, kb;   // kb = k / 32
  uint32_t sign_bits;
  Codebook cb;
};

typedef float float2v __attribute__((ext_vector_type(2)));

// two fp32 values to a packed fp16 pair, round to nearest even (one
// v_cvt_pk_f16_f32)
__device__ inline uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){lo, hi}, half2v));
}

// `lut` points at this lane's copy: entry e is lut[e * C].
template <int C = kLutCopies>
__device__ inline half8 dequant8(uint32_t codes, half2v scale, const uint32_t *lut) {
  const half2v p0 = __builtin_bit_cast(half2v, lut[(codes & 0xFFu) * C]) * scale;
  const half2v p1 = __builtin_bit_cast(half2v, lut[((codes >> 8) & 0xFFu) * C]) * scale;
  const half2v p2 = __builtin_bit_cast(half2v, lut[((codes >> 16) & 0xFFu) * C]) * scale;
  const half2v p3 = __builtin_bit_cast(half2v, lut[(codes >> 24) * C]) * scale;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The half-block scale as an fp16 pair, shifted by 2^kWeightShift (exact).
__device__ inline half2v scale_pair(uint32_t bf16_bits) {
  const float f = __uint_as_float(bf16_bits << 16) * kWeightScale;
  return __builtin_convertvector((float2v){f, f}, half2v);
}

// 4x4 transpose across the lane groups (rows of 16 lanes): on entry lane
// group g holds d[q] = D[g][q]; on exit it holds d[q] = D[q][g].
__device__ inline void transpose4(uint32_t (&d)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  d[0] = c[0];
  d[1] = c[1];
  d[2] = e[0];
  d[3] = e[1];
}

// CH >= chunks per consumer wave; XL >= ceil(k / 512) (loads per lane per x row).
template <int CH, int XL>
__global__ __launch_bounds__(kThreads) void skinny_kernel(SkinnyArgs g) {
  __shared__ uint32_t lut[256 * kLutCopies];
  __shared__ floatx4 red[kConsumers][kRowTiles][64];  // consumers' partial sums
  __shared__ uint16_t xs[16 * kXStrideMax];           // x rows

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int kb = g.kb;
  const int k = 32 * kb;
  // x row slot in LDS: k rounded up to whole KB, plus 8 halves, so that
  // consecutive rows start 4 banks apart (16-lane 16-byte reads of 16
  // different rows then hit 64 distinct banks)
  const int xstride = ((k + 511) / 512) * 512 + 8;

  if (wave >= kConsumers) {
    // ---------------------------------------------------------- producers
    const int pw = wave - kConsumers;
    const int ptid = tid - 64 * kConsumers;
    // rows pw, pw + 4, pw + 8, pw + 12, loaded straight into LDS (16 bytes
    // per lane, 1 KB per instruction).  Rows past m load row 0 (finite
    // values; their outputs are never stored); lanes past the row end re-read
    // piece 0 and land in the row's slack (the row slot is a whole number of
    // KB plus 16 bytes).
    const int row_pieces = k / 8;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int rr = pw + 4 * h;
      const uint16_t *src = g.x + (rr < g.m ? rr : 0) * k;
      uint16_t *dst = xs + rr * xstride;
#pragma unroll
      for (int i = 0; i < XL; ++i) {
        const int p = i * 64 + lane;
        __builtin_amdgcn_global_load_lds((const global_void *)(src + 8 * (p < row_pieces ? p : 0)),
                                         (lds_void *)(dst + 512 * i), 16, 0, 0);
      }
    }
    // 0: x requests are out; consumers may start on weights (orders issue only)
    __builtin_amdgcn_s_barrier();
    const float lut_lo = g.cb.c[ptid & 15];
    const float lut_hi = g.cb.c[ptid >> 4];
    {
      const uint32_t e = pack_f16x2(lut_lo, lut_hi);
      uint4 *dst = reinterpret_cast<uint4 *>(lut + ptid * kLutCopies);
#pragma unroll
      for (int c = 0; c < kLutCopies / 4; ++c) dst[c] = make_uint4(e, e, e, e);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the LDS-direct loads have landed
    __syncthreads();  // 1: x rows and pair table in LDS
    __syncthreads();  // 2: consumers' partial sums in LDS
    return;
  }

  // ------------------------------------------------------------ consumers
  const int chunks = (kb + 3) / 4;
  // workgroups rotate which wave takes which K range, so that they do not
  // all touch the same lines at the same moment
  const int q = (wave + static_cast<int>(blockIdx.x)) % kConsumers;
  const int c0 = (q * chunks) / kConsumers;
  const int c_end = ((q + 1) * chunks) / kConsumers;
  const int n_base = static_cast<int>(blockIdx.x) * kRowsPerWG + r;
  const uint8_t *wrow[kRowTiles];
  bool n_ok[kRowTiles];
#pragma unroll
  for (int j = 0; j < kRowTiles; ++j) {
    const int n = n_base + 16 * j;
    n_ok[j] = n < g.n;
    wrow[j] = g.w + static_cast<int64_t>(n_ok[j] ? n : 0) * kb * 20;
  }
  // rotation operand: MFMA row q stands for output element
  // pi(q) = 8 (q / 4) + q % 4 (+4 for the second MFMA), column kk for input kk
  bf16x8 h_lo, h_hi;
  {
    const int j_lo = 8 * (r >> 2) + (r & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = 8 * grp + i;
      const uint32_t sk = (g.sign_bits >> kk) & 1u;
      const uint32_t n_lo = (__builtin_popcount(j_lo & kk) & 1) ^ sk;
      const uint32_t n_hi = (__builtin_popcount((j_lo + 4) & kk) & 1) ^ sk;
      h_lo[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(kRotEntryBF16 | (n_lo << 15)));
      h_hi[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(kRotEntryBF16 | (n_hi << 15)));
    }
  }
  __builtin_amdgcn_s_barrier();  // 0

  // every weight block of this wave, chunk by chunk, no branches: a slot
  // without data re-reads a valid address and gets a zero scale below
  uint32_t wr[CH][kRowTiles][5];
  uint32_t ok_mask = 0;  // bit kRowTiles*i + j: weight slot (i, j) is real
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = c0 + i;
    const int b = 4 * c + grp;
    const bool b_ok = c < c_end && b < kb;
#pragma unroll
    for (int j = 0; j < kRowTiles; ++j) {
      const bool ok = b_ok && n_ok[j];
      ok_mask |= static_cast<uint32_t>(ok) << (kRowTiles * i + j);
      const uint32_t *p = reinterpret_cast<const uint32_t *>(wrow[j] + (ok ? b * 20 : 0));
#pragma unroll
      for (int v = 0; v < 5; ++v) wr[i][j][v] = p[v];
    }
  }
  __syncthreads();  // 1

  const uint32_t *my_lut = lut + (lane % kLutCopies);
  const uint16_t *xs_row = xs + r * xstride;
  floatx4 acc[kRowTiles];
#pragma unroll
  for (int j = 0; j < kRowTiles; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = c0 + i;
    // 1. rotated activations of blocks 4c + t (block 0 past the end: finite,
    //    and it meets zero weights)
    half8 a[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int b = 4 * c + t;
      const int col = (c < c_end && b < kb) ? 32 * b : 0;
      const bf16x8 xb8 =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(xs_row + col + 8 * grp));
      const floatx4 lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h_lo, xb8, zero, 0, 0, 0);
      const floatx4 hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h_hi, xb8, zero, 0, 0, 0);
      a[t] = __builtin_bit_cast(half8, make_uint4(pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3]),
                                                  pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3])));
    }
#pragma unroll
    for (int j = 0; j < kRowTiles; ++j) {
      // 2. word g of every block of the chunk into lane group g
      uint32_t codes[4] = {wr[i][j][0], wr[i][j][1], wr[i][j][2], wr[i][j][3]};
      const uint32_t sw = ((ok_mask >> (kRowTiles * i + j)) & 1u) ? wr[i][j][4] : 0u;
      uint32_t scales[4] = {sw, sw, sw, sw};
      transpose4(codes);
      transpose4(scales);
      // 3. decode elements 8g..8g+7 of block 4c + t (half g / 2) and multiply
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const half2v sc = scale_pair(grp < 2 ? (scales[t] & 0xFFFFu) : (scales[t] >> 16));
        const half8 bq = dequant8(codes[t], sc, my_lut);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], bq, acc[j], 0, 0, 0);
      }
    }
  }

  // the consumers' partial sums, in wave order; lane holds C[4grp+v][r]
#pragma unroll
  for (int j = 0; j < kRowTiles; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();  // 2
  if (wave < kRowTiles) {
    floatx4 s = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kConsumers; ++w) s += red[w][wave][lane];
    const int n = n_base + 16 * wave;
    if (n < g.n) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * grp + v;
        if (m < g.m) tail_apply(g.tail, g.y, m, n, g.n, s[v] * kSkinnyUnscale);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LDS-direct variant, for K a multiple of 128 up to kDmaMaxK.  Measured on
// this shape, the call is the time a compute unit takes to bring in its
// bytes (the weights of its 32 rows plus all of x, which every workgroup
// needs) and then to decode the chunks that land last.  LDS-direct loads of
// 16 bytes per lane, each instruction covering 1 KB of consecutive memory,
// take those in markedly faster than loads into registers, so this variant
// stages everything in LDS, chunk by chunk: a chunk slot holds the chunk's
// slice of x (16 rows x 256 bytes, its 16-byte parts XOR-swizzled by row so
// that fragment reads hit distinct banks) and its weights (32 rows x 80
// bytes).
//
//  * kDmaProducers waves keep the loads going: producer p takes chunks p,
//    p + kDmaProducers, ..., keeps kDmaDepth of them in flight, and as each
//    lands (its loads retire in issue order) raises that chunk's LDS flag and
//    issues the chunk kDmaDepth ahead.
//  * kDmaConsumers waves take chunks round robin (the last ones cut finer,
//    see the consumer loop); each waits for the chunk's flag, rotates the x
//    blocks (two bf16 MFMAs per block against the +-1 matrix, as in
//    skinny_kernel), decodes its lane's code words in registers
//    (decode8_perm: byte tables and v_perm_b32, so the LDS serves only the
//    stream and the chunk reads) and accumulates with f16 MFMAs.
//    Consumers issue no vector-memory loads, so nothing they do waits on the
//    stream.  Measured against the same kernel decoding through an LDS table
//    of level pairs: equal results bit for bit, 0.1-0.4 us faster per call.
// Producers and the chunks each keeps in flight.  Measured per call at
// K=2688 (graph replay, medians of five runs): 4 producers with 1, 2, 3, 4
// or 5 chunks each 7.52, 7.17, 7.32-7.40, 7.84, 8.24 us; 8 producers with 1
// or 2 chunks each 6.98-7.06 and 7.53 us.  About 8 chunks in flight per
// compute unit is best: more requests in flight only queue longer in front
// of the ones a consumer waits for, fewer leave the stream short.
constexpr int kDmaProducers = 8;
constexpr int kDmaConsumers = 8;
constexpr int kDmaDepth = 1;
static_assert(kDmaDepth >= 1 && kDmaDepth <= 3, "the producers' waits cover up to 3 chunks");
constexpr int kDmaThreads = 64 * (kDmaProducers + kDmaConsumers);
constexpr int kXSliceBytes = 16 * 256;                      // 16 rows x 128 k, bf16
constexpr int kChunkRowBytes = 80;                          // 4 blocks of one row
constexpr int kChunkBytes = kRowsPerWG * kChunkRowBytes;    // 2560
constexpr int kSlotBytes = kXSliceBytes + kChunkBytes;      // 6656
constexpr int kDmaMaxK = 2944;
constexpr int kDmaMaxChunks = kDmaMaxK / 128;               // 23
constexpr int kSimds = 4;  // SIMDs per compute unit

// Consumer arithmetic of skinny_dma_kernel.  The default is the library's
// product; the other two exist to measure the alternatives the format
// admits (tq4_linear_variant): the rotation undone on the weight tiles
// instead of applied to the activations, and the products on the VALU
// instead of MFMA.
constexpr int kArithDefault = 0;
constexpr int kArithWeightSide = 1;
constexpr int kArithValu = 2;
// element order of decode8_perm's output positions
constexpr int kPermOrder[8] = {0, 2, 4, 6, 1, 3, 5, 7};


template <int ARITH>
__global__ __launch_bounds__(kDmaThreads) void skinny_dma_kernel(SkinnyArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t slots[kDmaMaxChunks * kSlotBytes];
  __shared__ uint32_t ready[kDmaMaxChunks];
  // the VALU-product variant decodes through a table of fp16 level pairs
  __shared__ uint32_t pairs[ARITH == kArithValu ? 256 : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int r = lane % 16;
  const int grp = lane / 16;
  const int kb = g.kb;
  const int k = 32 * kb;
  const int chunks = kb / 4;
  const int n0 = static_cast<int>(blockIdx.x) * kRowsPerWG;

  if (wave >= kDmaConsumers) {
    // ---------------------------------------------------------- producers
    const int p = wave - kDmaConsumers;
    // chunk c into its slot: 4 loads of x (piece q: row q / 16, stored part
    // q % 16 = global part ^ row; rows past m copy row m - 1), then 3 loads
    // of weights (piece q: row q / 5, part q % 5; rows past n copy row n - 1).
    // The copies of other rows only reach outputs that are not stored.
    auto issue = [&](int c) {
      uint8_t *dst = slots + c * kSlotBytes;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int piece = 64 * s + lane;
        const int row = piece >> 4;
        const int part = (piece & 15) ^ row;
        const uint16_t *src = g.x + (row < g.m ? row : g.m - 1) * k + 128 * c + 8 * part;
        __builtin_amdgcn_global_load_lds((const global_void *)src, (lds_void *)(dst + 1024 * s),
                                         16, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int piece = 64 * s + lane;
        const int row = piece / 5;
        const int n = n0 + row < g.n ? n0 + row : g.n - 1;
        const uint8_t *src = g.w + n * kb * 20 + 80 * c + 16 * (piece - 5 * row);
        if (piece < 5 * kRowsPerWG)
          __builtin_amdgcn_global_load_lds((const global_void *)src,
                                           (lds_void *)(dst + kXSliceBytes + 1024 * s), 16, 0, 0);
      }
    };
    const uint32_t flag_addr = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint32_t *)ready));
    // the first chunk goes out before the barrier that publishes the cleared
    // flags and the pair table; then kDmaDepth of this producer's chunks stay
    // in flight: as each lands it is flagged and the chunk kDmaDepth ahead is
    // issued
    if (p < chunks) issue(p);
    __builtin_amdgcn_s_barrier();
    for (int i = 1; i < kDmaDepth; ++i)
      if (p + i * kDmaProducers < chunks) issue(p + i * kDmaProducers);
    for (int c = p; c < chunks; c += kDmaProducers) {
      // loads of chunk c are in once only the later chunks' (7 loads each)
      // are outstanding
      if (kDmaDepth > 2 && c + 2 * kDmaProducers < chunks)
        __builtin_amdgcn_s_waitcnt(0x0F7E);  // vmcnt(14)
      else if (kDmaDepth > 1 && c + kDmaProducers < chunks)
        __builtin_amdgcn_s_waitcnt(0x0F77);  // vmcnt(7)
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      // (written in asm: the compiler cannot tell this flag from the slots
      // still being filled and would wait for every load in flight first)
      asm volatile("ds_write_b32 %0, %1" ::"v"(flag_addr + 4 * c), "v"(1u) : "memory");
      if (c + kDmaDepth * kDmaProducers < chunks) issue(c + kDmaDepth * kDmaProducers);
    }
    __syncthreads();  // all chunks consumed
    __syncthreads();  // partial sums in LDS
    return;
  }

  // ------------------------------------------------------------ consumers
  if (tid < kDmaMaxChunks) ready[tid] = 0u;
  const PermTable pt = make_perm_table(g.cb);
  if constexpr (ARITH == kArithValu) {
    for (int i = tid; i < 256; i += 64 * kDmaConsumers)
      pairs[i] = pack_f16x2(g.cb.c[i & 15], g.cb.c[i >> 4]);
  }
  // rotation operand: lane group g of the rotated block must hold elements
  // 8g + (0, 2, 4, 6, 1, 3, 5, 7), the order decode8_perm yields the levels
  // in, so MFMA row q of the first product stands for element
  // 8 (q / 4) + 2 (q % 4) and of the second for the element after it
  bf16x8 h_lo, h_hi;
  {
    const int j_lo = 8 * (r >> 2) + 2 * (r & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = 8 * grp + i;
      const uint32_t sk = (g.sign_bits >> kk) & 1u;
      const uint32_t n_lo = (__builtin_popcount(j_lo & kk) & 1) ^ sk;
      const uint32_t n_hi = (__builtin_popcount((j_lo + 1) & kk) & 1) ^ sk;
      h_lo[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(kRotEntryBF16 | (n_lo << 15)));
      h_hi[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(kRotEntryBF16 | (n_hi << 15)));
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): flags (and pair table) written
  __builtin_amdgcn_s_barrier();

  const int half = grp >> 1;
  floatx4 acc[kRowTiles];
#pragma unroll
  for (int j = 0; j < kRowTiles; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  float vacc[4][16];  // kArithValu: rows 4 (lane % 8) + i, all 16 tokens
  if constexpr (ARITH == kArithValu) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < 16; ++m) vacc[i][m] = 0.f;
  }
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
  // acquire at workgroup scope: the slot reads after it cannot move above the
  // load that saw the flag set
  auto wait_chunk = [&](int c) {
    while (__hip_atomic_load(&ready[c], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u)
      __builtin_amdgcn_s_sleep(1);
  };
  // Default arithmetic on blocks t0 .. t0 + NT - 1 of chunk c: the blocks'
  // x parts, code words and scales from LDS, the rotation of the x blocks
  // (MFMA), then the register decode and the products.  Nothing here touches
  // global memory.
  auto default_blocks = [&](auto nt, int c, int t0) {
    constexpr int NT = decltype(nt)::value;
    wait_chunk(c);
    const uint8_t *sl = slots + c * kSlotBytes;
    bf16x8 xb[NT];
    uint32_t cw[kRowTiles][NT], sc[kRowTiles][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      xb[t] = __builtin_bit_cast(
          bf16x8,
          *reinterpret_cast<const uint4 *>(sl + 256 * r + 16 * ((4 * (t0 + t) + grp) ^ r)));
#pragma unroll
    for (int j = 0; j < kRowTiles; ++j) {
      const uint8_t *wr = sl + kXSliceBytes + (16 * j + r) * kChunkRowBytes + 20 * t0;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        cw[j][t] = *reinterpret_cast<const uint32_t *>(wr + 20 * t + 4 * grp);
        sc[j][t] = *reinterpret_cast<const uint16_t *>(wr + 20 * t + 16 + 2 * half);
      }
    }
    half8 a[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const floatx4 lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h_lo, xb[t], zero, 0, 0, 0);
      const floatx4 hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h_hi, xb[t], zero, 0, 0, 0);
      a[t] = __builtin_bit_cast(half8, make_uint4(pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3]),
                                                  pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3])));
    }
#pragma unroll
    for (int j = 0; j < kRowTiles; ++j)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const half2v sp = scale_pair(sc[j][t]);
        uint32_t d[4];
        decode8_perm(cw[j][t], pt, d);
        half8 bq;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const half2v q = __builtin_bit_cast(half2v, d[b]) * sp;
          bq[2 * b] = q[0];
          bq[2 * b + 1] = q[1];
        }
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], bq, acc[j], 0, 0, 0);
      }
  };
  if constexpr (ARITH == kArithDefault) {
    // A workgroup's waves go round robin over the SIMDs (measured), so
    // consumers w and w + kSimds share one, and whole chunks dealt round
    // robin give every SIMD the same share.  What the consumers still have to
    // do once the last chunk is in is the kernel's tail, so the last chunks
    // are cut finer: each chunk of the last two full rounds of kSimds
    // chunks is split in halves between the two consumers of one SIMD
    // (measured at K=2688: one round 6.84-6.88 us, two 6.79, three 6.94,
    // every chunk 6.99), and the chunks of a last, partial round (chunks %
    // kSimds of them) by block over consumers 0 .. kSimds - 1, one on each
    // SIMD: their whole chunks land first, so they are the ones done first
    // (measured: the kernel's consumers w >= kSimds finish about 1 us after
    // the others otherwise).
    const int full = chunks - chunks % kSimds;
    const int last = full >= 2 * kSimds ? full - 2 * kSimds : 0;
    for (int c = wave; c < last; c += kDmaConsumers)
      default_blocks(std::integral_constant<int, 4>{}, c, 0);
    for (int c = last + wave % kSimds; c < full; c += kSimds)
      default_blocks(std::integral_constant<int, 2>{}, c, wave < kSimds ? 0 : 2);
    if (wave < kSimds)
      for (int c = full; c < chunks; ++c)
        default_blocks(std::integral_constant<int, 1>{}, c, wave);
  }
  for (int c = wave; ARITH != kArithDefault && c < chunks; c += kDmaConsumers) {
    wait_chunk(c);
    uint8_t *sl = slots + c * kSlotBytes;
    if constexpr (ARITH == kArithWeightSide) {
      // The rotation on the weight side: every decoded block is rotated back
      // (w = s .* H z / sqrt(32)) by a butterfly across the wave (bits 0-2 of
      // the element index in-lane, bits 3 and 4 between lane groups), and
      // the activations enter the products unrotated, as fp16 with the signs
      // s applied (s .* x . H z = x . s .* H z).
      half8 a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4 q = *reinterpret_cast<const uint4 *>(sl + 256 * r + 16 * ((4 * t + grp) ^ r));
        const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int pos = 0; pos < 8; ++pos) {
          const int e = kPermOrder[pos];
          const uint32_t bits = (e & 1) ? (wv[e >> 1] & 0xFFFF0000u) : (wv[e >> 1] << 16);
          const float xv = __uint_as_float(bits ^ (((g.sign_bits >> (8 * grp + e)) & 1u) << 31));
          a[t][pos] = static_cast<_Float16>(xv);
        }
      }
      const float sg3 = (grp & 1) ? -1.f : 1.f;  // lower or upper lane of the bit-3 pairs
      const float sg4 = (grp & 2) ? -1.f : 1.f;  // ... of the bit-4 pairs
#pragma unroll
      for (int j = 0; j < kRowTiles; ++j) {
        const uint8_t *wr = sl + kXSliceBytes + (16 * j + r) * kChunkRowBytes;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t cw = *reinterpret_cast<const uint32_t *>(wr + 20 * t + 4 * grp);
          const uint32_t scb = *reinterpret_cast<const uint16_t *>(wr + 20 * t + 16 + 2 * half);
          // z_hat * 2^3 (a 2^5 smaller shift than the other products: the
          // butterfly's sums grow by up to 32)
          const float sf = __uint_as_float(scb << 16) * 8.0f;
          const half2v s = __builtin_convertvector((float2v){sf, sf}, half2v);
          uint32_t d[4];
          decode8_perm(cw, pt, d);
          float v[8];  // v[e]: element 8 grp + e of the block
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const half2v p = __builtin_bit_cast(half2v, d[b]) * s;
            v[kPermOrder[2 * b]] = static_cast<float>(p[0]);
            v[kPermOrder[2 * b + 1]] = static_cast<float>(p[1]);
          }
#pragma unroll
          for (int hb = 1; hb < 8; hb <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if ((e & hb) == 0) {
                const float lo = v[e], hi = v[e + hb];
                v[e] = lo + hi;
                v[e + hb] = lo - hi;
              }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t lo, hi;
            lane_pair16(__builtin_bit_cast(uint32_t, v[e]), lo, hi);
            v[e] = __builtin_fmaf(__uint_as_float(hi), sg3, __uint_as_float(lo));
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t lo, hi;
            lane_pair32(__builtin_bit_cast(uint32_t, v[e]), lo, hi);
            v[e] = __builtin_fmaf(__uint_as_float(hi), sg4, __uint_as_float(lo));
          }
          half8 bq;
#pragma unroll
          for (int pos = 0; pos < 8; ++pos) bq[pos] = static_cast<_Float16>(v[kPermOrder[pos]]);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], bq, acc[j], 0, 0, 0);
        }
      }
    } else if constexpr (ARITH == kArithValu) {
      // Products on the VALU.  1. Lane m + 16 t rotates block t of token m
      // in fp32 (signs, 32-point butterfly, times 2^-3) and writes the fp16
      // result over the x it read (the same swizzled 16-byte parts).
      {
        const int tm = lane % 16, tb = lane / 16;
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 d = *reinterpret_cast<const uint4 *>(sl + 256 * tm + 16 * ((4 * tb + q) ^ tm));
          const uint32_t wv[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[8 * q + 2 * i] = __uint_as_float(wv[i] << 16);
            v[8 * q + 2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int i = 0; i < 32; ++i)
          v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((g.sign_bits >> i) & 1u) << 31));
#pragma unroll
        for (int hb = 1; hb < 32; hb <<= 1)
#pragma unroll
          for (int i = 0; i < 32; ++i)
            if ((i & hb) == 0) {
              const float lo = v[i], hi = v[i + hb];
              v[i] = lo + hi;
              v[i + hb] = lo - hi;
            }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // this lane's reads are done
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint4 o;
          o.x = pack_f16x2(v[8 * q] * 0.125f, v[8 * q + 1] * 0.125f);
          o.y = pack_f16x2(v[8 * q + 2] * 0.125f, v[8 * q + 3] * 0.125f);
          o.z = pack_f16x2(v[8 * q + 4] * 0.125f, v[8 * q + 5] * 0.125f);
          o.w = pack_f16x2(v[8 * q + 6] * 0.125f, v[8 * q + 7] * 0.125f);
          *reinterpret_cast<uint4 *>(sl + 256 * tm + 16 * ((4 * tb + q) ^ tm)) = o;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the rotated activations are in LDS
      __builtin_amdgcn_wave_barrier();
      // 2. Lane rg + 8 kq: rows 4 rg .. 4 rg + 3, inputs 16 kq .. 16 kq + 15 of
      // the chunk (block kq / 2, half kq % 2); level pairs from the table.
      const int rg = lane % 8, kq = lane / 8;
      const int blk = kq >> 1, hf = kq & 1;
      half2v w[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint8_t *wr = sl + kXSliceBytes + (4 * rg + i) * kChunkRowBytes + 20 * blk;
        const uint2 cwp = *reinterpret_cast<const uint2 *>(wr + 8 * hf);
        const half2v s = scale_pair(*reinterpret_cast<const uint16_t *>(wr + 16 + 2 * hf));
        const uint32_t cws[2] = {cwp.x, cwp.y};
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            w[i][4 * q + b] = __builtin_bit_cast(half2v, pairs[(cws[q] >> (8 * b)) & 0xFFu]) * s;
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const uint4 x0 = *reinterpret_cast<const uint4 *>(sl + 256 * m + 16 * ((2 * kq) ^ m));
        const uint4 x1 = *reinterpret_cast<const uint4 *>(sl + 256 * m + 16 * ((2 * kq + 1) ^ m));
        const uint32_t xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int p = 0; p < 8; ++p)
            vacc[i][m] = __builtin_amdgcn_fdot2(w[i][p], __builtin_bit_cast(half2v, xv[p]),
                                                vacc[i][m], false);
      }
    }
  }

  __syncthreads();  // every chunk consumed; partial sums reuse the slots
  float *red = reinterpret_cast<float *>(slots);
  if constexpr (ARITH == kArithValu) {
    // red[wave][kq][rg * 4 + i][m]: 8 waves x 8 x 32 x 16 floats (128 KB)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < 16; ++m)
        red[(((wave * 8 + lane / 8) * 32) + 4 * (lane % 8) + i) * 16 + m] = vacc[i][m];
    __syncthreads();
    // thread n * 16 + m adds up row n, token m over the waves and lane groups
    const int o = tid;  // 512 outputs, 512 consumer threads
    const int n_l = o / 16, m = o % 16;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kDmaConsumers; ++w)
#pragma unroll
      for (int q = 0; q < 8; ++q) sum += red[(((w * 8 + q) * 32) + n_l) * 16 + m];
    const int n = n0 + n_l;
    if (n < g.n && m < g.m) tail_apply(g.tail, g.y, m, n, g.n, sum * kSkinnyUnscale);
    return;
  }
  // [kDmaConsumers][kRowTiles][4][64]
#pragma unroll
  for (int j = 0; j < kRowTiles; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * kRowTiles + j) * 4 + v) * 64 + lane] = acc[j][v];
  __syncthreads();
  // wave 4 v + j adds up C[4 grp + v][r] of row tile j over the consumers
  if (wave < 4 * kRowTiles) {
    const int j = wave % kRowTiles;
    const int v = wave / kRowTiles;
    float sum = red[(j * 4 + v) * 64 + lane];
#pragma unroll
    for (int w = 1; w < kDmaConsumers; ++w) sum += red[((w * kRowTiles + j) * 4 + v) * 64 + lane];
    const int n = n0 + r + 16 * j;
    const int m = 4 * grp + v;
    // weight-side: sum * 2^-3 / sqrt(32) (the 2^3 shift of its weight operand)
    const float unscale = ARITH == kArithWeightSide ? 0x1.6a09e6p-6f : kSkinnyUnscale;
    if (n < g.n && m < g.m) tail_apply(g.tail, g.y, m, n, g.n, sum * unscale);
  }
}

template <int CH, int XL>
hipError_t launch_cfg(const SkinnyArgs &a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.n + kRowsPerWG - 1) / kRowsPerWG);
  hipLaunchKernelGGL((skinny_kernel<CH, XL>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int CH>
hipError_t launch_ch(const SkinnyArgs &a, int xl, hipStream_t s) {
  switch (xl) {  // loads per lane per x row: ceil(k / 8 / 64)
    case 1: return launch_cfg<CH, 1>(a, s);
    case 2: return launch_cfg<CH, 2>(a, s);
    case 3: return launch_cfg<CH, 3>(a, s);
    case 4: return launch_cfg<CH, 4>(a, s);
    case 5: return launch_cfg<CH, 5>(a, s);
    case 6: return launch_cfg<CH, 6>(a, s);
    case 7: return launch_cfg<CH, 7>(a, s);
    case 8: return launch_cfg<CH, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool skinny_fits(int64_t m, int64_t k, int64_t n);

bool skinny_dma_fits(int64_t m, int64_t k, int64_t n, const void *x, const void *packed) {
  return skinny_fits(m, k, n) && (k / 32) % 4 == 0 && k <= kDmaMaxK &&
         reinterpret_cast<uintptr_t>(packed) % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
}

hipError_t launch_skinny_variant(int arith, const uint16_t *x, int64_t m, int64_t k,
                                 const uint8_t *packed, int64_t n, uint32_t sign_bits, float *y,
                                 hipStream_t s) {
  if (!skinny_dma_fits(m, k, n, x, packed)) return hipErrorInvalidValue;
  SkinnyArgs a{};
  a.x = x;
  a.w = packed;
  a.y = y;
  a.m = static_cast<int32_t>(m);
  a.n = static_cast<int32_t>(n);
  a.kb = static_cast<int32_t>(k / 32);
  a.sign_bits = sign_bits;
  a.cb = codebook();
  const unsigned grid = static_cast<unsigned>((n + kRowsPerWG - 1) / kRowsPerWG);
  switch (arith) {
    case kArithDefault:
      hipLaunchKernelGGL(skinny_dma_kernel<kArithDefault>, dim3(grid), dim3(kDmaThreads), 0, s, a);
      break;
    case kArithWeightSide:
      hipLaunchKernelGGL(skinny_dma_kernel<kArithWeightSide>, dim3(grid), dim3(kDmaThreads), 0, s,
                         a);
      break;
    case kArithValu:
      hipLaunchKernelGGL(skinny_dma_kernel<kArithValu>, dim3(grid), dim3(kDmaThreads), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool skinny_fits(int64_t m, int64_t k, int64_t n) {
  // 32-bit offsets inside the kernel: the packed matrix stays below 2 GiB
  return m >= 1 && m <= 16 && k >= 32 && k <= kMaxK && n >= 1 &&
         n * (k / 32) * 20 < (int64_t{1} << 31);
}

hipError_t launch_skinny(const uint16_t *x, int64_t m, int64_t k, const uint8_t *packed,
                         int64_t n, uint32_t sign_bits, float *y, hipStream_t s,
                         const Tail &tail) {
  SkinnyArgs a{};
  a.x = x;
  a.w = packed;
  a.y = y;
  a.tail = tail;
  a.m = static_cast<int32_t>(m);
  a.n = static_cast<int32_t>(n);
  a.kb = static_cast<int32_t>(k / 32);
  a.sign_bits = sign_bits;
  a.cb = codebook();
  if ((k / 32) % 4 == 0 && k <= kDmaMaxK && reinterpret_cast<uintptr_t>(packed) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(x) % 16 == 0) {
    const unsigned grid = static_cast<unsigned>((n + kRowsPerWG - 1) / kRowsPerWG);
    hipLaunchKernelGGL(skinny_dma_kernel<kArithDefault>, dim3(grid), dim3(kDmaThreads), 0, s, a);
    return hipGetLastError();
  }
  const int64_t chunks = (k / 32 + 3) / 4;                          // <= 32
  const int64_t per_wave = (chunks + kConsumers - 1) / kConsumers;  // <= 4
  const int xl = static_cast<int>((k / 8 + 63) / 64);               // <= 8
  switch (per_wave) {
    case 1: return launch_ch<1>(a, xl, s);
    case 2: return launch_ch<2>(a, xl, s);
    case 3: return launch_ch<3>(a, xl, s);
    case 4: return launch_ch<4>(a, xl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq4
