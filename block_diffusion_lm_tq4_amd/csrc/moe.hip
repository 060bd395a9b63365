// MoE routing and combine for the grouped TQ4_1S layer.
//
// Nemotron-TheHobbit-30B-A3B model card: section The model underneath
// (128-expert MoE, top-6) and section Running it ("sync-free MoE"; the stock
// loop synchronized host and device many times per token, section
// Performance & why it's slow).  Everything below stays on the device: the
// bucketing writes the expert counts, offsets, the stable permutation and the
// tile list that the grouped products read, and the host never looks at them.
#include "tq4_internal.h"

namespace tq4 {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxExperts = 512;

// Mask of the lanes (among `active`) whose key equals this lane's key.
__device__ inline uint64_t same_key_lanes(int key, uint64_t active, int key_bits) {
  uint64_t m = active;
  for (int b = 0; b < key_bits; ++b) {
    const uint64_t ones = __ballot((key >> b) & 1);
    m &= ((key >> b) & 1) ? ones : ~ones;
  }
  return m;
}

// The router in front of the layer (model card, The model underneath: 128
// experts, top-6) for one token, by one wave: softmax over all expert logits,
// then the topk largest logits with ties to the lower expert id, each gate the
// expert's softmax probability (not renormalized).  Lane l holds experts
// l, l + 64, ...; the max, the sum and every arg-max are xor-butterfly
// reductions, which leave bit-identical results in all lanes.
constexpr int kRouterPer = kMaxExperts / 64;

__device__ inline void route_one_token(const float *row, int32_t n_experts, int32_t topk,
                                       int lane, int32_t *ids, float *gates) {
  float v[kRouterPer];
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < kRouterPer; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < n_experts ? row[e] : -__builtin_inff();
    mx = fmaxf(mx, v[i]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kRouterPer; ++i)
    if (lane + 64 * i < n_experts) sum += expf(v[i] - mx);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
  uint32_t taken = 0;
  for (int j = 0; j < topk; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kRouterPer; ++i) {
      const int e = lane + 64 * i;
      if (e < n_experts && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d);
      const int oi = __shfl_xor(bi, d);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == bi % 64) taken |= 1u << (bi / 64);
    if (lane == 0) {
      ids[j] = bi;
      gates[j] = expf(bv - mx) / sum;
    }
  }
}

// One workgroup.  Pairs are split into kRouteWaves contiguous ranges, one per
// wave, walked in batches of 64 in pair order:
//   pass 1  per-wave expert histograms (LDS);
//   scan    per expert, over the waves in order, then over the experts;
//   pass 2  each pair's slot = offsets[e] + (pairs of e in earlier waves)
//           + (pairs of e earlier in this wave), the last term from ballots.
// This is a stable counting sort: inside an expert, pairs keep their order.
// With logits != nullptr the workgroup first routes the pairs / topk tokens
// itself (one wave per token, route_one_token) into ids and gates, which the
// bucketing then reads back.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    int32_t *ids, int64_t pairs, int32_t n_experts, int32_t *counts,
    int32_t *offsets, int32_t *perm, int32_t *inv, MoETile *tiles, int32_t *n_tiles,
    int32_t tile_rows, int32_t *status, const uint16_t *__restrict__ x, int64_t x_blocks,
    uint32_t sign_bits, uint16_t *__restrict__ xt, const float *__restrict__ logits,
    int32_t topk, float *gates) {
  __shared__ int32_t hist[kRouteWaves][kMaxExperts];
  __shared__ int32_t base[kMaxExperts + 1];
  __shared__ int32_t tile_base[kMaxExperts + 1];

  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    // the activation rotation of the same layer rides along in this launch
    const int64_t blk = static_cast<int64_t>(blockIdx.x - 1) * kRouteThreads + tid;
    if (blk < x_blocks) rotate_block_bf16(x + blk * 32, sign_bits, xt + blk * 32);
    return;
  }
  const int wave = tid / 64;
  const int lane = tid % 64;
  if (logits != nullptr) {
    for (int64_t tok = wave; tok < pairs / topk; tok += kRouteWaves)
      route_one_token(logits + tok * n_experts, n_experts, topk, lane, ids + tok * topk,
                      gates + tok * topk);
    // the ids are read back only by this workgroup's waves (one compute
    // unit): a workgroup-scope fence and the barrier make them visible
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __syncthreads();
  }
  int key_bits = 0;
  while ((1 << key_bits) < n_experts) ++key_bits;

  for (int i = tid; i < kRouteWaves * kMaxExperts; i += kRouteThreads)
    (&hist[0][0])[i] = 0;
  __syncthreads();

  const int64_t per_wave = (pairs + kRouteWaves - 1) / kRouteWaves;
  const int64_t p_begin = wave * per_wave;
  const int64_t p_end = (p_begin + per_wave < pairs) ? p_begin + per_wave : pairs;

  int32_t bad = 0;
  for (int64_t p0 = p_begin; p0 < p_end; p0 += 64) {
    const int64_t p = p0 + lane;
    const int e = (p < p_end) ? ids[p] : -1;
    const bool valid = (p < p_end) && e >= 0 && e < n_experts;
    if (valid) atomicAdd(&hist[wave][e], 1);
    if (p < p_end && !valid) ++bad;
  }
  __syncthreads();

  // per expert: exclusive scan over waves, total count
  for (int e = tid; e < n_experts; e += kRouteThreads) {
    int32_t run = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      const int32_t c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
    counts[e] = run;
    base[e] = run;
    tile_base[e] = tile_rows > 0 ? (run + tile_rows - 1) / tile_rows : 0;
  }
  __syncthreads();
  // exclusive scans of the counts and tile counts over the experts, by wave
  // 0: lane l sums experts 8l .. 8l + 7, then the lanes' totals are scanned
  if (wave == 0) {
    constexpr int kPer = kMaxExperts / 64;
    int32_t c[kPer], tc[kPer];
    int32_t sum = 0, tsum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = kPer * lane + i;
      c[i] = e < n_experts ? base[e] : 0;
      tc[i] = e < n_experts ? tile_base[e] : 0;
      sum += c[i];
      tsum += tc[i];
    }
    int32_t run = sum, trun = tsum;  // inclusive scan over lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t a = __shfl_up(run, d);
      const int32_t b = __shfl_up(trun, d);
      if (lane >= d) {
        run += a;
        trun += b;
      }
    }
    run -= sum;
    trun -= tsum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = kPer * lane + i;
      if (e < n_experts) {
        base[e] = run;
        tile_base[e] = trun;
        offsets[e] = run;
      }
      run += c[i];
      trun += tc[i];
    }
    if (lane == 63) {
      base[n_experts] = run;
      offsets[n_experts] = run;
      tile_base[n_experts] = trun;
      if (n_tiles != nullptr) *n_tiles = trun;
    }
  }
  __syncthreads();

  for (int64_t p0 = p_begin; p0 < p_end; p0 += 64) {
    const int64_t p = p0 + lane;
    const int e = (p < p_end) ? ids[p] : -1;
    const bool valid = (p < p_end) && e >= 0 && e < n_experts;
    const uint64_t active = __ballot(valid);
    const int key = valid ? e : 0;
    const uint64_t same = same_key_lanes(key, active, key_bits);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (valid) {
      const int rank = __popcll(same & below);
      const int32_t slot = base[e] + hist[wave][e] + rank;
      perm[slot] = static_cast<int32_t>(p);
      inv[p] = slot;
    } else if (p < p_end) {
      inv[p] = -1;
    }
    // the lowest lane of each key group advances the wave's running count
    if (valid && (same & below) == 0) hist[wave][e] += __popcll(same);
  }

  // tile list: expert e owns tiles tile_base[e] .. tile_base[e+1]-1
  for (int e = tid; tiles != nullptr && tile_rows > 0 && e < n_experts; e += kRouteThreads) {
    const int32_t c = base[e + 1] - base[e];
    for (int32_t i = 0; i * tile_rows < c; ++i) {
      MoETile t;
      t.expert = e;
      t.row0 = base[e] + i * tile_rows;
      t.rows = (c - i * tile_rows < tile_rows) ? c - i * tile_rows : tile_rows;
      t.pad = 0;
      tiles[tile_base[e] + i] = t;
    }
  }
  if (status != nullptr && bad != 0) atomicAdd(status, bad);
}

// out[t, :] = sum_j w[t, j] * o[inv[t*topk + j], :] in slot order; each thread
// owns four consecutive features of a token (grid: feature groups x tokens,
// tokens strided by the grid height).
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o,
                                                      const int32_t *__restrict__ inv,
                                                      const float *__restrict__ topk_w,
                                                      int64_t t, int32_t topk, int64_t k,
                                                      float *__restrict__ out) {
  const int64_t q = k / 4;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= q) return;
  for (int64_t tok = blockIdx.y; tok < t; tok += gridDim.y) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < topk; ++j) {
      const int32_t row = inv[tok * topk + j];
      if (row < 0) continue;
      const float gw = topk_w[tok * topk + j];
      const float4 v = reinterpret_cast<const float4 *>(o + static_cast<int64_t>(row) * k)[c];
      acc.x += gw * v.x;
      acc.y += gw * v.y;
      acc.z += gw * v.z;
      acc.w += gw * v.w;
    }
    reinterpret_cast<float4 *>(out + tok * k)[c] = acc;
  }
}

// The router in front of the layer, one wave per token (route_one_token).
__global__ __launch_bounds__(256) void router_kernel(const float *__restrict__ logits, int64_t t,
                                                     int32_t n_experts, int32_t topk,
                                                     int32_t *__restrict__ ids,
                                                     float *__restrict__ gates) {
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (tok >= t) return;
  route_one_token(logits + tok * n_experts, n_experts, topk, threadIdx.x % 64, ids + tok * topk,
                  gates + tok * topk);
}

}  // namespace

hipError_t launch_route(const int32_t *ids, int64_t pairs, int32_t topk, int32_t n_experts,
                        int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                        MoETile *tiles, int32_t *n_tiles, int32_t tile_rows, int32_t *status,
                        hipStream_t s, const uint16_t *x, int64_t x_blocks, uint32_t sign_bits,
                        uint16_t *xt, const float *logits, float *gates) {
  if (n_experts > kMaxExperts) return hipErrorInvalidValue;
  if (logits != nullptr && (gates == nullptr || topk < 1 || pairs % topk != 0))
    return hipErrorInvalidValue;
  const int64_t rot_wgs = x != nullptr ? (x_blocks + kRouteThreads - 1) / kRouteThreads : 0;
  // the ids are written by the kernel itself when it also routes
  hipLaunchKernelGGL(route_kernel, dim3(static_cast<unsigned>(1 + rot_wgs)), dim3(kRouteThreads),
                     0, s, const_cast<int32_t *>(ids), pairs, n_experts, counts, offsets, perm,
                     inv, tiles, n_tiles, tile_rows, status, x, x_blocks, sign_bits, xt, logits,
                     topk, gates);
  return hipGetLastError();
}

hipError_t launch_combine(const float *o, const int32_t *inv, const float *topk_w, int64_t t,
                          int32_t topk, int64_t k, float *out, hipStream_t s) {
  const int64_t q = k / 4;
  if (t == 0 || q == 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((q + threads - 1) / threads),
                                          static_cast<unsigned>(t < 65535 ? t : 65535)),
                     dim3(threads), 0, s, o, inv, topk_w, t, topk, k, out);
  return hipGetLastError();
}

hipError_t launch_router(const float *logits, int64_t t, int32_t n_experts, int32_t topk,
                         int32_t *ids, float *gates, hipStream_t s) {
  if (n_experts > kMaxExperts) return hipErrorInvalidValue;
  if (t == 0) return hipSuccess;
  hipLaunchKernelGGL(router_kernel, dim3(static_cast<unsigned>((t + 3) / 4)), dim3(256), 0, s,
                     logits, t, n_experts, topk, ids, gates);
  return hipGetLastError();
}

}  // namespace tq4
