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
#include "moe_route.h"

// Extra workgroups of the first bucketing launch rotate the activation rows
// of the same layer: one thread per 32-block.
__device__ inline void rotate_rows(int64_t group, int tid, const uint16_t *__restrict__ x,
                                   int64_t x_blocks, uint32_t sign_bits,
                                   uint16_t *__restrict__ xt) {
  const int64_t blk = group * kRouteThreads + tid;
  if (blk < x_blocks) rotate_block_bf16(x + blk * 32, sign_bits, xt + blk * 32);
}

// All of the bucketing in one workgroup (workgroup 0).  With logits !=
// nullptr it first routes the pairs / topk tokens itself (one wave per token,
// route_one_token) into ids and gates, which it then reads back.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    int32_t *ids, int64_t pairs, int32_t n_experts, int32_t *counts, int32_t *offsets,
    int32_t *perm, int32_t *inv, MoETile *tiles, int32_t *n_tiles, int32_t tile_rows,
    int32_t *status, const uint16_t *x, int64_t x_blocks, uint32_t sign_bits, uint16_t *xt,
    const float *__restrict__ logits, int32_t topk, float *gates) {
  __shared__ int32_t hist[kRouteWaves][kMaxExperts];
  __shared__ int32_t base[kMaxExperts + 1];
  __shared__ int32_t tile_base[kMaxExperts + 1];

  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    rotate_rows(blockIdx.x - 1, tid, x, x_blocks, sign_bits, xt);
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
  bucket_group<kRouteWaves>(hist, base, tile_base, ids, pairs, n_experts, counts, offsets, perm,
                            inv, tiles, n_tiles, tile_rows, status);
}

// Chunk g of n_chunks: pairs [g * chunk, (g + 1) * chunk), the last chunk
// running to the end (so every chunk holds at least `chunk` pairs).
__device__ inline void chunk_range(int64_t g, int64_t n_chunks, int64_t chunk, int64_t pairs,
                                   int64_t &begin, int64_t &end) {
  begin = g * chunk;
  end = (g + 1 == n_chunks) ? pairs : begin + chunk;
}

// Launch 1 of 3: each workgroup counts one chunk per expert and leaves the
// counts in inv[begin + e]; workgroups past the chunks rotate activations.
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(
    const int32_t *__restrict__ ids, int64_t pairs, int64_t chunk, int64_t n_chunks,
    int32_t n_experts, int32_t *inv, int32_t *status, const uint16_t *x, int64_t x_blocks,
    uint32_t sign_bits, uint16_t *xt) {
  __shared__ int32_t hist[kRouteWaves][kMaxExperts];
  const int tid = threadIdx.x;
  if (blockIdx.x >= n_chunks) {
    rotate_rows(blockIdx.x - n_chunks, tid, x, x_blocks, sign_bits, xt);
    return;
  }
  const int wave = tid / 64;
  const int lane = tid % 64;
  for (int i = tid; i < kRouteWaves * kMaxExperts; i += kRouteThreads) (&hist[0][0])[i] = 0;
  __syncthreads();
  int64_t begin, end, pb, pe;
  chunk_range(blockIdx.x, n_chunks, chunk, pairs, begin, end);
  wave_piece<kRouteWaves>(begin, end, wave, pb, pe);
  const int32_t bad = count_pairs(ids, pb, pe, lane, n_experts, hist[wave]);
  __syncthreads();
  for (int e = tid; e < n_experts; e += kRouteThreads) {
    int32_t c = 0;
    for (int w = 0; w < kRouteWaves; ++w) c += hist[w][e];
    inv[begin + e] = c;
  }
  if (status != nullptr && bad != 0) atomicAdd(status, bad);
}

// Launch 2 of 3, one workgroup: wave w sums the counts of chunks
// [w * per, (w + 1) * per) per expert; the expert totals give counts,
// offsets and the tile list; then each wave walks its chunks again and
// replaces every chunk's count of expert e by the chunk's first slot of e.
__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(
    int32_t *inv, int64_t chunk, int64_t n_chunks, int32_t n_experts, int32_t *counts,
    int32_t *offsets, MoETile *tiles, int32_t *n_tiles, int32_t tile_rows) {
  __shared__ int32_t hist[kRouteWaves][kMaxExperts];
  __shared__ int32_t base[kMaxExperts + 1];
  __shared__ int32_t tile_base[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  int64_t gb, ge;
  wave_piece<kRouteWaves>(0, n_chunks, wave, gb, ge);
  for (int e = lane; e < n_experts; e += 64) {
    int32_t c = 0;
    for (int64_t g = gb; g < ge; ++g) c += inv[g * chunk + e];
    hist[wave][e] = c;
  }
  __syncthreads();
  scan_over_waves<kRouteWaves>(hist, n_experts, tid, base);
  __syncthreads();
  scan_experts<kRouteWaves>(n_experts, tile_rows, tid, base, tile_base, counts, offsets, n_tiles);
  for (int e = lane; e < n_experts; e += 64) {
    int32_t run = base[e] + hist[wave][e];
    for (int64_t g = gb; g < ge; ++g) {
      const int32_t c = inv[g * chunk + e];
      inv[g * chunk + e] = run;
      run += c;
    }
  }
  write_tiles<kRouteWaves>(n_experts, tile_rows, tid, base, tile_base, tiles);
}

// Launch 3 of 3: each workgroup takes its chunk's first slots from
// inv[begin + e], then counts and scatters the chunk like route_kernel.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t *__restrict__ ids, int64_t pairs, int64_t chunk, int64_t n_chunks,
    int32_t n_experts, int32_t *perm, int32_t *inv) {
  __shared__ int32_t hist[kRouteWaves][kMaxExperts];
  __shared__ int32_t base[kMaxExperts];
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  int64_t begin, end, pb, pe;
  chunk_range(blockIdx.x, n_chunks, chunk, pairs, begin, end);
  for (int e = tid; e < n_experts; e += kRouteThreads) base[e] = inv[begin + e];
  for (int i = tid; i < kRouteWaves * kMaxExperts; i += kRouteThreads) (&hist[0][0])[i] = 0;
  // every start slot is read before any pair's slot overwrites inv
  __syncthreads();
  wave_piece<kRouteWaves>(begin, end, wave, pb, pe);
  count_pairs(ids, pb, pe, lane, n_experts, hist[wave]);
  __syncthreads();
  scan_over_waves<kRouteWaves>(hist, n_experts, tid, nullptr);
  __syncthreads();
  scatter_pairs(ids, pb, pe, lane, n_experts, key_bits_for(n_experts), base, hist[wave], perm,
                inv);
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
  for (int64_t tok = blockIdx.y; tok < t; tok += gridDim.y)
    combine_quad(o, inv, topk_w, tok, c, topk, k, out);
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
  if (n_experts < 1 || n_experts > kMaxExperts || pairs < 0) return hipErrorInvalidValue;
  if (logits != nullptr && (gates == nullptr || topk < 1 || pairs % topk != 0))
    return hipErrorInvalidValue;
  const int64_t rot_wgs = x != nullptr ? (x_blocks + kRouteThreads - 1) / kRouteThreads : 0;
  if (logits != nullptr || pairs <= kRouteOneGroupPairs) {
    // the ids are written by the kernel itself when it also routes
    hipLaunchKernelGGL(route_kernel, dim3(static_cast<unsigned>(1 + rot_wgs)),
                       dim3(kRouteThreads), 0, s, const_cast<int32_t *>(ids), pairs, n_experts,
                       counts, offsets, perm, inv, tiles, n_tiles, tile_rows, status, x,
                       x_blocks, sign_bits, xt, logits, topk, gates);
    return hipGetLastError();
  }
  // chunks of at least kRouteChunkMin pairs, at most 1024 of them
  int64_t chunk = kRouteChunkMin;
  while (pairs / chunk > 1024) chunk *= 2;
  const int64_t n_chunks = pairs / chunk;
  hipLaunchKernelGGL(route_count_kernel, dim3(static_cast<unsigned>(n_chunks + rot_wgs)),
                     dim3(kRouteThreads), 0, s, ids, pairs, chunk, n_chunks, n_experts, inv,
                     status, x, x_blocks, sign_bits, xt);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteThreads), 0, s, inv, chunk, n_chunks,
                     n_experts, counts, offsets, tiles, n_tiles, tile_rows);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(static_cast<unsigned>(n_chunks)),
                     dim3(kRouteThreads), 0, s, ids, pairs, chunk, n_chunks, n_experts, perm,
                     inv);
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
