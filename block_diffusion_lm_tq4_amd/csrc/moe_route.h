// Device routines of the MoE routing shared by the routing kernels (moe.hip)
// and the persistent MoE block kernel (gemm.hip): the router for one token,
// the stable bucketing of token-expert pairs by expert and the weighted
// combine.  Nemotron-TheHobbit-30B-A3B model card: section The model
// underneath (128-expert MoE, top-6) and section Running it ("sync-free
// MoE").  Included inside namespace tq4's anonymous namespace.
#pragma once

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

// Wave-wide reductions without LDS round trips: within each row of 16 lanes
// DPP moves pair lane l with l ^ 1, l ^ 2 (quad permutes), 7 - l (mirror
// within 8) and 15 - l (mirror within 16); then v_permlane16_swap and
// v_permlane32_swap pair the rows.  Each step combines a lane's value with
// its partner's by a commutative rule, so every lane ends with the same
// result, bit for bit.
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <class Combine>
__device__ inline float wave_reduce(float v, Combine f) {
  v = f(v, dpp_f<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = f(v, dpp_f<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = f(v, dpp_f<0x141>(v));  // row_half_mirror
  v = f(v, dpp_f<0x140>(v));  // row_mirror
  uint32_t lo, hi;
  lane_pair16(__builtin_bit_cast(uint32_t, v), lo, hi);
  v = f(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
  lane_pair32(__builtin_bit_cast(uint32_t, v), lo, hi);
  return f(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

// The larger (value, index) pair, ties to the lower index.
__device__ inline void better_pair(float &bv, int &bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

template <int CTRL>
__device__ inline void argmax_step(float &bv, int &bi) {
  const float ov = dpp_f<CTRL>(bv);
  const int oi = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xF, 0xF, false);
  better_pair(bv, bi, ov, oi);
}

__device__ inline void wave_argmax(float &bv, int &bi) {
  argmax_step<0xB1>(bv, bi);
  argmax_step<0x4E>(bv, bi);
  argmax_step<0x141>(bv, bi);
  argmax_step<0x140>(bv, bi);
  uint32_t vlo, vhi, ilo, ihi;
  lane_pair16(__builtin_bit_cast(uint32_t, bv), vlo, vhi);
  lane_pair16(static_cast<uint32_t>(bi), ilo, ihi);
  bv = __builtin_bit_cast(float, vlo);
  bi = static_cast<int>(ilo);
  better_pair(bv, bi, __builtin_bit_cast(float, vhi), static_cast<int>(ihi));
  lane_pair32(__builtin_bit_cast(uint32_t, bv), vlo, vhi);
  lane_pair32(static_cast<uint32_t>(bi), ilo, ihi);
  bv = __builtin_bit_cast(float, vlo);
  bi = static_cast<int>(ilo);
  better_pair(bv, bi, __builtin_bit_cast(float, vhi), static_cast<int>(ihi));
}

// The router in front of the layer (model card, The model underneath: 128
// experts, top-6) for one token, by one wave: softmax over all expert logits,
// then the topk largest logits with ties to the lower expert id, each gate the
// expert's softmax probability (not renormalized).  Lane l holds experts
// l, l + 64, ...; the max, the sum and every arg-max are the wave reductions
// above, which leave bit-identical results in all lanes.
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
  mx = wave_reduce(mx, [](float a, float b) { return fmaxf(a, b); });
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kRouterPer; ++i)
    if (lane + 64 * i < n_experts) sum += expf(v[i] - mx);
  sum = wave_reduce(sum, [](float a, float b) { return a + b; });
  uint32_t taken = 0;
  for (int j = 0; j < topk; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kRouterPer; ++i) {
      const int e = lane + 64 * i;
      if (e < n_experts && !((taken >> i) & 1u)) better_pair(bv, bi, v[i], e);
    }
    wave_argmax(bv, bi);
    if (lane == bi % 64) taken |= 1u << (bi / 64);
    if (lane == 0) {
      ids[j] = bi;
      gates[j] = expf(bv - mx) / sum;
    }
  }
}

// The bucketing is a stable counting sort of the pairs by expert id.  A range
// of pairs is split into one contiguous piece per wave of the workgroup, each
// walked in batches of 64 in pair order:
//   count    per-wave expert histograms (LDS);
//   scan     per expert over the waves in order, then over the experts;
//   scatter  each pair's slot = (start of its expert and piece) + (pairs of
//            the same expert earlier in its batch, from ballots).
// Inside an expert, pairs keep their order.  Up to kRouteOneGroupPairs pairs
// one workgroup does all of it (route_kernel); above, the pairs are cut into
// chunks of at least kRouteChunkMin pairs and three launches count the chunks
// (route_count_kernel), scan the counts (route_scan_kernel, one workgroup)
// and scatter each chunk (route_scatter_kernel).  Between the launches a
// chunk's per-expert counts, then its per-expert start slots, are kept in
// the first n_experts entries of the chunk's own range of inv, which only
// that chunk's scatter overwrites afterwards; so the bucketing needs no
// memory besides its outputs.
constexpr int64_t kRouteChunkMin = 4096;
constexpr int64_t kRouteOneGroupPairs = 2 * kRouteChunkMin - 1;
static_assert(kRouteChunkMin >= kMaxExperts, "a chunk's range of inv holds its counts");

// Adds the expert counts of pairs [p_begin, p_end) into hist_w (LDS) and
// returns the number of this lane's pairs whose id is outside [0, n_experts).
// Batches of 64 ids loaded back to back before any is used, so that a wave
// waits for one memory latency per group rather than per batch.
constexpr int kIdBatches = 4;

__device__ inline void load_ids(const int32_t *ids, int64_t p0, int64_t p_end, int lane,
                                int (&e)[kIdBatches]) {
#pragma unroll
  for (int u = 0; u < kIdBatches; ++u) {
    const int64_t p = p0 + 64 * u + lane;
    e[u] = (p < p_end) ? ids[p] : -1;
  }
}

__device__ inline int32_t count_pairs(const int32_t *ids, int64_t p_begin, int64_t p_end,
                                      int lane, int32_t n_experts, int32_t *hist_w) {
  int32_t bad = 0;
  for (int64_t g0 = p_begin; g0 < p_end; g0 += 64 * kIdBatches) {
    int eb[kIdBatches];
    load_ids(ids, g0, p_end, lane, eb);
#pragma unroll
    for (int u = 0; u < kIdBatches; ++u) {
      const int64_t p = g0 + 64 * u + lane;
      const int e = eb[u];
      const bool valid = (p < p_end) && e >= 0 && e < n_experts;
      if (valid) atomicAdd(&hist_w[e], 1);
      if (p < p_end && !valid) ++bad;
    }
  }
  return bad;
}

// Per expert, hist[w][e] becomes the exclusive prefix over the waves w; the
// total over the waves goes to tot[e] (LDS), when tot is given.
template <int NW>
__device__ inline void scan_over_waves(int32_t (*hist)[kMaxExperts], int32_t n_experts, int tid,
                                       int32_t *tot) {
  for (int e = tid; e < n_experts; e += 64 * NW) {
    int32_t run = 0;
    for (int w = 0; w < NW; ++w) {
      const int32_t c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
    if (tot != nullptr) tot[e] = run;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP moves, with no
// LDS round trips: shifts by 1, 2, 4 and 8 lanes inside each row of 16
// lanes, then the last lane of rows 0 and 2 into rows 1 and 3, and the last
// lane of row 1 into rows 2 and 3.  Lanes whose source lies outside the row
// add 0.
__device__ inline int32_t wave_inclusive_scan(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// From the per-expert totals in base[e]: counts, and (by wave 0) exclusive
// scans of the counts and tile counts over the experts into base, tile_base
// and offsets, with base[E] = offsets[E] = all valid pairs and
// tile_base[E] = *n_tiles = all tiles.  Lane l of wave 0 sums experts
// 8l .. 8l + 7, then the lanes' totals are scanned by shuffles.
template <int NW>
__device__ inline void scan_experts(int32_t n_experts, int32_t tile_rows, int tid, int32_t *base,
                                    int32_t *tile_base, int32_t *counts, int32_t *offsets,
                                    int32_t *n_tiles) {
  for (int e = tid; e < n_experts; e += 64 * NW) {
    const int32_t c = base[e];
    counts[e] = c;
    tile_base[e] = tile_rows > 0 ? (c + tile_rows - 1) / tile_rows : 0;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
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
    int32_t run = wave_inclusive_scan(sum);
    int32_t trun = wave_inclusive_scan(tsum);
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
}

// Slots of pairs [p_begin, p_end): pair p of expert e goes to base[e] +
// hist_w[e] + (pairs of e earlier in its batch of 64); hist_w[e] (this
// wave's start inside the expert, LDS) advances by each batch's count.
__device__ inline void scatter_pairs(const int32_t *ids, int64_t p_begin, int64_t p_end,
                                     int lane, int32_t n_experts, int key_bits,
                                     const int32_t *base, int32_t *hist_w, int32_t *perm,
                                     int32_t *inv) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t g0 = p_begin; g0 < p_end; g0 += 64 * kIdBatches) {
    int eb[kIdBatches];
    load_ids(ids, g0, p_end, lane, eb);
#pragma unroll
    for (int u = 0; u < kIdBatches; ++u) {
      const int64_t p = g0 + 64 * u + lane;
      const int e = eb[u];
      const bool valid = (p < p_end) && e >= 0 && e < n_experts;
      const uint64_t active = __ballot(valid);
      const int key = valid ? e : 0;
      const uint64_t same = same_key_lanes(key, active, key_bits);
      if (valid) {
        const int rank = __popcll(same & below);
        const int32_t slot = base[e] + hist_w[e] + rank;
        perm[slot] = static_cast<int32_t>(p);
        inv[p] = slot;
      } else if (p < p_end) {
        inv[p] = -1;
      }
      // the lowest lane of each key group advances the wave's running count
      if (valid && (same & below) == 0) hist_w[e] += __popcll(same);
    }
  }
}

// Tile list: expert e owns tiles tile_base[e] .. tile_base[e+1]-1, each of
// tile_rows bucket rows but the last.
template <int NW>
__device__ inline void write_tiles(int32_t n_experts, int32_t tile_rows, int tid,
                                   const int32_t *base, const int32_t *tile_base,
                                   MoETile *tiles) {
  for (int e = tid; tiles != nullptr && tile_rows > 0 && e < n_experts; e += 64 * NW) {
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
}

__device__ inline int key_bits_for(int32_t n_experts) {
  int b = 0;
  while ((1 << b) < n_experts) ++b;
  return b;
}

// Piece of wave `wave` when [begin, end) is split into NW.
template <int NW>
__device__ inline void wave_piece(int64_t begin, int64_t end, int wave, int64_t &pb,
                                  int64_t &pe) {
  const int64_t per = (end - begin + NW - 1) / NW;
  pb = begin + wave * per;
  if (pb > end) pb = end;
  pe = (pb + per < end) ? pb + per : end;
}

// The whole bucketing of pairs [0, pairs) by one workgroup of NW waves
// (every thread calls it): per-wave histograms, the scans, the stable
// scatter and the tile list.  hist, base and tile_base are the caller's LDS.
template <int NW>
__device__ inline void bucket_group(int32_t (*hist)[kMaxExperts], int32_t *base,
                                    int32_t *tile_base, const int32_t *ids, int64_t pairs,
                                    int32_t n_experts, int32_t *counts, int32_t *offsets,
                                    int32_t *perm, int32_t *inv, MoETile *tiles,
                                    int32_t *n_tiles, int32_t tile_rows, int32_t *status) {
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  for (int i = tid; i < NW * kMaxExperts; i += 64 * NW) (&hist[0][0])[i] = 0;
  __syncthreads();
  int64_t pb, pe;
  wave_piece<NW>(0, pairs, wave, pb, pe);
  const int32_t bad = count_pairs(ids, pb, pe, lane, n_experts, hist[wave]);
  __syncthreads();
  scan_over_waves<NW>(hist, n_experts, tid, base);
  __syncthreads();
  scan_experts<NW>(n_experts, tile_rows, tid, base, tile_base, counts, offsets, n_tiles);
  scatter_pairs(ids, pb, pe, lane, n_experts, key_bits_for(n_experts), base, hist[wave], perm,
                inv);
  write_tiles<NW>(n_experts, tile_rows, tid, base, tile_base, tiles);
  if (status != nullptr && bad != 0) atomicAdd(status, bad);
}

// Four consecutive outputs (features 4c .. 4c + 3) of token tok of the
// weighted combine: the token's slots in slot order, each its expert's row
// of o times the gate (slots that were not routed are skipped).
__device__ inline void combine_quad(const float *__restrict__ o, const int32_t *__restrict__ inv,
                                    const float *__restrict__ topk_w, int64_t tok, int64_t c,
                                    int32_t topk, int64_t k, float *__restrict__ out) {
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
