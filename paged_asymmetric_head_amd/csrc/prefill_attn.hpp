// Chunked causal prefill over a paged prefix on gfx950's matrix cores.
//
// "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000", What the kernels
// do: the prefill rows of a 4096-token chunk at 26K context, one block of
// 8 tokens x 16 GQA heads per program, FP8 K/V converted on the way in.
// Here a 512-thread workgroup owns 128 query rows of one (sequence, KV head)
// -- row r is new token r / G and query head g*G + r % G, so at G = 16 that
// is 8 tokens x 16 heads -- one 16-row tile per wave, two waves per SIMD, one
// workgroup per CU.  The 64-key K/V tiles are double-buffered in LDS: tile
// t + 1 is gathered and widened into one buffer while the matrix cores read
// tile t from the other.  Per tile each wave runs
//   S^T = K * Q^T   (16x16x32 bf16 MFMA, 4 key subtiles x 6)
//   one online-softmax update (rows live in lanes; keys across lane groups)
//   O^T += V^T P^T  (16x16x32 bf16 MFMA, 2 x 8), V^T from the transposing
//                    LDS read of the row-major V tile.
// Only tiles that cross a row's causal or window boundary (or hold padding
// rows) are masked; the others skip the compares.  The exp argument folds
// the scale into one FMA on the raw score (the scale is positive), the row
// sums of P come from an extra all-ones matrix-core tile, and the O rescale
// is skipped when no row's running max moved.
// The whole key range of a row block runs in one workgroup: no split, no
// merge; row blocks are issued latest-token first (they are the longest).
#pragma once

#include <type_traits>

#include "kv_tile.hpp"
#include "split_attn.hpp"

namespace diffkv {

constexpr int kPfRows = kPrefillRows;   // query rows per prefill workgroup
constexpr int kPfWaves = kPfRows / 16;   // one 16-row tile per wave
constexpr int kPfThreads = 64 * kPfWaves;
#ifndef DIFFKV_PREFILL_STAGES
#define DIFFKV_PREFILL_STAGES 2
#endif

template <bool FP8, bool UPAGE, bool COUNT>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void prefill_attn_kernel(const SplitArgs a) {
  using IO = KvTile<FP8, UPAGE, kPfThreads>;
  constexpr int NS = DIFFKV_PREFILL_STAGES;
  constexpr int LDS_TILE = kKLdsElems + kVLdsElems;

  // Two LDS tiles: the next tile is widened into one while the matrix cores
  // read the other, one barrier per tile.
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * LDS_TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int qb = a.n_qtiles - 1 - (int)blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.hkv, g = bg % a.hkv;
  const int G = a.group;

  const int L = a.seq_lens[b];
  const int n = a.q_lens ? a.q_lens[b] : 1;
  if (qb * kPfRows >= n * G) return;
  int kv_lo, kv_hi;
  qtile_key_range(L, n, G, qb, kPfRows, a.window, kv_lo, kv_hi);
  const int t_begin = kv_lo / kTileKeys;
  const int t_end = (kv_hi + kTileKeys - 1) / kTileKeys;

  // Tiles every row of the block sees whole: no key past the first row's
  // position, none before the last row's window start, no padding rows.
  const int r_first = qb * kPfRows;
  const int r_last = min(n * G, r_first + kPfRows) - 1;
  const bool has_pad = r_first + kPfRows > n * G;
  const int p_first = L - n + r_first / G;
  const int p_last = L - n + r_last / G;
  const int lo_last = a.window > 0 ? max(0, p_last - a.window + 1) : 0;

  const IO io(a.k_cache, a.v_cache, a.block_table + (size_t)b * a.bt_stride, a.hkv, g,
              a.log2_page, kv_lo, kv_hi, t_end, tid);
  // NS register stages of gathered tiles; page ids NS tiles ahead of them.
  typename IO::Pages pg[NS];
  typename IO::Stage st[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) io.fetch_pages(t_begin + i, pg[i]);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    io.fetch_data(t_begin + i, pg[i], st[i]);
    io.fetch_pages(t_begin + NS + i, pg[i]);
  }

  const int r0 = seq_row_start(a.q_lens, b);

  // This lane's query row.
  const int R = r_first + wave * 16 + col;
  const bool row_ok = R < n * G;
  const int tok = row_ok ? R / G : 0;
  const int hh = g * G + (row_ok ? R % G : 0);
  const int p_row = L - n + tok;
  const int lo_row = a.window > 0 ? max(0, p_row - a.window + 1) : 0;
  const int hi_row = row_ok ? p_row : -1;
  u32x4 qreg[6];
  {
    const uint16_t* qp = a.q + ((size_t)(r0 + tok) * a.hq + hh) * kHeadDimQK + 8 * grp;
#pragma unroll
    for (int c = 0; c < 6; ++c)
      qreg[c] = *reinterpret_cast<const u32x4*>(row_ok ? reinterpret_cast<const uint8_t*>(qp + 32 * c)
                                                       : g_zero_row);
  }

  // Tile t lives in LDS buffer t & 1 and, before that, in register stage
  // (t - t_begin) % NS.  Tile t_begin goes to LDS now.
  {
    uint16_t* first = lds + (t_begin & 1) * LDS_TILE;
    io.store(st[0], first, first + kKLdsElems);
  }
  io.fetch_data(t_begin + NS, pg[0], st[0]);
  io.fetch_pages(t_begin + 2 * NS, pg[0]);
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) o[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  int cnt = 0;
  const float scale = a.scale_log2;   // > 0 (checked on the host)

  auto compute_tile = [&](int t, const uint16_t* k_lds, const uint16_t* v_lds, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    f32x4 sacc[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) sacc[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 6; ++c)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
        sacc[sub] = mfma_16x16x32(
            *reinterpret_cast<const u32x4*>(k_lds + (sub * 16 + col) * kKLdsStride + 8 * grp + 32 * c),
            qreg[c], sacc[sub]);

    // sacc[sub][i] = raw score of key t*64 + sub*16 + 4*grp + i, row col.
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[sub][i];
        if constexpr (MASKED) {
          const int j = t * kTileKeys + sub * 16 + 4 * grp + i;
          const bool vis = j >= lo_row && j <= hi_row;
          x = vis ? x : -INFINITY;
          sacc[sub][i] = x;
          if constexpr (COUNT) cnt += vis ? 1 : 0;
        } else {
          if constexpr (COUNT) cnt += 1;
        }
        mx = fmaxf(mx, x);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m, mx * scale);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    u32x2 pb[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(__builtin_fmaf(sacc[sub][i], scale, -m_use));
      pb[sub] = u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
    }
    m = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) o[nn] *= alpha;
    }

    // O^T += V^T P^T over 32 keys per step: lane group grp contracts keys
    // 32c + 4grp + 0..3 and 32c + 16 + 4grp + 0..3, the P values it already
    // holds for subtiles 2c and 2c+1, and the matching V^T values come from
    // two transposing reads.  The row sums of this tile's (bf16) P come from
    // the matrix cores too: an all-ones V^T tile gives sum_k P[row][k] in
    // every element, across all four lane groups, with no shuffles.
    f32x4 psum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const u32x4 pt = cat(pb[2 * c], pb[2 * c + 1]);
      const uint16_t* vp = v_lds + (32 * c + 4 * grp + (col >> 2)) * kVLdsStride + 4 * (col & 3);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn)
        o[nn] = mfma_16x16x32(cat(lds_read_tr16(vp + 16 * nn), lds_read_tr16(vp + 16 * kVLdsStride + 16 * nn)),
                              pt, o[nn]);
      psum = mfma_16x16x32(kOnesBf16x8, pt, psum);
    }
    l = __builtin_fmaf(l, alpha, psum[0]);
  };

  // Every stage step runs in every round so the loads keep one fixed order
  // (the compiler then waits for exactly the stage it needs); only the math
  // of tiles past the end is skipped.
  for (int t0 = t_begin; t0 < t_end; t0 += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int t = t0 + i;
      uint16_t* cur = lds + (t & 1) * LDS_TILE;
      uint16_t* nxt = lds + ((t + 1) & 1) * LDS_TILE;
      if (t < t_end) {
        const bool whole = !has_pad && t * kTileKeys >= lo_last && t * kTileKeys + kTileKeys - 1 <= p_first;
        if (whole) compute_tile(t, cur, cur + kKLdsElems, std::false_type{});
        else compute_tile(t, cur, cur + kKLdsElems, std::true_type{});
      }
      // Widen tile t + 1 into the other buffer (its last readers passed the
      // barrier that ended the previous tile), then start loading t + 1 + NS.
      const int j = (i + 1) % NS;   // a constant once the loop is unrolled
      io.store(st[j], nxt, nxt + kKLdsElems);
      io.fetch_data(t + 1 + NS, pg[j], st[j]);
      io.fetch_pages(t + 1 + 2 * NS, pg[j]);
      __syncthreads();
    }
  }

  if constexpr (COUNT) {
    cnt += __shfl_xor(cnt, 16, 64);
    cnt += __shfl_xor(cnt, 32, 64);
    if (row_ok && grp == 0 && a.count_out)
      atomicAdd(a.count_out + (size_t)(r0 + tok) * a.hq + hh, cnt);
  }
  if (!row_ok) return;
  const size_t out_row = (size_t)(r0 + tok) * a.hq + hh;
  float coef;
  if (a.sinks) {
    const float s2 = a.sinks[hh] * kLog2e;
    const float M2 = fmaxf(m, s2);
    const float al = fast_exp2(m - M2);
    coef = al / (l * al + fast_exp2(s2 - M2));
  } else {
    coef = 1.f / l;
  }
  coef *= a.v_scale;
  uint16_t* op = a.out + out_row * kHeadDimV + 4 * grp;
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) {
    const f32x4 v = o[nn] * coef;
    *reinterpret_cast<u32x2*>(op + 16 * nn) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
  if (a.lse_out && grp == 0) a.lse_out[out_row] = (m + log2f(l)) * kLn2;
}

}  // namespace diffkv
