// Chunked causal prefill over a paged prefix on gfx950's matrix cores.
//
// "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000", What the kernels
// do: the prefill rows of a 4096-token chunk at 26K context, one block of
// 8 tokens x 16 GQA heads per program, FP8 K/V converted on the way in.
// Here a 512-thread workgroup owns 256 query rows of one (sequence, KV head)
// -- row r is new token r / G and query head g*G + r % G, so at G = 16 that
// is 16 tokens x 16 heads -- two 16-row tiles per wave, two waves per SIMD,
// one workgroup per CU.  The 64-key K/V tiles are double-buffered in LDS:
// tile t + 1 is gathered and widened into one buffer while the matrix cores
// read tile t from the other.  Per tile each wave runs, for both its row
// tiles,
//   S^T = K * Q^T   (16x16x32 bf16 MFMA, 4 key subtiles x 6)
//   one online-softmax update (rows live in lanes; keys across lane groups)
//   O^T += V^T P^T  (16x16x32 bf16 MFMA, 2 x 8), V^T from the transposing
//                    LDS read of the row-major V tile.
// Each K or V^T fragment read from LDS feeds the MFMAs of both row tiles:
// on gfx950 LDS read bandwidth, not the matrix cores, bounds a wave that
// reads the whole tile for only 16 rows.  Even so the eight waves read 320 KB
// of fragments from LDS per tile, about as long at the LDS's 128 bytes per
// clock as the matrix products take, so neither unit is ever idle for long
// without the other: the kernel runs at about 60% of both.
// The two waves of a SIMD do not progress alike: the older one wins issue
// ties, runs ahead through its phases and used to wait at the end-of-tile
// barrier for about a fifth of each tile while the younger one finished
// alone.  FP8 tiles are therefore gathered and widened by the four older
// waves only (waves 0-3 pair with 4-7 on the four SIMDs), which takes that
// work off the younger waves' path: 6% off the chunked-prefill workload,
// bit-identical outputs.  (Raising the younger waves' priority instead makes
// both waves move through the same phases together and was 7-16% slower.)
// bf16 tiles have twice the register stage and keep the even split.
// Only tiles that cross a row's causal or window boundary (or hold padding
// rows) are masked; the others skip the compares.  The exp argument folds
// the scale into one FMA on the raw score (the scale is positive), the row
// sums of P come from an extra all-ones matrix-core tile, and a row's
// reference max moves only when a tile's max exceeds it by more than 8 (a
// factor 2^8 in P), so the O rescale is rare.
// The whole key range of a row block runs in one workgroup: no split, no
// merge; row blocks are issued latest-token first (they are the longest).
#pragma once

#include "kv_tile.hpp"
#include "split_attn.hpp"

namespace diffkv {

constexpr int kPfRowTiles = 2;                               // 16-row tiles per wave
constexpr int kPfWaves = kPrefillRows / (16 * kPfRowTiles);  // waves per workgroup
constexpr int kPfThreads = 64 * kPfWaves;
// Register stages of gathered tiles beyond the two LDS buffers: one for
// both formats (two measured the same for FP8 and spill for bf16 beside two
// row tiles' accumulators at two waves per SIMD).
#ifndef DIFFKV_PREFILL_STAGES_FP8
#define DIFFKV_PREFILL_STAGES_FP8 1
#endif
#ifndef DIFFKV_PREFILL_STAGES_BF16
#define DIFFKV_PREFILL_STAGES_BF16 1
#endif

template <bool FP8, bool UPAGE, bool COUNT, int DQK>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void prefill_attn_kernel(const SplitArgs a) {
  constexpr int QC = DQK / 32;               // 32-dim contraction steps of QK^T
  // Threads that gather and widen the tiles: the older half of the waves
  // for FP8, all of them for bf16.
  constexpr int LT = FP8 ? kPfThreads / 2 : kPfThreads;
  using IO = KvTile<FP8, UPAGE, DQK, LT>;
  constexpr int NS = FP8 ? DIFFKV_PREFILL_STAGES_FP8 : DIFFKV_PREFILL_STAGES_BF16;
  constexpr int RT = kPfRowTiles;
  constexpr int LDS_TILE = kKLdsElems<DQK> + kVLdsElems;

  // Two LDS tiles: the next tile is widened into one while the matrix cores
  // read the other, one barrier per tile.
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * LDS_TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform (a scalar), so `loader` branches are scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = LT == kPfThreads || wave < kPfWaves / 2;
  const int col = lane & 15, grp = lane >> 4;
  const int qb = a.n_qtiles - 1 - (int)blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.hkv, g = bg % a.hkv;
  const int G = a.group;

#ifdef DIFFKV_DEBUG
  int L = a.seq_lens[b];
  int n = a.q_lens ? a.q_lens[b] : 1;
  DIFFKV_CHECK_LENGTHS(a, L, n);
#else
  const int L = a.seq_lens[b];
  const int n = a.q_lens ? a.q_lens[b] : 1;
#endif
  if (qb * kPrefillRows >= n * G || n < a.q_lo || n > a.q_hi) return;
  int kv_lo, kv_hi;
  qtile_key_range(L, n, G, qb, kPrefillRows, a.window, kv_lo, kv_hi);
  const int t_begin = kv_lo / kTileKeys;
  const int t_end = (kv_hi + kTileKeys - 1) / kTileKeys;

  // Tiles every row of the block sees whole: no key past the first row's
  // position, none before the last row's window start, no padding rows.
  const int r_first = qb * kPrefillRows;
  const int r_last = min(n * G, r_first + kPrefillRows) - 1;
  const bool has_pad = r_first + kPrefillRows > n * G;
  const int p_first = L - n + r_first / G;
  const int p_last = L - n + r_last / G;
  const int lo_last = a.window > 0 ? max(0, p_last - a.window + 1) : 0;

  const IO io(a.k_cache, a.v_cache, a.block_table + (size_t)b * a.bt_stride, a.hkv, g,
              a.log2_page, kv_lo, kv_hi, t_end, tid, 0, DIFFKV_PAGES(a));
  // NS register stages of gathered tiles; page ids NS tiles ahead of them.
  typename IO::Pages pg[NS];
  typename IO::Stage st[NS];
  if (loader) {
#pragma unroll
    for (int i = 0; i < NS; ++i) io.fetch_pages(t_begin + i, pg[i]);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      io.fetch_data(t_begin + i, pg[i], st[i]);
      io.fetch_pages(t_begin + NS + i, pg[i]);
    }
  }

  const int r0 = seq_row_start(a.q_lens, b);
#ifdef DIFFKV_DEBUG
  if (qb == 0) DIFFKV_CHECK_TOTAL_ROWS(a, b, r0, n);
#endif

  // This lane's query row in each of the wave's row tiles.
  bool row_ok[RT];
  int tok[RT], hh[RT], lo_row[RT], hi_row[RT];
  u32x4 qreg[RT][QC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int R = r_first + (wave * RT + rt) * 16 + col;
    row_ok[rt] = R < n * G && DIFFKV_ROW_IN_RANGE(a, r0 + R / G);
    tok[rt] = row_ok[rt] ? R / G : 0;
    hh[rt] = g * G + (row_ok[rt] ? R % G : 0);
    const int p_row = L - n + tok[rt];
    lo_row[rt] = a.window > 0 ? max(0, p_row - a.window + 1) : 0;
    hi_row[rt] = row_ok[rt] ? p_row : -1;
    const uint16_t* qp = a.q + ((size_t)(r0 + tok[rt]) * a.hq + hh[rt]) * DQK + 8 * grp;
#pragma unroll
    for (int c = 0; c < QC; ++c)
      qreg[rt][c] = *reinterpret_cast<const u32x4*>(
          row_ok[rt] ? reinterpret_cast<const uint8_t*>(qp + 32 * c) : g_zero_row);
  }

  // Tile t lives in LDS buffer t & 1 and, before that, in register stage
  // (t - t_begin) % NS.  Tile t_begin goes to LDS now.
  if (loader) {
    uint16_t* first = lds + (t_begin & 1) * LDS_TILE;
    io.store(st[0], first, first + kKLdsElems<DQK>);
    io.fetch_data(t_begin + NS, pg[0], st[0]);
    io.fetch_pages(t_begin + 2 * NS, pg[0]);
  }
  __syncthreads();

  float m[RT], l[RT];
  f32x4 o[RT][8];
  int cnt[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.f;
    cnt[rt] = 0;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) o[rt][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float scale = a.scale_log2;   // > 0 (checked on the host)

  auto compute_tile = [&](int t, const uint16_t* k_lds, const uint16_t* v_lds) {
    f32x4 sacc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) sacc[rt][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < QC; ++c)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const u32x4 kf =
            *reinterpret_cast<const u32x4*>(k_lds + (sub * 16 + col) * kKLdsStride<DQK> + 8 * grp + 32 * c);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sacc[rt][sub] = mfma_16x16x32(kf, qreg[rt][c], sacc[rt][sub]);
      }

    // sacc[rt][sub][i] = raw score of key t*64 + sub*16 + 4*grp + i for this
    // lane's row of row tile rt.  The mask branch is uniform over the
    // workgroup.
    if (has_pad || t * kTileKeys < lo_last || t * kTileKeys + kTileKeys - 1 > p_first) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = t * kTileKeys + sub * 16 + 4 * grp + i;
            const bool vis = j >= lo_row[rt] && j <= hi_row[rt];
            sacc[rt][sub][i] = vis ? sacc[rt][sub][i] : -INFINITY;
            if constexpr (COUNT) cnt[rt] += vis ? 1 : 0;
          }
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        if constexpr (COUNT) cnt[rt] += 16;
    }
    u32x4 pt[RT][2];
    float alpha[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[rt][sub][i]);
      mx = max_over_lane_groups(mx);
      const float m_new = next_reference(m[rt], mx * scale);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[rt] = fast_exp2(m[rt] - m_use);
      u32x2 pb[4];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(__builtin_fmaf(sacc[rt][sub][i], scale, -m_use));
        pb[sub] = u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
      }
      pt[rt][0] = cat(pb[0], pb[1]);
      pt[rt][1] = cat(pb[2], pb[3]);
      m[rt] = m_new;
      if (__ballot(alpha[rt] != 1.f)) {
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) o[rt][nn] *= alpha[rt];
      }
    }

    // O^T += V^T P^T over 32 keys per step: lane group grp contracts keys
    // 32c + 4grp + 0..3 and 32c + 16 + 4grp + 0..3, the P values it already
    // holds for subtiles 2c and 2c+1, and the matching V^T values come from
    // two transposing reads.  The row sums of this tile's (bf16) P come from
    // the matrix cores too: an all-ones V^T tile gives sum_k P[row][k] in
    // every element, across all four lane groups, with no shuffles.
    // The P*V products and the next tile's widening store run at raised
    // wave priority, QK^T and the softmax at the base level: of the two
    // waves on a SIMD, the one reaching its products or its store issues
    // first.  On the chunked-prefill workload this cut the waves' time spent
    // waiting to issue LDS instructions by a fifth and the kernel's time by
    // 2.4% (bit-identical outputs); MFMA/VALU co-execution stayed the same.
    __builtin_amdgcn_s_setprio(1);
    f32x4 psum[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) psum[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint16_t* vp = v_lds + (32 * c + 4 * grp + (col >> 2)) * kVLdsStride + 4 * (col & 3);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        const u32x4 vf = cat(lds_read_tr16(vp + 16 * nn), lds_read_tr16(vp + 16 * kVLdsStride + 16 * nn));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[rt][nn] = mfma_16x16x32(vf, pt[rt][c], o[rt][nn]);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) psum[rt] = mfma_16x16x32(kOnesBf16x8, pt[rt][c], psum[rt]);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l[rt] = __builtin_fmaf(l[rt], alpha[rt], psum[rt][0]);
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
      if (t < t_end) compute_tile(t, cur, cur + kKLdsElems<DQK>);
      // Widen tile t + 1 into the other buffer (its last readers passed the
      // barrier that ended the previous tile), then start loading t + 1 + NS.
      const int j = (i + 1) % NS;   // a constant once the loop is unrolled
      if (loader) {
        __builtin_amdgcn_s_setprio(1);
        io.store(st[j], nxt, nxt + kKLdsElems<DQK>);
        __builtin_amdgcn_s_setprio(0);
        io.fetch_data(t + 1 + NS, pg[j], st[j]);
        io.fetch_pages(t + 1 + 2 * NS, pg[j]);
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if constexpr (COUNT) {
      int c = cnt[rt];
      c += __shfl_xor(c, 16, 64);
      c += __shfl_xor(c, 32, 64);
      if (row_ok[rt] && grp == 0 && a.count_out)
        atomicAdd(a.count_out + (size_t)(r0 + tok[rt]) * a.hq + hh[rt], c);
    }
    if (!row_ok[rt]) continue;
    const size_t out_row = (size_t)(r0 + tok[rt]) * a.hq + hh[rt];
    float coef;
    if (a.sinks) {
      const float s2 = a.sinks[hh[rt]] * kLog2e;
      const float M2 = fmaxf(m[rt], s2);
      const float al = fast_exp2(m[rt] - M2);
      coef = al / (l[rt] * al + fast_exp2(s2 - M2));
    } else {
      coef = 1.f / l[rt];
    }
    coef *= a.v_scale;
    uint16_t* op = a.out + out_row * kHeadDimV + 4 * grp;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      const f32x4 v = o[rt][nn] * coef;
      *reinterpret_cast<u32x2*>(op + 16 * nn) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
    if (a.lse_out && grp == 0) a.lse_out[out_row] = (m[rt] + log2f(l[rt])) * kLn2;
  }
}

}  // namespace diffkv
