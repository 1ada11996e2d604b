// Chunked causal prefill over a paged prefix on gfx950's matrix cores.
//
// "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000", What the kernels
// do: the prefill rows of a 4096-token chunk at 26K context, one block of
// 8 tokens x 16 GQA heads per program, FP8 K/V converted on the way in.
// Here a 256-thread workgroup owns 128 query rows of one (sequence, KV head)
// -- row r is new token r / G and query head g*G + r % G, so at G = 16 that
// is 8 tokens x 16 heads -- and each wave owns two 16-row tiles, so every K
// or V operand read from LDS feeds two matrix-core products.  Per 64-key
// tile each wave runs
//   S^T = K * Q^T   (16x16x32 bf16 MFMA, 4 key subtiles x 2 row tiles x 6)
//   one online-softmax update (rows live in lanes; keys across lane groups)
//   O^T += V^T P^T  (16x16x16 bf16 MFMA, 4 x 8 x 2), V^T from the
//                    transposing LDS read of the row-major V tile.
// Only tiles that cross a row's causal or window boundary (or hold padding
// rows) are masked; the others skip the compares.  The exp argument folds
// the scale into one FMA on the raw score (the scale is positive), and the
// O rescale is skipped when no row's running max moved.
// The whole key range of a row block runs in one workgroup: no split, no
// merge; row blocks are issued latest-token first (they are the longest).
#pragma once

#include <type_traits>

#include "kv_tile.hpp"
#include "split_attn.hpp"

namespace diffkv {

constexpr int kPfRows = kPrefillRows;          // query rows per prefill workgroup
constexpr int kPfRowTiles = kPrefillRows / 64;  // 16-row tiles per wave (4 waves)
#ifndef DIFFKV_PREFILL_STAGES
#define DIFFKV_PREFILL_STAGES 2
#endif
#ifndef DIFFKV_PREFILL_WAVES_PER_EU
#define DIFFKV_PREFILL_WAVES_PER_EU 2
#endif

template <bool FP8, bool UPAGE, bool COUNT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DIFFKV_PREFILL_WAVES_PER_EU, 8)))
void prefill_attn_kernel(const SplitArgs a) {
  constexpr int RTW = kPfRowTiles;
  constexpr int NS = DIFFKV_PREFILL_STAGES;
  using IO = KvTile<FP8, UPAGE>;

  __shared__ __attribute__((aligned(16))) uint16_t lds[kKLdsElems + kVLdsElems];
  uint16_t* k_lds = lds;
  uint16_t* v_lds = lds + kKLdsElems;

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

  // This lane's query rows, one per row tile.
  bool row_ok[RTW];
  int tok[RTW], hh[RTW], lo_row[RTW], hi_row[RTW];
  u32x4 qreg[RTW][6];
#pragma unroll
  for (int rr = 0; rr < RTW; ++rr) {
    const int R = r_first + (wave * RTW + rr) * 16 + col;
    row_ok[rr] = R < n * G;
    tok[rr] = row_ok[rr] ? R / G : 0;
    hh[rr] = g * G + (row_ok[rr] ? R % G : 0);
    const int p = L - n + tok[rr];
    lo_row[rr] = a.window > 0 ? max(0, p - a.window + 1) : 0;
    hi_row[rr] = row_ok[rr] ? p : -1;
    const uint16_t* qp = a.q + ((size_t)(r0 + tok[rr]) * a.hq + hh[rr]) * kHeadDimQK + 8 * grp;
#pragma unroll
    for (int c = 0; c < 6; ++c)
      qreg[rr][c] = *reinterpret_cast<const u32x4*>(
          row_ok[rr] ? reinterpret_cast<const uint8_t*>(qp + 32 * c) : g_zero_row);
  }

  float m[RTW], l[RTW];
  f32x4 o[RTW][8];
  int cnt[RTW];
#pragma unroll
  for (int rr = 0; rr < RTW; ++rr) {
    m[rr] = -INFINITY;
    l[rr] = 0.f;
    cnt[rr] = 0;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) o[rr][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float scale = a.scale_log2;   // > 0 (checked on the host)

  auto compute_tile = [&](int t, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    f32x4 sacc[RTW][4];
#pragma unroll
    for (int rr = 0; rr < RTW; ++rr)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) sacc[rr][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 6; ++c)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const u32x4 kop = *reinterpret_cast<const u32x4*>(k_lds + (sub * 16 + col) * kKLdsStride + 8 * grp + 32 * c);
#pragma unroll
        for (int rr = 0; rr < RTW; ++rr) sacc[rr][sub] = mfma_16x16x32(kop, qreg[rr][c], sacc[rr][sub]);
      }

    u32x2 pb[RTW][4];
#pragma unroll
    for (int rr = 0; rr < RTW; ++rr) {
      // sacc[rr][sub][i] = raw score of key t*64 + sub*16 + 4*grp + i, row col.
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = sacc[rr][sub][i];
          if constexpr (MASKED) {
            const int j = t * kTileKeys + sub * 16 + 4 * grp + i;
            const bool vis = j >= lo_row[rr] && j <= hi_row[rr];
            x = vis ? x : -INFINITY;
            sacc[rr][sub][i] = x;
            if constexpr (COUNT) cnt[rr] += vis ? 1 : 0;
          } else {
            if constexpr (COUNT) cnt[rr] += 1;
          }
          mx = fmaxf(mx, x);
        }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m[rr], mx * scale);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m[rr] - m_use);
      float ps = 0.f;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = fast_exp2(__builtin_fmaf(sacc[rr][sub][i], scale, -m_use));
          ps += pr[i];
        }
        pb[rr][sub] = u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l[rr] = l[rr] * alpha + ps;
      m[rr] = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) o[rr][nn] *= alpha;
      }
    }

#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const uint16_t* vp = v_lds + (sub * 16 + 4 * grp + (col >> 2)) * kVLdsStride + 4 * (col & 3);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        const u32x2 vop = lds_read_tr16(vp + 16 * nn);
#pragma unroll
        for (int rr = 0; rr < RTW; ++rr) o[rr][nn] = mfma_16x16x16(vop, pb[rr][sub], o[rr][nn]);
      }
    }
  };

  for (int t = t_begin; t < t_end; t += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __syncthreads();
      io.store(st[i], k_lds, v_lds);
      __syncthreads();
      io.fetch_data(t + i + NS, pg[i], st[i]);
      io.fetch_pages(t + i + 2 * NS, pg[i]);
      const int tt = t + i;
      if (tt < t_end) {
        const bool whole = !has_pad && tt * kTileKeys >= lo_last && tt * kTileKeys + kTileKeys - 1 <= p_first;
        if (whole) compute_tile(tt, std::false_type{});
        else compute_tile(tt, std::true_type{});
      }
    }
  }

#pragma unroll
  for (int rr = 0; rr < RTW; ++rr) {
    if constexpr (COUNT) {
      int c = cnt[rr];
      c += __shfl_xor(c, 16, 64);
      c += __shfl_xor(c, 32, 64);
      if (row_ok[rr] && grp == 0 && a.count_out)
        atomicAdd(a.count_out + (size_t)(r0 + tok[rr]) * a.hq + hh[rr], c);
    }
    if (!row_ok[rr]) continue;
    const size_t out_row = (size_t)(r0 + tok[rr]) * a.hq + hh[rr];
    float coef;
    if (a.sinks) {
      const float s2 = a.sinks[hh[rr]] * kLog2e;
      const float M2 = fmaxf(m[rr], s2);
      const float al = fast_exp2(m[rr] - M2);
      coef = al / (l[rr] * al + fast_exp2(s2 - M2));
    } else {
      coef = 1.f / l[rr];
    }
    coef *= a.v_scale;
    uint16_t* op = a.out + out_row * kHeadDimV + 4 * grp;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      const f32x4 v = o[rr][nn] * coef;
      *reinterpret_cast<u32x2*>(op + 16 * nn) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
    if (a.lse_out && grp == 0) a.lse_out[out_row] = (m[rr] + log2f(l[rr])) * kLn2;
  }
}

}  // namespace diffkv
