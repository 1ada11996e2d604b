// Split-KV paged attention for decode and speculative verify on gfx950, plus
// the log-sum-exp merge of the split partials.  K rows are DQK wide (192, or
// 128 for symmetric heads), V rows 128.
//
// Work decomposition ("diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000",
// What the kernels do: without split-KV a multi-token verify ran on a handful
// of workgroups; split-KV fixed that): one workgroup per (key split, query
// tile, sequence * KV head).  A query tile is up to 64 rows; row r of a
// (sequence, KV head) is new token r / G and query head g*G + r % G, so a
// whole verify block of all G heads shares one pass over the keys (one
// program per whole verify, same page).
//
// Per 64-key tile the workgroup gathers K (192 wide) and V (128 wide) rows
// through the block table with 16-byte loads and writes them row-major into
// LDS as bf16 (FP8 E4M3 widened on the way).  Each wave owns one 16-row
// query tile and a quarter, half or all of the 64 keys (4, 2 or 1 row tiles
// per workgroup) and runs
//   S^T = K * Q^T        (v_mfma_f32_16x16x32_bf16, 6 steps over 192 dims)
//   mask -> online softmax in base 2 (rows live in lanes, keys across the
//           4 lane groups: a row max is two lane-row swaps on the VALU)
//   O^T += V^T * P^T     (v_mfma_f32_16x16x32_bf16 when a wave holds 32 or
//                         more keys of the tile, else 16x16x16; 8 tiles over
//                         the 128 dims; V^T comes from transposing LDS reads
//                         of the row-major V tile)
// Keeping S and O transposed puts one query row in each lane, so the softmax
// rescale needs no data movement between lanes.
// The global loads of the next NS tiles are in flight in registers while a
// tile is converted into LDS and multiplied.  A one-chunk launch whose pairs
// span at most four tiles (sliding windows, short sequences) takes the
// short-range pass instead: all of a pair's loads at once, K straight into
// the MFMA operands, one softmax update.
#pragma once

#include <type_traits>

#include "kv_tile.hpp"

namespace diffkv {

struct SplitArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* q_lens;
  const float* sinks;
  uint16_t* part_o;     // fp16 partial rows [.., 128]: normalised row * 2^-e
  f32x2* part_lse;      // per partial row: base-2 log-sum-exp, exponent e
  i32x2* pair_chunks;   // per (sequence, query tile): first chunk id, chunk count
  uint16_t* out;
  float* lse_out;
  int32_t* count_out;
  int batch, hq, hkv, group, log2_page, bt_stride, window;
  int n_qtiles;       // query tiles per (sequence, KV head) the launch covers
  int slots;          // balanced plan: target chunks per KV head (one resident round)
  int force_splits;   // > 0: every (sequence, query tile) takes exactly this many chunks
  int chunk_bound;    // chunk ids stay below this (the workspace holds that many)
  // Context partials: keys outside [key_lo[b], key_hi[b]) stay invisible
  // (NULL: no bound), and with part_out set the rows are written as fp32
  // normalised outputs (0 for a row that sees no key) with their natural
  // log-sum-exp in lse_out (-inf there); the sink is not applied.
  const int32_t* key_lo;
  const int32_t* key_hi;
  float* part_out;
  int q_lo, q_hi;     // this launch takes the sequences with q_lo <= q_len <= q_hi
  float scale_log2;   // softmax_scale * k_scale * log2(e)
  float v_scale;      // v_scale for FP8 caches, 1 for bf16
#ifdef DIFFKV_DEBUG
  int max_seq_len, max_q_len, total_q, num_pages;   // the descriptor's bounds
#endif
};

// Debug builds (-DDIFFKV_DEBUG) check a sequence's lengths against the
// descriptor's bounds and make them safe (seq_len clamped to [0,
// max_seq_len], q_len to at most seq_len, so no position is negative and no
// block-table index passes the row), drop packed rows outside [0, total_q),
// let the last sequence's workgroup check that the rows add up to total_q,
// and bound block-table entries by the page count.  In release builds the
// macros below expand to nothing (or to true), so the kernels are the same
// code as without them.
#ifdef DIFFKV_DEBUG
__device__ __forceinline__ void check_lengths(const SplitArgs& a, int& L, int& n) {
  uint32_t bad = 0;
  if (L < 0 || L > a.max_seq_len) {
    bad |= kDbgSeqLen;
    L = min(max(L, 0), a.max_seq_len);
  }
  if (n < 1 || n > L || n > a.max_q_len) bad |= kDbgQLen;
  if (n > L) n = L;
  if (bad) debug_flag(bad);
}
__device__ __forceinline__ bool row_in_range(const SplitArgs& a, int row) {
  if ((unsigned)row < (unsigned)a.total_q) return true;
  debug_flag(kDbgRows);
  return false;
}
__device__ __forceinline__ void check_total_rows(const SplitArgs& a, int b, int r0, int n) {
  if (b == a.batch - 1 && threadIdx.x == 0 && r0 + n != a.total_q) debug_flag(kDbgRows);
}
#define DIFFKV_CHECK_LENGTHS(a, L, n) check_lengths(a, L, n)
#define DIFFKV_ROW_IN_RANGE(a, row) row_in_range(a, row)
#define DIFFKV_CHECK_TOTAL_ROWS(a, b, r0, n) check_total_rows(a, b, r0, n)
#define DIFFKV_PAGES(a) (a).num_pages
#else
#define DIFFKV_CHECK_LENGTHS(a, L, n) ((void)0)
#define DIFFKV_ROW_IN_RANGE(a, row) true
#define DIFFKV_CHECK_TOTAL_ROWS(a, b, r0, n) ((void)0)
#define DIFFKV_PAGES(a) 1
#endif

// Tiles of chunk s among S equal shares of the aligned tile range.
__device__ __forceinline__ void split_tiles(int kv_lo, int kv_hi, int S, int s, int& t_begin,
                                            int& t_end) {
  const int t0 = kv_lo / kTileKeys;
  const int t1 = (kv_hi + kTileKeys - 1) / kTileKeys;
  const int tps = (t1 - t0 + S - 1) / S;
  t_begin = t0 + s * tps;
  t_end = min(t1, t_begin + tps);
}

// Balanced split plan.  The keys a (sequence, query tile) pair sees span
// nt 64-key tiles; over the pairs of the launch (sequences with q_lo <=
// q_len <= q_hi) they total T.  With C = max(kMinTilesPerSplit, ceil(T /
// slots)), lengthened while the chunks would not fit one resident round of
// slots, a pair is cut into k = ceil(nt / C) chunks of equal tile counts
// (force_splits fixes k instead), and chunk ids number the chunks pair by
// pair in (sequence, query tile) order.  Every split workgroup derives the
// same plan from seq_lens and q_lens (the first chunk of each pair records
// its chunk range for the merge), so which workgroup sums which keys
// depends on the lengths alone (results repeat bit for bit) while the
// launch shape depends on host bounds alone.  Long
// and short sequences in one batch get chunks of about the same length,
// where equal shares per sequence would leave the longest one as the tail.
// Each wave computes the plan for itself (no LDS, no barrier).
template <int ROWS>
struct SplitPlanner {
  const SplitArgs& a;
  const FastDiv& G;     // the GQA group
  int C = 0;            // tiles per chunk; 0 with forced splits
  FastDiv Cd{1};        // division by C (set with C)
  int L0 = 0, n0 = 0;   // this lane's sequence (b = lane) of the first pass
  int lo0 = 0, hi0 = 0; // its key bounds

  __device__ __forceinline__ SplitPlanner(const SplitArgs& args, const FastDiv& group) : a(args), G(group) {}
  __device__ __forceinline__ void set_chunk(int c) {
    C = c;
    Cd = FastDiv((uint32_t)c);
  }

  // Lengths and key bounds of sequence b0 + lane (new tokens 0 past the batch).
  __device__ __forceinline__ void load(int b0, int& L, int& n, int& klo, int& khi) const {
    const int b = b0 + lane_id();
    L = 0;
    n = 0;
    klo = 0;
    khi = INT32_MAX;
    if (b < a.batch) {
      L = a.seq_lens[b];
      n = a.q_lens ? a.q_lens[b] : 1;
      if (a.key_lo) klo = a.key_lo[b];
      if (a.key_hi) khi = a.key_hi[b];
      DIFFKV_CHECK_LENGTHS(a, L, n);
    }
  }
  __device__ __forceinline__ int qtiles(int n) const {
    return n >= a.q_lo && n <= a.q_hi ? min((n * G.value() + ROWS - 1) / ROWS, a.n_qtiles) : 0;
  }
  __device__ __forceinline__ int tiles(int L, int n, int qt, int klo, int khi) const {
    int lo, hi;
    pair_key_range(L, n, G, qt, ROWS, a.window, klo, khi, lo, hi);
    return hi > lo ? (hi + kTileKeys - 1) / kTileKeys - lo / kTileKeys : 0;
  }
  // At least one chunk per pair, so a pair with no key in range still
  // writes its rows.
  __device__ __forceinline__ int chunks(int L, int n, int qt, int klo, int khi) const {
    return a.force_splits > 0 ? a.force_splits : max(1, (int)Cd.div((uint32_t)(tiles(L, n, qt, klo, khi) + C - 1)));
  }
  // Chunks of all query tiles of a sequence (0 for one this launch skips).
  __device__ __forceinline__ int seq_chunks(int L, int n, int klo, int khi) const {
    int k = 0;
    const int nq = qtiles(n);
    for (int qt = 0; qt < nq; ++qt) k += chunks(L, n, qt, klo, khi);
    return k;
  }

  __device__ __forceinline__ void init() {
    load(0, L0, n0, lo0, hi0);
    if (a.force_splits > 0) return;
    int T = 0;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      int L = L0, n = n0, klo = lo0, khi = hi0;
      if (b0 > 0) load(b0, L, n, klo, khi);
      const int nq = qtiles(n);
      for (int qt = 0; qt < nq; ++qt) T += tiles(L, n, qt, klo, khi);
    }
    T = wave_sum_int(T);
    set_chunk(max(kMinTilesPerSplit, (T + a.slots - 1) / a.slots));
    // Rounding every pair up to whole chunks can give more chunks than the
    // slots of one resident round (up to slots + pairs, which the grid
    // covers); the chunks past the round would start only when others end
    // and run as a tail after them (decode at 64K tokens per sequence: 524
    // chunks for 512 slots).  Lengthen the chunks by about 3% a step until
    // they fit; a few steps at most, none for the usual near-uniform batch.
    // Up to 64 sequences the check rides on find()'s own prefix sum, which
    // already counts every chunk; larger batches count here.
    if (a.batch > 64)
      for (int it = 0; it < kFitSteps && total_chunks() > a.slots; ++it) set_chunk(C + max(1, C >> 5));
  }
  static constexpr int kFitSteps = 8;

  // Chunks of the whole launch at the current chunk length C.
  __device__ __forceinline__ int total_chunks() const {
    int S = 0;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      int L = L0, n = n0, klo = lo0, khi = hi0;
      if (b0 > 0) load(b0, L, n, klo, khi);
      S += seq_chunks(L, n, klo, khi);
    }
    return wave_sum_int(S);
  }

  // The pair and chunk of chunk id w, with the sequence's lengths, key
  // bounds and first packed query row; false when w is past the last chunk.
  __device__ __forceinline__ bool find(int w, int& b, int& qt, int& c, int& base, int& k, int& L_b,
                                       int& n_b, int& klo_b, int& khi_b, int& r0) {
    int before = 0;                           // chunks of the earlier passes
    int rows_before = 0;                      // new tokens of the earlier passes
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      int L = L0, n = n0, klo = lo0, khi = hi0;
      if (b0 > 0) load(b0, L, n, klo, khi);
      // Inclusive prefix sums over the lanes (chunks, and new tokens for the
      // packed row start).
      auto prefix = [](int v) { return wave_scan_int(v); };
      int kb = seq_chunks(L, n, klo, khi);
      int incl = prefix(kb);
      // One pass holds the whole batch: its count decides whether the
      // chunks fit one resident round (see init).
      if (a.batch <= 64 && a.force_splits <= 0) {
        for (int it = 0; it < kFitSteps && read_lane(incl, 63) > a.slots; ++it) {
          set_chunk(C + max(1, C >> 5));
          kb = seq_chunks(L, n, klo, khi);
          incl = prefix(kb);
        }
      }
      int nincl = n;
      if (a.q_lens) nincl = prefix(n);
      const int total = read_lane(incl, 63);
      if (w < before + total) {
        const int owner = __builtin_ctzll(__ballot(before + incl > w));
        b = b0 + owner;
        base = before + read_lane(incl - kb, owner);
        L_b = read_lane(L, owner);
        n_b = read_lane(n, owner);
        klo_b = read_lane(klo, owner);
        khi_b = read_lane(khi, owner);
        r0 = a.q_lens ? rows_before + read_lane(nincl - n, owner) : b;
        const int nq = qtiles(n_b);
        for (qt = 0; qt < nq; ++qt) {
          k = chunks(L_b, n_b, qt, klo_b, khi_b);
          if (w < base + k) {
            c = w - base;
            return true;
          }
          base += k;
        }
        return false;                         // not reached
      }
      before += total;
      rows_before += a.q_lens ? read_lane(nincl, 63) : 0;
    }
    return false;
  }
};

// Short key ranges: a pair whose keys span at most kWinTiles 64-key tiles
// (a sliding window of a few hundred keys, a short sequence) in a launch of
// one workgroup per pair with 16-row query tiles.  Every tile's loads go out
// at once and each wave runs one softmax update over all of them, instead of
// a chain of dependent per-tile steps, each waiting for its own tile.  Wave w
// takes keys 16w .. 16w+15 of every tile, as the wave-local loop does.  K
// goes from memory straight into the MFMA operand registers: lane group grp
// holds the contiguous dims DQK/4 * grp .. + DQK/4 of the lane's key, and the
// query rows are loaded with the same assignment of dims to contraction
// steps (S^T = K Q^T only needs both operands to agree), so K makes no LDS
// round trip.  V goes through LDS for the transposing reads, one region per
// tile.  NT slots (the pair's tiles; one tile takes two): a slot past the
// pair's last tile, and keys outside [kv_lo, kv_hi), read the zero row; the
// row masks drop every key a row does not see.
constexpr int kWinTiles = 4;

template <bool FP8, bool UPAGE, bool COUNT, int DQK, int NT>
__device__ __forceinline__ void window_pass(const SplitArgs& a, int b, int g, int kv_lo, int kv_hi,
                                            int t_begin, int t_end, int wave, int lane,
                                            const uint16_t* q_row, bool row_ok, int lo_row, int hi_row,
                                            uint16_t* v_lds, float& m, float& l, f32x4 (&o)[8], int& cnt) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int QC = DQK / 32;             // contraction steps of 8 dims per lane
  constexpr int KD = DQK / 4;              // dims of a K row per lane group
  constexpr int KL = KD * ESZ / 16;        // 16-byte K loads per lane and tile
  constexpr int VL = 32 * ESZ / 16;        // 16-byte V loads per lane and tile (32 dims)
  const int col = lane & 15, grp = lane >> 4;
  const uint8_t* k_head = a.k_cache + (size_t)g * DQK * ESZ;
  const uint8_t* v_head = a.v_cache + (size_t)g * kHeadDimV * ESZ;
  const size_t k_slot = (size_t)a.hkv * DQK * ESZ, v_slot = (size_t)a.hkv * kHeadDimV * ESZ;
  const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
  const int lp = a.log2_page, pmask = (1 << lp) - 1;
  const int nt = t_end - t_begin;
  // Keys this lane loads: K row (the lane's column of the K fragment) and
  // V piece (16 keys x 4 pieces of 32 dims).
  const int k_key = 16 * wave + col, v_key = 16 * wave + (lane >> 2), v_piece = lane & 3;
  auto readable = [&](int i, int j) { return i < nt && j >= kv_lo && j < kv_hi; };

  static_assert(NT >= 1 && NT <= kWinTiles, "slots of the short-range pass");
  int pk[NT], pv[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int t = min(t_begin + i, t_end - 1);
    if constexpr (UPAGE) {
      pk[i] = scalar_load(bt, (t * kTileKeys) >> lp);   // a tile lies inside one page
      pv[i] = pk[i];
    } else {
      const int jk = (t_begin + i) * kTileKeys + k_key, jv = (t_begin + i) * kTileKeys + v_key;
      pk[i] = bt[(readable(i, jk) ? jk : kv_lo) >> lp];
      pv[i] = bt[(readable(i, jv) ? jv : kv_lo) >> lp];
    }
#ifdef DIFFKV_DEBUG
    if ((unsigned)pk[i] >= (unsigned)a.num_pages || (unsigned)pv[i] >= (unsigned)a.num_pages) {
      debug_flag(kDbgPage);
      pk[i] = 0;
      pv[i] = 0;
    }
#endif
  }
  // Query rows: step c carries dims KD * grp + 8c .. + 7.
  u32x4 qreg[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c)
    qreg[c] = *reinterpret_cast<const u32x4*>(row_ok ? reinterpret_cast<const uint8_t*>(q_row + KD * grp + 8 * c)
                                                     : g_zero_row);
  // Every K load, then every V load: the products wait for K alone (loads
  // complete in issue order), and V arrives while QK^T and the softmax run.
  u32x4 kr[NT][KL], vr[NT][VL];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int jk = (t_begin + i) * kTileKeys + k_key;
    const uint8_t* kp = k_head + (((size_t)pk[i] << lp) | (size_t)(jk & pmask)) * k_slot + KD * grp * ESZ;
    const bool rk = readable(i, jk);
#pragma unroll
    for (int u = 0; u < KL; ++u) kr[i][u] = *reinterpret_cast<const u32x4*>(rk ? kp + 16 * u : g_zero_row);
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int jv = (t_begin + i) * kTileKeys + v_key;
    const uint8_t* vp = v_head + (((size_t)pv[i] << lp) | (size_t)(jv & pmask)) * v_slot + 32 * v_piece * ESZ;
    const bool rv = readable(i, jv);
#pragma unroll
    for (int u = 0; u < VL; ++u) vr[i][u] = *reinterpret_cast<const u32x4*>(rv ? vp + 16 * u : g_zero_row);
  }

  DIFFKV_STAMP_AFTER(3, kr[NT - 1][KL - 1].x);
  // S^T of every tile: independent MFMA chains.
  f32x4 sacc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < QC; ++c)
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      u32x4 kf;
      if constexpr (FP8) {
        const uint32_t w0 = (c & 1) ? kr[i][c >> 1].z : kr[i][c >> 1].x;
        const uint32_t w1 = (c & 1) ? kr[i][c >> 1].w : kr[i][c >> 1].y;
        kf = cat(e4m3x4_to_bf16x4(w0), e4m3x4_to_bf16x4(w1));
      } else {
        kf = kr[i][c];
      }
      sacc[i] = mfma_16x16x32(kf, qreg[c], sacc[i]);
    }

  // sacc[i][r] = raw score of key (t_begin + i) * 64 + 16 wave + 4 grp + r.
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = (t_begin + i) * kTileKeys + 16 * wave + 4 * grp + r;
      const bool vis = j >= lo_row && j <= hi_row;
      sacc[i][r] = vis ? sacc[i][r] : -INFINITY;
      if constexpr (COUNT) cnt += vis ? 1 : 0;
      mx = fmaxf(mx, sacc[i][r]);
    }
  mx = max_over_lane_groups(mx);
  const float scale = a.scale_log2;
  m = next_reference(-INFINITY, mx * scale);
  const float m_use = m == -INFINITY ? 0.f : m;
  u32x2 pb[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(__builtin_fmaf(sacc[i][r], scale, -m_use));
    pb[i] = u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
  }

  // V rows into LDS (bf16, row-major), this wave's 16 rows of each tile's
  // region; only this wave reads them, so program order suffices.
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    uint16_t* dst = v_lds + i * kVLdsElems + v_key * kVLdsStride + 32 * v_piece;
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      if constexpr (FP8) {
        const u32x2 c0 = e4m3x4_to_bf16x4(vr[i][u].x), c1 = e4m3x4_to_bf16x4(vr[i][u].y);
        const u32x2 c2 = e4m3x4_to_bf16x4(vr[i][u].z), c3 = e4m3x4_to_bf16x4(vr[i][u].w);
        *reinterpret_cast<u32x4*>(dst + 16 * u) = u32x4{c0.x, c0.y, c1.x, c1.y};
        *reinterpret_cast<u32x4*>(dst + 16 * u + 8) = u32x4{c2.x, c2.y, c3.x, c3.y};
      } else {
        *reinterpret_cast<u32x4*>(dst + 8 * u) = vr[i][u];
      }
    }
  }

  // O^T = V^T P^T over two tiles' 16 keys per step (32 keys, as the loop's
  // paired subtiles; an odd last tile alone), the row sums from the all-ones
  // tile.
  f32x4 psum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NT; i += 2) {
    const uint16_t* vp = v_lds + i * kVLdsElems + (16 * wave + 4 * grp + (col >> 2)) * kVLdsStride + 4 * (col & 3);
    if constexpr (NT % 2 == 1) {
      if (i + 1 == NT) {
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) o[nn] = mfma_16x16x16(lds_read_tr16(vp + 16 * nn), pb[i], o[nn]);
        psum = mfma_16x16x16(kOnesBf16x4, pb[i], psum);
        break;
      }
    }
    const u32x4 pt = cat(pb[i], pb[min(i + 1, NT - 1)]);
#pragma unroll
    for (int nn = 0; nn < 8; ++nn)
      o[nn] = mfma_16x16x32(cat(lds_read_tr16(vp + 16 * nn), lds_read_tr16(vp + kVLdsElems + 16 * nn)), pt, o[nn]);
    psum = mfma_16x16x32(kOnesBf16x8, pt, psum);
  }
  l = psum[0];
  DIFFKV_STAMP_AFTER(4, l);
}

template <bool FP8, int RT, bool DIRECT, bool COUNT, bool UPAGE, int NS, int DQK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kSplitWavesPerEu, 8)))
void split_attn_kernel(const SplitArgs a) {
  constexpr int ROWS = 16 * RT;
  constexpr int KW = 4 / RT;                 // waves splitting the keys of one row tile
  constexpr int SUBS = kTileKeys / 16 / KW;  // 16-key subtiles per wave per tile
  constexpr int QC = DQK / 32;               // 32-dim contraction steps of QK^T
  // 16-row tiles: each wave reads only its own 16 keys of a tile, so it
  // gathers them itself into its own LDS rows and streams without waiting
  // for the other waves (no barrier per tile; a wave's LDS reads and writes
  // stay in program order).  Larger row tiles share every key between waves
  // and gather the tile together, with barriers.
  constexpr bool WAVE_LOCAL = RT == 1;
  using IO = std::conditional_t<WAVE_LOCAL, KvTile<FP8, UPAGE, DQK, 64, 16>, KvTile<FP8, UPAGE, DQK>>;
  // One K/V tile, or, for the short-range pass of one-chunk launches, the V
  // regions of kWinTiles tiles.
  constexpr int LDS_ELEMS = DIRECT && WAVE_LOCAL && kWinTiles * kVLdsElems > kKLdsElems<DQK> + kVLdsElems
                                ? kWinTiles * kVLdsElems
                                : kKLdsElems<DQK> + kVLdsElems;
  // Waves that split the keys of a row tile combine in a region of their
  // own, so none has to wait for the others' last tile before writing:
  // (m, l, row max of |O|) and the unscaled O per wave and lane.
  constexpr int ML_ELEMS = 4 * 64 * 8;         // f32x4 per wave and lane, in uint16 units
  constexpr int OB_ELEMS = 4 * 8 * 64 * 8;     // f32x4 per wave, column block and lane
  constexpr int COMB_ELEMS = KW > 1 ? ML_ELEMS + OB_ELEMS : 0;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS + COMB_ELEMS];
  uint16_t* k_lds = lds;
  uint16_t* v_lds = lds + kKLdsElems<DQK>;

  DIFFKV_STAMP_BEGIN();
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int rt = wave % RT, kg = wave / RT;
  const int g = blockIdx.y;
  const int G = a.group;
  const FastDiv gdiv((uint32_t)G);

  // Which pair and chunk: one chunk per pair when DIRECT (grid.x = pairs),
  // else the balanced plan.
  int b, qt, c = 0, base = 0, k = 1, L, n, klo, khi, r0;
  if constexpr (DIRECT) {
    b = blockIdx.x / a.n_qtiles;
    qt = blockIdx.x % a.n_qtiles;
    L = scalar_load(a.seq_lens, b);
    n = a.q_lens ? scalar_load(a.q_lens, b) : 1;
    klo = a.key_lo ? scalar_load(a.key_lo, b) : 0;
    khi = a.key_hi ? scalar_load(a.key_hi, b) : INT32_MAX;
    DIFFKV_CHECK_LENGTHS(a, L, n);
    // The packed row start, summed now so that the query rows can be
    // requested together with the first K/V tile (summed after the tile's
    // loads, its own loads waited for the tile in the in-order load counter
    // and put the query rows a round trip behind it).
    r0 = seq_row_start(a.q_lens, b);
    DIFFKV_STAMP_AFTER(1, L + r0);
  } else {
    SplitPlanner<ROWS> plan(a, gdiv);
    plan.init();
    DIFFKV_STAMP_AFTER(1, plan.C);
    if (!plan.find(blockIdx.x, b, qt, c, base, k, L, n, klo, khi, r0) || base + c >= a.chunk_bound)
      return;
    // The pair's first chunk records where the merge finds the pair.
    if (c == 0 && tid == 0) a.pair_chunks[(size_t)b * a.n_qtiles + qt] = i32x2{base, k};
  }
  if (qt * ROWS >= n * G || n < a.q_lo || n > a.q_hi) return;
  // A pair of one chunk writes its output here; the merge skips it.
  const bool direct = DIRECT || k == 1;
  int kv_lo, kv_hi, t_begin = 0, t_end = 0;
  pair_key_range(L, n, gdiv, qt, ROWS, a.window, klo, khi, kv_lo, kv_hi);
  if (kv_hi > kv_lo) split_tiles(kv_lo, kv_hi, k, c, t_begin, t_end);
  DIFFKV_STAMP_AFTER(2, t_end);
  // Partial row of this chunk for row r of the tile.
  const size_t prow0 = ((size_t)(base + c) * a.hkv + g) * ROWS;
  if (t_begin >= t_end) {
    // An empty chunk (forced splits, or a key range the tile's rows do not
    // reach) still marks its rows: log-sum-exp -inf for the merge, or, when
    // it is the pair's only chunk, the empty rows of a context partial.
    const bool row = tid < ROWS && qt * ROWS + tid < n * G;
    if (!direct) {
      if (row) a.part_lse[prow0 + tid] = f32x2{-INFINITY, 0.f};
    } else if (a.part_out) {                  // uniform: whole waves take this branch
      if (row && DIFFKV_ROW_IN_RANGE(a, r0 + (qt * ROWS + tid) / G)) {
        const int R = qt * ROWS + tid;
        const size_t out_row = (size_t)(r0 + R / G) * a.hq + g * G + R % G;
        for (int d = 0; d < kHeadDimV; d += 4)
          *reinterpret_cast<f32x4*>(a.part_out + out_row * kHeadDimV + d) = f32x4{0.f, 0.f, 0.f, 0.f};
        a.lse_out[out_row] = -INFINITY;
      }
    }
    return;
  }

  // The query row this lane owns in S^T / O^T.
  const int R = qt * ROWS + rt * 16 + col;
  const bool row_ok = R < n * G && DIFFKV_ROW_IN_RANGE(a, r0 + R / G);
#ifdef DIFFKV_DEBUG
  if (qt == 0 && (DIRECT || c == 0)) DIFFKV_CHECK_TOTAL_ROWS(a, b, r0, n);
#endif
  const int tok = row_ok ? (int)gdiv.div((uint32_t)R) : 0;
  const int h = g * G + (row_ok ? R - tok * G : 0);
  const int p_row = L - n + tok;
  const int lo_row = max(a.window > 0 ? max(0, p_row - a.window + 1) : 0, klo);
  const int hi_row = row_ok ? min(p_row, khi - 1) : -1;   // empty interval for padding rows

  // This row's sink logit, used by a pair of one chunk: loaded here, not
  // in the epilogue, where it would add a round trip after the last tile.
  const float sink = *(a.sinks ? a.sinks + h : reinterpret_cast<const float*>(g_zero_row));

  float m = -INFINITY, l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  int cnt = 0;

  bool windowed = false;
  if constexpr (DIRECT && WAVE_LOCAL) windowed = t_end - t_begin <= kWinTiles;   // uniform
  if (windowed) {
    // Only the pair's own tiles are multiplied (a window of 128 keys spans
    // three tiles unless it starts in a tile's last two keys).
    auto pass = [&](auto nt) {
      window_pass<FP8, UPAGE, COUNT, DQK, decltype(nt)::value>(
          a, b, g, kv_lo, kv_hi, t_begin, t_end, wave, lane, a.q + ((size_t)(r0 + tok) * a.hq + h) * DQK,
          row_ok, lo_row, hi_row, lds, m, l, o, cnt);
    };
    const int nt = t_end - t_begin;         // 1 .. kWinTiles, uniform
    if (nt <= 2) pass(std::integral_constant<int, 2>{});
    else if (nt == 3) pass(std::integral_constant<int, 3>{});
    else pass(std::integral_constant<int, 4>{});
  } else {
    const IO io(a.k_cache, a.v_cache, a.block_table + (size_t)b * a.bt_stride, a.hkv, g,
                a.log2_page, kv_lo, kv_hi, t_end, WAVE_LOCAL ? lane : tid, WAVE_LOCAL ? 16 * wave : 0,
                DIFFKV_PAGES(a));

    // NS tiles of K/V in flight in registers; page ids NS tiles ahead of the
    // data they address.  Order of the first requests: (the sink,) page ids,
    // query rows, K/V data, so that neither the query rows nor the data wait
    // for the other.
    typename IO::Pages pg[NS];
    typename IO::Stage st[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) io.fetch_pages(t_begin + i, pg[i]);

    // Q^T operand: contraction chunk c carries dims 32c + 8*grp .. +7.
    u32x4 qreg[QC];
    {
      const uint16_t* qp = a.q + ((size_t)(r0 + tok) * a.hq + h) * DQK + 8 * grp;
#pragma unroll
      for (int c = 0; c < QC; ++c)
        qreg[c] = *reinterpret_cast<const u32x4*>(row_ok ? reinterpret_cast<const uint8_t*>(qp + 32 * c)
                                                         : g_zero_row);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      io.fetch_data(t_begin + i, pg[i], st[i]);
      io.fetch_pages(t_begin + NS + i, pg[i]);
    }

    // Tiles every row of the workgroup sees whole (no key past the first row's
    // position, none before the last row's window start) skip the mask.
    // Padding rows past n*G may then score keys they would not see; their
    // results stay in their own lanes and are never written.
    const int r_first = qt * ROWS;
    const int r_last = min(n * G, r_first + ROWS) - 1;
    const int p_first = min(L - n + token_of_row(r_first, gdiv), khi - 1);
    const int lo_last = max(a.window > 0 ? max(0, L - n + token_of_row(r_last, gdiv) - a.window + 1) : 0, klo);
    const float scale = a.scale_log2;   // > 0 (checked on the host)

    // One online-softmax update per tile: the S^T tiles of all this wave's
    // 16-key subtiles first (independent MFMA chains), one max / rescale / sum
    // over them, then all the P*V products.
    auto compute_tile = [&](int t) {
      f32x4 sacc[SUBS];
#pragma unroll
      for (int sub = 0; sub < SUBS; ++sub) sacc[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < QC; ++c)
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) {
          const uint16_t* kp = k_lds + ((kg * SUBS + sub) * 16 + col) * kKLdsStride<DQK> + 8 * grp + 32 * c;
          sacc[sub] = mfma_16x16x32(*reinterpret_cast<const u32x4*>(kp), qreg[c], sacc[sub]);
        }

      // sacc[sub][i] = raw S^T[key (kg*SUBS+sub)*16 + 4*grp + i][row col].
      // The branch is uniform over the workgroup.
      if (t * kTileKeys < lo_last || t * kTileKeys + kTileKeys - 1 > p_first) {
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = t * kTileKeys + (kg * SUBS + sub) * 16 + 4 * grp + i;
            const bool vis = j >= lo_row && j <= hi_row;
            sacc[sub][i] = vis ? sacc[sub][i] : -INFINITY;
            if constexpr (COUNT) cnt += vis ? 1 : 0;
          }
      } else {
        if constexpr (COUNT) cnt += 4 * SUBS;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < SUBS; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[sub][i]);
      mx = max_over_lane_groups(mx);
      const float m_new = next_reference(m, mx * scale);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      u32x2 pb[SUBS];
#pragma unroll
      for (int sub = 0; sub < SUBS; ++sub) {
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

      // V^T operand straight from the row-major tile: in each 16-lane group the
      // transposing read hands lane col the dim 16*nn + col of keys
      // 4*grp + 0..3 when source lane col reads 4 dims (16*nn + 4*(col%4))
      // of key 4*grp + col/4.  The row sums of the (bf16) P come from an extra
      // all-ones V^T tile: every element of psum is sum_k P[row][k].
      // With two or more subtiles per wave the products contract 32 keys at a
      // time: lane group grp takes keys 4grp + 0..3 of subtiles 2c and 2c+1 (the
      // P values it holds), and two transposing reads give the matching V^T.
      f32x4 psum = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (SUBS % 2 == 0) {
#pragma unroll
        for (int c = 0; c < SUBS / 2; ++c) {
          const u32x4 pt = cat(pb[2 * c], pb[2 * c + 1]);
          const uint16_t* vp =
              v_lds + ((kg * SUBS + 2 * c) * 16 + 4 * grp + (col >> 2)) * kVLdsStride + 4 * (col & 3);
#pragma unroll
          for (int nn = 0; nn < 8; ++nn)
            o[nn] = mfma_16x16x32(cat(lds_read_tr16(vp + 16 * nn), lds_read_tr16(vp + 16 * kVLdsStride + 16 * nn)),
                                  pt, o[nn]);
          psum = mfma_16x16x32(kOnesBf16x8, pt, psum);
        }
      } else {
#pragma unroll
        for (int sub = 0; sub < SUBS; ++sub) {
          const uint16_t* vp = v_lds + ((kg * SUBS + sub) * 16 + 4 * grp + (col >> 2)) * kVLdsStride + 4 * (col & 3);
#pragma unroll
          for (int nn = 0; nn < 8; ++nn)
            o[nn] = mfma_16x16x16(lds_read_tr16(vp + 16 * nn), pb[sub], o[nn]);
          psum = mfma_16x16x16(kOnesBf16x4, pb[sub], psum);
        }
      }
      l = __builtin_fmaf(l, alpha, psum[0]);
    };

    // Every stage step runs in every round that has tiles beyond it (loads
    // stay in one fixed order, so the compiler waits for exactly the stage it
    // needs).  The last round issues no look-ahead loads: they would only hold
    // the waves at their exit (sliding-window verify 7.2 -> 7.0 us).  Page ids
    // are requested after the tile's products: with large pages they are
    // scalar loads, which share the LDS reads' completion counter and return
    // out of order, so a page id requested before the products would make
    // their first LDS read wait for its whole memory round trip.
    int t = t_begin;
    DIFFKV_STAMP_AFTER(3, st[0].k[0].x);
    for (; t + NS < t_end; t += NS) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if constexpr (!WAVE_LOCAL) __syncthreads();
        io.store(st[i], k_lds, v_lds);
        if constexpr (!WAVE_LOCAL) __syncthreads();
        // With wave-local tiles a wave issues its next loads at raised
        // priority, ahead of the other waves' products on its SIMD, so the
        // next tile is requested as soon as this one is in LDS (batched decode
        // 37.5 -> 36.7 us; the shared 32- and 64-row tiles gain nothing).
        if constexpr (WAVE_LOCAL) __builtin_amdgcn_s_setprio(1);
        io.fetch_data(t + i + NS, pg[i], st[i]);
        if constexpr (WAVE_LOCAL) __builtin_amdgcn_s_setprio(0);
        compute_tile(t + i);
        if (t + i == t_begin) DIFFKV_STAMP(4);
        io.fetch_pages(t + i + 2 * NS, pg[i]);
      }
    }
    DIFFKV_STAMP(5);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (t + i < t_end) {                       // uniform over the workgroup
        if constexpr (!WAVE_LOCAL) __syncthreads();
        io.store(st[i], k_lds, v_lds);
        if constexpr (!WAVE_LOCAL) __syncthreads();
        compute_tile(t + i);
      }
    }
  }

  DIFFKV_STAMP(6);
  if constexpr (COUNT) {
    cnt += __shfl_xor(cnt, 16, 64);
    cnt += __shfl_xor(cnt, 32, 64);
    if (row_ok && grp == 0 && a.count_out)
      atomicAdd(a.count_out + (size_t)(r0 + tok) * a.hq + h, cnt);
  }

  // Waves that split the keys of one row tile combine through LDS: each
  // publishes its (m, l), the row maximum of its |O| and its O; after one
  // barrier each of the KW waves weights and sums 8 / KW of the eight
  // 16-column blocks for its rows and stores them, so the reads, adds and
  // output stores are spread over the waves.  The published row maxima give
  // the partial rows' fp16 exponent a bound (the combined row's largest
  // magnitude is at most sum_k f_k max|O_k|) without a second exchange.
  constexpr int NNW = 8 / KW;                  // column blocks a wave stores
  int nn0 = 0;                                 // its first block
  float amax_bound = 0.f;                      // bound on the row's max |O| (KW > 1)
  if constexpr (KW > 1) {
    f32x4* ml = reinterpret_cast<f32x4*>(lds + LDS_ELEMS);
    f32x4* ob = reinterpret_cast<f32x4*>(lds + LDS_ELEMS + ML_ELEMS);
    float am = 0.f;
    if (!direct) {
#pragma unroll
      for (int nn = 0; nn < 8; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(o[nn][i]));
      am = max_over_lane_groups(am);
    }
    ml[wave * 64 + lane] = f32x4{m, l, am, 0.f};
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) ob[(wave * 8 + nn) * 64 + lane] = o[nn];
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < KW; ++k) M = fmaxf(M, ml[(rt + k * RT) * 64 + lane].x);
    const float M_use = M == -INFINITY ? 0.f : M;
    float f[KW];
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      const f32x4 e = ml[(rt + k * RT) * 64 + lane];
      f[k] = fast_exp2(e.x - M_use);
      L += f[k] * e.y;
      A += f[k] * e.z;
    }
    nn0 = kg * NNW;
#pragma unroll
    for (int j = 0; j < NNW; ++j) {
      f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KW; ++k) sum += f[k] * ob[((rt + k * RT) * 8 + nn0 + j) * 64 + lane];
      o[j] = sum;
    }
    m = M;
    l = L;
    amax_bound = A;
  }

  // o[j] now holds column block nn0 + j of this lane's row: dims
  // 16 (nn0 + j) + 4 grp + 0..3.  The row's lse goes out once, from kg 0.
  const size_t out_row = (size_t)(r0 + tok) * a.hq + h;
  if (direct) {
    if (!row_ok) return;
    float coef;
    if (a.sinks) {
      const float s2 = sink * kLog2e;
      const float M2 = fmaxf(m, s2);
      const float al = fast_exp2(m - M2);
      coef = al / (l * al + fast_exp2(s2 - M2));
    } else {
      coef = l > 0.f ? 1.f / l : 0.f;         // l == 0 only for a context partial's empty row
    }
    coef *= a.v_scale;
    if (a.part_out) {
      float* op = a.part_out + out_row * kHeadDimV + 16 * nn0 + 4 * grp;
#pragma unroll
      for (int j = 0; j < NNW; ++j) *reinterpret_cast<f32x4*>(op + 16 * j) = o[j] * coef;
      if (kg == 0 && grp == 0) a.lse_out[out_row] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
      DIFFKV_STAMP(7);
      DIFFKV_STAMP_FLUSH();
      return;
    }
    uint16_t* op = a.out + out_row * kHeadDimV + 16 * nn0 + 4 * grp;
#pragma unroll
    for (int j = 0; j < NNW; ++j) {
      const f32x4 v = o[j] * coef;
      *reinterpret_cast<u32x2*>(op + 16 * j) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
    if (a.lse_out && kg == 0 && grp == 0) a.lse_out[out_row] = (m + log2f(l)) * kLn2;
    DIFFKV_STAMP(7);
    DIFFKV_STAMP_FLUSH();
  } else {
    const size_t prow = prow0 + rt * 16 + col;
    // The normalised partial row (a convex combination of V rows) is stored
    // in fp16 as a block-floating-point row: scaled by 2^-e so its largest
    // magnitude lies in [2^14, 2^15), e kept beside the row's log-sum-exp.
    // Each element then keeps fp16's 11 bits relative to the row maximum,
    // so the merge adds far less than the output's own bf16 rounding (a bf16
    // partial would round every row twice at 8 bits), and any finite V fits.
    // With the blocks spread over KW waves, e comes from the bound above.
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float amax = amax_bound;
    if constexpr (KW == 1) {
#pragma unroll
      for (int j = 0; j < NNW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[j][i]));
      amax = max_over_lane_groups(amax);
    }
    amax *= inv;
    if (!row_ok) return;
    int e = 0;
    if (amax > 0.f) {
      int k;
      frexpf(amax, &k);                       // amax in [2^(k-1), 2^k)
      e = max(k - 15, -100);                  // 2^-e stays a normal float
    }
    const float p2 = __builtin_amdgcn_ldexpf(1.f, -e);
    uint16_t* pp = a.part_o + prow * kHeadDimV + 16 * nn0 + 4 * grp;
#pragma unroll
    for (int j = 0; j < NNW; ++j) {
      const f32x4 v = (o[j] * inv) * p2;
      *reinterpret_cast<u32x2*>(pp + 16 * j) = u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
    }
    if (kg == 0 && grp == 0) a.part_lse[prow] = f32x2{l > 0.f ? m + log2f(l) : -INFINITY, (float)e};
    DIFFKV_STAMP(7);
    DIFFKV_STAMP_FLUSH();
  }
}

// Combines the split partials of one query row: weights 2^(lse_s - M) (times
// 2^e_s on the stored fp16 row), the sink joining the denominator, v_scale,
// bf16 store.  One workgroup of W
// waves per row.  Every split wrote its row (an empty split an lse of -inf),
// so a pass over up to W*K splits issues all of its loads before any
// arithmetic: every wave reads all the pass's lse values (so each has the
// pass max and the weight sum), wave w the partial rows of splits
// w, w+W, ..., two output dims per lane.  Passes combine with a running
// maximum; the waves' sums meet in LDS in a fixed order (deterministic).
// One wave (no LDS, no barrier) when the splits fit its K loads.
template <int ROWS, int W, int K>
__global__ __launch_bounds__(64 * W) void split_merge_kernel(const SplitArgs a) {
  constexpr int PASS = W * K;               // splits per pass
  constexpr int LI = (PASS + 63) / 64;      // lse values per lane per pass
  __shared__ f32x2 red[W > 1 ? W - 1 : 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = blockIdx.x;                 // row of this (sequence, KV head)
  const int qt = R / ROWS, r = R % ROWS;
  const int bg = blockIdx.y;
  const int b = bg / a.hkv, g = bg % a.hkv;
  const int G = a.group;
  // The sequence's length, its pair's chunk range, its packed row start and
  // the row's sink are independent loads: all go out before any is tested,
  // so the partials are one memory round trip away and nothing waits on
  // memory after them.  The pair entry is read even for rows past the
  // sequence's own (in bounds: every pair of the launch has one); those
  // rows return before using it.
  const int tok = R / G, h = g * G + R % G;
#ifdef DIFFKV_DEBUG
  int n = a.q_lens ? a.q_lens[b] : 1;
#else
  const int n = a.q_lens ? a.q_lens[b] : 1;
#endif
  const i32x2 pc = a.pair_chunks[(size_t)b * a.n_qtiles + qt];
  const int r0 = seq_row_start(a.q_lens, b);
  const float sink = *(a.sinks ? a.sinks + h : reinterpret_cast<const float*>(g_zero_row));
#ifdef DIFFKV_DEBUG
  {
    int L = a.seq_lens[b];
    DIFFKV_CHECK_LENGTHS(a, L, n);
  }
#endif
  if (n < a.q_lo || n > a.q_hi || R >= n * G) return;   // uniform over the workgroup
#ifdef DIFFKV_DEBUG
  if (!DIFFKV_ROW_IN_RANGE(a, r0 + R / G)) return;      // uniform as well
#endif
  const int base = pc.x, S = pc.y;
  if (S <= 1) return;                       // written by the split kernel itself
  if (base < 0 || base + S > a.chunk_bound) return;
  // Waves in use: one when its K loads cover every chunk of the pair.
  const int nw = S <= K ? 1 : W;
  if (wave >= nw) return;

  // Chunk j's partial row: chunk ids are consecutive within the pair.
  const size_t prow0 = ((size_t)base * a.hkv + g) * ROWS + r;
  const size_t pstride = (size_t)a.hkv * ROWS;
  const uint16_t* po0 = a.part_o + prow0 * kHeadDimV + 2 * lane;
  float m_run = -INFINITY, ksum = 0.f;
  f32x2 acc = f32x2{0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += nw * K) {
    const int s1 = min(S, s0 + nw * K);     // chunks [s0, s1) in this pass
    float lse_l[LI], e_l[LI];
#pragma unroll
    for (int i = 0; i < LI; ++i) {
      const int j = s0 + lane + 64 * i;
      const f32x2 le = j < s1 ? a.part_lse[prow0 + (size_t)j * pstride] : f32x2{-INFINITY, 0.f};
      lse_l[i] = le.x;
      e_l[i] = le.y;
    }
    uint32_t raw[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int j = min(s0 + wave + nw * k, S - 1);
      raw[k] = *reinterpret_cast<const uint32_t*>(po0 + (size_t)j * pstride * kHeadDimV);
    }
    float mx = lse_l[0];
#pragma unroll
    for (int i = 1; i < LI; ++i) mx = fmaxf(mx, lse_l[i]);
    const float m_new = fmaxf(m_run, wave_max_all(mx));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float f = fast_exp2(m_run - m_use);
    acc *= f;
    ksum *= f;
    float wl[LI];
#pragma unroll
    for (int i = 0; i < LI; ++i) {
      const float w = fast_exp2(lse_l[i] - m_use);
      ksum += w;
      wl[i] = __builtin_amdgcn_ldexpf(w, (int)e_l[i]);   // weight of the stored row
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = wave + nw * k;          // split within the pass (wave-uniform)
      float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl[0]), i & 63));
#pragma unroll
      for (int li = 1; li < LI; ++li) {
        const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl[li]), i & 63));
        w = (i >> 6) == li ? wi : w;
      }
      if (s0 + i < s1 && w > 0.f) acc += w * unpack_f16x2(raw[k]);
    }
    m_run = m_new;
  }
  if (W > 1 && nw > 1) {                   // uniform: every wave of the workgroup is here
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < W - 1; ++w) acc += red[w][lane];
  }
  ksum = wave_sum_all(ksum);
  const float s2 = a.sinks ? sink * kLog2e : -INFINITY;
  const float Mt = fmaxf(m_run, s2);
  const float Mt_use = Mt == -INFINITY ? 0.f : Mt;   // a context partial's row with no key
  const float f = fast_exp2(m_run - Mt_use);
  const float den = ksum * f + (a.sinks ? fast_exp2(s2 - Mt_use) : 0.f);
  const float coef = den > 0.f ? a.v_scale * f / den : 0.f;
  const size_t out_row = (size_t)(r0 + tok) * a.hq + h;
  if (a.part_out) {
    *reinterpret_cast<f32x2*>(a.part_out + out_row * kHeadDimV + 2 * lane) = acc * coef;
    if (lane == 0) a.lse_out[out_row] = ksum > 0.f ? (m_run + log2f(ksum)) * kLn2 : -INFINITY;
    return;
  }
  *reinterpret_cast<uint32_t*>(a.out + out_row * kHeadDimV + 2 * lane) = pack_bf16x2(acc.x * coef, acc.y * coef);
  if (a.lse_out && lane == 0) a.lse_out[out_row] = (m_run + log2f(ksum)) * kLn2;
}

__global__ void fill_i32_kernel(int32_t* p, size_t n, int32_t v) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace diffkv
