// Host-side launch planning for the paged attention kernels.
//
// Everything here is a pure function of the descriptor (plus the window of
// the call), never of device data, so a launch can be captured in a HIP
// graph and replayed with new sequence lengths and block tables that stay
// within the descriptor's bounds.
#pragma once

#include <cstddef>
#include <cstdint>

#include "diffkv_attn.h"

namespace diffkv {

constexpr int kHeadDimQK = 192;
constexpr int kHeadDimV = 128;
constexpr int kTileKeys = 64;        // keys per split-kernel tile
constexpr int kTargetCUs = 256;      // MI355X: 256 compute units in 8 XCDs
constexpr int kMaxGridYZ = 65535;

// Query rows per split-kernel workgroup: 16 * row_tiles, row_tiles in {1,2,4}.
inline int split_row_tiles(int rows_per_pair) {
  return rows_per_pair <= 16 ? 1 : (rows_per_pair <= 32 ? 2 : 4);
}

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

struct SplitPlan {
  int row_tiles = 1;      // 16-row MFMA tiles per workgroup
  int rows = 16;          // query rows per workgroup (16 * row_tiles)
  int n_qtiles = 1;       // workgroups along the query rows of one (sequence, KV head)
  int num_splits = 1;     // workgroups along the key axis
  size_t part_o_bytes = 0, part_lse_bytes = 0, workspace_bytes = 0;
};

// Upper bound on the keys one (sequence, KV head, query tile) reads.
inline long long max_keys_bound(const diffkv_attn_desc& d, int window) {
  long long full = d.max_seq_len;
  if (window > 0) {
    long long w = (long long)window + d.max_q_len - 1;
    return w < full ? w : full;
  }
  return full;
}

// Register stages of the split kernel (tiles of K/V in flight per
// workgroup, beyond the one in LDS) and the waves per SIMD it is compiled
// for, which is also the number of its 256-thread workgroups resident per
// CU.  Both K/V formats keep a single register stage: with a resident round
// of workgroups that is enough loads in flight for HBM, and deeper stages
// measured slower (the opening burst of loads delays every workgroup's
// first tile).  Two workgroups per CU for every page size (three measured no
// better).
#ifndef DIFFKV_BF16_STAGES
#define DIFFKV_BF16_STAGES 1
#endif
#ifndef DIFFKV_FP8_STAGES
#define DIFFKV_FP8_STAGES 1
#endif
#ifndef DIFFKV_SPLIT_WAVES_PER_EU
#define DIFFKV_SPLIT_WAVES_PER_EU 2
#endif
template <bool FP8> constexpr int kSplitStages = FP8 ? DIFFKV_FP8_STAGES : DIFFKV_BF16_STAGES;
constexpr int kSplitWavesPerEu = DIFFKV_SPLIT_WAVES_PER_EU;

// Split count: one resident round of workgroups over the 256 CUs (a second
// round would pay the start-up chain seq_lens -> block table -> data again),
// but never fewer than `kMinTilesPerSplit` tiles per split (the split
// partials are extra traffic, so short splits do not pay).  Monotone in the
// key bound, so the workspace sized for full attention covers every window;
// the workspace is sized for the largest target (4 workgroups per CU).
constexpr int kMinTilesPerSplit = 4;

inline SplitPlan plan_split(const diffkv_attn_desc& d, int window, bool allow_split,
                            int wgs_per_cu = 4) {
  SplitPlan p;
  const int G = d.num_q_heads / d.num_kv_heads;
  const long long rows_pair = (long long)d.max_q_len * G;
  p.row_tiles = split_row_tiles((int)(rows_pair < 64 ? rows_pair : 64));
  p.rows = 16 * p.row_tiles;
  p.n_qtiles = ceil_div(rows_pair, p.rows);
  const long long pairs = (long long)d.batch * d.num_kv_heads * p.n_qtiles;
  const long long tiles = ceil_div(max_keys_bound(d, window), kTileKeys) + 1;
  int s = 1;
  if (allow_split) {
    if (d.force_num_splits > 0) {
      s = d.force_num_splits;
    } else {
      const long long target = (long long)kTargetCUs * wgs_per_cu;
      long long want = (target + pairs - 1) / pairs;
      long long cap = tiles / kMinTilesPerSplit;
      if (cap < 1) cap = 1;
      if (want > cap) want = cap;
      if (want < 1) want = 1;
      s = (int)want;
    }
  }
  p.num_splits = s;
  if (s > 1) {
    const size_t prow = (size_t)pairs * s * p.rows;
    p.part_o_bytes = prow * kHeadDimV * sizeof(uint16_t);   // bf16 partial rows
    p.part_lse_bytes = prow * sizeof(float);
    p.workspace_bytes = ((p.part_o_bytes + 255) / 256) * 256 + ((p.part_lse_bytes + 255) / 256) * 256;
  }
  return p;
}

// Prefill: workgroups of kPrefillRows query rows along one (sequence, KV
// head), one 16-row tile per wave.
constexpr int kPrefillRows = 256;
inline int prefill_row_blocks(const diffkv_attn_desc& d) {
  return ceil_div((long long)d.max_q_len * (d.num_q_heads / d.num_kv_heads), kPrefillRows);
}

}  // namespace diffkv
