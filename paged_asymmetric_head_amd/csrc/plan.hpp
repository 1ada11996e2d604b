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

constexpr int kHeadDimQK = 192;      // key head dim of the asymmetric layers
constexpr int kHeadDimQKSym = 128;   // key head dim of symmetric (128/128) heads
constexpr int kHeadDimV = 128;
constexpr int kTileKeys = 64;        // keys per split-kernel tile
constexpr int kDefaultCUs = 256;     // MI355X: 256 compute units in 8 XCDs (the count used
                                     // when no device can be queried)
constexpr int kMaxCUs = 1024;        // largest CU count a descriptor is validated for
constexpr int kMaxGridYZ = 65535;
constexpr int kMaxForcedSplits = 1 << 16;   // force_num_splits bound (a test hook)

// Query rows per split-kernel workgroup: 16 * row_tiles, row_tiles in {1,2,4}.
inline int split_row_tiles(int rows_per_pair) {
  return rows_per_pair <= 16 ? 1 : (rows_per_pair <= 32 ? 2 : 4);
}

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

struct SplitPlan {
  int row_tiles = 1;      // 16-row MFMA tiles per workgroup
  int rows = 16;          // query rows per workgroup (16 * row_tiles)
  int n_qtiles = 1;       // query tiles per (sequence, KV head)
  bool direct = true;     // one chunk per pair: no partials, no merge
  int slots = 1;          // balanced plan: target chunks per KV head
  int max_chunks = 1;     // bound on the chunks of one pair (picks the merge shape)
  long long grid_x = 1;   // workgroups per KV head
  size_t part_o_bytes = 0, part_lse_bytes = 0, pair_bytes = 0, workspace_bytes = 0;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

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
// measured slower at the common sizes (the opening burst of loads delays
// every workgroup's first tile; two bf16 stages cost 2% on decode at 8K
// tokens per sequence for 2% at 64K).  Two workgroups per CU (three spill).
#ifndef DIFFKV_BF16_STAGES
#define DIFFKV_BF16_STAGES 1
#endif
#ifndef DIFFKV_FP8_STAGES
#define DIFFKV_FP8_STAGES 1
#endif
#ifndef DIFFKV_SPLIT_WAVES_PER_EU
#define DIFFKV_SPLIT_WAVES_PER_EU 2
#endif
#ifndef DIFFKV_SPLIT_SLOTS_PER_CU
#define DIFFKV_SPLIT_SLOTS_PER_CU DIFFKV_SPLIT_WAVES_PER_EU
#endif
#ifndef DIFFKV_SPLIT_SLOTS_PER_CU_64
#define DIFFKV_SPLIT_SLOTS_PER_CU_64 1
#endif
#ifndef DIFFKV_MIN_TILES_PER_SPLIT
#define DIFFKV_MIN_TILES_PER_SPLIT 4
#endif
template <bool FP8> constexpr int kSplitStages = FP8 ? DIFFKV_FP8_STAGES : DIFFKV_BF16_STAGES;
constexpr int kSplitWavesPerEu = DIFFKV_SPLIT_WAVES_PER_EU;
constexpr int kSplitSlotsPerCu = DIFFKV_SPLIT_SLOTS_PER_CU;
// Workgroups of 64 query rows (4 row tiles: a verify block at GQA 8 or
// more) over a bf16 cache plan one chunk per CU instead while those chunks
// stay short (host bound: at most kSlots64MaxTilesPerCu tiles each): each
// workgroup then has every SIMD to itself for its four times larger
// products, and the fewer chunks halve the partials the merge reads (4
// verify blocks at 40K-50K tokens: the call 36.2 vs 38.1 us with two per
// CU).  Longer work goes back to two per CU, which keeps twice the loads in
// flight (32 such blocks: the kernel 173 vs 180 us).  FP8 caches keep two:
// the widening adds VALU work per tile that a second workgroup hides (the
// split part of a mixed FP8 batch took 148 instead of 121 us with one).
constexpr int kSplitSlotsPerCu64 = DIFFKV_SPLIT_SLOTS_PER_CU_64;
constexpr long long kSlots64MaxTilesPerCu = 16;
// plan_split's wgs_per_cu for a launch: slots chosen from the row tiles and
// the cache format.
constexpr int kLaunchSlots = -1;

// Split plan from host bounds and the device's CU count (a pure function of
// both).  The kernels cut the keys on the device (balanced chunks of
// C = max(kMinTilesPerSplit, ceil(T / slots)) tiles, T the key tiles of the
// whole call), so the host fixes only the bounds: slots = one resident round
// of workgroups over the num_cus CUs per KV head (a second round would pay
// the start-up chain seq_lens -> block table -> data again), at most
// slots + pairs chunks per KV head (each pair's last chunk may be short), and
// no split at all when no pair can hold more than kMinTilesPerSplit tiles
// (short windows).  A larger wgs_per_cu only grows the bounds, so the
// workspace sized for 4 workgroups per CU covers every launch on that device.
constexpr int kMinTilesPerSplit = DIFFKV_MIN_TILES_PER_SPLIT;
constexpr int kWorkspaceWgsPerCu = kSplitSlotsPerCu > 4 ? kSplitSlotsPerCu : 4;

inline SplitPlan plan_split(const diffkv_attn_desc& d, int window, int num_cus,
                            int wgs_per_cu = kWorkspaceWgsPerCu) {
  SplitPlan p;
  const int G = d.num_q_heads / d.num_kv_heads;
  const long long rows_pair = (long long)d.max_q_len * G;
  const long long max_tiles = ceil_div(max_keys_bound(d, window), kTileKeys) + 1;
  // Short windows (no pair can hold more than kMinTilesPerSplit tiles, so
  // one chunk per pair) take 16-row query tiles whatever the rows per pair:
  // such a launch has few workgroups, each walking its few tiles as a chain
  // of dependent steps, and 16-row tiles give more workgroups whose waves
  // each gather and multiply their own keys with no barrier per tile (the
  // window reads are repeated per query tile, a few MB at most).  On the
  // sliding-window workloads (64 sequences, 4 new tokens x 8 heads, window
  // 128, FP8) the call went from 9.4 to 7.8 us (pages of 1) and from 8.5 to
  // 7.0 us (pages of 128).
  const bool short_keys = d.force_num_splits <= 0 && max_tiles <= kMinTilesPerSplit;
  p.row_tiles = short_keys ? 1 : split_row_tiles((int)(rows_pair < 64 ? rows_pair : 64));
  p.rows = 16 * p.row_tiles;
  p.n_qtiles = ceil_div(rows_pair, p.rows);
  const long long pairs = (long long)d.batch * p.n_qtiles;
  if (wgs_per_cu == kLaunchSlots)   // bound on the tiles one CU's single chunk would hold
    wgs_per_cu = p.row_tiles == 4 && d.kv_dtype == DIFFKV_KV_BF16 &&
                         pairs * max_tiles * d.num_kv_heads <= (long long)kSlots64MaxTilesPerCu * num_cus
                     ? kSplitSlotsPerCu64
                     : kSplitSlotsPerCu;
  const long long per_head = (long long)num_cus * wgs_per_cu / d.num_kv_heads;
  p.slots = per_head > 1 ? (int)per_head : 1;
  if (d.force_num_splits > 0) {
    p.direct = d.force_num_splits == 1;
    p.max_chunks = d.force_num_splits;
    p.grid_x = pairs * d.force_num_splits;
  } else {
    p.direct = max_tiles <= kMinTilesPerSplit;
    const long long kmax = ceil_div(max_tiles, kMinTilesPerSplit);
    p.max_chunks = p.direct ? 1 : (int)(kmax < p.slots ? kmax : p.slots);
    p.grid_x = p.direct ? pairs : p.slots + pairs;
  }
  if (!p.direct) {
    const size_t prow = (size_t)p.grid_x * d.num_kv_heads * p.rows;
    p.part_o_bytes = prow * kHeadDimV * sizeof(uint16_t);   // fp16 partial rows
    p.part_lse_bytes = prow * 2 * sizeof(float);             // lse and row exponent
    p.pair_bytes = (size_t)pairs * 2 * sizeof(int32_t);      // first chunk id, chunk count
    p.workspace_bytes = align256(p.part_o_bytes) + align256(p.part_lse_bytes) + align256(p.pair_bytes);
  }
  return p;
}

// Prefill: workgroups of kPrefillRows query rows along one (sequence, KV
// head), two 16-row tiles per wave.
constexpr int kPrefillRows = 256;

// Mixed batches: sequences with at most this many new tokens (the verify
// limit) go to the split kernel, longer ones to the prefill kernel.
constexpr int kMixedSplitMaxQ = 16;

// The descriptor the split part of a call is planned from: a mixed call's
// split kernel sees only sequences of at most kMixedSplitMaxQ new tokens.
inline diffkv_attn_desc split_part_desc(const diffkv_attn_desc& d, int entry) {
  diffkv_attn_desc s = d;
  if (entry == DIFFKV_ENTRY_MIXED && s.max_q_len > kMixedSplitMaxQ) s.max_q_len = kMixedSplitMaxQ;
  return s;
}
inline int prefill_row_blocks(const diffkv_attn_desc& d) {
  return ceil_div((long long)d.max_q_len * (d.num_q_heads / d.num_kv_heads), kPrefillRows);
}

}  // namespace diffkv
