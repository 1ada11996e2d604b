// Synchronous descriptor checks of the C ABI.  Host code only (no HIP call,
// no device type), so it also builds with a plain C++ compiler: the CPU
// tests compile it with the address and undefined-behaviour sanitizers and
// feed it seeded random descriptors.
#pragma once

#include <cstdint>

#include "diffkv_attn.h"
#include "plan.hpp"

namespace diffkv {

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// log2 of a power of two in [1, 256].
inline int ilog2(int x) {
  int r = 0;
  while (r < 30 && (1 << r) < x) ++r;
  return r;
}

// DIFFKV_OK, or the status the entry returns for this descriptor.  The
// launch-shape limits hold on every device of up to kMaxCUs compute units.
inline int validate_desc(const diffkv_attn_desc* d, int entry) {
  if (d == nullptr) return DIFFKV_INVALID_ARGUMENT;
  if (entry < DIFFKV_ENTRY_DECODE || entry > DIFFKV_ENTRY_MIXED) return DIFFKV_INVALID_ARGUMENT;
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return DIFFKV_INVALID_ARGUMENT;
  if (d->num_q_heads % d->num_kv_heads != 0) return DIFFKV_INVALID_ARGUMENT;
  if ((d->head_dim_qk != kHeadDimQK && d->head_dim_qk != kHeadDimQKSym) || d->head_dim_v != kHeadDimV)
    return DIFFKV_UNSUPPORTED;
  if (!is_pow2(d->page_size) || d->page_size > 256) return DIFFKV_UNSUPPORTED;
  if (d->kv_dtype != DIFFKV_KV_BF16 && d->kv_dtype != DIFFKV_KV_FP8_E4M3) return DIFFKV_UNSUPPORTED;
  if (d->num_pages < 1 || d->max_seq_len < 1 || d->max_q_len < 1 || d->total_q < 1)
    return DIFFKV_INVALID_ARGUMENT;
  if (d->max_q_len > d->max_seq_len) return DIFFKV_INVALID_ARGUMENT;
  if (d->block_table_stride < 1) return DIFFKV_INVALID_ARGUMENT;
  if ((long long)d->block_table_stride * d->page_size < d->max_seq_len) return DIFFKV_INVALID_ARGUMENT;
  if (d->total_q < d->batch || (long long)d->total_q > (long long)d->batch * d->max_q_len)
    return DIFFKV_INVALID_ARGUMENT;
  if (d->force_num_splits < 0 || d->force_num_splits > kMaxForcedSplits) return DIFFKV_INVALID_ARGUMENT;
  if ((d->profile_start == nullptr) != (d->profile_stop == nullptr)) return DIFFKV_INVALID_ARGUMENT;
  if (entry == DIFFKV_ENTRY_DECODE && d->max_q_len != 1) return DIFFKV_INVALID_ARGUMENT;
  if (entry == DIFFKV_ENTRY_VERIFY && d->max_q_len > 16) return DIFFKV_INVALID_ARGUMENT;
  // Launch-shape limits: grid y and z, 32-bit element offsets into q and out
  // (which also bound one sequence's query rows), then the split grid's x.
  // The planner runs only on descriptors inside the first ones, so its
  // 64-bit products cannot overflow.
  if ((long long)d->batch * d->num_kv_heads > kMaxGridYZ) return DIFFKV_UNSUPPORTED;
  if ((long long)d->total_q * d->num_q_heads > (1LL << 31) / kHeadDimQK) return DIFFKV_UNSUPPORTED;
  if ((long long)d->max_q_len * (d->num_q_heads / d->num_kv_heads) > (1LL << 31) / kHeadDimQK)
    return DIFFKV_UNSUPPORTED;
  if (entry != DIFFKV_ENTRY_PREFILL) {
    const SplitPlan p = plan_split(split_part_desc(*d, entry), 0, kMaxCUs);
    if (p.grid_x > INT32_MAX) return DIFFKV_UNSUPPORTED;
  }
  return DIFFKV_OK;
}

}  // namespace diffkv
