// Paged KV write: the new tokens' K and V rows stored into their cache slots.
//
// The FP8 KV cache of "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000"
// (intro: E4M3 K/V with per-tensor scales) is filled one step before
// attention reads it; K (192 wide, or 128 for symmetric heads) and V (128
// wide) live in two caches
// ("sglang PR 32818, Route asymmetric-KV models to fa4 on SM100").  New token
// i of sequence b sits at position p = L - n + i and goes to slot p % P of
// page block_table[b][p / P].  bf16 caches take the rows as they are; FP8
// caches take E4M3FN codes of x / scale (division in fp32, clamped to +-448,
// round to nearest even, NaN kept with its sign).
//
// A row is cut into 8-value units (K 24 or 16, V 16 per KV head); one thread per
// unit, the units of one sequence's new tokens numbered token-major over a
// grid of (ceil(max_q_len * units per token / 256), batch) workgroups, so
// consecutive threads read and write contiguous runs of each row.  A
// token whose position, packed row or page falls outside its bounds is
// skipped, so bad device data never turns into a stray write.
#pragma once

#include "device_common.hpp"
#include "plan.hpp"

namespace diffkv {

struct KvWriteArgs {
  const uint16_t* k_new;     // bf16 [total_q, Hkv, DQK]
  const uint16_t* v_new;     // bf16 [total_q, Hkv, 128]
  uint8_t* k_cache;          // [pages, P, Hkv, DQK] bf16 or E4M3 codes
  uint8_t* v_cache;          // [pages, P, Hkv, 128]
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* q_lens;     // NULL: one new token per sequence
  int hkv, log2_page, bt_stride, num_pages, total_q;
  float k_scale, v_scale;    // FP8 only
};

constexpr int kVUnits = kHeadDimV / 8;      // 8-value units per V row

// Eight fp32 values -> eight E4M3FN codes (byte j = value j): clamp to
// +-448 (NaN kept), v_cvt_pk_fp8_f32 rounds to nearest even; NaN lanes get
// the code 0x7F with the value's sign.
__device__ __forceinline__ u32x2 encode8_e4m3(const float (&y)[8]) {
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float c[4];
    uint32_t nan_fix = 0, nan_mask = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = y[4 * h + j];
      const bool nan = v != v;
      c[j] = nan ? 0.f : fminf(fmaxf(v, -448.f), 448.f);
      const uint32_t sign = (__builtin_bit_cast(uint32_t, v) >> 31) << 7;
      nan_mask |= nan ? 0xFFu << (8 * j) : 0u;
      nan_fix |= nan ? (0x7Fu | sign) << (8 * j) : 0u;
    }
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], packed, true);
    w[h] = ((uint32_t)packed & ~nan_mask) | nan_fix;
  }
  return u32x2{w[0], w[1]};
}

template <bool FP8, int DQK>
__global__ __launch_bounds__(256) void kv_write_kernel(const KvWriteArgs a) {
  constexpr int kKUnits = DQK / 8;          // 8-value units per K row
  const int b = blockIdx.y;
  const int n = a.q_lens ? a.q_lens[b] : 1;
  const int per_token = a.hkv * (kKUnits + kVUnits);
  if ((int)blockIdx.x * 256 >= n * per_token) return;     // whole workgroup past the end
  const int r0 = seq_row_start(a.q_lens, b);              // needs every lane of the wave
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= n * per_token) return;
  const int i = u / per_token;
  const int rem = u - i * per_token;
  const int g = rem / (kKUnits + kVUnits);
  const int c = rem - g * (kKUnits + kVUnits);
  const bool is_k = c < kKUnits;
  const int piece = is_k ? c : c - kKUnits;
  const int width = is_k ? DQK : kHeadDimV;
  const int p = a.seq_lens[b] - n + i;
  if (p < 0 || (p >> a.log2_page) >= a.bt_stride || r0 + i >= a.total_q) return;
  const int page = a.block_table[(size_t)b * a.bt_stride + (p >> a.log2_page)];
  if (page < 0 || page >= a.num_pages) return;
  const size_t slot = ((size_t)page << a.log2_page) | (size_t)(p & ((1 << a.log2_page) - 1));
  const uint16_t* src = (is_k ? a.k_new : a.v_new) + ((size_t)(r0 + i) * a.hkv + g) * width + piece * 8;
  const u32x4 in = *reinterpret_cast<const u32x4*>(src);
  if constexpr (FP8) {
    uint8_t* dst = (is_k ? a.k_cache : a.v_cache) + (slot * a.hkv + g) * width + piece * 8;
    const float scale = is_k ? a.k_scale : a.v_scale;
    float y[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 x = unpack_bf16x2(in[j]);
      y[2 * j] = x.x / scale;
      y[2 * j + 1] = x.y / scale;
    }
    *reinterpret_cast<u32x2*>(dst) = encode8_e4m3(y);
  } else {
    uint8_t* dst = (is_k ? a.k_cache : a.v_cache) + ((slot * a.hkv + g) * width + piece * 8) * 2;
    *reinterpret_cast<u32x4*>(dst) = in;
  }
}

}  // namespace diffkv
