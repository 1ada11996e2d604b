// Split-KV paged attention for decode and speculative verify on gfx950, plus
// the log-sum-exp merge of the split partials.
//
// Work decomposition ("diffkv/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000",
// What the kernels do: without split-KV a multi-token verify ran on a handful
// of workgroups; split-KV fixed that): one workgroup per (key split, query
// tile, sequence * KV head).  A query tile is up to 64 rows; row r of a
// (sequence, KV head) is new token r / G and query head g*G + r % G, so a
// whole verify block of all G heads shares one pass over the keys (one
// program per whole verify, same page).
//
// Per 64-key tile the workgroup gathers K (192 wide) and V (128 wide) rows
// through the block table with 16-byte loads, converts FP8 E4M3 to bf16 on
// the way into LDS, and stores V transposed so it can feed the matrix cores.
// Each wave owns one 16-row query tile and a quarter, half or all of the 64
// keys (4, 2 or 1 row tiles per workgroup) and runs
//   S^T = K * Q^T        (v_mfma_f32_16x16x32_bf16, 6 steps over 192 dims)
//   mask -> online softmax in base 2 (rows live in lanes, keys across the
//           4 lane groups: two xor-shuffles per reduction)
//   O^T += V^T * P^T     (v_mfma_f32_16x16x16_bf16, 8 tiles over 128 dims)
// Keeping S and O transposed puts one query row in each lane, so the softmax
// rescale needs no data movement between lanes.
// The next tile's global loads are issued before the current tile's math.
#pragma once

#include "device_common.hpp"
#include "plan.hpp"

namespace diffkv {

constexpr int kKLdsStride = kHeadDimQK + 8;   // bf16 per K row in LDS (400 B, conflict-free reads)
constexpr int kVtLdsStride = kTileKeys + 4;    // bf16 per V^T row in LDS (136 B)
constexpr int kKLdsElems = kTileKeys * kKLdsStride;
constexpr int kVtLdsElems = kHeadDimV * kVtLdsStride;

struct SplitArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* q_lens;
  const float* sinks;
  float* part_o;
  float* part_lse;
  uint16_t* out;
  float* lse_out;
  int32_t* count_out;
  int hq, hkv, group, log2_page, bt_stride, window;
  int n_qtiles, num_splits;
  float scale_log2;   // softmax_scale * k_scale * log2(e)
  float v_scale;      // v_scale for FP8 caches, 1 for bf16
};

// Keys one query tile can see: the union of its rows' ranges.
__device__ __forceinline__ void qtile_key_range(int L, int n, int G, int qt, int rows, int window,
                                                int& kv_lo, int& kv_hi) {
  const int r_lo = qt * rows;
  const int r_hi = min(n * G, r_lo + rows) - 1;
  const int p_lo = L - n + r_lo / G;
  const int p_hi = L - n + r_hi / G;
  kv_lo = window > 0 ? max(0, p_lo - window + 1) : 0;
  kv_hi = p_hi + 1;
}

// Tiles of split s among S equal shares of the aligned tile range.
__device__ __forceinline__ void split_tiles(int kv_lo, int kv_hi, int S, int s, int& t_begin,
                                            int& t_end, int& n_valid) {
  const int t0 = kv_lo / kTileKeys;
  const int t1 = (kv_hi + kTileKeys - 1) / kTileKeys;
  const int nt = t1 - t0;
  const int tps = (nt + S - 1) / S;
  t_begin = t0 + s * tps;
  t_end = min(t1, t_begin + tps);
  n_valid = (nt + tps - 1) / tps;
}

template <bool FP8, int RT, bool DIRECT, bool COUNT>
__global__ __launch_bounds__(256) void split_attn_kernel(const SplitArgs a) {
  constexpr int ROWS = 16 * RT;
  constexpr int KW = 4 / RT;                 // waves splitting the keys of one row tile
  constexpr int SUBS = kTileKeys / 16 / KW;  // 16-key subtiles per wave per tile
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int K_UPR = kHeadDimQK * ESZ / 16;   // 16-byte units per K row
  constexpr int V_UPR = kHeadDimV * ESZ / 16;
  constexpr int KU = kTileKeys * K_UPR / 256;    // units per thread per tile
  constexpr int VU = kTileKeys * V_UPR / 256;
  static_assert(kTileKeys * K_UPR % 256 == 0 && kTileKeys * V_UPR % 256 == 0, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t lds[kKLdsElems + kVtLdsElems];
  uint16_t* k_lds = lds;
  uint16_t* vt_lds = lds + kKLdsElems;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int rt = wave % RT, kg = wave / RT;
  const int s = blockIdx.x, qt = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.hkv, g = bg % a.hkv;
  const int G = a.group;

  const int L = a.seq_lens[b];
  const int n = a.q_lens ? a.q_lens[b] : 1;
  if (qt * ROWS >= n * G) return;
  int kv_lo, kv_hi, t_begin, t_end, n_valid;
  qtile_key_range(L, n, G, qt, ROWS, a.window, kv_lo, kv_hi);
  split_tiles(kv_lo, kv_hi, a.num_splits, s, t_begin, t_end, n_valid);
  if (t_begin >= t_end) return;
  const int r0 = seq_row_start(a.q_lens, b);

  // The query row this lane owns in S^T / O^T.
  const int R = qt * ROWS + rt * 16 + col;
  const bool row_ok = R < n * G;
  const int tok = row_ok ? R / G : 0;
  const int h = g * G + (row_ok ? R % G : 0);
  const int p_row = L - n + tok;
  const int lo_row = a.window > 0 ? max(0, p_row - a.window + 1) : 0;
  const int hi_row = row_ok ? p_row : -1;     // empty interval for padding rows

  // Q^T operand: contraction chunk c carries dims 32c + 8*grp .. +7.
  u32x4 qreg[6];
  {
    const uint16_t* qp = a.q + ((size_t)(r0 + tok) * a.hq + h) * kHeadDimQK + 8 * grp;
#pragma unroll
    for (int c = 0; c < 6; ++c)
      qreg[c] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 32 * c) : u32x4{0, 0, 0, 0};
  }

  float m = -INFINITY, l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  int cnt = 0;

  const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
  const int pmask = (1 << a.log2_page) - 1;
  const size_t k_row_bytes = (size_t)kHeadDimQK * ESZ, v_row_bytes = (size_t)kHeadDimV * ESZ;
  u32x4 kbuf[KU], vbuf[VU];

  // Gather one tile's K and V rows into registers; keys outside the union
  // range are never touched (their pages may be unmapped) and read as zero.
  auto load_tile = [&](int t) {
    const int base = t * kTileKeys;
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      const int u = tid + 256 * k;
      const int row = u / K_UPR, piece = u % K_UPR;
      const int j = base + row;
      kbuf[k] = u32x4{0, 0, 0, 0};
      if (j >= kv_lo && j < kv_hi) {
        const size_t slot = ((size_t)bt[j >> a.log2_page] << a.log2_page) | (size_t)(j & pmask);
        kbuf[k] = *reinterpret_cast<const u32x4*>(a.k_cache + (slot * a.hkv + g) * k_row_bytes + piece * 16);
      }
    }
#pragma unroll
    for (int k = 0; k < VU; ++k) {
      const int u = tid + 256 * k;
      const int row = u / V_UPR, piece = u % V_UPR;
      const int j = base + row;
      vbuf[k] = u32x4{0, 0, 0, 0};
      if (j >= kv_lo && j < kv_hi) {
        const size_t slot = ((size_t)bt[j >> a.log2_page] << a.log2_page) | (size_t)(j & pmask);
        vbuf[k] = *reinterpret_cast<const u32x4*>(a.v_cache + (slot * a.hkv + g) * v_row_bytes + piece * 16);
      }
    }
  };

  // Registers -> LDS as bf16: K row-major, V transposed (dims x keys).
  auto store_tile = [&]() {
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      const int u = tid + 256 * k;
      const int row = u / K_UPR, piece = u % K_UPR;
      if constexpr (FP8) {
        const u32x2 c0 = e4m3x4_to_bf16x4(kbuf[k].x), c1 = e4m3x4_to_bf16x4(kbuf[k].y);
        const u32x2 c2 = e4m3x4_to_bf16x4(kbuf[k].z), c3 = e4m3x4_to_bf16x4(kbuf[k].w);
        u32x4* dst = reinterpret_cast<u32x4*>(k_lds + row * kKLdsStride + piece * 16);
        dst[0] = u32x4{c0.x, c0.y, c1.x, c1.y};
        dst[1] = u32x4{c2.x, c2.y, c3.x, c3.y};
      } else {
        *reinterpret_cast<u32x4*>(k_lds + row * kKLdsStride + piece * 8) = kbuf[k];
      }
    }
#pragma unroll
    for (int k = 0; k < VU; ++k) {
      const int u = tid + 256 * k;
      const int row = u / V_UPR, piece = u % V_UPR;
      if constexpr (FP8) {
        const u32x2 c[4] = {e4m3x4_to_bf16x4(vbuf[k].x), e4m3x4_to_bf16x4(vbuf[k].y),
                            e4m3x4_to_bf16x4(vbuf[k].z), e4m3x4_to_bf16x4(vbuf[k].w)};
        uint16_t* dst = vt_lds + (piece * 16) * kVtLdsStride + row;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[(4 * e + 0) * kVtLdsStride] = (uint16_t)(c[e].x & 0xffff);
          dst[(4 * e + 1) * kVtLdsStride] = (uint16_t)(c[e].x >> 16);
          dst[(4 * e + 2) * kVtLdsStride] = (uint16_t)(c[e].y & 0xffff);
          dst[(4 * e + 3) * kVtLdsStride] = (uint16_t)(c[e].y >> 16);
        }
      } else {
        const uint32_t w[4] = {vbuf[k].x, vbuf[k].y, vbuf[k].z, vbuf[k].w};
        uint16_t* dst = vt_lds + (piece * 8) * kVtLdsStride + row;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[(2 * e + 0) * kVtLdsStride] = (uint16_t)(w[e] & 0xffff);
          dst[(2 * e + 1) * kVtLdsStride] = (uint16_t)(w[e] >> 16);
        }
      }
    }
  };

  load_tile(t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < t_end) load_tile(t + 1);

#pragma unroll
    for (int sub = 0; sub < SUBS; ++sub) {
      const int kb = (kg * SUBS + sub) * 16;
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kp = k_lds + (kb + col) * kKLdsStride + 8 * grp;
#pragma unroll
      for (int c = 0; c < 6; ++c)
        sacc = mfma_16x16x32(*reinterpret_cast<const u32x4*>(kp + 32 * c), qreg[c], sacc);

      // sacc[i] = S^T[key kb + 4*grp + i][row col].  Masked by select only.
      const int j0 = t * kTileKeys + kb + 4 * grp;
      float x[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + i;
        const bool vis = j >= lo_row && j <= hi_row;
        x[i] = vis ? sacc[i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[i]);
        if constexpr (COUNT) cnt += vis ? 1 : 0;
      }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float pr[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = fast_exp2(x[i] - m_use);
        ps += pr[i];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l = l * alpha + ps;
      m = m_new;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) o[nn] *= alpha;

      const u32x2 pb = u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
      const uint16_t* vp = vt_lds + col * kVtLdsStride + kb + 4 * grp;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn)
        o[nn] = mfma_16x16x16(*reinterpret_cast<const u32x2*>(vp + nn * 16 * kVtLdsStride), pb, o[nn]);
    }
  }

  if constexpr (COUNT) {
    cnt += __shfl_xor(cnt, 16, 64);
    cnt += __shfl_xor(cnt, 32, 64);
    if (row_ok && grp == 0 && a.count_out)
      atomicAdd(a.count_out + (size_t)(r0 + tok) * a.hq + h, cnt);
  }

  // Waves that split the keys of one row tile combine through LDS.
  if constexpr (KW > 1) {
    constexpr int STR = 34;
    static_assert(4 * 64 * STR * 4 <= (kKLdsElems + kVtLdsElems) * 2, "reduction fits");
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
    float* mine = red + (wave * 64 + lane) * STR;
    mine[0] = m;
    mine[1] = l;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[2 + 4 * nn + i] = o[nn][i];
    __syncthreads();
    if (kg != 0) return;
    float M = m;
#pragma unroll
    for (int k = 1; k < KW; ++k) M = fmaxf(M, red[((rt + k * RT) * 64 + lane) * STR]);
    const float M_use = M == -INFINITY ? 0.f : M;
    const float f0 = fast_exp2(m - M_use);
    l *= f0;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) o[nn] *= f0;
#pragma unroll
    for (int k = 1; k < KW; ++k) {
      const float* other = red + ((rt + k * RT) * 64 + lane) * STR;
      const float fk = fast_exp2(other[0] - M_use);
      l += fk * other[1];
#pragma unroll
      for (int nn = 0; nn < 8; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nn][i] += fk * other[2 + 4 * nn + i];
    }
    m = M;
  }

  if (!row_ok) return;
  const size_t out_row = (size_t)(r0 + tok) * a.hq + h;
  if constexpr (DIRECT) {
    float coef;
    if (a.sinks) {
      const float s2 = a.sinks[h] * kLog2e;
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
  } else {
    const size_t prow = (((size_t)bg * a.n_qtiles + qt) * a.num_splits + s) * ROWS + rt * 16 + col;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* pp = a.part_o + prow * kHeadDimV + 4 * grp;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) *reinterpret_cast<f32x4*>(pp + 16 * nn) = o[nn] * inv;
    if (grp == 0) a.part_lse[prow] = l > 0.f ? m + log2f(l) : -INFINITY;
  }
}

// Combines the split partials of one query row: weights 2^(lse_s - M), the
// sink joining the denominator, v_scale, bf16 store.  One wave per row, two
// output dims per lane.  Splits are read in a fixed order (deterministic).
template <int ROWS>
__global__ __launch_bounds__(64) void split_merge_kernel(const SplitArgs a) {
  const int lane = threadIdx.x;
  const int qt = blockIdx.x / ROWS, r = blockIdx.x % ROWS;
  const int bg = blockIdx.y;
  const int b = bg / a.hkv, g = bg % a.hkv;
  const int G = a.group;
  const int L = a.seq_lens[b];
  const int n = a.q_lens ? a.q_lens[b] : 1;
  const int R = qt * ROWS + r;
  if (R >= n * G) return;
  int kv_lo, kv_hi, t_begin, t_end, n_valid;
  qtile_key_range(L, n, G, qt, ROWS, a.window, kv_lo, kv_hi);
  split_tiles(kv_lo, kv_hi, a.num_splits, 0, t_begin, t_end, n_valid);
  const int r0 = seq_row_start(a.q_lens, b);
  const int tok = R / G, h = g * G + R % G;

  const size_t prow0 = ((size_t)bg * a.n_qtiles + qt) * a.num_splits * ROWS + r;
  float M = -INFINITY;
  for (int s = 0; s < n_valid; ++s) M = fmaxf(M, a.part_lse[prow0 + (size_t)s * ROWS]);
  const float s2 = a.sinks ? a.sinks[h] * kLog2e : -INFINITY;
  const float Mt = fmaxf(M, s2);
  f32x2 acc = f32x2{0.f, 0.f};
  float ksum = 0.f;
  for (int s = 0; s < n_valid; ++s) {
    const size_t pr = prow0 + (size_t)s * ROWS;
    const float w = fast_exp2(a.part_lse[pr] - Mt);
    ksum += w;
    acc += w * *reinterpret_cast<const f32x2*>(a.part_o + pr * kHeadDimV + 2 * lane);
  }
  const float den = ksum + (a.sinks ? fast_exp2(s2 - Mt) : 0.f);
  const float coef = a.v_scale / den;
  const size_t out_row = (size_t)(r0 + tok) * a.hq + h;
  *reinterpret_cast<uint32_t*>(a.out + out_row * kHeadDimV + 2 * lane) = pack_bf16x2(acc.x * coef, acc.y * coef);
  if (a.lse_out && lane == 0) a.lse_out[out_row] = (Mt + log2f(ksum)) * kLn2;
}

__global__ void fill_i32_kernel(int32_t* p, size_t n, int32_t v) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace diffkv
