// Gathers 64-key tiles of the paged K (192 wide) and V (128 wide) caches
// into LDS as bf16, shared by the split-KV and the prefill kernels.
//
// K and V live in two caches because their rows differ in width
// ("sglang PR 32818, Route asymmetric-KV models to fa4 on SM100"); FP8 E4M3
// rows are widened to bf16 on the way into LDS ("diffbot/MiMo-V2.6-Flash-RL-
// FP8KV-W4A8-2x-RTX-PRO-6000", What the kernels do).  A workgroup of NT
// threads (256 or 512) moves a tile as 16-byte units, consecutive lanes on
// consecutive pieces of a row, through registers: the caller keeps the next
// tiles' loads in flight (`Stage`s) and writes the oldest into LDS.  When
// the threads do not divide the tile evenly, whole waves take one unit fewer.
#pragma once

#include "device_common.hpp"
#include "plan.hpp"

namespace diffkv {

// bf16 per K row in LDS: the row plus 16 bytes (400 B at QK 192, 272 B at
// 128), so the 16 rows a K-fragment read touches fall in distinct banks.
template <int DQK> constexpr int kKLdsStride = DQK + 8;
constexpr int kVLdsStride = kHeadDimV + 16;   // bf16 per V row in LDS (288 B: the 16 rows of
                                               // a transposing read fall in distinct bank windows)
template <int DQK> constexpr int kKLdsElems = kTileKeys * kKLdsStride<DQK>;
constexpr int kVLdsElems = kTileKeys * kVLdsStride;

// Sixteen zero bytes (static device memory is zero-filled at load): the
// source of every load whose key lies outside the range a tile may read.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[16];

// NT threads move TK keys of each 64-key tile: all of it (TK = 64), or, for
// a loader private to one wave (NT = 64), the slice of TK keys starting at
// key_off that only this wave reads, so no barrier orders it against the
// other waves.
template <bool FP8, bool UPAGE, int DQK, int NT = 256, int TK = kTileKeys>
struct KvTile {
  static constexpr int ESZ = FP8 ? 1 : 2;
  static constexpr int K_UPR = DQK * ESZ / 16;          // 16-byte units per K row
  static constexpr int V_UPR = kHeadDimV * ESZ / 16;
  static constexpr int K_UNITS = TK * K_UPR;            // units per tile (slice)
  static constexpr int V_UNITS = TK * V_UPR;
  static constexpr int KU = (K_UNITS + NT - 1) / NT;    // units per thread per tile
  static constexpr int VU = (V_UNITS + NT - 1) / NT;
  static constexpr int NPK = UPAGE ? 1 : KU;            // page ids held per thread per tile
  static constexpr int NPV = UPAGE ? 1 : VU;
  // A thread's last unit may not exist when NT does not divide the tile;
  // the split is by whole waves (units come in multiples of 64).
  static_assert(K_UNITS % 64 == 0 && V_UNITS % 64 == 0 && NT % 64 == 0, "wave-uniform split");
  __device__ __forceinline__ bool k_has(int k) const { return tid + NT * k < K_UNITS; }
  __device__ __forceinline__ bool v_has(int k) const { return tid + NT * k < V_UNITS; }

  struct Pages { int k[NPK]; int v[NPV]; };
  struct Stage { u32x4 k[KU]; u32x4 v[VU]; };

  const uint8_t* k_head;     // k_cache + g * row bytes
  const uint8_t* v_head;
  const int32_t* bt;         // this sequence's block-table row
  size_t k_slot_bytes, v_slot_bytes;   // Hkv rows per slot
  int lp, pmask, kv_lo, kv_hi, t_last, tid;
  int koff;                  // first key of this loader's slice in each tile
#ifdef DIFFKV_DEBUG
  int num_pages = 1;         // entries outside [0, num_pages) read page 0
#endif
  // Large pages: byte offset of each of this thread's units from the tile's
  // first slot (the tile lies inside one page, so rows are slot-contiguous).
  uint32_t k_off[UPAGE ? KU : 1], v_off[UPAGE ? VU : 1];

  __device__ __forceinline__ KvTile(const uint8_t* k_cache, const uint8_t* v_cache,
                                    const int32_t* bt_row, int hkv, int g, int log2_page,
                                    int lo, int hi, int t_end, int thread, int key_off = 0,
                                    int pages = 1)
      : k_head(k_cache + (size_t)g * DQK * ESZ),
        v_head(v_cache + (size_t)g * kHeadDimV * ESZ),
        bt(bt_row),
        k_slot_bytes((size_t)hkv * DQK * ESZ),
        v_slot_bytes((size_t)hkv * kHeadDimV * ESZ),
        lp(log2_page), pmask((1 << log2_page) - 1), kv_lo(lo), kv_hi(hi), t_last(t_end - 1),
        tid(thread), koff(key_off) {
#ifdef DIFFKV_DEBUG
    num_pages = pages;
#else
    (void)pages;
#endif
    if constexpr (UPAGE) {
#pragma unroll
      for (int k = 0; k < KU; ++k) k_off[k] = (uint32_t)(k_row(k) * k_slot_bytes + k_piece(k) * 16);
#pragma unroll
      for (int k = 0; k < VU; ++k) v_off[k] = (uint32_t)(v_key(k) * v_slot_bytes + v_piece(k) * 16);
    }
  }

  // Key of unit k within the 64-key tile (this loader's slice starts at
  // koff); units past the slice (k_has false) map to its first key and read
  // the zero row.
  __device__ __forceinline__ int k_row(int k) const { return koff + (k_has(k) ? (tid + NT * k) / K_UPR : 0); }
  __device__ __forceinline__ int k_piece(int k) const { return (tid + NT * k) % K_UPR; }
  __device__ __forceinline__ int v_key(int k) const { return koff + (v_has(k) ? (tid + NT * k) / V_UPR : 0); }
  __device__ __forceinline__ int v_piece(int k) const { return (tid + NT * k) % V_UPR; }
  __device__ __forceinline__ bool readable(int j) const { return j >= kv_lo && j < kv_hi; }

  // Physical page ids of tile t.  Every load here and in fetch_data is
  // unconditional (a branch around a load makes the compiler wait for all
  // loads in flight): tiles past the last re-read the last tile, and keys
  // outside [kv_lo, kv_hi) read the zero row instead of their page, so a
  // page that holds no readable key is never touched.
  __device__ __forceinline__ void fetch_pages(int t, Pages& p) const {
    const int tc = min(t, t_last);
    if constexpr (UPAGE) {
      p.k[0] = scalar_load(bt, (tc * kTileKeys) >> lp);
      p.v[0] = p.k[0];
    } else {
#pragma unroll
      for (int k = 0; k < KU; ++k) {
        const int j = tc * kTileKeys + k_row(k);
        p.k[k] = bt[(readable(j) ? j : kv_lo) >> lp];
      }
#pragma unroll
      for (int k = 0; k < VU; ++k) {
        const int j = tc * kTileKeys + v_key(k);
        p.v[k] = bt[(readable(j) ? j : kv_lo) >> lp];
      }
    }
#ifdef DIFFKV_DEBUG
    auto check = [&](int& page) {
      if ((unsigned)page >= (unsigned)num_pages) {
        debug_flag(kDbgPage);
        page = 0;
      }
    };
#pragma unroll
    for (int k = 0; k < NPK; ++k) check(p.k[k]);
#pragma unroll
    for (int k = 0; k < NPV; ++k) check(p.v[k]);
#endif
  }

  // Gather tile t's K and V rows into registers.
  __device__ __forceinline__ void fetch_data(int t, const Pages& p, Stage& st) const {
    const int tc = min(t, t_last);
    if constexpr (UPAGE) {
      const size_t slot0 = ((size_t)p.k[0] << lp) + (size_t)((tc * kTileKeys) & pmask);
      const uint8_t* kb = k_head + slot0 * k_slot_bytes;
      const uint8_t* vb = v_head + slot0 * v_slot_bytes;
#pragma unroll
      for (int k = 0; k < KU; ++k) {
        const uint8_t* src = k_has(k) && readable(tc * kTileKeys + k_row(k)) ? kb + k_off[k] : g_zero_row;
        st.k[k] = *reinterpret_cast<const u32x4*>(src);
      }
#pragma unroll
      for (int k = 0; k < VU; ++k) {
        const uint8_t* src = v_has(k) && readable(tc * kTileKeys + v_key(k)) ? vb + v_off[k] : g_zero_row;
        st.v[k] = *reinterpret_cast<const u32x4*>(src);
      }
      return;
    }
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      const int j = tc * kTileKeys + k_row(k);
      const size_t slot = ((size_t)(UPAGE ? p.k[0] : p.k[k]) << lp) | (size_t)(j & pmask);
      const uint8_t* src = k_has(k) && readable(j) ? k_head + slot * k_slot_bytes + k_piece(k) * 16 : g_zero_row;
      st.k[k] = *reinterpret_cast<const u32x4*>(src);
    }
#pragma unroll
    for (int k = 0; k < VU; ++k) {
      const int j = tc * kTileKeys + v_key(k);
      const size_t slot = ((size_t)(UPAGE ? p.v[0] : p.v[k]) << lp) | (size_t)(j & pmask);
      const uint8_t* src = v_has(k) && readable(j) ? v_head + slot * v_slot_bytes + v_piece(k) * 16 : g_zero_row;
      st.v[k] = *reinterpret_cast<const u32x4*>(src);
    }
  }

  // Registers -> LDS as bf16, both row-major (FP8 widened on the way).
  __device__ __forceinline__ void store(const Stage& st, uint16_t* k_lds, uint16_t* v_lds) const {
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      if (!k_has(k)) continue;
      const int row = k_row(k), piece = k_piece(k);
      if constexpr (FP8) {
        const u32x2 c0 = e4m3x4_to_bf16x4(st.k[k].x), c1 = e4m3x4_to_bf16x4(st.k[k].y);
        const u32x2 c2 = e4m3x4_to_bf16x4(st.k[k].z), c3 = e4m3x4_to_bf16x4(st.k[k].w);
        u32x4* dst = reinterpret_cast<u32x4*>(k_lds + row * kKLdsStride<DQK> + piece * 16);
        dst[0] = u32x4{c0.x, c0.y, c1.x, c1.y};
        dst[1] = u32x4{c2.x, c2.y, c3.x, c3.y};
      } else {
        *reinterpret_cast<u32x4*>(k_lds + row * kKLdsStride<DQK> + piece * 8) = st.k[k];
      }
    }
#pragma unroll
    for (int k = 0; k < VU; ++k) {
      if (!v_has(k)) continue;
      const int key = v_key(k), piece = v_piece(k);
      if constexpr (FP8) {
        const u32x2 c0 = e4m3x4_to_bf16x4(st.v[k].x), c1 = e4m3x4_to_bf16x4(st.v[k].y);
        const u32x2 c2 = e4m3x4_to_bf16x4(st.v[k].z), c3 = e4m3x4_to_bf16x4(st.v[k].w);
        u32x4* dst = reinterpret_cast<u32x4*>(v_lds + key * kVLdsStride + piece * 16);
        dst[0] = u32x4{c0.x, c0.y, c1.x, c1.y};
        dst[1] = u32x4{c2.x, c2.y, c3.x, c3.y};
      } else {
        *reinterpret_cast<u32x4*>(v_lds + key * kVLdsStride + piece * 8) = st.v[k];
      }
    }
  }
};

// Rows per new token (the GQA group) as a plain int or a FastDiv.
__device__ __forceinline__ int group_size(int G) { return G; }
__device__ __forceinline__ int group_size(const FastDiv& G) { return G.value(); }
// r / G for r >= -1 (truncating: -1 / G = 0).
__device__ __forceinline__ int token_of_row(int r, int G) { return r / G; }
__device__ __forceinline__ int token_of_row(int r, const FastDiv& G) { return r > 0 ? (int)G.div((uint32_t)r) : 0; }

// Keys one block of query rows can see: the union of its rows' ranges.
// Row r of a (sequence, KV head) is new token r / G.
template <class Group>
__device__ __forceinline__ void qtile_key_range(int L, int n, const Group& G, int qt, int rows, int window,
                                                int& kv_lo, int& kv_hi) {
  const int r_lo = qt * rows;
  const int r_hi = min(n * group_size(G), r_lo + rows) - 1;
  const int p_lo = L - n + token_of_row(r_lo, G);
  const int p_hi = L - n + token_of_row(r_hi, G);
  kv_lo = window > 0 ? max(0, p_lo - window + 1) : 0;
  kv_hi = p_hi + 1;
}

// The same range cut to the keys [klo, khi) (a context partial's share); it
// may come out empty (hi <= lo).
template <class Group>
__device__ __forceinline__ void pair_key_range(int L, int n, const Group& G, int qt, int rows, int window,
                                               int klo, int khi, int& kv_lo, int& kv_hi) {
  qtile_key_range(L, n, G, qt, rows, window, kv_lo, kv_hi);
  kv_lo = max(kv_lo, klo);
  kv_hi = min(kv_hi, khi);
}

}  // namespace diffkv
