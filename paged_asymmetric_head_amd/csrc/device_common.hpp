// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// wrappers, storage-format conversion and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "fast_div.hpp"

namespace diffkv {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// S/O tiles: D(16x16, fp32) += A(16 x K) * B(K x 16) on the matrix cores.
// Operand layout shared by both shapes: lane l supplies row (l % 16) of A and
// column (l % 16) of B, its lane group (l / 16) a slice of the contraction;
// D comes back as rows 4*(l/16)+i, column l%16 for i = 0..3.  On gfx950 one
// 16x16x16 takes about as long as one 16x16x32 (half the rate), so the
// contractions use K = 32 wherever a wave holds 32 keys.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Four / eight bf16 ones: MFMA operands that sum the other operand's columns.
constexpr u32x2 kOnesBf16x4 = u32x2{0x3F803F80u, 0x3F803F80u};
constexpr u32x4 kOnesBf16x8 = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

__device__ __forceinline__ u32x4 cat(u32x2 lo, u32x2 hi) { return u32x4{lo.x, lo.y, hi.x, hi.y}; }

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of
// 16 lanes the four 16-bit values each lane reads are concatenated in lane
// order into S[0..64); lane i of the group receives S[i], S[16+i], S[32+i],
// S[48+i].
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax reference point (base-2 logit domain).  A row keeps its
// reference m while the tile max stays within kStaleMaxSlack of it, so the
// unnormalised P = 2^(x - m) stays below 2^kStaleMaxSlack (well inside bf16
// and fp32 range) and O, l need no rescale for most tiles; m, l and O stay
// mutually consistent, so the normalised result is the same.  A row with no
// visible key yet has m = -inf and takes the first finite max.
constexpr float kStaleMaxSlack = 8.f;
__device__ __forceinline__ float next_reference(float m, float tile_max) {
  return tile_max > m + kStaleMaxSlack ? tile_max : m;
}

// Two fp32 -> two bf16 in one word, round to nearest even (one
// v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Two bf16 codes in one word (low half first) -> two floats, exactly.
__device__ __forceinline__ f32x2 unpack_bf16x2(uint32_t w) {
  return f32x2{__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xFFFF0000u)};
}

// Two fp32 -> two fp16 in one word (round to nearest even), and back.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
__device__ __forceinline__ f32x2 unpack_f16x2(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}

// Four OCP E4M3FN codes (one 32-bit word, byte 0 first) -> four bf16 codes in
// two words, with gfx950's packed converter at scale 1.0.  Every finite
// E4M3 value has at most 4 significant bits and an exponent in [-9, 8], so
// it is exact in bf16; NaN codes give NaN.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// v_max_f32 of two raw registers.  Written out because fmaxf here costs
// three more instructions: the compiler cannot tell that the row-swap
// results below are canonical floats, so it re-canonicalises both operands
// (v_max x, x) before the max.  The operands are scores, -inf or magnitudes,
// never NaN, so no quieting is needed.  Also opaque to the compiler: with
// fmaxf on the swap results this compiler (ROCm 7.2 clang) once replaced
// the second result by the first and the max silently disappeared.
__device__ __forceinline__ float max_raw(uint32_t a, uint32_t b) {
  float r;
  asm volatile("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Max over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48) on
// the VALU, with gfx950's row swaps instead of LDS permutes.  Called with
// both operands equal, v_permlane16_swap returns the values of the even and
// the odd row of each row pair, v_permlane32_swap those of the low and the
// high half-wave.
__device__ __forceinline__ float max_over_lane_groups(float v) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const uint32_t y = __builtin_bit_cast(uint32_t, max_raw(a[0], a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return max_raw(b[0], b[1]);
}

// Wave-wide scans and reductions on the VALU: DPP row shifts inside each
// 16-lane row (lanes whose source lies before the row start keep `fill`),
// then the four row totals read with v_readlane.  A __shfl_xor / __shfl_up
// ladder compiles to one LDS permute per step, six dependent LDS round trips
// per ladder, and the split plan runs three ladders before its first K/V
// load.  The reductions return the same value in every lane.
template <int N>
__device__ __forceinline__ int row_shr(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, 0x110 + N, 0xf, 0xf, false);   // DPP row_shr:N
}
template <int N>
__device__ __forceinline__ float row_shr(float v, float fill) {
  return __builtin_bit_cast(float, row_shr<N>(__builtin_bit_cast(int, v), __builtin_bit_cast(int, fill)));
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_scan_int(int v) {
  v += row_shr<1>(v, 0);
  v += row_shr<2>(v, 0);
  v += row_shr<4>(v, 0);
  v += row_shr<8>(v, 0);
  const int t0 = __builtin_amdgcn_readlane(v, 15);
  const int t1 = __builtin_amdgcn_readlane(v, 31);
  const int t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane_id() >> 4;
  return v + (row > 0 ? t0 : 0) + (row > 1 ? t1 : 0) + (row > 2 ? t2 : 0);
}

__device__ __forceinline__ int wave_sum_int(int v) {
  v += row_shr<1>(v, 0);
  v += row_shr<2>(v, 0);
  v += row_shr<4>(v, 0);
  v += row_shr<8>(v, 0);
  return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) +
         __builtin_amdgcn_readlane(v, 47) + __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_max_all(float v) {
  v = fmaxf(v, row_shr<1>(v, -INFINITY));
  v = fmaxf(v, row_shr<2>(v, -INFINITY));
  v = fmaxf(v, row_shr<4>(v, -INFINITY));
  v = fmaxf(v, row_shr<8>(v, -INFINITY));
  return fmaxf(fmaxf(readlane_f(v, 15), readlane_f(v, 31)), fmaxf(readlane_f(v, 47), readlane_f(v, 63)));
}

__device__ __forceinline__ float wave_sum_all(float v) {
  v += row_shr<1>(v, 0.f);
  v += row_shr<2>(v, 0.f);
  v += row_shr<4>(v, 0.f);
  v += row_shr<8>(v, 0.f);
  return (readlane_f(v, 15) + readlane_f(v, 31)) + (readlane_f(v, 47) + readlane_f(v, 63));
}

// p[i] for a wave-uniform i, as a scalar load through the constant address
// space, for arrays the kernels only read (block tables, sequence lengths).
// Through a plain pointer such a load becomes a vector load followed by
// v_readfirstlane; the wait for it then also waits for every vector load
// issued before it (that counter is in order), and the compiler may place
// that wait right behind the next tile's data loads, so the current tile's
// products wait for the next tile (one build of the long-verify kernel took
// 36.5 instead of 29.9 us that way).
__device__ __forceinline__ int32_t scalar_load(const int32_t* p, long long i) {
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  return ((const_i32*)p)[i];
}

// Debug builds (-DDIFFKV_DEBUG) check the preconditions on device data that
// the host cannot see: each violation sets a bit in a device-wide word (read
// and cleared by diffkv_attn_debug_flags) and the offending value is replaced
// by one that keeps every access in bounds, so the call finishes with a
// meaningless result instead of touching memory it must not.  Release
// builds compile none of this.
#ifdef DIFFKV_DEBUG
__device__ uint32_t g_debug_flags;
constexpr uint32_t kDbgQLen = 1;      // q_len outside [1, seq_len] or above max_q_len
constexpr uint32_t kDbgSeqLen = 2;    // seq_len outside [0, max_seq_len]
constexpr uint32_t kDbgPage = 4;      // a block-table entry read outside [0, num_pages)
constexpr uint32_t kDbgRows = 8;      // sum(q_lens) != total_q (a row outside [0, total_q))
__device__ __forceinline__ void debug_flag(uint32_t bits) { atomicOr(&g_debug_flags, bits); }
#endif

// Value of x in lane `lane` (wave-uniform) for every lane.
__device__ __forceinline__ int read_lane(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }

// Timeline builds (-DDIFFKV_TIMELINE, shipped as libdiffkv_attn_timeline.so)
// stamp the shader real-time counter (100 MHz) at fixed points of the split
// kernel: thread 0 keeps kTlSlots stamps in LDS (zero until stamped) and
// writes them out when its workgroup finishes a chunk, to slot (blockIdx.y * gridDim.x + blockIdx.x) *
// kTlSlots of a buffer registered with diffkv_attn_timeline_buffer.  A stamp
// after a value waits for that value (the empty asm takes it as an operand).
// In other builds the macros expand to nothing.
constexpr int kTlSlots = 8;
#ifdef DIFFKV_TIMELINE
__device__ uint64_t* g_tl_buf;
__device__ uint64_t g_tl_entries;
__shared__ uint64_t g_tl_stamps[kTlSlots];
#define DIFFKV_STAMP(k)                                                              \
  do {                                                                               \
    if (threadIdx.x == 0) ::diffkv::g_tl_stamps[k] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define DIFFKV_STAMP_AFTER(k, v)         \
  do {                                   \
    asm volatile("" ::"v"(v));           \
    DIFFKV_STAMP(k);                     \
  } while (0)
#define DIFFKV_STAMP_BEGIN()                                                       \
  do {                                                                             \
    if (threadIdx.x == 0)                                                          \
      for (int k_ = 1; k_ < ::diffkv::kTlSlots; ++k_) ::diffkv::g_tl_stamps[k_] = 0; \
    DIFFKV_STAMP(0);                                                               \
  } while (0)
#define DIFFKV_STAMP_FLUSH()                                                                      \
  do {                                                                                            \
    if (threadIdx.x == 0 && ::diffkv::g_tl_buf) {                                                 \
      const uint64_t w_ = ((uint64_t)blockIdx.y * gridDim.x + blockIdx.x) * ::diffkv::kTlSlots;   \
      for (int k_ = 0; k_ < ::diffkv::kTlSlots; ++k_)                                             \
        if (w_ + k_ < ::diffkv::g_tl_entries) ::diffkv::g_tl_buf[w_ + k_] = ::diffkv::g_tl_stamps[k_]; \
    }                                                                                             \
  } while (0)
#else
#define DIFFKV_STAMP_BEGIN() \
  do {                       \
  } while (0)
#define DIFFKV_STAMP(k) \
  do {                  \
  } while (0)
#define DIFFKV_STAMP_AFTER(k, v) \
  do {                           \
  } while (0)
#define DIFFKV_STAMP_FLUSH() \
  do {                       \
  } while (0)
#endif

// Packed query row where sequence b starts: sum of q_lens[0..b).  One wave
// computes it cooperatively (a strided sum and a wave reduction).
__device__ __forceinline__ int seq_row_start(const int32_t* q_lens, int b) {
  if (q_lens == nullptr) return b;
  int s = 0;
  for (int k = lane_id(); k < b; k += 64) s += q_lens[k];
  return wave_sum_int(s);
}

}  // namespace diffkv
