// Combine of context partials: the log-sum-exp merge of the partial outputs
// several key ranges produced for the same rows (on one GPU, or gathered from
// the GPUs that each hold a range of a sequence's keys; "diffbot/MiMo-V2.6-
// Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000", What the kernels do: split-KV, here
// cut across key ranges).  With M = max(max_s lse_s, sink) and w_s =
// e^(lse_s - M):
//     out = sum_s w_s out_s / (sum_s w_s + e^(sink - M)),   lse = M + ln sum_s w_s
// One wave per row: lane s holds part s's lse (up to 64 parts), two output
// dims per lane, parts summed in a fixed order.
#pragma once

#include "device_common.hpp"
#include "plan.hpp"

namespace diffkv {

struct CombineArgs {
  const float* out_parts;   // fp32 [parts, rows, 128]
  const float* lse_parts;   // fp32 [parts, rows], natural log, -inf for no key
  const float* sinks;       // fp32 [Hq] or NULL
  uint16_t* out;            // bf16 [rows, 128]
  float* lse_out;           // fp32 [rows] or NULL
  int parts, rows, hq;
};

constexpr int kMaxCombineParts = 64;

__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;                // whole waves
  const float lse = lane < a.parts ? a.lse_parts[(size_t)lane * a.rows + row] : -INFINITY;
  const float s = a.sinks ? a.sinks[row % a.hq] : -INFINITY;
  const float M = wave_max_all(lse);
  const float Mt = fmaxf(M, s);
  const float Mu = Mt == -INFINITY ? 0.f : Mt;
  const float w = lse == -INFINITY ? 0.f : fast_exp2((lse - Mu) * kLog2e);
  const float ksum = wave_sum_all(w);
  f32x2 acc = f32x2{0.f, 0.f};
  const float* op = a.out_parts + (size_t)row * kHeadDimV + 2 * lane;
  for (int p = 0; p < a.parts; ++p) {
    const float wp = readlane_f(w, p);
    const f32x2 v = *reinterpret_cast<const f32x2*>(op + (size_t)p * a.rows * kHeadDimV);
    if (wp > 0.f) acc += wp * v;
  }
  const float den = ksum + (a.sinks ? fast_exp2((s - Mu) * kLog2e) : 0.f);
  const float coef = den > 0.f ? 1.f / den : 0.f;
  *reinterpret_cast<uint32_t*>(a.out + (size_t)row * kHeadDimV + 2 * lane) =
      pack_bf16x2(acc.x * coef, acc.y * coef);
  if (a.lse_out && lane == 0) a.lse_out[row] = ksum > 0.f ? Mu + logf(ksum) : -INFINITY;
}

}  // namespace diffkv
