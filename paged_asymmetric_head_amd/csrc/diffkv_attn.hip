// C ABI of the paged asymmetric-head attention library: argument checks,
// launch planning and kernel dispatch onto the caller's stream.
//
// The host side never allocates, frees, synchronises or reads device memory;
// it derives every launch from the descriptor, so calls can be captured in a
// HIP graph.  Errors are status codes; no exception crosses the ABI.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <mutex>

#include "diffkv_attn.h"
#include "plan.hpp"
#include "validate.hpp"
#include "split_attn.hpp"
#include "prefill_attn.hpp"
#include "kv_write.hpp"
#include "combine.hpp"

using namespace diffkv;

namespace {

#ifdef DIFFKV_DEBUG
// Copies the debug builds' violation bits to the caller's word and clears
// them (a kernel, so the call stays in stream order and capturable).
__global__ void take_debug_flags_kernel(uint32_t* flags) {
  *flags = g_debug_flags;
  g_debug_flags = 0;
}
#endif

// Compute units per device, queried once per device (the planner's one
// resident round of workgroups is sized from it).  kDefaultCUs when the
// device cannot be queried (no GPU, or an ordinal past kMaxDevices).
constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];

int device_cu_count(int device) {
  if (device < 0 || device >= kMaxDevices) return kDefaultCUs;
  std::call_once(g_cu_once[device], [device] {
    int n = 0;
    const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    g_cu_count[device] = e == hipSuccess && n > 0 ? n : kDefaultCUs;
  });
  return g_cu_count[device];
}

// CUs of the device a stream belongs to (the current device for the null
// stream, and for workspace sizing, which has no stream).
int stream_cu_count(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) == hipSuccess) return device_cu_count(dev);
  }
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();                 // leave no sticky error for the caller
    return kDefaultCUs;
  }
  return device_cu_count(dev);
}

// Workspace of diffkv_attn_verify_noalloc: one static array per device (the
// code object's zero-filled data, held until the process ends), for callers
// that cannot allocate.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device, with
// that device current, and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device `dev` (nullptr if it cannot be
// looked up).
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess)
      g_scratch_ptr[dev] = ptr;
    else
      (void)hipGetLastError();
    if (cur != dev) (void)hipSetDevice(cur);
  });
  return g_scratch_ptr[dev];
}

// Ordinal of the device a stream belongs to (the current device for the
// null stream); -1 if it cannot be found.
int stream_device(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) == hipSuccess) return dev;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return dev;
}

// The measurement events of a call (the descriptor's profile_start and
// profile_stop), or none.
struct Profile {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Launches the main kernel of a call.  With measurement events, the
// dispatch itself stamps them (hipExtLaunchKernel), so their elapsed time is
// the kernel's execution alone.
hipError_t launch_main(const void* fn, dim3 grid, dim3 block, void** args, hipStream_t stream,
                       const Profile& pf) {
  if (pf.start != nullptr)
    return hipExtLaunchKernel(fn, grid, block, args, 0, stream, pf.start, pf.stop, 0);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

template <bool FP8, int RT, bool DIRECT, bool COUNT, bool UPAGE, int DQK>
hipError_t launch_split_kernel(const SplitArgs& a, dim3 grid, hipStream_t stream, const Profile& pf) {
  void* args[] = {const_cast<SplitArgs*>(&a)};
  constexpr int NS = kSplitStages<FP8>;
  return launch_main(
      reinterpret_cast<const void*>(&split_attn_kernel<FP8, RT, DIRECT, COUNT, UPAGE, NS, DQK>),
      grid, dim3(256), args, stream, pf);
}

template <bool FP8, int RT, bool UPAGE, int DQK>
hipError_t dispatch_split_rt(const SplitArgs& a, dim3 grid, bool direct, bool count, hipStream_t st,
                             const Profile& pf) {
  if (direct) return count ? launch_split_kernel<FP8, RT, true, true, UPAGE, DQK>(a, grid, st, pf)
                           : launch_split_kernel<FP8, RT, true, false, UPAGE, DQK>(a, grid, st, pf);
  return count ? launch_split_kernel<FP8, RT, false, true, UPAGE, DQK>(a, grid, st, pf)
               : launch_split_kernel<FP8, RT, false, false, UPAGE, DQK>(a, grid, st, pf);
}

// UPAGE: pages of at least one 64-key tile, so a tile never straddles pages.
template <bool FP8, int DQK>
hipError_t dispatch_split_dqk(const SplitArgs& a, int rt, bool upage, dim3 grid, bool direct,
                              bool count, hipStream_t st, const Profile& pf) {
  if (upage) {
    switch (rt) {
      case 1: return dispatch_split_rt<FP8, 1, true, DQK>(a, grid, direct, count, st, pf);
      case 2: return dispatch_split_rt<FP8, 2, true, DQK>(a, grid, direct, count, st, pf);
      default: return dispatch_split_rt<FP8, 4, true, DQK>(a, grid, direct, count, st, pf);
    }
  }
  switch (rt) {
    case 1: return dispatch_split_rt<FP8, 1, false, DQK>(a, grid, direct, count, st, pf);
    case 2: return dispatch_split_rt<FP8, 2, false, DQK>(a, grid, direct, count, st, pf);
    default: return dispatch_split_rt<FP8, 4, false, DQK>(a, grid, direct, count, st, pf);
  }
}

template <bool FP8>
hipError_t dispatch_split(const SplitArgs& a, int dqk, int rt, bool upage, dim3 grid, bool direct,
                          bool count, hipStream_t st, const Profile& pf) {
  return dqk == kHeadDimQKSym
             ? dispatch_split_dqk<FP8, kHeadDimQKSym>(a, rt, upage, grid, direct, count, st, pf)
             : dispatch_split_dqk<FP8, kHeadDimQK>(a, rt, upage, grid, direct, count, st, pf);
}

// Merge shape by the chunks a pair is expected to have: one wave with 16
// loads per pass when that is at most 16, else four waves with 32 loads each
// (128 chunks per pass), of which a pair of at most 32 chunks uses one.
// Either shape takes any chunk count (more passes).  The expectation is the
// plan's slots over its pairs (the balanced plan gives near-uniform batches
// about that many each; decode at 8K tokens: 16, where the worst-case bound
// is 37 and picked the four-wave shape, 1 us slower per call); forced splits
// are exact.
int expected_chunks_per_pair(const SplitPlan& plan, const diffkv_attn_desc& d) {
  if (d.force_num_splits > 0) return plan.max_chunks;
  const long long pairs = (long long)d.batch * plan.n_qtiles;
  const long long e = (plan.slots + pairs - 1) / pairs;
  return (int)(e < plan.max_chunks ? e : plan.max_chunks);
}

template <int ROWS>
const void* merge_kernel_for(int splits, int& threads) {
  if (splits <= 16) { threads = 64; return reinterpret_cast<const void*>(&split_merge_kernel<ROWS, 1, 16>); }
  threads = 256;
  return reinterpret_cast<const void*>(&split_merge_kernel<ROWS, 4, 32>);
}

hipError_t launch_merge(const SplitArgs& a, int rows, int max_chunks, dim3 grid,
                        hipStream_t stream) {
  void* args[] = {const_cast<SplitArgs*>(&a)};
  int threads = 0;
  const void* fn = rows == 16 ? merge_kernel_for<16>(max_chunks, threads)
                 : rows == 32 ? merge_kernel_for<32>(max_chunks, threads)
                              : merge_kernel_for<64>(max_chunks, threads);
  return hipLaunchKernel(fn, grid, dim3(threads), args, 0, stream);
}

template <bool FP8, bool UPAGE, bool COUNT, int DQK>
hipError_t launch_prefill_kernel(const SplitArgs& a, dim3 grid, hipStream_t stream, const Profile& pf) {
  void* args[] = {const_cast<SplitArgs*>(&a)};
  return launch_main(reinterpret_cast<const void*>(&prefill_attn_kernel<FP8, UPAGE, COUNT, DQK>),
                     grid, dim3(kPfThreads), args, stream, pf);
}

template <bool FP8, int DQK>
hipError_t dispatch_prefill_dqk(const SplitArgs& a, bool upage, bool count, dim3 grid,
                                hipStream_t st, const Profile& pf) {
  if (upage) return count ? launch_prefill_kernel<FP8, true, true, DQK>(a, grid, st, pf)
                          : launch_prefill_kernel<FP8, true, false, DQK>(a, grid, st, pf);
  return count ? launch_prefill_kernel<FP8, false, true, DQK>(a, grid, st, pf)
               : launch_prefill_kernel<FP8, false, false, DQK>(a, grid, st, pf);
}

template <bool FP8>
hipError_t dispatch_prefill(const SplitArgs& a, int dqk, bool upage, bool count, dim3 grid,
                            hipStream_t st, const Profile& pf) {
  return dqk == kHeadDimQKSym ? dispatch_prefill_dqk<FP8, kHeadDimQKSym>(a, upage, count, grid, st, pf)
                              : dispatch_prefill_dqk<FP8, kHeadDimQK>(a, upage, count, grid, st, pf);
}

hipError_t launch_fill(int32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int32_t zero = 0;
  void* args[] = {&p, &n, &zero};
  const unsigned blocks = (unsigned)((n + 255) / 256);
  return hipLaunchKernel(reinterpret_cast<const void*>(&fill_i32_kernel), dim3(blocks), dim3(256),
                         args, 0, stream);
}

// Context partials (part_out set) run as a verify call restricted to the key
// ranges [key_lo[b], key_hi[b]), without sinks, writing fp32 partial rows.
struct PartialMode {
  const int32_t* key_lo = nullptr;
  const int32_t* key_hi = nullptr;
  float* part_out = nullptr;
};

int run_entry(int entry, const diffkv_attn_desc* d, const void* q, const void* k_cache,
              const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
              const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
              float v_scale, float softmax_scale, void* out, float* lse_out, int32_t* count_out,
              void* workspace, size_t workspace_bytes, hipStream_t stream,
              const PartialMode& pm = PartialMode()) {
  const int st = validate_desc(d, entry);
  if (st != DIFFKV_OK) return st;
  // The measurement events go to the call's first main kernel.
  const Profile pf{d->profile_start, d->profile_stop};
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !(out || pm.part_out))
    return DIFFKV_INVALID_ARGUMENT;
  if (!q_lens && d->max_q_len != 1) return DIFFKV_INVALID_ARGUMENT;
  const bool fp8 = d->kv_dtype == DIFFKV_KV_FP8_E4M3;
  const float ks = fp8 ? k_scale : 1.f;
  const float vs = fp8 ? v_scale : 1.f;
  if (!std::isfinite(softmax_scale) || !std::isfinite(ks) || !std::isfinite(vs) ||
      !(softmax_scale > 0.f) || !(ks > 0.f))
    return DIFFKV_INVALID_ARGUMENT;
  const int G = d->num_q_heads / d->num_kv_heads;

  if (count_out) {
    const hipError_t e = launch_fill(count_out, (size_t)d->total_q * d->num_q_heads, stream);
    if (e != hipSuccess) return DIFFKV_HIP_ERROR;
  }

  const bool upage = d->page_size >= kTileKeys;
  const bool count = count_out != nullptr;
  SplitArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.q_lens = q_lens;
  a.sinks = sinks;
  a.out = static_cast<uint16_t*>(out);
  a.lse_out = lse_out;
  a.count_out = count_out;
  a.batch = d->batch;
  a.hq = d->num_q_heads;
  a.hkv = d->num_kv_heads;
  a.group = G;
  a.log2_page = ilog2(d->page_size);
  a.bt_stride = d->block_table_stride;
  a.window = window;
  a.q_lo = 1;
  a.q_hi = INT32_MAX;
  a.key_lo = pm.key_lo;
  a.key_hi = pm.key_hi;
  a.part_out = pm.part_out;
  a.scale_log2 = softmax_scale * ks * kLog2e;
  a.v_scale = vs;
#ifdef DIFFKV_DEBUG
  a.max_seq_len = d->max_seq_len;
  a.max_q_len = d->max_q_len;
  a.total_q = d->total_q;
  a.num_pages = d->num_pages;
#endif

  // Split-KV part: decode and verify, and a mixed call's short sequences.
  if (entry != DIFFKV_ENTRY_PREFILL) {
    const diffkv_attn_desc sd = split_part_desc(*d, entry);
    const SplitPlan plan = plan_split(sd, window, stream_cu_count(stream), kLaunchSlots);
    if (!plan.direct && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
      return DIFFKV_WORKSPACE_TOO_SMALL;
    SplitArgs sa = a;
    if (!plan.direct) {
      char* ws = static_cast<char*>(workspace);
      sa.part_o = reinterpret_cast<uint16_t*>(ws);
      sa.part_lse = reinterpret_cast<f32x2*>(ws + align256(plan.part_o_bytes));
      sa.pair_chunks = reinterpret_cast<i32x2*>(ws + align256(plan.part_o_bytes) +
                                                align256(plan.part_lse_bytes));
    }
    sa.n_qtiles = plan.n_qtiles;
    sa.slots = plan.slots;
    sa.force_splits = d->force_num_splits;
    sa.chunk_bound = (int)plan.grid_x;
    if (entry == DIFFKV_ENTRY_MIXED) sa.q_hi = kMixedSplitMaxQ;
    const dim3 grid((unsigned)plan.grid_x, d->num_kv_heads);
    hipError_t e =
        fp8 ? dispatch_split<true>(sa, d->head_dim_qk, plan.row_tiles, upage, grid, plan.direct, count,
                                   stream, pf)
            : dispatch_split<false>(sa, d->head_dim_qk, plan.row_tiles, upage, grid, plan.direct, count,
                                    stream, pf);
    if (e == hipSuccess && !plan.direct)
      e = launch_merge(sa, plan.rows, expected_chunks_per_pair(plan, *d),
                       dim3(sd.max_q_len * G, d->batch * d->num_kv_heads), stream);
    if (e != hipSuccess) return DIFFKV_HIP_ERROR;
  }

  // Prefill part: one workgroup per 256 query rows of a (sequence, KV head);
  // the many rows of a chunk fill the GPU without splitting the keys.
  const bool prefill_part = entry == DIFFKV_ENTRY_PREFILL ||
                            (entry == DIFFKV_ENTRY_MIXED && d->max_q_len > kMixedSplitMaxQ);
  if (prefill_part) {
    SplitArgs pa = a;
    pa.n_qtiles = prefill_row_blocks(*d);
    if (entry == DIFFKV_ENTRY_MIXED) pa.q_lo = kMixedSplitMaxQ + 1;
    const dim3 grid(pa.n_qtiles, d->batch * d->num_kv_heads);
    // A mixed call's events went to its split-KV kernel.
    const Profile ppf = entry == DIFFKV_ENTRY_PREFILL ? pf : Profile{};
    const hipError_t e = fp8 ? dispatch_prefill<true>(pa, d->head_dim_qk, upage, count, grid, stream, ppf)
                             : dispatch_prefill<false>(pa, d->head_dim_qk, upage, count, grid, stream, ppf);
    if (e != hipSuccess) return DIFFKV_HIP_ERROR;
  }
  return DIFFKV_OK;
}

int run_kv_write(const diffkv_attn_desc* d, const void* k_new, const void* v_new, void* k_cache,
                 void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                 const int32_t* q_lens, float k_scale, float v_scale, hipStream_t stream) {
  const int st = validate_desc(d, DIFFKV_ENTRY_PREFILL);
  if (st != DIFFKV_OK) return st;
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !seq_lens)
    return DIFFKV_INVALID_ARGUMENT;
  if (!q_lens && d->max_q_len != 1) return DIFFKV_INVALID_ARGUMENT;
  const bool fp8 = d->kv_dtype == DIFFKV_KV_FP8_E4M3;
  if (fp8 && !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return DIFFKV_INVALID_ARGUMENT;
  KvWriteArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.q_lens = q_lens;
  a.hkv = d->num_kv_heads;
  a.log2_page = ilog2(d->page_size);
  a.bt_stride = d->block_table_stride;
  a.num_pages = d->num_pages;
  a.total_q = d->total_q;
  a.k_scale = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  void* args[] = {&a};
  const long long units = (long long)d->max_q_len * d->num_kv_heads * (d->head_dim_qk / 8 + kVUnits);
  const dim3 grid((unsigned)((units + 255) / 256), d->batch);
  const bool sym = d->head_dim_qk == kHeadDimQKSym;
  const void* fn = fp8 ? (sym ? reinterpret_cast<const void*>(&kv_write_kernel<true, kHeadDimQKSym>)
                              : reinterpret_cast<const void*>(&kv_write_kernel<true, kHeadDimQK>))
                       : (sym ? reinterpret_cast<const void*>(&kv_write_kernel<false, kHeadDimQKSym>)
                              : reinterpret_cast<const void*>(&kv_write_kernel<false, kHeadDimQK>));
  return launch_main(fn, grid, dim3(256), args, stream, Profile{d->profile_start, d->profile_stop}) ==
                 hipSuccess
             ? DIFFKV_OK
             : DIFFKV_HIP_ERROR;
}

}  // namespace

extern "C" {

int diffkv_attn_decode(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
                       float v_scale, float softmax_scale, void* out, float* lse_out,
                       int32_t* count_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return run_entry(DIFFKV_ENTRY_DECODE, desc, q, k_cache, v_cache, block_table, seq_lens, q_lens,
                   window, sinks, k_scale, v_scale, softmax_scale, out, lse_out, count_out,
                   workspace, workspace_bytes, stream);
}

int diffkv_attn_verify(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
                       float v_scale, float softmax_scale, void* out, float* lse_out,
                       int32_t* count_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return run_entry(DIFFKV_ENTRY_VERIFY, desc, q, k_cache, v_cache, block_table, seq_lens, q_lens,
                   window, sinks, k_scale, v_scale, softmax_scale, out, lse_out, count_out,
                   workspace, workspace_bytes, stream);
}

int diffkv_attn_prefill(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
                        float v_scale, float softmax_scale, void* out, float* lse_out,
                        int32_t* count_out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return run_entry(DIFFKV_ENTRY_PREFILL, desc, q, k_cache, v_cache, block_table, seq_lens, q_lens,
                   window, sinks, k_scale, v_scale, softmax_scale, out, lse_out, count_out,
                   workspace, workspace_bytes, stream);
}

int diffkv_kv_write(const diffkv_attn_desc* desc, const void* k_new, const void* v_new,
                    void* k_cache, void* v_cache, const int32_t* block_table,
                    const int32_t* seq_lens, const int32_t* q_lens, float k_scale, float v_scale,
                    hipStream_t stream) {
  return run_kv_write(desc, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_lens,
                      k_scale, v_scale, stream);
}

int diffkv_attn_partial(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* q_lens, const int32_t* key_lo, const int32_t* key_hi,
                        int32_t window, float k_scale, float v_scale, float softmax_scale,
                        float* out_part, float* lse_part, int32_t* count_out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (out_part == nullptr || lse_part == nullptr) return DIFFKV_INVALID_ARGUMENT;
  PartialMode pm;
  pm.key_lo = key_lo;
  pm.key_hi = key_hi;
  pm.part_out = out_part;
  return run_entry(DIFFKV_ENTRY_VERIFY, desc, q, k_cache, v_cache, block_table, seq_lens, q_lens,
                   window, nullptr, k_scale, v_scale, softmax_scale, nullptr, lse_part, count_out,
                   workspace, workspace_bytes, stream, pm);
}

int diffkv_attn_combine(int32_t num_parts, int32_t rows, int32_t num_q_heads,
                        const float* out_parts, const float* lse_parts, const float* sinks,
                        void* out, float* lse_out, hipStream_t stream) {
  if (num_parts < 1 || rows < 1 || num_q_heads < 1 || rows % num_q_heads != 0)
    return DIFFKV_INVALID_ARGUMENT;
  if (num_parts > kMaxCombineParts) return DIFFKV_UNSUPPORTED;
  if (!out_parts || !lse_parts || !out) return DIFFKV_INVALID_ARGUMENT;
  CombineArgs a{out_parts, lse_parts, sinks, static_cast<uint16_t*>(out), lse_out,
                num_parts, rows, num_q_heads};
  void* args[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel),
                                       dim3((unsigned)((rows + 3) / 4)), dim3(256), args, 0, stream);
  return e == hipSuccess ? DIFFKV_OK : DIFFKV_HIP_ERROR;
}

int diffkv_attn_verify_noalloc(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* q_lens, int32_t window,
                               const float* sinks, float k_scale, float v_scale,
                               float softmax_scale, void* out, float* lse_out, int32_t* count_out,
                               hipStream_t stream) {
  const int st = validate_desc(desc, DIFFKV_ENTRY_VERIFY);
  if (st != DIFFKV_OK) return st;
  // The workspace this launch needs (the plan of the call itself, on the
  // stream's device) must fit the static array; nothing is allocated.
  const int dev = stream_device(stream);
  const SplitPlan plan = plan_split(*desc, window, dev >= 0 ? device_cu_count(dev) : kDefaultCUs,
                                    kLaunchSlots);
  if (plan.workspace_bytes > kScratchBytes) return DIFFKV_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    ws = device_scratch(dev);
    if (ws == nullptr) return DIFFKV_HIP_ERROR;
  }
  return run_entry(DIFFKV_ENTRY_VERIFY, desc, q, k_cache, v_cache, block_table, seq_lens, q_lens,
                   window, sinks, k_scale, v_scale, softmax_scale, out, lse_out, count_out, ws,
                   ws ? kScratchBytes : 0, stream);
}

int diffkv_attn_mixed(const diffkv_attn_desc* desc, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* q_lens, int32_t window, const float* sinks, float k_scale,
                      float v_scale, float softmax_scale, void* out, float* lse_out,
                      int32_t* count_out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return run_entry(DIFFKV_ENTRY_MIXED, desc, q, k_cache, v_cache, block_table, seq_lens, q_lens,
                   window, sinks, k_scale, v_scale, softmax_scale, out, lse_out, count_out,
                   workspace, workspace_bytes, stream);
}

size_t diffkv_attn_workspace_bytes(const diffkv_attn_desc* desc, int entry) {
  if (validate_desc(desc, entry) != DIFFKV_OK) return 0;
  if (entry == DIFFKV_ENTRY_PREFILL) return 0;
  return plan_split(split_part_desc(*desc, entry), 0, stream_cu_count(nullptr)).workspace_bytes;
}

int diffkv_attn_validate(const diffkv_attn_desc* desc, int entry) {
  return validate_desc(desc, entry);
}

int diffkv_attn_num_splits(const diffkv_attn_desc* desc, int entry, int32_t window) {
  if (validate_desc(desc, entry) != DIFFKV_OK) return 0;
  if (entry == DIFFKV_ENTRY_PREFILL) return 1;
  return plan_split(split_part_desc(*desc, entry), window, stream_cu_count(nullptr), kLaunchSlots)
      .max_chunks;
}

int diffkv_attn_timeline_buffer(uint64_t* stamps, size_t entries) {
#ifdef DIFFKV_TIMELINE
  if ((stamps == nullptr) != (entries == 0)) return DIFFKV_INVALID_ARGUMENT;
  const uint64_t n = entries;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_tl_buf), &stamps, sizeof(stamps)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(g_tl_entries), &n, sizeof(n)) != hipSuccess)
    return DIFFKV_HIP_ERROR;
  return DIFFKV_OK;
#else
  (void)stamps;
  (void)entries;
  return DIFFKV_UNSUPPORTED;
#endif
}

int diffkv_attn_debug_flags(uint32_t* flags, hipStream_t stream) {
#ifdef DIFFKV_DEBUG
  if (flags == nullptr) return DIFFKV_INVALID_ARGUMENT;
  void* args[] = {&flags};
  return hipLaunchKernel(reinterpret_cast<const void*>(&take_debug_flags_kernel), dim3(1), dim3(1),
                         args, 0, stream) == hipSuccess
             ? DIFFKV_OK
             : DIFFKV_HIP_ERROR;
#else
  (void)flags;
  (void)stream;
  return DIFFKV_UNSUPPORTED;
#endif
}

const char* diffkv_attn_strerror(int status) {
  switch (status) {
    case DIFFKV_OK: return "success";
    case DIFFKV_INVALID_ARGUMENT: return "invalid argument";
    case DIFFKV_UNSUPPORTED: return "unsupported shape, page size or dtype";
    case DIFFKV_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DIFFKV_HIP_ERROR: return "HIP launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
