// Host-side checks of the library's descriptor validation and split planner,
// built with a plain C++ compiler under the address and undefined-behaviour
// sanitizers (tests/test_host_sanitized.py).  No GPU and no HIP call: it
// includes only the host headers the library's entry points use.
//
//   fuzz <seed> <count>   seeded random descriptors (extreme values mixed in):
//                         validation returns a status code, and every valid
//                         descriptor plans within its bounds at several CU counts
//   scale                 the planner's grid, workspace and one-resident-round
//                         bound at 32, 80 and 256 CUs for the decode and verify
//                         workloads' shapes
//   fastdiv               the kernels' multiply-high division (fast_div.hpp)
//                         against the division operator: every dividend below
//                         2^16 for divisors 1..1024, dividends at and around
//                         multiples of the divisor and at the top of the range,
//                         and seeded random (dividend, divisor) pairs
// Exits 0 when every check holds; prints the first failure and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fast_div.hpp"
#include "plan.hpp"
#include "validate.hpp"

using namespace diffkv;

namespace {

int g_fail = 0;

void check(bool ok, const char* what, const diffkv_attn_desc& d, int entry, int cus) {
  if (ok || g_fail) return;
  g_fail = 1;
  std::printf("FAIL %s: entry=%d cus=%d batch=%d hq=%d hkv=%d dqk=%d dv=%d P=%d pages=%d stride=%d "
              "max_seq=%d max_q=%d total_q=%d dtype=%d force=%d\n",
              what, entry, cus, d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim_qk, d.head_dim_v,
              d.page_size, d.num_pages, d.block_table_stride, d.max_seq_len, d.max_q_len, d.total_q,
              d.kv_dtype, d.force_num_splits);
}

// splitmix64: a small counter-based generator (Steele, Lea and Flood, 2014).
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int range(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }
  // A field value: usually plausible, sometimes extreme.
  int field(int lo, int hi) {
    static const int kExtreme[] = {0, -1, 1, 2, 16, 127, 128, 129, 255, 256, 65535, 65536,
                                   1 << 20, (1 << 30) - 1, 1 << 30, INT32_MAX, INT32_MIN, -65536};
    const uint64_t r = next() % 8;
    if (r == 0) return kExtreme[next() % (sizeof(kExtreme) / sizeof(kExtreme[0]))];
    if (r == 1) return (int)(uint32_t)next();
    return range(lo, hi);
  }
};

// A plausible descriptor (valid more often than not), then zero to two of
// its fields replaced by extreme or random values.
diffkv_attn_desc random_desc(Rng& g) {
  diffkv_attn_desc d{};
  d.batch = g.range(1, 200);
  d.num_kv_heads = g.range(1, 8);
  d.num_q_heads = d.num_kv_heads * g.range(1, 16);
  d.head_dim_qk = (g.next() % 2) ? 192 : 128;
  d.head_dim_v = 128;
  d.page_size = 1 << g.range(0, 8);
  d.max_seq_len = g.range(1, 300000);
  d.max_q_len = g.range(1, (g.next() % 2) ? 16 : 5000);
  if (d.max_q_len > d.max_seq_len) d.max_q_len = d.max_seq_len;
  d.block_table_stride = (d.max_seq_len + d.page_size - 1) / d.page_size + g.range(0, 3);
  d.num_pages = g.range(1, 1 << 22);
  d.total_q = d.batch * g.range(1, d.max_q_len < 64 ? d.max_q_len : 64);
  if (d.total_q < d.batch) d.total_q = d.batch;
  d.kv_dtype = (int)(g.next() % 2);
  d.force_num_splits = (g.next() % 4) ? 0 : g.range(1, 300);
  int32_t* fields[] = {&d.batch, &d.num_q_heads, &d.num_kv_heads, &d.head_dim_qk, &d.head_dim_v,
                       &d.page_size, &d.num_pages, &d.block_table_stride, &d.max_seq_len,
                       &d.max_q_len, &d.total_q, &d.kv_dtype, &d.force_num_splits};
  const int n_fields = sizeof(fields) / sizeof(fields[0]);
  const int mutations = (int)(g.next() % 3);
  for (int k = 0; k < mutations; ++k) *fields[g.next() % n_fields] = g.field(-3, 1 << 16);
  return d;
}

void check_plan(const diffkv_attn_desc& d, int entry, int window, int cus) {
  if (entry == DIFFKV_ENTRY_PREFILL || entry == DIFFKV_ENTRY_MIXED) {
    const long long blocks = prefill_row_blocks(d);
    check(blocks >= 1 && blocks <= INT32_MAX, "prefill row blocks", d, entry, cus);
    if (entry == DIFFKV_ENTRY_PREFILL) return;             // no split-KV part
  }
  const diffkv_attn_desc sd = split_part_desc(d, entry);
  const SplitPlan ws = plan_split(sd, 0, cus);                      // what workspace_bytes sizes
  const SplitPlan run = plan_split(sd, window, cus, kLaunchSlots);  // what a launch uses
  check(run.grid_x >= 1 && run.grid_x <= INT32_MAX, "grid_x range", d, entry, cus);
  // One resident round of workgroups per launch (at least one slot per KV head).
  const long long round = (long long)cus * kWorkspaceWgsPerCu / d.num_kv_heads;
  check(run.slots >= 1 && run.slots <= (round > 1 ? round : 1), "slots within one resident round", d,
        entry, cus);
  check(run.rows == 16 * run.row_tiles && (run.rows == 16 || run.rows == 32 || run.rows == 64),
        "row tile", d, entry, cus);
  check(run.max_chunks >= 1, "max_chunks", d, entry, cus);
  check(run.workspace_bytes <= ws.workspace_bytes, "launch workspace within the sized one", d, entry,
        cus);
  if (!run.direct) {
    check(run.workspace_bytes >= run.part_o_bytes + run.part_lse_bytes + run.pair_bytes,
          "workspace holds its regions", d, entry, cus);
    check(run.workspace_bytes % 256 == 0, "workspace alignment", d, entry, cus);
  }
}

int fuzz(uint64_t seed, long count) {
  Rng g{seed};
  long valid = 0;
  for (long i = 0; i < count && !g_fail; ++i) {
    const diffkv_attn_desc d = random_desc(g);
    for (int entry = -1; entry <= 4; ++entry) {
      const int st = validate_desc(&d, entry);
      check(st == DIFFKV_OK || st == DIFFKV_INVALID_ARGUMENT || st == DIFFKV_UNSUPPORTED,
            "status code", d, entry, 0);
      if (st != DIFFKV_OK) continue;
      ++valid;
      const int window = g.field(-5, 300);
      for (int cus : {1, 32, 80, 256, 1024}) check_plan(d, entry, window, cus);
    }
  }
  check(validate_desc(nullptr, DIFFKV_ENTRY_DECODE) == DIFFKV_INVALID_ARGUMENT, "null descriptor",
        diffkv_attn_desc{}, 0, 0);
  std::printf("fuzz: %ld descriptors, %ld valid (descriptor, entry) pairs\n", count, valid);
  return g_fail;
}

diffkv_attn_desc shape(int batch, int max_seq, int q_len) {
  diffkv_attn_desc d{};
  d.batch = batch;
  d.num_q_heads = 8;
  d.num_kv_heads = 1;
  d.head_dim_qk = 192;
  d.head_dim_v = 128;
  d.page_size = 128;
  d.max_seq_len = max_seq;
  d.block_table_stride = (max_seq + 127) / 128;
  d.num_pages = batch * d.block_table_stride;
  d.max_q_len = q_len;
  d.total_q = batch * q_len;
  d.kv_dtype = DIFFKV_KV_BF16;
  return d;
}

int scale() {
  struct Case { const char* name; diffkv_attn_desc d; int entry; };
  const Case cases[] = {{"batched decode", shape(32, 9216, 1), DIFFKV_ENTRY_DECODE},
                        {"long verify", shape(4, 50000, 8), DIFFKV_ENTRY_VERIFY}};
  for (const Case& c : cases) {
    check(validate_desc(&c.d, c.entry) == DIFFKV_OK, "valid shape", c.d, c.entry, 0);
    const SplitPlan base = plan_split(c.d, 0, 32);
    for (int cus : {32, 80, 256}) {
      const SplitPlan ws = plan_split(c.d, 0, cus);
      const SplitPlan run = plan_split(c.d, 0, cus, kLaunchSlots);
      const long long pairs = (long long)c.d.batch * run.n_qtiles;
      // Workspace bound: 4 workgroups per CU plus one chunk per pair, per KV head.
      check(ws.slots == cus * kWorkspaceWgsPerCu / c.d.num_kv_heads, "sized slots", c.d, c.entry, cus);
      check(ws.grid_x == ws.slots + pairs, "sized grid", c.d, c.entry, cus);
      check(ws.workspace_bytes >= base.workspace_bytes, "workspace grows with the CUs", c.d, c.entry,
            cus);
      // The launch: one resident round of slots (the verify rows' 64-row
      // tiles take one workgroup per CU while chunks stay short, decode two).
      const int per_cu = run.row_tiles == 4 && (long long)pairs * (ceil_div(c.d.max_seq_len, kTileKeys) + 1) <=
                                                   kSlots64MaxTilesPerCu * cus
                             ? kSplitSlotsPerCu64 : kSplitSlotsPerCu;
      check(run.slots == cus * per_cu / c.d.num_kv_heads, "launch slots = one resident round", c.d,
            c.entry, cus);
      check(run.grid_x == run.slots + pairs, "launch grid", c.d, c.entry, cus);
      check(!run.direct, "split", c.d, c.entry, cus);
      std::printf("%s at %d CUs: slots %d, grid %lld, workspace %zu (sized %zu)\n", c.name, cus,
                  run.slots, run.grid_x, run.workspace_bytes, ws.workspace_bytes);
    }
  }
  return g_fail;
}

}  // namespace

int fastdiv() {
  long checked = 0;
  auto one = [&](uint32_t x, uint32_t d) {
    ++checked;
    const uint32_t got = FastDiv(d).div(x), want = x / d;
    if (got != want && !g_fail) {
      g_fail = 1;
      std::printf("FAIL fastdiv: %u / %u = %u, got %u\n", x, d, want, got);
    }
  };
  for (uint32_t d = 1; d <= 1024 && !g_fail; ++d)
    for (uint32_t x = 0; x < 65536u; ++x) one(x, d);
  Rng rng{12345};
  for (int i = 0; i < 200000 && !g_fail; ++i) {
    uint32_t d = (uint32_t)rng.next();
    if (i % 3 == 0) d >>= (uint32_t)(rng.next() % 32);
    if (d == 0) d = 1;
    const uint32_t q = 0xffffffffu / d;
    const uint32_t edges[] = {0u, 1u, d - 1, d, d + 1, q * d, q * d - 1, 0xffffffffu, 0xfffffffeu,
                              (uint32_t)rng.next()};
    for (uint32_t x : edges) one(x, d);
  }
  std::printf("fastdiv: %ld (dividend, divisor) pairs\n", checked);
  return g_fail;
}

int main(int argc, char** argv) {
  if (argc >= 2 && std::strcmp(argv[1], "fuzz") == 0) {
    const uint64_t seed = argc >= 3 ? std::strtoull(argv[2], nullptr, 10) : 1;
    const long count = argc >= 4 ? std::strtol(argv[3], nullptr, 10) : 100000;
    return fuzz(seed, count);
  }
  if (argc >= 2 && std::strcmp(argv[1], "scale") == 0) return scale();
  if (argc >= 2 && std::strcmp(argv[1], "fastdiv") == 0) return fastdiv();
  std::printf("usage: %s fuzz <seed> <count> | scale | fastdiv\n", argv[0]);
  return 2;
}
