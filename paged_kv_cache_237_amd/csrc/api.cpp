// C-ABI entry points of libpa: host-side argument checks, launch sizing and
// error reporting.  Declarations and the contract of every call are in
// include/pa.h.  Nothing here allocates device memory; the only state is a
// per-device cache of the compute-unit count and the debug-check switch (the
// host block manager in block_manager.cpp owns its own host memory).
#include "pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "pa_internal.hpp"
#include "pa_prefill.hpp"

namespace {

thread_local std::string g_detail;

int fail(int code, const std::string& msg) {
  g_detail = msg;
  return code;
}

}  // namespace

namespace pa {
int report_error(int code, const std::string& msg) { return fail(code, msg); }
}  // namespace pa

namespace {

int ok() {
  g_detail.clear();
  return PA_OK;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                              hipGetErrorString(e) + ")");
}

// Compute units of the current device (cached per device).
int current_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static std::mutex mu;
  static std::vector<int> cache;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && size_t(dev) < cache.size() && cache[dev] > 0) {
    *cus = cache[dev];
    return PA_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
  if (n <= 0) return fail(PA_ERR_HIP, "device reports no compute units");
  if (size_t(dev) >= cache.size()) cache.resize(size_t(dev) + 1, 0);
  cache[dev] = n;
  *cus = n;
  return PA_OK;
}

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Debug checks: -1 = not yet decided (PA_DEBUG is read at the first call).
std::atomic<int> g_debug_checks{-1};

bool debug_checks_on() {
  int v = g_debug_checks.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("PA_DEBUG");
    v = (e != nullptr && e[0] == '1') ? 1 : 0;
    int expected = -1;
    if (!g_debug_checks.compare_exchange_strong(expected, v)) v = expected;
  }
  return v == 1;
}

// PA_ERR_PRECONDITION naming the conditions whose bits are set.
int precondition_fail(int flags) {
  std::string d = "device checks:";
  if (flags & pa::kCheckSlot) d += " a slot past the pool;";
  if (flags & pa::kCheckCtx) d += " a context length outside [0, cap];";
  if (flags & pa::kCheckTable) d += " a used block-table entry outside the pool;";
  if (flags & pa::kCheckRows) d += " query rows inconsistent with cu_seqlens_q or the context;";
  return fail(PA_ERR_PRECONDITION, d);
}

int check_geometry(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int* group) {
  if (num_kv_heads <= 0 || num_q_heads <= 0)
    return fail(PA_ERR_BAD_SHAPE, "head counts must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_BAD_SHAPE, "num_q_heads must be a multiple of num_kv_heads");
  if (head_dim != PA_HEAD_DIM) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (block_size != PA_BLOCK_SIZE) return fail(PA_ERR_UNSUPPORTED, "block_size must be 256");
  const int g = num_q_heads / num_kv_heads;
  if (!supported_group(g))
    return fail(PA_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads must be 1, 2, 4 or 8");
  *group = g;
  return PA_OK;
}

// Runs the decode's work list is cut into when set (> 0) by
// pa_set_decode_waves, a testing aid; 0 = the automatic count.
std::atomic<int> g_decode_waves{0};

int64_t decode_waves(int cus, int32_t batch, int32_t num_kv_heads, int32_t max_context_len, int group) {
  const int fixed = g_decode_waves.load(std::memory_order_relaxed);
  // every workspace is sized for kDecodeWavesPerCU waves per CU
  if (fixed > 0) return std::min<int64_t>(fixed, int64_t(cus) * pa::kDecodeWavesPerCU);
  const int64_t tiles_upper =
      int64_t(batch) * num_kv_heads * ((int64_t(max_context_len) + pa::kTile - 1) / pa::kTile);
  // one workgroup per CU
  const int64_t w = int64_t(cus) * pa::decode_group_waves(group);
  return std::max<int64_t>(1, std::min(w, tiles_upper));
}

// Workspace: the partial records (batch*Hkv + waves of them) from its start,
// one int arrival counter per (sequence, kv head) segment at its end (the
// last 256-byte-aligned counter region that fits).  Records never reach the
// counters of a later call that the same workspace covers: a call's records
// end where a workspace sized for the largest call's records and counters
// leaves room for its counters, whatever the batch of the calls before it
// (with the counters first, a call with a small batch would write records
// over counter slots that a later, larger batch expects to be zero).
size_t decode_counter_bytes(int32_t batch, int32_t num_kv_heads) {
  const size_t bytes = size_t(int64_t(batch) * num_kv_heads) * sizeof(int);
  return (bytes + 255) & ~size_t(255);
}

size_t decode_ws_bytes(int32_t batch, int32_t num_kv_heads, int group, int64_t waves) {
  const int64_t records = int64_t(batch) * num_kv_heads + waves;
  const size_t bytes = size_t(records) * size_t(pa::partial_floats(group)) * sizeof(float);
  return decode_counter_bytes(batch, num_kv_heads) + ((bytes + 255) & ~size_t(255));
}

// Prefill context split: parts per query block and tiles per part.  Only a
// launch with fewer query blocks than workgroup slots (2 per CU; the
// 256-CU gfx950 part is assumed, so that the workspace size does not depend
// on which device is current -- the split only affects speed) can leave CUs
// idle while a few blocks stream long contexts; only then are blocks split,
// into as many parts as fill every slot once: floor(slots / blocks), at most
// kPrefillMaxSplits (every other launch gets max_splits = 1: no records, no
// merge, no empty workgroups).  One workgroup per slot beat several: with
// ~4 per slot the extra parts added merge traffic and prologues, and a
// count that is not a multiple of the slots leaves some slots a second
// workgroup while the rest idle.
//
// Longest-first plan: when the query lengths are ragged (total_q_rows below
// batch * max_seqlen_q) the grid's blocks differ in length in ways only the
// device sees (a chunked-prefill batch mixes one-token decode rows with long
// chunks), and grid order can dispatch a long block after a round of short
// ones, or a block far longer than the rest can end the launch alone.  A
// small kernel then plans the launch on the device (prefill.hip): it cuts
// blocks longer than the launch's share of tiles per slot into parts and
// sorts the items longest-first into the workspace (plan_bytes); the
// attention kernel takes them in that order and the last part of a cut
// block to finish merges it.  Launches whose contexts fit 4 blocks (16 tiles per query block at
// most) are left in grid order: no block is long enough to end the launch
// late.
struct PrefillSplit {
  int split_tiles, max_splits, nqb_max;
  size_t ml_bytes, o_bytes, plan_bytes;
  bool plan;
  int64_t cands, plan_items;  // plan: query-block candidates, grid items
};

constexpr int64_t kPrefillSlots = 2 * 256;
// Key tiles of the shortest split part, and parts per query block at most.
constexpr int kPrefillSplitTiles = 16;
constexpr int kPrefillMaxSplits = 16;

PrefillSplit prefill_split(int32_t batch, int64_t total_q_rows, int32_t max_seqlen_q,
                           int32_t num_q_heads, int32_t num_kv_heads, int group,
                           int32_t max_blocks_per_seq) {
  PrefillSplit ps;
  const int64_t max_tiles = int64_t(max_blocks_per_seq) * (PA_BLOCK_SIZE / pa::kTile);
  ps.split_tiles = int(std::max<int64_t>(kPrefillSplitTiles,
                                         (max_tiles + kPrefillMaxSplits - 1) / kPrefillMaxSplits));
  const int qb = pa::kPrefillRows / group;
  ps.nqb_max = (max_seqlen_q + qb - 1) / qb;
  const int64_t slots = kPrefillSlots;
  const int64_t blocks = std::max<int64_t>(1, int64_t(batch) * num_kv_heads * ps.nqb_max);
  // no block has more parts than its longest context has split_tiles runs
  const int64_t cap = std::max<int64_t>(
      1, std::min<int64_t>(kPrefillMaxSplits, (max_tiles + ps.split_tiles - 1) / ps.split_tiles));
  int64_t want = 1;
  if (2 * blocks <= slots) {
    want = slots / blocks;  // every slot once
  } else if (blocks < slots) {
    // Between half and all of the slots, one part per block leaves slots
    // idle, and two parts need two rounds.  With p parts the launch takes
    // ceil(blocks * p / slots) rounds of 1/p of a block plus a prologue and
    // merge share per round (taken as 2 % of a block, which makes 8 parts
    // in one round beat 16 in two, as measured); split into the p with the
    // fewest block-times, and only when that beats one part by 30 % (304
    // blocks over 16K-token prefixes ran 21 % faster in 5 parts; 400 blocks
    // over 8K-token prefixes were no faster in any number of parts).  Only
    // part counts the blocks can take are weighed: a count above `cap` would
    // be cut back to it after the choice, where the model may predict no gain.
    constexpr double kRoundCost = 0.02;
    const double one = 1.0 + kRoundCost;
    double best = one;
    for (int64_t p = 2; p <= cap; ++p) {
      const double rounds = double((blocks * p + slots - 1) / slots);
      const double c = rounds * (1.0 / double(p) + kRoundCost);
      if (c < best - 1e-9) {
        best = c;
        want = p;
      }
    }
    if (best > 0.7 * one) want = 1;
  }
  ps.max_splits = int(std::min<int64_t>(want, cap));
  // A plan (ragged query lengths, contexts beyond 4 blocks) decides the
  // split on the device instead: parts of at least kPrefillSplitTiles tiles,
  // at most kPrefillMaxSplits per block, records in 2 * slots slots of
  // kPrefillRows rows per kv head (enough for any cut the plan makes).  Its
  // grid holds every (query block) candidate plus the extra parts (fewer
  // than 2 * slots / num_kv_heads), at most 2^24 workgroups of 256 threads.
  ps.cands = int64_t(batch) * ps.nqb_max;
  ps.plan_items = ps.cands + (2 * pa::kPlanShareDiv * slots + num_kv_heads - 1) / num_kv_heads;
  ps.plan = total_q_rows < int64_t(batch) * max_seqlen_q && max_blocks_per_seq > 4 &&
            ps.plan_items * num_kv_heads < (int64_t(1) << 24);
  if (ps.plan) {
    static_assert(kPrefillMaxSplits <= 16, "a plan item keeps its part in 4 bits");
    ps.split_tiles = kPrefillSplitTiles;
    ps.max_splits = kPrefillMaxSplits;
    ps.plan_bytes =
        (size_t(pa::kPlanHeader + ps.plan_items + ps.cands + 2 * pa::kPlanShareDiv * slots) * sizeof(int32_t) +
         255) & ~size_t(255);
    // (slot * Hkv + g) < 2 * kPlanShareDiv * slots
    const size_t rows = size_t(2 * pa::kPlanShareDiv * slots) * pa::kPrefillRows;
    ps.ml_bytes = (rows * 2 * sizeof(float) + 255) & ~size_t(255);
    ps.o_bytes = (rows * size_t(pa::kDim) * sizeof(float) + 255) & ~size_t(255);
    return ps;
  }
  ps.plan_bytes = 0;
  if (ps.max_splits == 1) {
    ps.ml_bytes = ps.o_bytes = 0;
    return ps;
  }
  const size_t rows = size_t(ps.max_splits) * size_t(std::max<int64_t>(total_q_rows, 0)) * size_t(num_q_heads);
  ps.ml_bytes = (rows * 2 * sizeof(float) + 255) & ~size_t(255);
  ps.o_bytes = (rows * size_t(pa::kDim) * sizeof(float) + 255) & ~size_t(255);
  return ps;
}

// Virtual heads per (sequence, kv head) of a decode of q_per_seq rows: 32
// for 17 to 32 rows and 16 for 9 to 16 (the matrix-core kernels), also 16
// for 5 to 8 rows of several query tokens; otherwise group * q_per_seq
// rounded up to a power of two (the vector-ALU kernel: every pa_decode and
// pa_decode_append, and pa_decode_multi up to 4 rows); 0 beyond 32.  At 5
// to 8 rows the 16-row kernel measured 16-20 % faster than the vector-ALU
// one (4 tokens at 2 q heads per kv head over U{512..4096}: 139.2 -> 117.4
// us; over 8 x 131,072 tokens: 783.0 -> 625.9 us), at 4 rows 3 % slower.
constexpr int kMfmaRows = 32;
constexpr int kMfma16Rows = 16;
int virtual_group(int group, int32_t q_per_seq) {
  if (q_per_seq < 1 || q_per_seq > kMfmaRows) return 0;
  const int rows = group * q_per_seq;
  if (rows > kMfmaRows) return 0;
  if (rows > kMfma16Rows) return kMfmaRows;
  if (rows > 8 || (rows > 4 && q_per_seq > 1)) return kMfma16Rows;
  int gv = 1;
  while (gv < rows) gv *= 2;
  return gv;
}

// Decode of q_per_seq query rows per sequence (1 for pa_decode); with k_new
// set (one row per sequence), the newest position of each sequence is the
// appended token (pa_decode_append) and the caches are written.  With
// noalloc, the workspace is the library's per-device scratch, looked up once
// every argument has been checked.
int decode_rows(void* out, const void* q, const void* k_new, const void* v_new, const void* k_cache,
                const void* v_cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t batch, int32_t q_per_seq, int32_t max_context_len,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int64_t num_blocks, float scale, void* workspace, size_t workspace_bytes, void* stream,
                bool noalloc = false) {
  try {
    if (batch < 0) return fail(PA_ERR_BAD_SHAPE, "batch < 0");
    int group = 0;
    int r = check_geometry(num_q_heads, num_kv_heads, head_dim, block_size, &group);
    if (r != PA_OK) return r;
    if (q_per_seq < 1) return fail(PA_ERR_BAD_SHAPE, "q_per_seq must be >= 1");
    const int gv = virtual_group(group, q_per_seq);
    if (gv == 0)
      return fail(PA_ERR_UNSUPPORTED, "q_per_seq * num_q_heads / num_kv_heads must be at most 32");
    if (max_blocks_per_seq <= 0) return fail(PA_ERR_BAD_SHAPE, "max_blocks_per_seq must be positive");
    if (num_blocks <= 0) return fail(PA_ERR_BAD_SHAPE, "num_blocks must be positive");
    if (max_context_len < 0 || int64_t(max_context_len) > int64_t(max_blocks_per_seq) * PA_BLOCK_SIZE)
      return fail(PA_ERR_BAD_SHAPE, "max_context_len outside [0, max_blocks_per_seq*block_size]");
    if (!std::isfinite(scale)) return fail(PA_ERR_BAD_SHAPE, "scale is not finite");
    if (batch == 0) return ok();
    if (!out || !q || !k_cache || !v_cache || !block_table || !context_lens)
      return fail(PA_ERR_NULL_PTR, "pa_decode: a pointer argument is NULL");
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_table, 4) || !aligned(context_lens, 4))
      return fail(PA_ERR_ALIGN, "bf16 arrays must be 16-byte aligned, int32 arrays 4-byte");
    const bool append = k_new != nullptr || v_new != nullptr;
    if (append) {
      if (!k_new || !v_new) return fail(PA_ERR_NULL_PTR, "pa_decode_append: k_new or v_new is NULL");
      if (!aligned(k_new, 16) || !aligned(v_new, 16))
        return fail(PA_ERR_ALIGN, "k_new and v_new must be 16-byte aligned");
      if (q_per_seq != 1) return fail(PA_ERR_UNSUPPORTED, "an appended token needs one query row per sequence");
    }
    // every tile index of the flattened work list must fit an int
    if (int64_t(batch) * num_kv_heads * max_blocks_per_seq * (PA_BLOCK_SIZE / pa::kTile) >
        int64_t(INT32_MAX) / 2)
      return fail(PA_ERR_BAD_SHAPE, "batch * num_kv_heads * max_blocks_per_seq too large");
    int cus = 0;
    r = current_cus(&cus);
    if (r != PA_OK) return r;
    const int64_t waves = decode_waves(cus, batch, num_kv_heads, max_context_len, gv);
    const size_t need = decode_ws_bytes(batch, num_kv_heads, gv, waves);
    if (noalloc) {
      if (need > pa::kNoAllocScratchBytes)
        return fail(PA_ERR_WORKSPACE, "pa_decode_append_noalloc: this batch needs " + std::to_string(need) +
                                          " bytes of workspace, more than the library's " +
                                          std::to_string(pa::kNoAllocScratchBytes) +
                                          "-byte scratch; use pa_decode_append with a workspace");
      const hipError_t se = pa::noalloc_scratch(static_cast<hipStream_t>(stream), &workspace);
      if (se != hipSuccess) return hip_fail(se, "decode scratch lookup");
      workspace_bytes = pa::kNoAllocScratchBytes;
    }
    if (workspace == nullptr) return fail(PA_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(PA_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                        std::to_string(workspace_bytes));
    pa::DecodeArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint4*>(k_cache);
    a.v_cache = static_cast<const uint4*>(v_cache);
    a.block_table = block_table;
    a.ctx_lens = context_lens;
    a.out = static_cast<uint16_t*>(out);
    a.ws = static_cast<float*>(workspace);
    a.counters = reinterpret_cast<int*>(
        static_cast<char*>(workspace) +
        ((workspace_bytes - decode_counter_bytes(batch, num_kv_heads)) & ~size_t(255)));
    a.num_blocks = num_blocks;
    a.batch = batch;
    a.hkv = num_kv_heads;
    a.mbps = max_blocks_per_seq;
    a.n_waves = int(waves);
    a.run_w_even = pa::kRunWeightEven;
    a.run_w_odd = pa::kRunWeightOdd;
    a.scale_log2 = float(double(scale) * 1.4426950408889634);
    a.ql = q_per_seq;
    a.gr = group;
    a.gr_shift = group == 1 ? 0 : (group == 2 ? 1 : (group == 4 ? 2 : 3));
    a.hq = num_q_heads;
    a.k_new = static_cast<const uint4*>(k_new);
    a.v_new = static_cast<const uint4*>(v_new);
    // written only when a token is appended (the caller then passes writable caches)
    a.k_store = append ? static_cast<uint4*>(const_cast<void*>(k_cache)) : nullptr;
    a.v_store = append ? static_cast<uint4*>(const_cast<void*>(v_cache)) : nullptr;
    if (debug_checks_on()) {
      pa::SeqCheckArgs c{};
      c.ctx_lens = context_lens;
      c.block_table = block_table;
      c.cu_q = nullptr;
      c.num_blocks = num_blocks;
      c.batch = batch;
      c.mbps = max_blocks_per_seq;
      c.max_context_len = max_context_len;
      c.rows_per_seq = q_per_seq;
      int flags = 0;
      const hipError_t ce = pa::check_seqs(c, static_cast<hipStream_t>(stream), &flags);
      if (ce != hipSuccess) return hip_fail(ce, "decode checks");
      if (flags) return precondition_fail(flags);
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = gv == kMfmaRows     ? pa::launch_decode_mfma(a, st)
                         : gv == kMfma16Rows ? pa::launch_decode_mfma16(a, st)
                                             : pa::launch_decode(a, gv, st);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected host exception");
  }
}

}  // namespace

extern "C" {

int pa_set_decode_waves(int32_t waves) {
  return g_decode_waves.exchange(waves > 0 ? waves : 0);
}

int pa_set_debug_checks(int enabled) {
  const int prev = debug_checks_on() ? 1 : 0;
  g_debug_checks.store(enabled ? 1 : 0);
  return prev;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL_PTR: return "PA_ERR_NULL_PTR";
    case PA_ERR_BAD_SHAPE: return "PA_ERR_BAD_SHAPE";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_SLOT_RANGE: return "PA_ERR_SLOT_RANGE";
    case PA_ERR_DUPLICATE_SLOT: return "PA_ERR_DUPLICATE_SLOT";
    case PA_ERR_BLOCK_CONFLICT: return "PA_ERR_BLOCK_CONFLICT";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS";
    case PA_ERR_PRECONDITION: return "PA_ERR_PRECONDITION";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error_detail(void) { return g_detail.c_str(); }

int pa_validate_slots(const int32_t* host_slots, int64_t n, int64_t num_slots) {
  try {
    if (n < 0 || num_slots < 0) return fail(PA_ERR_BAD_SHAPE, "negative size");
    if (n == 0) return ok();
    if (host_slots == nullptr) return fail(PA_ERR_NULL_PTR, "host_slots is NULL");
    std::vector<int32_t> s;
    s.reserve(size_t(n));
    for (int64_t i = 0; i < n; ++i) {
      const int32_t v = host_slots[i];
      if (v < 0) continue;
      if (int64_t(v) >= num_slots)
        return fail(PA_ERR_SLOT_RANGE, "slot_mapping[" + std::to_string(i) + "] = " +
                                           std::to_string(v) + " >= " + std::to_string(num_slots));
      s.push_back(v);
    }
    std::sort(s.begin(), s.end());
    for (size_t i = 1; i < s.size(); ++i)
      if (s[i] == s[i - 1])
        return fail(PA_ERR_DUPLICATE_SLOT, "slot " + std::to_string(s[i]) + " appears twice");
    return ok();
  } catch (...) {
    return fail(PA_ERR_BAD_SHAPE, "host allocation failed");
  }
}

int pa_validate_block_pairs(const int32_t* host_pairs, int64_t n_pairs, int64_t num_blocks) {
  try {
    if (n_pairs < 0 || num_blocks < 0) return fail(PA_ERR_BAD_SHAPE, "negative size");
    if (n_pairs == 0) return ok();
    if (host_pairs == nullptr) return fail(PA_ERR_NULL_PTR, "host_pairs is NULL");
    std::vector<int32_t> srcs, dsts;
    for (int64_t i = 0; i < n_pairs; ++i) {
      const int32_t a = host_pairs[2 * i], b = host_pairs[2 * i + 1];
      if (a < 0 || b < 0 || a == b) continue;  // skipped by the copy
      if (int64_t(a) >= num_blocks || int64_t(b) >= num_blocks)
        return fail(PA_ERR_SLOT_RANGE, "pair " + std::to_string(i) + " = (" + std::to_string(a) +
                                           ", " + std::to_string(b) + ") outside " +
                                           std::to_string(num_blocks) + " blocks");
      srcs.push_back(a);
      dsts.push_back(b);
    }
    std::sort(dsts.begin(), dsts.end());
    for (size_t i = 1; i < dsts.size(); ++i)
      if (dsts[i] == dsts[i - 1])
        return fail(PA_ERR_BLOCK_CONFLICT, "block " + std::to_string(dsts[i]) +
                                               " is the destination of two pairs");
    std::sort(srcs.begin(), srcs.end());
    for (int32_t d : dsts)
      if (std::binary_search(srcs.begin(), srcs.end(), d))
        return fail(PA_ERR_BLOCK_CONFLICT, "block " + std::to_string(d) +
                                               " is both a source and a destination");
    return ok();
  } catch (...) {
    return fail(PA_ERR_BAD_SHAPE, "host allocation failed");
  }
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int64_t n_pairs,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, void* stream) {
  try {
    if (n_pairs < 0) return fail(PA_ERR_BAD_SHAPE, "n_pairs < 0");
    if (num_kv_heads <= 0 || num_kv_heads > 65535)
      return fail(PA_ERR_BAD_SHAPE, "num_kv_heads must be in 1..65535");
    if (head_dim != PA_HEAD_DIM) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 128");
    if (block_size != PA_BLOCK_SIZE) return fail(PA_ERR_UNSUPPORTED, "block_size must be 256");
    if (num_blocks <= 0) return fail(PA_ERR_BAD_SHAPE, "num_blocks must be positive");
    if (n_pairs == 0) return ok();
    if (n_pairs > INT32_MAX) return fail(PA_ERR_BAD_SHAPE, "n_pairs too large");
    if (!k_cache || !v_cache || !pairs)
      return fail(PA_ERR_NULL_PTR, "pa_copy_blocks: a pointer argument is NULL");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(pairs, 4))
      return fail(PA_ERR_ALIGN, "caches must be 16-byte aligned, pairs 4-byte");
    pa::CopyBlocksArgs a;
    a.pairs = pairs;
    a.n_pairs = n_pairs;
    a.k_cache = static_cast<uint4*>(k_cache);
    a.v_cache = static_cast<uint4*>(v_cache);
    a.num_blocks = num_blocks;
    a.hkv = num_kv_heads;
    const hipError_t e = pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected host exception");
  }
}

int pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int32_t* host_pairs, int64_t n_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, void* stream) {
  try {
    if (n_pairs < 0) return fail(PA_ERR_BAD_SHAPE, "n_pairs < 0");
    if (num_kv_heads <= 0) return fail(PA_ERR_BAD_SHAPE, "num_kv_heads must be positive");
    if (head_dim != PA_HEAD_DIM) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 128");
    if (block_size != PA_BLOCK_SIZE) return fail(PA_ERR_UNSUPPORTED, "block_size must be 256");
    if (src_num_blocks <= 0 || dst_num_blocks <= 0)
      return fail(PA_ERR_BAD_SHAPE, "pools must have a positive number of blocks");
    if (n_pairs == 0) return ok();
    if (!src_k || !src_v || !dst_k || !dst_v || !host_pairs)
      return fail(PA_ERR_NULL_PTR, "pa_swap_blocks: a pointer argument is NULL");
    for (int64_t i = 0; i < n_pairs; ++i) {
      const int32_t a = host_pairs[2 * i], b = host_pairs[2 * i + 1];
      if (a < 0 || int64_t(a) >= src_num_blocks || b < 0 || int64_t(b) >= dst_num_blocks)
        return fail(PA_ERR_SLOT_RANGE, "pair " + std::to_string(i) + " = (" + std::to_string(a) +
                                           ", " + std::to_string(b) + ") outside its pool");
    }
    // one block of one cache, all kv heads: contiguous in both layouts
    const size_t bytes = size_t(num_kv_heads) * PA_BLOCK_SIZE * PA_HEAD_DIM * 2;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // runs of consecutive (src, dst) blocks become one transfer
    int64_t i = 0;
    while (i < n_pairs) {
      int64_t j = i + 1;
      while (j < n_pairs && host_pairs[2 * j] == host_pairs[2 * i] + (j - i) &&
             host_pairs[2 * j + 1] == host_pairs[2 * i + 1] + (j - i))
        ++j;
      const size_t so = size_t(host_pairs[2 * i]) * bytes, dof = size_t(host_pairs[2 * i + 1]) * bytes;
      const size_t len = size_t(j - i) * bytes;
      hipError_t e = hipMemcpyAsync(static_cast<char*>(dst_k) + dof,
                                    static_cast<const char*>(src_k) + so, len, hipMemcpyDefault, st);
      if (e != hipSuccess) return hip_fail(e, "swap K copy");
      e = hipMemcpyAsync(static_cast<char*>(dst_v) + dof, static_cast<const char*>(src_v) + so, len,
                         hipMemcpyDefault, st);
      if (e != hipSuccess) return hip_fail(e, "swap V copy");
      i = j;
    }
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected host exception");
  }
}

int pa_store_kv(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                int64_t num_tokens, void* k_cache, void* v_cache, int64_t num_blocks,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, void* stream) {
  try {
    if (num_tokens < 0) return fail(PA_ERR_BAD_SHAPE, "num_tokens < 0");
    if (num_kv_heads <= 0) return fail(PA_ERR_BAD_SHAPE, "num_kv_heads must be positive");
    if (head_dim != PA_HEAD_DIM) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 128");
    if (block_size != PA_BLOCK_SIZE) return fail(PA_ERR_UNSUPPORTED, "block_size must be 256");
    if (num_blocks <= 0) return fail(PA_ERR_BAD_SHAPE, "num_blocks must be positive");
    if (num_blocks > (int64_t(INT32_MAX) + 1) / PA_BLOCK_SIZE)
      return fail(PA_ERR_BAD_SHAPE, "pool has more slots than an int32 slot can address");
    if (num_kv_heads > 65535) return fail(PA_ERR_BAD_SHAPE, "num_kv_heads > 65535");
    if (num_tokens == 0) return ok();
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
      return fail(PA_ERR_NULL_PTR, "pa_store_kv: a pointer argument is NULL");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(slot_mapping, 4))
      return fail(PA_ERR_ALIGN, "bf16 arrays must be 16-byte aligned, slot_mapping 4-byte");
    if ((num_tokens + pa::kTile - 1) / pa::kTile > INT32_MAX)
      return fail(PA_ERR_BAD_SHAPE, "num_tokens too large");
    pa::StoreArgs a;
    a.k_new = static_cast<const uint4*>(k_new);
    a.v_new = static_cast<const uint4*>(v_new);
    a.slots = slot_mapping;
    a.k_cache = static_cast<uint4*>(k_cache);
    a.v_cache = static_cast<uint4*>(v_cache);
    a.n = num_tokens;
    a.num_slots = num_blocks * PA_BLOCK_SIZE;
    a.hkv = num_kv_heads;
    if (debug_checks_on()) {
      int flags = 0;
      const hipError_t ce = pa::check_slots(slot_mapping, num_tokens, a.num_slots,
                                            static_cast<hipStream_t>(stream), &flags);
      if (ce != hipSuccess) return hip_fail(ce, "store_kv checks");
      if (flags) return precondition_fail(flags);
    }
    const hipError_t e = pa::launch_store_kv(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "store_kv launch");
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected host exception");
  }
}

size_t pa_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size) {
  return pa_decode_multi_workspace_size(batch, 1, num_q_heads, num_kv_heads, head_dim, block_size);
}

size_t pa_decode_multi_workspace_size(int32_t batch, int32_t q_per_seq, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
  try {
    int group = 0;
    if (batch < 0) return 0;
    if (check_geometry(num_q_heads, num_kv_heads, head_dim, block_size, &group) != PA_OK) return 0;
    const int gv = virtual_group(group, q_per_seq);
    if (gv == 0) return 0;
    int cus = 0;
    if (current_cus(&cus) != PA_OK) return 0;
    const int64_t waves = int64_t(cus) * pa::kDecodeWavesPerCU;
    return decode_ws_bytes(batch, num_kv_heads, gv, waves);
  } catch (...) {
    return 0;
  }
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t batch, int32_t max_context_len,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int64_t num_blocks, float scale, void* workspace, size_t workspace_bytes,
              void* stream) {
  return decode_rows(out, q, nullptr, nullptr, k_cache, v_cache, block_table, max_blocks_per_seq, context_lens,
                     batch, 1, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     workspace, workspace_bytes, stream);
}

int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                     void* v_cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int64_t num_blocks, float scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (batch > 0 && (k_new == nullptr || v_new == nullptr))
    return fail(PA_ERR_NULL_PTR, "pa_decode_append: k_new or v_new is NULL");
  return decode_rows(out, q, k_new, v_new, k_cache, v_cache, block_table, max_blocks_per_seq, context_lens,
                     batch, 1, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     scale, workspace, workspace_bytes, stream);
}

int pa_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* block_table,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                             int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                             void* stream) {
  static_assert(pa::kNoAllocScratchBytes == PA_DECODE_NOALLOC_SCRATCH_BYTES,
                "scratch size differs from the header's");
  if (batch > 0 && (k_new == nullptr || v_new == nullptr))
    return fail(PA_ERR_NULL_PTR, "pa_decode_append_noalloc: k_new or v_new is NULL");
  return decode_rows(out, q, k_new, v_new, k_cache, v_cache, block_table, max_blocks_per_seq, context_lens,
                     batch, 1, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     scale, nullptr, 0, stream, true);
}

int pa_decode_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t batch, int32_t q_per_seq,
                    int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_rows(out, q, nullptr, nullptr, k_cache, v_cache, block_table, max_blocks_per_seq, context_lens,
                     batch, q_per_seq, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, scale, workspace, workspace_bytes, stream);
}

size_t pa_prefill_workspace_size(int32_t batch, int64_t total_q_rows, int32_t max_seqlen_q,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq) {
  try {
    int group = 0;
    if (batch < 0 || total_q_rows < 0 || max_seqlen_q < 0 || max_blocks_per_seq <= 0) return 0;
    if (check_geometry(num_q_heads, num_kv_heads, head_dim, block_size, &group) != PA_OK) return 0;
    const PrefillSplit ps = prefill_split(batch, total_q_rows, max_seqlen_q, num_q_heads,
                                          num_kv_heads, group, max_blocks_per_seq);
    return ps.ml_bytes + ps.o_bytes + ps.plan_bytes;
  } catch (...) {
    return 0;
  }
}

int pa_prefill(void* out, const void* q, const int32_t* cu_seqlens_q,
               const int32_t* context_lens, int32_t batch, int32_t max_seqlen_q,
               int64_t total_q_rows, const void* k_cache, const void* v_cache,
               const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
               float scale, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (batch < 0) return fail(PA_ERR_BAD_SHAPE, "batch < 0");
    if (total_q_rows < 0) return fail(PA_ERR_BAD_SHAPE, "total_q_rows < 0");
    int group = 0;
    int r = check_geometry(num_q_heads, num_kv_heads, head_dim, block_size, &group);
    if (r != PA_OK) return r;
    if (max_blocks_per_seq <= 0) return fail(PA_ERR_BAD_SHAPE, "max_blocks_per_seq must be positive");
    if (num_blocks <= 0) return fail(PA_ERR_BAD_SHAPE, "num_blocks must be positive");
    if (max_seqlen_q < 0 || int64_t(max_seqlen_q) > int64_t(max_blocks_per_seq) * PA_BLOCK_SIZE)
      return fail(PA_ERR_BAD_SHAPE, "max_seqlen_q outside [0, max_blocks_per_seq*block_size]");
    if (!std::isfinite(scale)) return fail(PA_ERR_BAD_SHAPE, "scale is not finite");
    if (batch == 0 || max_seqlen_q == 0 || total_q_rows == 0) return ok();
    if (!out || !q || !cu_seqlens_q || !context_lens || !k_cache || !v_cache || !block_table)
      return fail(PA_ERR_NULL_PTR, "pa_prefill: a pointer argument is NULL");
    const PrefillSplit ps = prefill_split(batch, total_q_rows, max_seqlen_q, num_q_heads,
                                          num_kv_heads, group, max_blocks_per_seq);
    const size_t need = ps.ml_bytes + ps.o_bytes + ps.plan_bytes;
    if (need > 0) {
      if (workspace == nullptr) return fail(PA_ERR_WORKSPACE, "workspace is NULL");
      if (!aligned(workspace, 256)) return fail(PA_ERR_ALIGN, "workspace must be 256-byte aligned");
      if (workspace_bytes < need)
        return fail(PA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                          std::to_string(workspace_bytes));
    }
    if (int64_t(batch) * ps.max_splits > int64_t(INT32_MAX) || 2 * int64_t(ps.nqb_max) > 65535 ||
        num_kv_heads > 65535)
      return fail(PA_ERR_BAD_SHAPE, "launch grid too large");
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(cu_seqlens_q, 4))
      return fail(PA_ERR_ALIGN, "bf16 arrays must be 16-byte aligned, int32 arrays 4-byte");
    pa::PrefillArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint4*>(k_cache);
    a.v_cache = static_cast<const uint4*>(v_cache);
    a.block_table = block_table;
    a.cu_q = cu_seqlens_q;
    a.ctx_lens = context_lens;
    a.out = static_cast<uint16_t*>(out);
    a.num_blocks = num_blocks;
    a.batch = batch;
    a.hq = num_q_heads;
    a.hkv = num_kv_heads;
    a.mbps = max_blocks_per_seq;
    a.max_q = max_seqlen_q;
    a.scale_log2 = float(double(scale) * 1.4426950408889634);
    a.split_tiles = ps.split_tiles;
    a.max_splits = ps.max_splits;
    a.total_q = total_q_rows;
    char* wsb = static_cast<char*>(workspace);
    a.rec_ml = ps.ml_bytes > 0 ? reinterpret_cast<float*>(wsb) : nullptr;
    a.rec_o = ps.o_bytes > 0 ? reinterpret_cast<float*>(wsb + ps.ml_bytes) : nullptr;
    a.plan = ps.plan ? reinterpret_cast<int32_t*>(wsb + ps.ml_bytes + ps.o_bytes) : nullptr;
    a.plan_rec = ps.plan ? a.plan + pa::kPlanHeader + ps.plan_items : nullptr;
    a.plan_cnt = ps.plan ? a.plan_rec + ps.cands : nullptr;
    a.plan_items = int(ps.plan_items);
    a.slots = int(kPrefillSlots);
    if (debug_checks_on()) {
      pa::SeqCheckArgs c{};
      c.ctx_lens = context_lens;
      c.block_table = block_table;
      c.cu_q = cu_seqlens_q;
      c.num_blocks = num_blocks;
      c.total_q = total_q_rows;
      c.batch = batch;
      c.mbps = max_blocks_per_seq;
      c.max_context_len = int(std::min<int64_t>(int64_t(max_blocks_per_seq) * PA_BLOCK_SIZE, INT32_MAX));
      c.max_q = max_seqlen_q;
      c.rows_per_seq = 1;
      int flags = 0;
      const hipError_t ce = pa::check_seqs(c, static_cast<hipStream_t>(stream), &flags);
      if (ce != hipSuccess) return hip_fail(ce, "prefill checks");
      if (flags) return precondition_fail(flags);
    }
    const hipError_t e = pa::launch_prefill(a, group, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return fail(PA_ERR_UNSUPPORTED, "prefill kernel not available");
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected host exception");
  }
}

}  // extern "C"
