// Internal interface between the C-ABI host layer (api.cpp) and the kernel
// translation units.  Launchers validate nothing: api.cpp has already checked
// every argument.  Each returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "pa_common.hpp"

namespace pa {


// Partial-state record of one decode work piece: G rows of D fp32 weighted
// values, then G maxima, then G sums (floats).
__host__ __device__ constexpr int partial_floats(int g) { return (g * (kDim + 2) + 3) & ~3; }

struct StoreArgs {
  const uint4* k_new;
  const uint4* v_new;
  const int32_t* slots;
  uint4* k_cache;
  uint4* v_cache;
  int64_t n;
  int64_t num_slots;
  int hkv;
};

struct DecodeArgs {
  const uint16_t* q;
  const uint4* k_cache;
  const uint4* v_cache;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  uint16_t* out;
  float* ws;         // partial records (after the counters)
  int* counters;     // one arrival counter per segment; zero between calls
  int64_t num_blocks;
  int batch;
  int hkv;
  int mbps;        // max_blocks_per_seq
  int n_waves;     // waves in the split-context grid
  int run_w_even;  // relative run length of waves on even- / odd-numbered XCDs
  int run_w_odd;
  float scale_log2;  // scale * log2(e)
  // Query rows: ql per sequence (1 for decode), gr q heads per kv head, hq q
  // heads.  The kernel's G = gr * ql rounded up to a power of two "virtual
  // heads" per (sequence, kv head): virtual head v is query token
  // b*ql + (v >> gr_shift), head g*gr + (v & (gr-1)); it sees keys
  // 0 .. ctx - ql + (v >> gr_shift).  Virtual heads past ql rows are padding.
  int ql;
  int gr;
  int gr_shift;
  int hq;
  // Appended token (one query row per sequence only): when k_new is set, the
  // token at position ctx-1 of every sequence is new.  Its K/V rows
  // k_new/v_new [batch][hkv][kDim] take part in the attention directly (the
  // kernel streams positions 0 .. ctx-2 from the cache) and are written into
  // the cache at that position through the block table.
  const uint4* k_new;
  const uint4* v_new;
  uint4* k_store;
  uint4* v_store;
};


struct CopyBlocksArgs {
  const int32_t* pairs;  // [n_pairs][2] (src, dst)
  int64_t n_pairs;
  uint4* k_cache;
  uint4* v_cache;
  int64_t num_blocks;
  int hkv;
};

// Waves per CU the decode grid is sized for.  A workgroup holds the waves of
// one CU: 8, or 4 for G = 8 (whose waves need twice the registers).
constexpr int kDecodeWavesPerCU = 8;
// Workgroup b of a launch runs on XCD b % 8, and the odd-numbered XCDs
// stream about 9 % slower than the even ones under the same load (measured
// per XCD with the hardware's realtime counter on every MI355X we ran on), so
// their waves get runs 11/12 as long and all XCDs finish together.
constexpr int kRunWeightEven = 12;
constexpr int kRunWeightOdd = 11;
// The matrix-core decodes of 5..16 and 17..32 rows per (sequence, kv head)
// (decode_mfma16.hip, "G" = 16; decode_mfma.hip, "G" = 32) run 4 waves per
// CU, one per SIMD.
__host__ __device__ constexpr int decode_group_waves(int g) { return g >= 8 ? 4 : 8; }

// Records a status and its detail string for pa_last_error_detail (thread
// local); returns the status.
int report_error(int code, const std::string& msg);

// Device-side precondition checks (debug mode): bits of the violated
// conditions, read back synchronously.
constexpr int kCheckSlot = 1;   // a slot past the pool
constexpr int kCheckCtx = 2;    // a context length outside [0, cap]
constexpr int kCheckTable = 4;  // a used block-table entry outside the pool
constexpr int kCheckRows = 8;   // cu_seqlens_q / rows per sequence inconsistent
struct SeqCheckArgs {
  const int32_t* ctx_lens;
  const int32_t* block_table;
  const int32_t* cu_q;  // varlen calls, else nullptr
  int64_t num_blocks;
  int64_t total_q;
  int batch;
  int mbps;
  int max_context_len;
  int max_q;
  int rows_per_seq;     // decode: query rows per sequence
};
hipError_t check_slots(const int32_t* slots, int64_t n, int64_t num_slots, hipStream_t s, int* flags);
hipError_t check_seqs(const SeqCheckArgs& a, hipStream_t s, int* flags);

hipError_t launch_store_kv(const StoreArgs& a, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int group, hipStream_t s);
// pa_decode_multi with 17 to 32 rows per (sequence, kv head), on the matrix
// cores (records of 32 rows).
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s);
// ... with 5 to 16 rows (records of 16 rows).
hipError_t launch_decode_mfma16(const DecodeArgs& a, hipStream_t s);

// Library-owned decode workspace of the allocation-free decode step: the
// bytes of the per-device array (decode.hip), and its device address on the
// current device, found once per device and cleared on `s` at that first
// use (later calls find it as the previous call left it: records are
// scratch, counters are back at zero).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(hipStream_t s, void** ptr);

}  // namespace pa
