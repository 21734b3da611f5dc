// Internal interface between the C-ABI layer (pa_api.cpp) and the HIP kernel
// launchers (kv_write.hip, decode.hip, prefill.hip). Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

// Set the calling thread's pa_last_error() text and return `st`; report_ok()
// clears it and returns PA_OK.
pa_status report(pa_status st, const char* fmt, ...);
pa_status report_ok();

constexpr int kBlockTokens = 16;  // token slots per KV block
constexpr int kWaves = 4;         // waves per workgroup (KV write, reduce, prefill)
constexpr int kThreads = 64 * kWaves;
constexpr int kDecodeWaves = 8;   // waves per decode workgroup
constexpr int kDecodeThreads = 64 * kDecodeWaves;
// Largest split-K partition (256 blocks). Batches with many sequences run
// most of them as one partition (no partial results to write and combine);
// the cap bounds how long the last workgroups of a launch can run.
constexpr int64_t kMaxPartitionTokens = 4096;

// The decode kernel's MFMA tiles have 16 columns: (new token, query head)
// pairs of one KV head. A sequence whose n new tokens times G query heads fit
// them (every decode, and short chunks such as speculative-decode
// verification) is attended by the decode kernel, with a causal limit per
// column; longer chunks go to the prefill kernel.
constexpr int kMaxDecodeColumns = 16;
__host__ __device__ inline bool decode_path(int64_t n, int64_t G) { return n >= 1 && n * G <= kMaxDecodeColumns; }

// KV heads one decode workgroup serves: the largest power of two <= 8 that
// divides Hkv (each head gets 8 / that many waves).
inline int decode_heads_per_workgroup(int64_t Hkv) {
  for (int hw : {8, 4, 2}) if (Hkv % hw == 0) return hw;
  return 1;
}

enum class Elem : int { F32 = 0, BF16 = 1 };

// KV write: all strides in bytes.
struct WriteArgs {
  const char* k;
  const char* v;
  char* kc;
  char* vc;
  const int64_t* slots;
  int64_t T, Hkv, D, NB;
  int64_t k_st, k_sh, v_st, v_sh;        // k/v: token and head strides
  int64_t kc_sb, kc_sr, kc_sh;           // key cache: block, row, head strides
  int64_t vc_sb, vc_sr, vc_sh;           // value cache
  int es;                                // element bytes of k and v
  bool kv8;                              // the caches hold fp8 codes: each element is quantized
  float k_scale, v_scale;                // fp8 only: code = nearest(x / scale)
};

// Attention: all tensor strides in bytes except the int32 tables (elements).
struct AttnArgs {
  char* out;
  const char* q;
  const char* kc;
  const char* vc;
  const int32_t* block_tables;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* ctx_lens;
  int64_t T, S, MB, NB, Hq, Hkv, D;
  int64_t out_st, out_sh, q_st, q_sh;
  int64_t kc_sb, kc_sr, kc_sh, vc_sb, vc_sr, vc_sh;
  int64_t bt_row;  // block-table row stride (elements)
  float scale;
  Elem elem;              // q, out and the compute path
  bool kv8;               // the caches hold fp8 codes (elem is bf16)
  float k_scale, v_scale;  // fp8 only: a cached element reads back as value(code) * scale
  // split-K decode
  int64_t part_tokens;  // tokens per partition (multiple of 16)
  int64_t max_parts;    // partitions per sequence at most: ceil(MB * 16 / part_tokens)
  float* ws_o;          // [S][Hq][max_parts][D] unnormalised partial outputs
  float2* ws_ml;        // [S][Hq][max_parts] (running max in log2 units, sum of weights)
  // prefill work list
  int32_t* tile_start;    // [S + 1] exclusive prefix sum of prefill q-tiles per sequence
  int32_t* tile_order;    // [kMaxSortedTiles][kTileRecord] per rank of the q-tiles by decreasing key count (if
                          // they fit): sequence, tile, query start, query count, cached context, length,
                          // 2 unused, then the sequence's first 8 block-table entries
  int32_t* work_counter;  // [0] prefill work-queue head, zeroed by the plan kernel; [1] prefill workgroups that
                          // run beside the decode kernel (set by the plan kernel); [2], [3] the bf16 prefill's
                          // cost capacity per workgroup (int64, low word first)
  int32_t* sched;         // [kMaxPrefillWorkgroups] first item of each bf16 prefill workgroup, then
                          // [kMaxPrefillWorkgroups] merge counters of split items (both set by the plan kernel)
  int32_t* dorder;        // the decode workgroups' work, longest first: [0] count, [1] the decode's claim
                          // counter (zeroed), then from word kDecodeOrderHeader one kDecodeOrderRecord-word
                          // record per unit (set by decode_order_kernel; read by the decode kernel when
                          // its launch is ordered)
};

// Rates measured on MI355X at head size 128, for the choice and sizing of
// the prefill beside the decode: a CU of the bf16 prefill kernel computes
// about 4.7 TFLOP/s; the decode kernel reads about 6.6 TB/s over all 256 CUs.
constexpr float kPrefillFlopPerCuUs = 4.7e6f;
constexpr float kDecodeBytePerCuUs = 6.6e6f / 256.0f;

// The bf16 prefill launches at most one workgroup per CU.
constexpr int kMaxPrefillWorkgroups = 256;

// Up to this many prefill q-tiles are sorted by cost (longest first) before
// the prefill kernel takes them from a queue; beyond it they go in order.
constexpr int kMaxSortedTiles = 4096;
constexpr int kTileRecord = 16;  // int32 words per ranked-tile record

// Decode work order: a launch whose grid holds more than one round of
// workgroups takes its (sequence, head group, partition) units longest
// first. A record: unit x = sequence * head groups + group, partition, the
// sequence's query start and end, its length and cached context (as in the
// caller's arrays), 2 unused. At most kMaxOrderedUnits units are ordered.
constexpr int kDecodeOrderHeader = 64;  // int32 words before the first record
constexpr int kDecodeOrderRecord = 8;   // int32 words per record
constexpr int64_t kMaxOrderedUnits = int64_t(1) << 20;

struct WorkspaceLayout {
  size_t tile_start_off, counter_off, order_off, sched_off, dorder_off, ml_off, o_off, total;
};

// Tokens per split-K decode partition. per_cu: decode workgroups a CU holds at
// once (decode_workgroups_per_cu; 0 if unknown); the workspace is sized for 2.
int64_t partition_tokens(int64_t S, int64_t Hkv, int64_t MB, int per_cu);
WorkspaceLayout workspace_layout(int64_t S, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int64_t MB);

// Optional per-kernel HIP-event timing (include/pa_profile.h).
enum KernelId { kKvWrite = 0, kDecode = 1, kReduce = 2, kPlan = 3, kPrefill = 4, kWritePlan = 5, kDecodeOrder = 6 };
bool profiling();
void profile_mark(int id, bool end, hipStream_t stream);
struct ProfileScope {
  int id;
  hipStream_t stream;
  bool on;
  ProfileScope(int id_, hipStream_t s) : id(id_), stream(s), on(profiling()) {
    if (on) profile_mark(id, false, stream);
  }
  ~ProfileScope() {
    if (on) profile_mark(id, true, stream);
  }
};

// pa_step / pa_step_fp8 (pa_api.cpp). allow_side = false keeps every launch
// on `stream` (no stream or event of the library's own is created or used).
pa_status step_impl(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                    const pa_tensor* key_cache, const pa_tensor* value_cache, const pa_tensor* slot_mapping,
                    const pa_tensor* block_tables, const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                    const pa_tensor* context_lens, float scale, bool fp8, float k_scale, float v_scale,
                    void* workspace, size_t workspace_bytes, pa_stream stream, bool allow_side);

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream);
// Decode kernel, then (with_reduce) the partition reduce (decode.hip).
hipError_t launch_decode(const AttnArgs& a, hipStream_t stream, bool with_reduce);
// Workgroups of the decode kernel for these element types and head size that
// one CU holds at once (HIP occupancy query); 0 when unknown.
int decode_workgroups_per_cu(Elem elem, bool kv8, int64_t D);
// The partition reduce alone (decode.hip).
hipError_t launch_reduce(const AttnArgs& a, hipStream_t stream);
// prefill.hip: the plan kernel (prefill tile list and queue, and the
// prefill's share of the CUs when it runs `beside` the decode on another
// stream); the plan and the KV write in one launch (when the prefill runs
// after the decode); the chunked-prefill kernel, after a plan, which first
// combines the decode's partitions when `fold_reduce` (it then runs after the
// decode on the same stream); and whether a prefill launch has any workgroup.
hipError_t launch_plan(const AttnArgs& a, hipStream_t stream, bool beside);
hipError_t launch_write_plan(const WriteArgs& w, const AttnArgs& a, hipStream_t stream);
hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream, bool beside, bool fold_reduce);
bool prefill_launches(const AttnArgs& a);

}  // namespace pa
