// Chunked-prefill attention: sequences with more than one new token. Query i
// of a chunk that follows C cached tokens sits at position C + i and sees keys
// 0 .. C + i: the whole cached context plus the chunk's own earlier tokens
// (ngrok "Serving models at scale with vLLM", section "Chunked prefill": a
// later chunk reads the earlier chunks' K/V from the cache, and a token
// depends only on the tokens before it). A dense contraction, compute-bound
// ("Inside vLLM", section "Scheduler": prefill is usually compute-bound).
//
// Design for gfx950 (the pages give no kernel design):
//  - A plan kernel lists the q-tiles of every prefill sequence, sorts them by
//    key count (longest first, when they fit in one workgroup's sort) and
//    records each rank's (sequence, tile), so the host never reads lengths.
//    For the bf16 kernel it also splits the items' total cost into one equal
//    share per workgroup (McNaughton's wrap-around rule over the ranked
//    items): an item that straddles two shares is cut along its keys, each
//    workgroup computes its piece, and the piece that finishes last combines
//    the pieces' partial results. The 9x spread of chunk contexts then leaves
//    no longest-item tail, and a few long items still fill every CU. The fp32
//    kernel takes tiles from a work queue instead.
//  - bf16: one workgroup of 8 waves per CU (two per SIMD) owns one (q-tile,
//    KV head, group of HW query heads); wave w takes query head w % HW and
//    32 tokens of sub-tile w / HW. The waves share K/V tiles of 64 keys.
//  - K and V tiles go from HBM straight into LDS (buffer loads that write
//    LDS), four stages deep: a tile is requested two tiles before its use and
//    no registers hold data in flight. Rows are stored with a 16-byte XOR
//    swizzle that keeps both fragment read patterns free of bank conflicts.
//  - S^T = K . Q^T on 32x32x16 bf16 MFMA (keys as rows): each lane owns one
//    query token, so the row max needs one cross-lane exchange and the output
//    rescale none. The scores are already the B operand of O^T = V^T . P^T; the
//    V^T operand comes straight from the row-major tile through gfx950's
//    transposing LDS read (ds_read_b64_tr_b16), two per MFMA.
//  - Each wave runs a software pipeline over 32-key slices: step j computes
//    the weights of slice j while its MFMAs are the score chain of slice
//    j + 1 and P.V of slice j - 1. The MFMAs go out one at a time between
//    shares of the vector work, dependent chain MFMAs alternating with
//    independent P.V ones, and fragment reads run a few MFMAs ahead.
//  - Online softmax in log2 units with the scale folded into one FMA before
//    exp2, the same lazy rescale as decode, and the causal mask only on
//    slices that cross the wave's diagonal.
//  - fp32 inputs take a simpler exact kernel (fp32 MFMA, V transposed while
//    staging); it exists for accuracy, not speed.
#include <algorithm>
#include <type_traits>

#include "pa_internal.h"
#include "step_parts.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) const uint4 lds_u4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) int lds_int;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;
// The bf16 kernel keeps its reference maximum while a slice's weights (16
// per lane) sum to at most 2^8; each weight is then at most 2^8 as well.
constexpr float kRescaleBound = 256.0f;
// Word 3 of a raw (unformatted, unswizzled) buffer resource on gfx9-family
// parts: 32-bit data format, no index stride.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of a buffer access that other XCDs' workgroups must see: sc1,
// which the compiler also gives agent-scope atomic loads and stores (each XCD
// has its own L2).
constexpr int kCoherent = 16;
constexpr int kWaveTokens = 32;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Tokens per workgroup tile for a given number of heads per workgroup.
constexpr int tile_tokens(int hw) { return kWaveTokens * (kWaves / hw); }
// The bf16 kernel runs 8 waves per workgroup (one workgroup per CU, two
// waves per SIMD): twice the query rows share each staged K/V tile.
constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int bf16_tile_tokens(int hw) { return kWaveTokens * (kPWaves / hw); }

// CUs of the prefill beside the decode kernel (bf16 steps over a bf16 pool
// whose prefill is large enough, chosen on the host): ratio * 256 * prefill
// work / (prefill + decode work), with the rates kPrefillFlopPerCuUs and
// kDecodeBytePerCuUs, the prefill also paying about 6 us per item outside
// its key loop. Ratio 2: the share would finish in about half the decode's
// time alone; beside the decode's HBM stream it takes most of it, and the
// HBM-bound decode barely notices the CUs it lost (ratio 4 ran 1.5-3.5%
// slower on prefill-heavy steps).
constexpr float kBesideRatio = 2.0f;
constexpr float kPrefillItemCuUs = 6.0f;

// Static schedule of the bf16 prefill kernel. Costs are in quarters of a
// 64-key tile: an item costs kItemFixedQ for its start and end plus 4 per
// K/V tile it reads (measured on MI355X at head size 128: about 4.4 us per
// item and 1.86 us per tile).
constexpr int kPrefillKeyTile = 64;
constexpr int64_t kItemFixedQ = 9;
__device__ inline int64_t item_cost_q(int64_t key_tiles) { return kItemFixedQ + 4 * key_tiles; }
// Workgroup b runs on XCD b mod 8, and each XCD has its own L2. The schedule
// keeps the items of KV head g on the workgroups with b = g (mod nclass):
// the token tiles of a chunk that read the same K/V then share one L2. Each
// class splits its own items among its nwg / nclass workgroups (every rank
// holds the same number of items of each class, so the classes' loads are
// equal).
__device__ inline int schedule_classes(int64_t Hkv, int nwg) {
  const int c = Hkv % 8 == 0 ? 8 : Hkv % 4 == 0 ? 4 : Hkv % 2 == 0 ? 2 : 1;
  return nwg % c == 0 ? c : 1;
}

// One block of 1024 threads: per-sequence tile counts, exclusive scan into
// tile_start, cost-sorted tile order (if it fits), queue head reset, and the
// number of prefill workgroups to run when the prefill shares the GPU with
// the decode kernel: enough CUs that the prefill work takes about half as
// long as the decode work on the rest (all slots when there is no decode
// work). With sorted tiles it also lays out the bf16 kernel's static
// schedule: the cost prefix of every rank, each workgroup's equal share of
// the total cost (its capacity) and the item in which each share starts.
__device__ void plan_body(const int32_t* qsl, const int32_t* ctx_lens,
                                                    const int32_t* seq_lens, const int32_t* block_tables,
                                                    int64_t bt_row, int64_t S, int64_t T, int64_t MB,
                                                    int64_t G, int qtile, int64_t Hq, int64_t D,
                                                    int64_t kv_token_bytes, int items_per_tile, int slots,
                                                    int beside, float flop_per_cu_us, int wg_per_cu, float ratio,
                                                    int32_t* tile_start, int32_t* tile_order,
                                                    int32_t* counter, int32_t* sched) {
  __shared__ int32_t part[1024];
  __shared__ int32_t n_active;
  __shared__ float red_dec[1024], red_pre[1024];
  __shared__ uint64_t keys[kMaxSortedTiles];
  // sequence of each tile (sorted case); later reused as int64 scratch, hence 8-byte aligned
  __shared__ __attribute__((aligned(8))) int32_t tile_seq[kMaxSortedTiles];
  const int tid = threadIdx.x;
  const int64_t per = (S + 1023) / 1024;
  const int64_t s0 = min(S, tid * per), s1 = min(S, s0 + per);
  auto qlen = [&](int64_t s) -> int64_t {
    const int64_t a = min(max(static_cast<int64_t>(qsl[s]), int64_t(0)), T);
    const int64_t b = min(max(static_cast<int64_t>(qsl[s + 1]), a), T);
    return b - a;
  };
  // sequences on the decode kernel's path get no prefill tiles
  auto tiles = [&](int64_t n) -> int32_t {
    return n >= 1 && !decode_path(n, G) ? static_cast<int32_t>((n + qtile - 1) / qtile) : 0;
  };
  int32_t sum = 0;
  float dec_tokens = 0.f, pre_token_keys = 0.f;  // decode keys; prefill (query token, key) pairs (upper bound)
  for (int64_t s = s0; s < s1; ++s) {
    const int64_t n = qlen(s);
    const int32_t nt = tiles(n);
    sum += nt;
    if (!beside || n < 1) continue;
    const int64_t Lc = min(max(static_cast<int64_t>(seq_lens[s]), int64_t(0)), MB * kBlockTokens);
    if (nt == 0) {
      dec_tokens += static_cast<float>(Lc);
    } else {
      const int64_t C = min(max(static_cast<int64_t>(ctx_lens[s]), int64_t(0)), Lc);
      for (int64_t i0 = 0; i0 < n; i0 += qtile)
        pre_token_keys += static_cast<float>(min(int64_t(qtile), n - i0)) *
                          static_cast<float>(min(C + min(n, i0 + qtile), Lc));
    }
  }
  part[tid] = sum;
  red_dec[tid] = dec_tokens;
  red_pre[tid] = pre_token_keys;
  __syncthreads();
  if (beside) {
    for (int off = 512; off > 0; off >>= 1) {
      if (tid < off) {
        red_dec[tid] += red_dec[tid + off];
        red_pre[tid] += red_pre[tid + off];
      }
      __syncthreads();
    }
  }
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int32_t total = part[1023];
  int len = 1;  // the sort covers the next power of two >= total
  while (len < total) len <<= 1;
  if (total <= kMaxSortedTiles)
    for (int i = total + tid; i < len; i += 1024) keys[i] = 0;  // empty slots sort last
  int32_t run = part[tid] - sum;
  for (int64_t s = s0; s < s1; ++s) {
    tile_start[s] = run;
    const int64_t n = qlen(s);
    const int32_t nt = tiles(n);
    if (total <= kMaxSortedTiles) {
      const int64_t C = max(static_cast<int64_t>(ctx_lens[s]), int64_t(0));
      const int64_t Lc = min(max(static_cast<int64_t>(seq_lens[s]), int64_t(0)), MB * kBlockTokens);
      for (int32_t lt = 0; lt < nt; ++lt) {
        const int64_t cost = max(int64_t(0), min(C + min(n, int64_t(lt + 1) * qtile), Lc));
        const uint32_t t = static_cast<uint32_t>(run + lt);
        keys[t] = (static_cast<uint64_t>(cost) << 32) | (0xffffffffu - t);
        tile_seq[t] = static_cast<int32_t>(s);
      }
    }
    run += nt;
  }
  if (tid == 1023) tile_start[S] = total;
  if (tid == 0) {
    counter[0] = 0;
    const float pre = red_pre[0] * 4.f * static_cast<float>(D * Hq) / flop_per_cu_us +
                      static_cast<float>(total) * items_per_tile * kPrefillItemCuUs;
    const float dec = red_dec[0] * static_cast<float>(kv_token_bytes) / kDecodeBytePerCuUs;
    int active = 0;
    if (total > 0)
      active = (beside && dec > 0.f) ? static_cast<int>(ceilf(ratio * 256.f * pre / (pre + dec))) : slots;
    n_active = min(max(active * wg_per_cu, total > 0 ? 1 : 0), slots);  // CUs -> workgroups
    counter[1] = n_active;
  }
  if (total > kMaxSortedTiles) return;  // uniform: tiles go in sequence order
  __syncthreads();
  // bitonic sort, descending (empty slots hold key 0 and sort last)
  for (int k = 2; k <= len; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < len; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = keys[i], y = keys[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? x < y : x > y) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  // One record per rank: the tile, its sequence's clamped lengths and the
  // block ids of its first key tiles, so that a workgroup can start an item's
  // first K/V loads after a single load.
  for (int i = tid; i < total; i += 1024) {
    const int32_t t = static_cast<int32_t>(0xffffffffu - uint32_t(keys[i]));
    const int32_t sq = tile_seq[t];
    const int64_t q0 = min(max(static_cast<int64_t>(qsl[sq]), int64_t(0)), T);
    const int64_t n = min(max(static_cast<int64_t>(qsl[sq + 1]), q0), T) - q0;
    const int64_t Lc = min(max(static_cast<int64_t>(seq_lens[sq]), int64_t(0)), MB * kBlockTokens);
    const int64_t C = min(max(static_cast<int64_t>(ctx_lens[sq]), int64_t(0)), Lc);
    int4* rec = reinterpret_cast<int4*>(tile_order + kTileRecord * i);
    rec[0] = make_int4(sq, t - tile_start[sq], static_cast<int32_t>(q0), static_cast<int32_t>(n));
    rec[1] = make_int4(static_cast<int32_t>(C), static_cast<int32_t>(Lc), 0, 0);
    // the block ids of the first two key tiles (8 blocks), as the table has them
    const int32_t* row = block_tables + sq * bt_row;
    auto id = [&](int j) { return row[min(int64_t(j), MB - 1)]; };
    rec[2] = make_int4(id(0), id(1), id(2), id(3));
    rec[3] = make_int4(id(4), id(5), id(6), id(7));
  }
  if (sched == nullptr) return;
  if (total == 0) {  // no prefill items: every workgroup's first item is past the end
    for (int b = tid; b < kMaxPrefillWorkgroups; b += 1024) sched[b] = 0;
    return;
  }
  // Cost prefix over the ranks (each rank stands for items_per_tile items of
  // equal cost), kept in keys[] once every record is written.
  __syncthreads();
  int64_t* const pre = reinterpret_cast<int64_t*>(tile_seq);  // 1024 of its 2048 int64 slots
  int64_t cr[kMaxSortedTiles / 1024];
  int64_t csum = 0;
#pragma unroll
  for (int k = 0; k < kMaxSortedTiles / 1024; ++k) {
    const int r = (kMaxSortedTiles / 1024) * tid + k;
    const int64_t keys_r = r < total ? static_cast<int64_t>(keys[r] >> 32) : 0;
    cr[k] = r < total ? item_cost_q((keys_r + kPrefillKeyTile - 1) / kPrefillKeyTile) * items_per_tile : 0;
    csum += cr[k];
  }
  pre[tid] = csum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t v = tid >= off ? pre[tid - off] : 0;
    __syncthreads();
    pre[tid] += v;
    __syncthreads();
  }
  int64_t pos = pre[tid] - csum;
  const int64_t p_total = pre[1023];
#pragma unroll
  for (int k = 0; k < kMaxSortedTiles / 1024; ++k) {
    const int r = (kMaxSortedTiles / 1024) * tid + k;
    if (r < total) {
      keys[r] = static_cast<uint64_t>(pos);
      int4* rec = reinterpret_cast<int4*>(tile_order + kTileRecord * r);
      rec[1].z = static_cast<int32_t>(pos & 0xffffffff);
      rec[1].w = static_cast<int32_t>(pos >> 32);
    }
    pos += cr[k];
  }
  __syncthreads();
  // Equal shares within each class of items (schedule_classes): workgroup
  // b = w nclass + x owns costs [w cap, (w + 1) cap) of class x, whose
  // items in rank order have the cost prefix P_rank / nclass (+ the cost of
  // the class's items before it in the rank); its first item (class-local
  // index) is the one whose cost range holds w cap.
  const int nwg = max(1, min(n_active, kMaxPrefillWorkgroups));
  const int nclass = schedule_classes(Hq / G, nwg);
  const int64_t cap = max(int64_t(1), (p_total + nwg - 1) / nwg);
  // Cut items only when the longest one (rank 0) outlasts an equal share by
  // more than a cut costs (a second item start, the partial result's write,
  // count and combine: together about an eighth of a share here). Otherwise
  // the longest-first queue balances the items whole.
  const int64_t longest = (total > 1 ? static_cast<int64_t>(keys[1]) : p_total) / items_per_tile;
  const bool cut = longest > cap + cap / 8;
  if (tid == 0) {
    counter[2] = cut ? static_cast<int32_t>(cap & 0xffffffff) : 0;
    counter[3] = cut ? static_cast<int32_t>(cap >> 32) : 0;
  }
  if (!cut) return;
  const int64_t per_class = items_per_tile / nclass;  // items of one class per rank
  const int64_t class_items = int64_t(total) * per_class;
  const int64_t class_total = p_total / nclass;
  for (int b = tid; b < kMaxPrefillWorkgroups; b += 1024) {
    sched[kMaxPrefillWorkgroups + b] = 0;  // merge counters
    const int64_t at = int64_t(b / nclass) * cap;
    int64_t first = class_items;
    if (b < nwg && at < class_total) {
      int lo = 0, hi = total - 1;  // last rank with class prefix <= at
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(keys[mid]) / nclass <= at) lo = mid; else hi = mid - 1;
      }
      const int64_t p0 = static_cast<int64_t>(keys[lo]) / nclass;
      const int64_t p1 = (lo + 1 < total ? static_cast<int64_t>(keys[lo + 1]) : p_total) / nclass;
      const int64_t per_item = (p1 - p0) / per_class;
      first = int64_t(lo) * per_class + min(per_class - 1, (at - p0) / per_item);
    }
    sched[b] = static_cast<int32_t>(first);
  }
}

// The plan parameters a launch passes to plan_body.
struct PlanArgs {
  const int32_t* qsl;
  const int32_t* ctx_lens;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int64_t bt_row, S, T, MB, G;
  int qtile;
  int64_t Hq, D, kv_token_bytes;
  int items_per_tile, slots, beside;
  float flop_per_cu_us;
  int wg_per_cu;
  float ratio;
  int32_t *tile_start, *tile_order, *counter;
  int32_t* sched;  // the bf16 kernel's static schedule; nullptr for the fp32 kernel (queue)
};

__device__ inline void plan_with(const PlanArgs& p) {
  plan_body(p.qsl, p.ctx_lens, p.seq_lens, p.block_tables, p.bt_row, p.S, p.T, p.MB, p.G, p.qtile, p.Hq, p.D,
            p.kv_token_bytes, p.items_per_tile, p.slots, p.beside, p.flop_per_cu_us, p.wg_per_cu, p.ratio,
            p.tile_start, p.tile_order, p.counter, p.sched);
}

__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs p) { plan_with(p); }

// One launch for a step whose prefill runs after its decode: workgroup 0
// plans (as plan_kernel), the others write the step's new K/V into the pool
// (as the KV write kernels, 1024 lanes per workgroup). Nothing reads the
// pool before the launch has ended, so the two need no ordering.
__global__ __launch_bounds__(1024) void write_plan_kernel(WriteArgs w, int vec_per_head, int tpb, PlanArgs p) {
  if (blockIdx.x == 0) {
    plan_with(p);
    return;
  }
  if (w.kv8) kv_write_fp8_tokens(w, vec_per_head, tpb, int64_t(blockIdx.x) - 1, 1024);
  else kv_write_tokens(w, vec_per_head, tpb, int64_t(blockIdx.x) - 1, 1024);
}

// Which sequence and local tile a queue item names, with the sequence's
// clamped query start, query count, cached context and length.
struct TileRef {
  int64_t s, lt, g, hg, rank;
  int64_t q0, n, C, Lc;
  int64_t P;            // cost prefix of the rank (plan record; bf16 kernel only)
  bool ranked;          // from a plan record, which also holds
  int4 ids_lo, ids_hi;  // the sequence's table entries 0 .. 3 and 4 .. 7
};

__device__ inline TileRef locate(const AttnArgs& a, int64_t item, int n_hg, int64_t total_tiles) {
  TileRef r;
  r.g = item % a.Hkv;
  const int64_t rest = item / a.Hkv;
  r.hg = rest % n_hg;
  const int64_t rank = rest / n_hg;
  r.rank = rank;
  r.P = 0;
  if (total_tiles <= kMaxSortedTiles) {  // the plan kernel wrote one record per rank
    const int4* rec = reinterpret_cast<const int4*>(a.tile_order + kTileRecord * rank);
    const int4 r0 = rec[0], r1 = rec[1], r2 = rec[2], r3 = rec[3];
    r.s = r0.x;
    r.lt = r0.y;
    r.q0 = r0.z;
    r.n = r0.w;
    r.C = r1.x;
    r.Lc = r1.y;
    r.P = (static_cast<int64_t>(r1.w) << 32) | static_cast<uint32_t>(r1.z);
    r.ranked = true;
    r.ids_lo = r2;
    r.ids_hi = r3;
    return r;
  }
  const int64_t t = rank;
  int64_t lo = 0, hi = a.S - 1;  // last s with tile_start[s] <= t
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (a.tile_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  r.s = lo;
  r.lt = t - a.tile_start[lo];
  r.ranked = false;
  r.ids_lo = r.ids_hi = make_int4(0, 0, 0, 0);
  r.q0 = min(max(static_cast<int64_t>(a.qsl[lo]), int64_t(0)), a.T);
  r.n = min(max(static_cast<int64_t>(a.qsl[lo + 1]), r.q0), a.T) - r.q0;
  r.Lc = min(max(static_cast<int64_t>(a.seq_lens[lo]), int64_t(0)), a.MB * kBlockTokens);
  r.C = min(max(static_cast<int64_t>(a.ctx_lens[lo]), int64_t(0)), r.Lc);
  return r;
}

// Pull the next queue item for the whole workgroup.
__device__ inline int64_t next_item(const AttnArgs& a, int* item_sh) {
  if (threadIdx.x == 0) *item_sh = atomicAdd(a.work_counter, 1);
  __syncthreads();
  // uniform across the workgroup: keep it (and all that derives from it) scalar
  const int item = __builtin_amdgcn_readfirstlane(*item_sh);
  __syncthreads();
  return item;
}

// ---------------------------------------------------------------- bf16 ----

template <int D>
struct Bf16Tile {
  static constexpr int KT = 64;                        // keys per tile
  static constexpr int STAGES = 4;                     // LDS stages, for K and for V
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int CHUNKS = KT * CPR;              // per K or V tile
  static constexpr uint32_t TB = CHUNKS * 16;          // bytes of one K or V tile
  static constexpr uint32_t HALF = TB / 2;             // bytes of a 32-key slice
  static constexpr uint32_t V0 = STAGES * TB;          // the V stages follow the K stages
  static constexpr int DPW = CHUNKS / (64 * kPWaves);  // LDS loads per wave per K (or V) tile
  // Chunk c of row r sits at r * CPR + (c ^ swz(r)). LDS has 64 banks of 4
  // bytes, so a 256-byte span is one pass. swz depends on r mod 16 only and
  // keeps the two read patterns at one pass per 256 bytes: 16 rows read at
  // one chunk (K fragments) and 4 consecutive rows x 4 consecutive chunks
  // (transposing V reads).
  __device__ static int swz(int r) {
    return CPR == 16 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  __device__ static int chunk(int r, int c) { return r * CPR + (c ^ swz(r)); }
  static_assert(CPR == 8 || CPR == 16, "head size 64 or 128");
  static_assert(DPW >= 1 && (64 / CPR) <= kBlockTokens, "one load instruction stays inside one cache block");
};

template <int D>
constexpr size_t bf16_lds_bytes() {
  // K and V stages, then each wave's (max, sum) rows of a cut item's partial
  // result, and the schedule's state
  return 2 * Bf16Tile<D>::STAGES * Bf16Tile<D>::TB + kPWaves * 256 + 32;
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// dst + 16 l (dst is wave-uniform); reads at or past rec bytes deliver zeros.
__device__ inline void load_lds16(const char* base, uint32_t rec, uint32_t off, lds_char* dst) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, static_cast<int>(rec), kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, reinterpret_cast<lds_void*>(dst), 16, off, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (s_waitcnt with the export and LDS counts left open).
// The memory clobber keeps the compiler from moving loads across the wait.
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier with no wait of its own. The memory clobber keeps the
// compiler from moving LDS accesses across it; the caller waits for what
// must have landed.
__device__ inline void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }

// f(integral_constant<int, i>) for i = I .. N - 1, unrolled at compile time.
template <int I, int N, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The workgroup's items one after another. dma and rd are two views of the same LDS:
// the tile loads write through dma, the fragment reads go through rd. Between
// two barriers a stage is either being loaded or being read, never both, so
// the two kinds of access are independent; handing the compiler two distinct
// restrict pointers lets it see that (otherwise it waits for every load in
// flight before each LDS read).
template <int D, int HW, bool KV8, bool CUTS>
__device__ __attribute__((always_inline)) inline void prefill_bf16_items(const AttnArgs& a,
                                                                        const int32_t* __restrict__ bt_all,
                                                                        lds_char* __restrict__ dma,
                                                                        const lds_char* __restrict__ rd,
                                                                        int nwg) {
  using Tl = Bf16Tile<D>;
  constexpr int KT = Tl::KT, CPR = Tl::CPR, DPW = Tl::DPW;
  constexpr uint32_t TB = Tl::TB, HALF = Tl::HALF, V0 = Tl::V0;
  constexpr int QTB = bf16_tile_tokens(HW);
  constexpr int QS = D / 16;   // k-steps of S^T
  constexpr int DT = D / 32;   // 32-row tiles of O^T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = lane & 31;  // query token of this lane (B/C column)
  const int hh = lane >> 5;   // lane half
  const int j16 = lane & 15, g16 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave % HW, tw = wave / HW;
  const int G = static_cast<int>(a.Hq / a.Hkv);
  const int n_hg = G / HW;
  const int64_t total_tiles = a.tile_start[a.S];
  const int64_t n_items = total_tiles * a.Hkv * n_hg;
  // an 8-bit pool reads back as value(code) * k_scale: the factor joins Q's scale
  const float c_scale = a.scale * kLog2e * (KV8 ? a.k_scale : 1.f);
  const uint32_t NB = static_cast<uint32_t>(min(a.NB, int64_t(0x7fffffff)));
  static_assert(!KV8 || D == 128, "8-bit pools take this kernel at head size 128");

  // Per-lane fragment addresses in stage 0 (K: slice 0; V: rows of slice 0).
  // The swizzle term depends only on the row modulo 16, which no slice or
  // stage offset changes, so these hold everywhere; the empty asm keeps each
  // in a register so that stage and slice offsets fold into the reads'
  // immediate offsets.
  uint32_t k_rd[QS];
#pragma unroll
  for (int st = 0; st < QS; ++st) {
    k_rd[st] = 16u * Tl::chunk(col, 2 * st + hh);
    asm volatile("" : "+v"(k_rd[st]));
  }
  uint32_t v_rd[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      // lane j16 of 16-lane group g16 points at V[row][d .. d + 3]; the
      // transposing read hands it V[row0 + e][32 dt + 16 (g16 & 1) + j16], e = 0..3
      const int row = 4 * hh + (j16 >> 2) + 8 * w;
      const int d = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3);
      v_rd[dt][w] = V0 + 16u * Tl::chunk(row, d >> 3) + 2u * (d & 7);
      asm volatile("" : "+v"(v_rd[dt][w]));
    }
  // Tile loads: load i of this wave fills LDS chunks [64 (wave + 8 i), +64)
  // of a K (or V) tile; lane l fills chunk slot p = (64 (wave + 8 i) + l) mod
  // CPR of row r, i.e. it fetches the row's logical chunk p ^ swz(r). The
  // rows of one load lie in one 16-token block (blk_of), so the block and
  // its address are wave-uniform; only the in-block offset is per lane.
  uint32_t dk[DPW], dv[DPW];
  auto row_of = [&](int i) { return 64 * (wave + kPWaves * i) / CPR + lane / CPR; };  // tile row of lane's chunk
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int r = row_of(i), c = (lane % CPR) ^ Tl::swz(r);
    dk[i] = static_cast<uint32_t>((r % kBlockTokens) * a.kc_sr + 16 * c);
    dv[i] = static_cast<uint32_t>((r % kBlockTokens) * a.vc_sr + 16 * c);
  }
  auto blk_of = [&](int i) { return (64 * (wave + kPWaves * i) / CPR) / kBlockTokens; };
  // 8-bit pool: lane (wave, lane) fetches the 16 codes 16 c8 .. +15 of tile
  // row r8 (8 lanes per 128-code row; a wave's 8 rows lie in block wave / 2 of
  // the tile) and writes them widened to bf16 as chunks 2 c8, 2 c8 + 1 of that
  // row, the layout the fragment reads expect.
  const int r8 = (64 * wave + lane) / 8, c8 = lane % 8;
  const uint32_t dk8 = static_cast<uint32_t>((r8 % kBlockTokens) * a.kc_sr + 16 * c8);
  const uint32_t dv8 = static_cast<uint32_t>((r8 % kBlockTokens) * a.vc_sr + 16 * c8);
  const uint32_t wk8 = 16u * Tl::chunk(r8, 2 * c8), wk8b = 16u * Tl::chunk(r8, 2 * c8 + 1);

  // Two schedules, chosen by the plan kernel.
  //  - Queue (the usual case): longest-first greedy assignment of whole items
  //    (below).
  //  - Cuts, when the longest item outlasts an equal share of the work (a few
  //    long items, as in a long-context prefill): workgroup w of class x owns
  //    the cost range [w cap, (w + 1) cap) of the class's items in rank order,
  //    the items inside it whole and, of an item that a range boundary cuts,
  //    the key tiles on its side of the cut (McNaughton's wrap-around rule). A
  //    cut never lies past the position of the tile's first token, so both
  //    pieces of an item see a key for every token: the first piece only keys
  //    every token sees, the last piece the causal diagonal. Each piece of a
  //    cut item writes its partial result (running maximum, weight sum and
  //    unnormalised output per token and head) to the rows of its tokens in
  //    the split-K workspace, at its piece index; the piece that counts in
  //    last combines them in piece order, so the result does not depend on
  //    which finishes first.
  static_assert(KT == kPrefillKeyTile, "the plan's cost model counts 64-key tiles");
  // No prefill items (the launch only combined the decode's partitions): the
  // schedule may not have been written, so nothing of it is read.
  if (n_items <= 0) return;
  const int b = static_cast<int>(blockIdx.x);
  const int64_t items_per_rank = a.Hkv * n_hg;
  // Pieces per item: at most the workspace's partial slots per row, and none
  // (no cut) when the 32-bit offsets of the partial stores could overflow.
  const int max_pieces = 32 * a.Hq * a.max_parts * D * 4 < (int64_t(1) << 31) ? static_cast<int>(a.max_parts) : 1;
  // Queue: workgroup b starts on item b (items are ranked longest first, so
  // this is the first round of a longest-first assignment), later items come
  // from the queue. The next item is claimed while the current one's last
  // key tile is in flight (thread 0 issues the atomic and keeps the result),
  // so the claim's round trip overlaps compute. Item b of the first round
  // reads KV head b mod Hkv, and workgroup b runs on XCD b mod 8: the ranked
  // token tiles of a chunk that read the same K/V start on one L2.
  //
  // The schedule's state lives in LDS, read where it is needed, so that none
  // of it occupies scalar registers through the key loop: [0] merge count,
  // [1] the loop's next index, [3..4] capacity, [5] pieces of the
  // current item, [6] its piece index, [7] its merge counter.
  lds_int* const st = reinterpret_cast<lds_int*>(dma + 2 * V0 + kPWaves * 256u);
  const lds_int* const st_rd = reinterpret_cast<const lds_int*>(rd + 2 * V0 + kPWaves * 256u);
  if (tid == 0) {
    st[1] = CUTS ? a.sched[b] : b;  // class-local index of the schedule (cuts), or item index (queue)
    if constexpr (CUTS) {  // the plan's capacity per workgroup
      st[3] = a.work_counter[2];
      st[4] = a.work_counter[3];
    }
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  for (;;) {
    const int64_t ci = __builtin_amdgcn_readfirstlane(st_rd[1]);
    constexpr bool cuts = CUTS;
    const int64_t cap = cuts ? max(int64_t(1), (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(st_rd[4])) << 32) |
                                                   static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(st_rd[3])))
                             : int64_t(1);
    // This workgroup's class x (the KV heads g = x mod nclass) and its place
    // w among the class's workgroups; with cuts, items are counted within
    // the class.
    const int nclass = schedule_classes(a.Hkv, nwg);
    const int cx = b % nclass, w = b / nclass;
    const int64_t heads_per_class = a.Hkv / nclass;
    const int64_t per_class = items_per_rank / nclass;
    if (cuts ? ci >= total_tiles * per_class : ci >= n_items) break;
    const int64_t range_lo = int64_t(w) * cap, range_hi = range_lo + cap;
    int64_t item = ci, k_in_rank = 0;
    if (cuts) {  // class-local index -> item (rank, head group, KV head g = cx + nclass m)
      const int64_t rank = ci / per_class;
      k_in_rank = ci - rank * per_class;
      const int64_t hg_c = k_in_rank / heads_per_class, m = k_in_rank - hg_c * heads_per_class;
      item = rank * items_per_rank + hg_c * a.Hkv + cx + nclass * m;
    }
    const TileRef tr = locate(a, item, n_hg, total_tiles);
    // Positions fit in 32 bits: keys are bounded by MB * 16 (checked on the host).
    const int64_t s = tr.s, g = tr.g;
    const int lt = static_cast<int>(tr.lt), hg = static_cast<int>(tr.hg);
    const int64_t q0 = tr.q0;
    const int n = static_cast<int>(tr.n);
    const int Lc = static_cast<int>(tr.Lc);
    const int C_item = static_cast<int>(tr.C);
    const int blk_last = min(n, (lt + 1) * QTB) - 1;                 // last token of the tile
    const int kend_item = min(C_item + blk_last + 1, Lc);             // keys [0, kend_item) needed by the tile
    const int nkt_item = (kend_item + KT - 1) / KT;
    // This workgroup's piece of the item: key tiles [t_lo, t_hi), piece
    // pidx of npieces.
    int t_lo = 0, t_hi = nkt_item, pidx = 0, npieces = 1;
    int64_t merge_slot = 0;  // first range boundary inside the item: its merge counter
    int claimed = 0;  // queue: thread 0's claim of the next item
    auto claim = [&] {
      if (!cuts && tid == 0) claimed = atomicAdd(a.work_counter, 1);
    };
    if (cuts) {
      const int64_t cost = item_cost_q(nkt_item);
      const int64_t p_item = tr.P / nclass + k_in_rank * cost;
      if (p_item >= range_hi) break;
      if (p_item < range_lo || p_item + cost > range_hi) {
        // The cut at range boundary x: the key tiles whose cost lies before x,
        // at most up to the tile's first token position (and short of the
        // last tile); 0 is no cut. Cuts grow with x; at most max_pieces - 1
        // distinct ones are kept (one partial slot per piece), a boundary
        // past them cuts nothing.
        const int smax = max(0, min(nkt_item - 1, (C_item + lt * QTB) / KT));
        auto cut_at = [&](int64_t x) {
          return static_cast<int>(min(max((x - p_item - kItemFixedQ) >> 2, int64_t(0)), int64_t(smax)));
        };
        const int64_t j0 = p_item / cap + 1, j1 = (p_item + cost - 1) / cap;  // boundaries inside the item
        merge_slot = j0 * nclass + cx;  // the workgroup whose share starts at the first of them
        int prev = 0, ncut = 0;
        for (int64_t j = j0; j <= j1; ++j) {
          int c = cut_at(j * cap);
          if (c > prev) {
            if (ncut + 1 < max_pieces) {
              ++ncut;
              prev = c;
            } else {
              c = nkt_item;  // dropped
            }
          }
          if (j == w) {
            t_lo = c;
            pidx = ncut;
          }
          if (j == w + 1) t_hi = c;
          if (c == nkt_item) {
            if (j <= w) t_lo = nkt_item;
            break;
          }
        }
        npieces = ncut + 1;
      }
    }
    if (cuts && t_lo >= t_hi) {  // this workgroup has no piece of the item
      asm volatile("s_barrier" ::: "memory");  // every wave has read the index
      if (tid == 0) st[1] = static_cast<int>(ci + 1);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      continue;
    }
    if (CUTS && tid == 0) {
      st[5] = npieces;
      st[6] = pidx;
      st[7] = static_cast<int>(merge_slot);
    }
    // The piece as an item of its own: keys shifted down by k0, the block
    // table advanced by the tiles before it.
    const int k0 = KT * t_lo;
    const int C = C_item - k0;
    const int kend = (t_hi == nkt_item ? kend_item : KT * t_hi) - k0;  // keys [0, kend) of the piece
    const int nkt = t_hi - t_lo;
    const int64_t h = g * G + hg * HW + hw;
    const int i0 = lt * QTB + tw * kWaveTokens;  // first token of this wave
    const bool wave_active = i0 < n;
    const int wave_first = C + min(i0, n - 1);  // smallest position among the wave's lanes
    const int my_i = min(i0 + col, n - 1);      // clamped token of this lane
    const int my_pos = C + my_i;                // last key this lane sees

    const int32_t* bt = bt_all + s * a.bt_row + (KT / kBlockTokens) * t_lo;
    const char* kc = a.kc + g * a.kc_sh;
    const char* vc = a.vc + g * a.vc_sh;
    const int last_blk = (kend - 1) / kBlockTokens;
    // bytes of one block's head slice, from its first row
    constexpr int CES = KV8 ? 1 : 2;  // cache element bytes
    const uint32_t k_rec = static_cast<uint32_t>((kBlockTokens - 1) * a.kc_sr + a.D * CES);
    const uint32_t v_rec = static_cast<uint32_t>((kBlockTokens - 1) * a.vc_sr + a.D * CES);
    int32_t ids[DPW];  // block ids of the next tile to load (scalar)
    auto load_ids = [&](int t) {
#pragma unroll
      for (int i = 0; i < DPW; ++i) ids[i] = bt[min(t * (KT / kBlockTokens) + blk_of(i), last_blk)];
    };
    // Tiles 0 and 1 (blocks 0 .. 7) take their ids from the item's plan
    // record when it has one (read together with the item, picked by register
    // selects), not from the table: no round trip before the first loads.
    const bool rec_ids = tr.ranked && t_lo == 0;  // the plan record holds the piece's first block ids
    auto first_ids = [&](int t) {
      if (!rec_ids) return load_ids(t);
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int j = min(t * (KT / kBlockTokens) + blk_of(i), last_blk);
        const int4 q = j < 4 ? tr.ids_lo : tr.ids_hi;
        const int jj = j & 3;
        ids[i] = jj == 0 ? q.x : jj == 1 ? q.y : jj == 2 ? q.z : q.w;
      }
    };
    // 8-bit pool: the codes of two tiles in flight in registers (slot t % 2),
    // and the block id of the next tile to load (scalar).
    uint4 rk8[2], rv8[2];
    int32_t id8 = 0;
    auto load_id8 = [&](int t) { id8 = bt[min(t * (KT / kBlockTokens) + wave / 2, last_blk)]; };
    auto first_id8 = [&](int t) {
      if (!rec_ids) return load_id8(t);
      const int j = min(t * (KT / kBlockTokens) + wave / 2, last_blk);
      const int4 q = j < 4 ? tr.ids_lo : tr.ids_hi;
      const int jj = j & 3;
      id8 = jj == 0 ? q.x : jj == 1 ? q.y : jj == 2 ? q.z : q.w;
    };
    auto load_regs8 = [&](int t, int slot) {
      const uint32_t u = static_cast<uint32_t>(id8);
      const int64_t pid = u < NB ? int64_t(u) : 0;
      uint32_t ok = dk8, ov = dv8;
      if (t == nkt - 1 && t * KT + r8 >= kend) ok = ov = 0x80000000u;  // past the keys: zeros
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kc + pid * a.kc_sb), 0, static_cast<int>(k_rec), kBufferFlags);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vc + pid * a.vc_sb), 0, static_cast<int>(v_rec), kBufferFlags);
      rk8[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, ok, 0, 0));
      rv8[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, ov, 0, 0));
    };
    // Codes 2 SEL, 2 SEL + 1 of w as bf16 (exact).
    auto widen2 = [](uint32_t w, auto sel_c) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, decltype(sel_c)::value));
    };
    auto write_regs8 = [&](int slot, uint32_t stage_off) {
      using f = std::false_type;
      using t = std::true_type;
      const uint4 k = rk8[slot], v = rv8[slot];
      *reinterpret_cast<lds_u32x4*>(dma + stage_off + wk8) =
          u32x4{widen2(k.x, f{}), widen2(k.x, t{}), widen2(k.y, f{}), widen2(k.y, t{})};
      *reinterpret_cast<lds_u32x4*>(dma + stage_off + wk8b) =
          u32x4{widen2(k.z, f{}), widen2(k.z, t{}), widen2(k.w, f{}), widen2(k.w, t{})};
      *reinterpret_cast<lds_u32x4*>(dma + V0 + stage_off + wk8) =
          u32x4{widen2(v.x, f{}), widen2(v.x, t{}), widen2(v.y, f{}), widen2(v.y, t{})};
      *reinterpret_cast<lds_u32x4*>(dma + V0 + stage_off + wk8b) =
          u32x4{widen2(v.z, f{}), widen2(v.z, t{}), widen2(v.w, f{}), widen2(v.w, t{})};
    };
    // Rows at or past kend (only in the last tile) read past the resource and
    // land as zeros; their block index is clamped to a block the tile needs.
    auto load_tile = [&](int t, uint32_t stage_off) {
      const bool last = t == nkt - 1;
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const uint32_t u = static_cast<uint32_t>(ids[i]);
        const int64_t pid = u < NB ? int64_t(u) : 0;
        uint32_t ok = dk[i], ov = dv[i];
        if (last && t * KT + row_of(i) >= kend) ok = ov = 0x80000000u;
        lds_char* dst = dma + stage_off + 1024u * (wave + kPWaves * i);
        load_lds16(kc + pid * a.kc_sb, k_rec, ok, dst);
        load_lds16(vc + pid * a.vc_sb, v_rec, ov, dst + V0);
      }
    };

    bf16x8 qf[QS];  // Q^T (B operand): token col, d = 16 st + 8 hh .. +8
    // Q comes in through LDS: loaded as whole rows (16 lanes per 256-byte
    // row at D = 128), where loading the B operand directly would fetch 16
    // bytes of each of 32 rows per instruction. Each wave stages its own 32
    // rows in a half stage of K or V stages 2 and 3, which no tile uses before
    // the item's first barrier; row r's 16-byte chunk c sits at chunk slot
    // c ^ (r mod QCH), so that the fragment reads (32 rows at one chunk) are
    // one pass per 256 bytes. Rows past the item's tokens repeat its last.
    constexpr int QCH = D / 8;     // 16-byte chunks per Q row
    constexpr int QRI = 64 / QCH;  // rows per 1 KiB load
    const uint32_t qst = static_cast<uint32_t>((wave >> 1) < 2 ? (2 + (wave >> 1)) * TB : V0 + (wave >> 1) * TB) +
                         (wave & 1) * HALF;
    // (the lane index passes through an empty asm in both, so that their
    // per-lane offsets are computed here, not kept across the item loop)
    auto load_q = [&] {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int w0 = min(i0, n - 1);  // the wave's first (clamped) token
      const char* qb = a.q + (q0 + w0) * a.q_st + h * a.q_sh;
      const uint32_t qrec = static_cast<uint32_t>((n - 1 - w0) * a.q_st + 2 * D);
#pragma unroll
      for (int i = 0; i < 32 / QRI; ++i) {
        const int r = i * QRI + ln / QCH;
        const int tok = min(i0 + r, n - 1);
        const int c = (ln % QCH) ^ (r % QCH);
        load_lds16(qb, qrec, static_cast<uint32_t>((tok - w0) * a.q_st + 16 * c), dma + qst + 1024u * i);
      }
    };
    auto read_q = [&] {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int qc = ln & 31, qh = ln >> 5;
#pragma unroll
      for (int st = 0; st < QS; ++st)
        qf[st] = *reinterpret_cast<const lds_bf16x8*>(rd + qst + 16u * (qc * QCH + ((2 * st + qh) ^ (qc % QCH))));
    };
    // Pre-scaled by scale * log2(e) once the loads have landed (after the
    // first tiles' loads are out), so the scores come out in log2 units.
    // Rounding the scaled Q to bf16 perturbs each product term by at most
    // 2^-9 relative, far below the bf16 rounding of the weights.
    auto scale_q = [&] {
#pragma unroll
      for (int st = 0; st < QS; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[st][e] = static_cast<__bf16>(static_cast<float>(qf[st][e]) * c_scale);
    };
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float l_run = 0.f;
    // Scores are kept relative to the running maximum m in log2 units: every
    // score chain after the first starts from negm = -m (all 16 entries)
    // instead of zero, so the weights are plain exp2 of the chain's result.
    f32x16 negm;

    // Software pipeline over 32-key slices j: step j runs the softmax of
    // slice j, the score chain of slice j + 1 and P.V of slice j - 1, so the
    // matrix core has independent work while the vector ALU computes weights.
    f32x16 s_cur;     // S^T[key 32 j + 8 q + 4 hh + r][token col] in s_cur[4 q + r]
    bf16x8 p_prev[2];  // weights of slice j - 1, the two B operands of its P.V
    auto read_k = [&](uint32_t ko, int st) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<lds_u4*>(rd + k_rd[st] + ko));
    };
    auto read_v = [&](uint32_t vo, int q2, int dt) {
      // rows 16 q2 + [4 hh, 4 hh + 4) and the same + 8 of the slice at vo
      const uint32_t off = vo + 16u * q2 * CPR * 16;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<lds_i16x4*>(const_cast<lds_char*>(rd + v_rd[dt][0] + off)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<lds_i16x4*>(const_cast<lds_char*>(rd + v_rd[dt][1] + off)));
      const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
      return __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
    };
    // Weights of a slice; four partial sums keep the adds from forming one
    // serial chain.
    auto weights = [&](const float (&sc)[16], float (&w)[16]) {
      float part[4];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        w[i] = fast_exp2(sc[i]);
        part[i & 3] = i < 4 ? w[i] : part[i & 3] + w[i];
      }
      return (part[0] + part[1]) + (part[2] + part[3]);
    };
    // key slots of lane half hh in P^T: e < 4 -> 16 q2 + 4 hh + e,
    // e >= 4 -> 16 q2 + 8 + 4 hh + (e - 4), i.e. w[8 q2 + e]
    auto pack = [&](const float (&w)[16], bf16x8 (&p)[2]) {
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int e = 0; e < 8; ++e) p[q2][e] = static_cast<__bf16>(w[8 * q2 + e]);
    };
    // The reference m stands while no weight of the slice exceeds 2^8
    // (checked through the lane's sum, which also catches inf and NaN).
    // Otherwise the slice's maximum is taken across the two lane halves of
    // each token; where it is above m, m moves up to it: the accumulators
    // (which already hold P.V of the previous slice) and l are rescaled, and
    // the slice's scores, negm and sn (the next slice's chain, started from
    // the old m) are shifted. Then the weights are recomputed.
    auto settle = [&](float (&sc)[16], float (&w)[16], float& lsum, bf16x8 (&p)[2], f32x16* sn) {
      if (__any(!(lsum <= kRescaleBound))) {
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[i]);
        const float delta = fmaxf(fmaxf(tmax, __shfl_xor(tmax, 32)), 0.f);
        if (delta > 0.f) {
          const float alpha = fast_exp2(-delta);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            negm[i] -= delta;
            sc[i] -= delta;
          }
          if (sn != nullptr) *sn -= delta;
        }
        lsum = weights(sc, w);
        pack(w, p);
      }
      l_run += lsum;
    };

    // Keys above the lane's own position (including every key at or past
    // kend, which lies above every position) get -inf in s_cur.
    auto mask_cur = [&](int j) {
      const int t = my_pos - 32 * j - 4 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i) s_cur[i] = 8 * (i >> 2) + (i & 3) <= t ? s_cur[i] : -INFINITY;
    };
    // Step j: softmax of slice j with P.V of slice j - 1 and (QK) the score
    // chain of slice j + 1. Every wave runs every slice of the tile's keys;
    // keys a lane must not see are masked, so slices past a wave's last
    // token cost work but change nothing (their weights are zero and their V
    // rows finite: real keys, or zeros past kend).
    //
    // Scheduled by hand: the MFMAs go out one at a time, each followed by a
    // share of the softmax's vector work (weights, their sum, the bf16
    // packing), and fragment reads run ahead of their MFMAs. Scheduling
    // fences hold that order; left alone, the compiler bunches the vector
    // work ahead of the first MFMA.
    auto step = [&](auto qk_c, int j, uint32_t ko, uint32_t vo) {
      constexpr bool QK = decltype(qk_c)::value;
      if (32 * j + 31 > wave_first) mask_cur(j);
      constexpr int M = 2 * DT + QS;  // MFMA slots (the score chain's only with QK)
      // Vector work items. Item k < 18 runs two independent operations: exp2
      // of element k and the partial sum of element k - 2. Then the total
      // (item 18) and the eight bf16 pairs (19 .. 26).
      constexpr int NW = 18 + 1 + 8;
      float sc[16], w[16], part[4], lsum = 0.f;
      bf16x8 p[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = s_cur[i];
      auto work = [&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        if constexpr (k < 18) {
          if constexpr (k < 16) w[k] = fast_exp2(sc[k]);
          if constexpr (k >= 2 && k < 6) part[k - 2] = w[k - 2];
          if constexpr (k >= 6) part[(k - 2) & 3] += w[k - 2];
        } else if constexpr (k == 18) {
          lsum = (part[0] + part[1]) + (part[2] + part[3]);
        } else {
          constexpr int e = k - 19;  // weights 2e, 2e + 1 -> P^T slots of p[e / 4]
          p[e / 4][2 * (e % 4)] = static_cast<__bf16>(w[2 * e]);
          p[e / 4][2 * (e % 4) + 1] = static_cast<__bf16>(w[2 * e + 1]);
        }
      };
      auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
      // MFMA m of the step: even m is k-step m / 2 of the score chain, odd m
      // is P.V tile i = (m - 1) / 2 (16-key group i / DT, rows 32 (i % DT)).
      // The chain's dependent MFMAs thus alternate with independent ones,
      // which keeps the matrix core busy from this wave alone (a dependent
      // MFMA waits for its predecessor's result, longer than the issue
      // interval). Each fragment is read L MFMAs ahead of its use.
      constexpr int L = 5;
      static_assert(QS == 2 * DT, "score and P.V MFMAs alternate one for one");
      bf16x8 fr[M];
      auto issue_read = [&](auto m_c) {
        constexpr int m = decltype(m_c)::value;
        if constexpr (m % 2 == 0) {
          if constexpr (QK) fr[m] = read_k(ko, m / 2);
        } else {
          constexpr int i = (m - 1) / 2;
          fr[m] = read_v(vo, i / DT, i % DT);
        }
      };
      static_for<0, L>(issue_read);
      fence();
      static_for<0, 4>(work);  // while the reads land
      fence();
      f32x16 sn;
      static_for<0, M>([&](auto m_c) {
        constexpr int m = decltype(m_c)::value;
        if constexpr (m % 2 == 0) {
          constexpr int st = m / 2;
          if constexpr (QK) sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m], qf[st], st == 0 ? negm : sn, 0, 0, 0);
        } else {
          constexpr int i = (m - 1) / 2, q2 = i / DT, dt = i % DT;
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m], p_prev[q2], o[dt], 0, 0, 0);
        }
        if constexpr (m + L < M) issue_read(std::integral_constant<int, m + L>{});
        // this MFMA's share of the remaining work items 4 .. NW - 1
        static_for<4 + (NW - 4) * m / M, 4 + (NW - 4) * (m + 1) / M>(work);
        fence();
      });
      settle(sc, w, lsum, p, QK ? &sn : nullptr);
      p_prev[0] = p[0];
      p_prev[1] = p[1];
      if constexpr (QK) s_cur = sn;
    };
    // The score chain of slice 0 from zero; then the first softmax, which
    // sets m to the slice's maximum (finite: every lane sees key 0), and the
    // chain of slice 1 from -m.
    auto first_steps = [&](uint32_t ko) {
      bf16x8 kf[QS];
#pragma unroll
      for (int st = 0; st < QS; ++st) kf[st] = read_k(ko, st);
#pragma unroll
      for (int i = 0; i < 16; ++i) s_cur[i] = 0.f;
#pragma unroll
      for (int st = 0; st < QS; ++st) s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s_cur, 0, 0, 0);
      if (31 > wave_first) mask_cur(0);
      float sc[16], w[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] = s_cur[i];
        tmax = fmaxf(tmax, sc[i]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        negm[i] = -tmax;
        sc[i] -= tmax;
      }
      l_run = weights(sc, w);
      pack(w, p_prev);
#pragma unroll
      for (int st = 0; st < QS; ++st) kf[st] = read_k(ko + HALF, st);
      s_cur = negm;
#pragma unroll
      for (int st = 0; st < QS; ++st) s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s_cur, 0, 0, 0);
    };
    // P.V of the last slice alone.
    auto pv_only = [&](uint32_t vo) {
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        bf16x8 va[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) va[dt] = read_v(vo, q2, dt);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], p_prev[q2], o[dt], 0, 0, 0);
      }
    };
    using yes = std::true_type;
    using no = std::false_type;

    if (nkt > 0) {
      // Prologue: Q, then tiles 0 and 1 in flight; wait for Q and tile 0,
      // read this wave's Q fragments before the barrier (tile 2 may go into
      // their stage after it). An 8-bit pool's tile goes through registers:
      // its codes are widened into the stage just before the barrier that
      // publishes it.
      load_q();
      if constexpr (KV8) {
        first_id8(0);
        load_regs8(0, 0);
        if (nkt > 1) {
          first_id8(1);
          load_regs8(1, 1);
          wait_vmem<2>();
        } else {
          wait_vmem<0>();
        }
        read_q();
        write_regs8(0, 0);
      } else {
        first_ids(0);
        load_tile(0, 0);
        if (nkt > 1) {
          first_ids(1);
          load_tile(1, TB);
          wait_vmem<2 * DPW>();
        } else {
          wait_vmem<0>();
        }
        read_q();
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      raw_barrier();
      // Claim point for short items: after the last tile's loads went out.
      if (nkt <= 2) claim();
      if (nkt > 2) {
        if constexpr (KV8) {
          load_id8(2);
          load_regs8(2, 0);
        } else {
          load_ids(2);
          load_tile(2, 2 * TB);
        }
      }
      if (nkt > 3) {
        if constexpr (KV8) load_id8(3);
        else load_ids(3);
      }
      scale_q();
      first_steps(0);                       // scores of slices 0 and 1, softmax 0
      // Tile u: wait for it (tile u + 1 may stay in flight), start loading
      // tile u + 2 into the stage that held tile u - 2 (last read by the P.V
      // steps of tile u - 1, which every wave has finished at the barrier),
      // then steps 2u - 1 and 2u: scores from tile u, P.V from tile u - 1.
      auto tile_body = [&](auto stage_c, int u) {
        constexpr int S = decltype(stage_c)::value;
        constexpr uint32_t kst = S * TB, vst = ((S + 3) % 4) * TB, nst = ((S + 2) % 4) * TB;
        // Wave 0's claim (issued after the last tile's loads) may stay in
        // flight through the last tile.
        if (u + 1 < nkt)
          wait_vmem<KV8 ? 2 : 2 * DPW>();
        else if (wave == 0 && !cuts)
          wait_vmem<1>();
        else
          wait_vmem<0>();
        if constexpr (KV8) {  // tile u's codes (slot u % 2) into its stage, published by the barrier
          write_regs8(S % 2, kst);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        raw_barrier();
        if (u + 2 < nkt) {
          if constexpr (KV8) load_regs8(u + 2, S % 2);
          else load_tile(u + 2, nst);
        }
        if (u + 2 == nkt) claim();
        step(yes{}, 2 * u - 1, kst, vst);
        step(yes{}, 2 * u, kst + HALF, vst + HALF);
        if (u + 3 < nkt) {
          if constexpr (KV8) load_id8(u + 3);
          else load_ids(u + 3);
        }
      };
      static_assert(Tl::STAGES == 4, "the tile loop is unrolled over four stages");
      for (int u0 = 0; u0 < nkt; u0 += 4) {
        if (u0 > 0) tile_body(std::integral_constant<int, 0>{}, u0);
        if (u0 + 1 < nkt) tile_body(std::integral_constant<int, 1>{}, u0 + 1);
        if (u0 + 2 < nkt) tile_body(std::integral_constant<int, 2>{}, u0 + 2);
        if (u0 + 3 < nkt) tile_body(std::integral_constant<int, 3>{}, u0 + 3);
      }
      // Epilogue: the last two P.V steps read V of the last tile.
      const uint32_t vst = static_cast<uint32_t>((nkt - 1) % 4) * TB;
      step(no{}, 2 * nkt - 1, 0, vst);
      pv_only(vst + HALF);
    }

    if (nkt <= 0) claim();
    // The claimed item goes to LDS before this item's output stores, so that
    // waiting for the claim does not also wait for them (queue items follow
    // the first round).
    if (tid == 0) st[1] = cuts ? st[1] + 1 : nwg + claimed;
    // A cut item: this piece's partial result goes to the workspace, and the
    // piece that counts in last combines every piece's.
    // (the piece's index and count and its item's counter, from LDS)
    const int cut_n = CUTS ? __builtin_amdgcn_readfirstlane(st_rd[5]) : 1;
    if (cut_n > 1) {
      const int cut_i = __builtin_amdgcn_readfirstlane(st_rd[6]);
      const int64_t cut_slot = __builtin_amdgcn_readfirstlane(st_rd[7]);
      const int64_t row_bytes = a.Hq * a.max_parts * D * 4;  // workspace stride between tokens
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave is done with the stages
      // The wave's unnormalised 32 x D output, fp32, as rows in LDS (one
      // stage-sized region per wave): lane (col, hh) holds 16-byte chunk
      // 8 dt + 2 q + hh of row col, at chunk position c ^ (row mod FCH); the
      // row's running maximum and weight sum go to a small area after the
      // stages.
      constexpr int FCH = D / 4;       // 16-byte chunks per fp32 row
      constexpr int RPR = 64 / FCH;    // rows per 16-byte-per-lane access
      const uint32_t prow = static_cast<uint32_t>(wave) * TB;
      const uint32_t pml = 2 * V0 + static_cast<uint32_t>(wave) * 256u;
      {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int pc = ln & 31, ph = ln >> 5;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = 8 * dt + 2 * q + ph;
            *reinterpret_cast<lds_u32x4*>(dma + prow + 16u * (pc * FCH + (c ^ (pc % FCH)))) =
                u32x4{__float_as_uint(o[dt][4 * q]), __float_as_uint(o[dt][4 * q + 1]),
                      __float_as_uint(o[dt][4 * q + 2]), __float_as_uint(o[dt][4 * q + 3])};
          }
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        if (ph == 0) *reinterpret_cast<lds_u32x2*>(dma + pml + 8u * pc) = u32x2{__float_as_uint(-negm[0]), __float_as_uint(l_tot)};
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // Rows to the workspace at this piece's index (cache-coherent stores:
      // the combining workgroup may run on another XCD).
      // The wave's rows: token q0 + i0 + r, head h; offsets from its first
      // row fit 32 bits (max_pieces is 1 otherwise).
      const int64_t row0 = (q0 + i0) * a.Hq + h;
      const uint32_t ml_stride = static_cast<uint32_t>(a.Hq * a.max_parts * 8);  // between tokens
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<char*>(a.ws_o + row0 * a.max_parts * D), 0, 0x7fffffff, kBufferFlags);
      const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<char*>(a.ws_ml + row0 * a.max_parts), 0, 0x7fffffff, kBufferFlags);
      if (wave_active) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int c = ln % FCH;
#pragma unroll
        for (int i = 0; i < 32 / RPR; ++i) {
          const int r = i * RPR + ln / FCH;
          const u32x4 v = *reinterpret_cast<const lds_u32x4*>(rd + prow + 16u * (r * FCH + (c ^ (r % FCH))));
          if (i0 + r < n)
            __builtin_amdgcn_raw_buffer_store_b128(
                v, ors, static_cast<uint32_t>(r * row_bytes + (cut_i * D + 4 * c) * 4), 0, kCoherent);
        }
        if (ln < 32 && i0 + ln < n) {
          const u32x2 v = *reinterpret_cast<const lds_u32x2*>(rd + pml + 8u * ln);
          __builtin_amdgcn_raw_buffer_store_b64(v, mrs, static_cast<uint32_t>(ln) * ml_stride + 8u * cut_i, 0, kCoherent);
        }
      }
      // Count this piece in once every wave's stores have completed.
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (tid == 0)
        st[0] = __hip_atomic_fetch_add(a.sched + kMaxPrefillWorkgroups + cut_slot, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const bool merge = __builtin_amdgcn_readfirstlane(st_rd[0]) == cut_n - 1;
      if (merge && wave_active) {
        // Combine the pieces in piece order (online: rescale the running sum
        // to each new maximum), this one's rows from LDS, the others' from the
        // workspace with coherent loads, issued for four passes over the
        // wave's rows at a time.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int c = ln % FCH;
        const float vs = KV8 ? a.v_scale : 1.f;
        constexpr int NP = 4;  // passes per group
        static_assert((32 / RPR) % NP == 0, "whole groups of passes");
#pragma unroll 1
        for (int half = 0; half < 32 / RPR / NP; ++half) {
          float M[NP], L[NP], acc[NP][4];
          uint32_t o_off[NP], m_off[NP];
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            // rows past the item's tokens read the wave's last row instead
            // (their results are not stored)
            const int rr = min((half * NP + i) * RPR + ln / FCH, n - 1 - i0);
            o_off[i] = static_cast<uint32_t>(rr * row_bytes + 16 * c);
            m_off[i] = static_cast<uint32_t>(rr) * ml_stride;
          }
#pragma unroll 1
          for (int p = 0; p < cut_n; ++p) {
            float mp[NP], lp[NP], op[NP][4];
            if (p == cut_i) {
#pragma unroll
              for (int i = 0; i < NP; ++i) {
                const int r = (half * NP + i) * RPR + ln / FCH;
                const u32x2 ml = *reinterpret_cast<const lds_u32x2*>(rd + pml + 8u * r);
                const u32x4 o4 = *reinterpret_cast<const lds_u32x4*>(rd + prow + 16u * (r * FCH + (c ^ (r % FCH))));
                mp[i] = __uint_as_float(ml.x);
                lp[i] = __uint_as_float(ml.y);
#pragma unroll
                for (int e = 0; e < 4; ++e) op[i][e] = __uint_as_float(o4[e]);
              }
            } else {
#pragma unroll
              for (int i = 0; i < NP; ++i) {
                const float2 ml = __builtin_bit_cast(
                    float2, __builtin_amdgcn_raw_buffer_load_b64(mrs, m_off[i] + 8u * p, 0, kCoherent));
                const u32x4 o4 =
                    __builtin_amdgcn_raw_buffer_load_b128(ors, o_off[i] + static_cast<uint32_t>(p * D * 4), 0, kCoherent);
                mp[i] = ml.x;
                lp[i] = ml.y;
#pragma unroll
                for (int e = 0; e < 4; ++e) op[i][e] = __uint_as_float(o4[e]);
              }
            }
#pragma unroll
            for (int i = 0; i < NP; ++i) {
              if (p == 0) {
                M[i] = mp[i];
                L[i] = lp[i];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][e] = op[i][e];
              } else {
                const float m_new = fmaxf(M[i], mp[i]);
                const float wa = fast_exp2(M[i] - m_new), wb = fast_exp2(mp[i] - m_new);
                M[i] = m_new;
                L[i] = L[i] * wa + lp[i] * wb;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][e] = acc[i][e] * wa + op[i][e] * wb;
              }
            }
          }
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            const int r = (half * NP + i) * RPR + ln / FCH;
            const float inv = vs / L[i];
            if (i0 + r < n)
              *reinterpret_cast<u32x2*>(a.out + (q0 + i0 + r) * a.out_st + h * a.out_sh + 8 * c) =
                  u32x2{pack_bf16(acc[i][0] * inv, acc[i][1] * inv), pack_bf16(acc[i][2] * inv, acc[i][3] * inv)};
          }
        }
      }
    }
    if (cut_n == 1 && wave_active) {
      // The wave's 32 x D output tile goes out as whole rows: the lanes hold
      // it transposed (lane (col, hh) has O^T[d = 32 dt + 8 q + 4 hh + r][token
      // col], 8-byte pieces of 32 different rows per store), so it passes
      // through LDS first. Row col's 16-byte chunk c = 4 dt + q sits at chunk
      // position c ^ (col mod OCH): the writes (32 rows at one chunk) and the
      // row reads (OCH lanes per row) are then one pass per 256 bytes.
      // Its place: a half stage no wave reads any more. Every wave is past
      // the last tile's barrier, so only the K stage of the last tile and
      // the V stages of the last two tiles may still be read; no load is in
      // flight. That leaves three K stages and two V stages, ten halves.
      constexpr int OCH = D / 8;     // 16-byte chunks per output row
      constexpr int RPI = 64 / OCH;  // rows per 16-byte-per-lane read
      const int ls = (nkt + 3) & 3;  // stage of the last tile
      const uint32_t ot = wave < 6 ? static_cast<uint32_t>(((ls + 1 + wave / 2) & 3) * TB + (wave & 1) * HALF)
                                   : static_cast<uint32_t>(V0 + ((ls + 1) & 3) * TB + (wave & 1) * HALF);
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const float inv = (KV8 ? a.v_scale : 1.f) / l_tot;
      // The lane index passes through an empty asm here, so that the
      // addresses below are computed here and not kept in registers across
      // the whole item loop.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int ocol = ln & 31, ohh = ln >> 5;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 4 * dt + q;
          *reinterpret_cast<lds_u32x2*>(dma + ot + 16u * (ocol * OCH + (c ^ (ocol % OCH))) + 8u * ohh) =
              u32x2{pack_bf16(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv),
                    pack_bf16(o[dt][4 * q + 2] * inv, o[dt][4 * q + 3] * inv)};
        }
      const int c = ln % OCH;
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int row = i * RPI + ln / OCH;
        const u32x4 val = *reinterpret_cast<const lds_u32x4*>(dma + ot + 16u * (row * OCH + (c ^ (row % OCH))));
        const int tok = i0 + row;
        if (tok < n) *reinterpret_cast<u32x4*>(a.out + (q0 + tok) * a.out_st + h * a.out_sh + 16 * c) = val;
      }
    }
    // The next item reuses the stages: every wave's LDS accesses must be
    // done, and the claimed item is in LDS (the barrier does not wait for
    // this item's output stores). Every wave reads the slot before its next
    // barrier, and the slot is next written after one.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// block_tables comes in again as a restrict pointer: nothing in the kernel
// writes it, so its wave-uniform entries are read with scalar loads. When the
// prefill runs beside the decode kernel (`beside`), only the first
// counter[1] workgroups (the plan kernel's share of the CUs) take items; the
// others exit at once and leave their CUs to the decode.
template <int D, int HW, bool KV8>
__global__ __launch_bounds__(kPThreads) void prefill_bf16_kernel(AttnArgs a, const int32_t* __restrict__ bt_all,
                                                                 int beside, int fold_reduce) {
  const int active = beside ? min(a.work_counter[1], static_cast<int>(gridDim.x)) : static_cast<int>(gridDim.x);
  if (static_cast<int>(blockIdx.x) >= active) return;
  // After the decode on the same stream, the waves first combine the decode's
  // split-K partitions (one (sequence, query head) per wave at a time).
  if (fold_reduce) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t it = int64_t(blockIdx.x) * kPWaves + wave; it < a.S * a.Hq; it += int64_t(gridDim.x) * kPWaves)
      reduce_partitions<true, D>(a, it, threadIdx.x & 63);
  }
  // No static LDS: the dynamic array starts at address 0, so fragment
  // addresses are a per-lane offset plus an immediate.
  extern __shared__ uint4 lds[];
  // The load view is offset by an opaque zero so that the two views are
  // distinct values (identical arguments would defeat the restrict hint).
  uint32_t zero = 0;
  asm volatile("" : "+s"(zero));
  // The plan's schedule: cuts when it wrote a capacity (ranked items only),
  // else the queue. Each is its own instance of the item loop, so that the
  // queue's key loop carries none of the cuts' state.
  const int64_t total_tiles = a.tile_start[a.S];
  const bool cut_mode = total_tiles > 0 && total_tiles <= kMaxSortedTiles &&
                        (a.work_counter[2] != 0 || a.work_counter[3] != 0);
  if (cut_mode)
    prefill_bf16_items<D, HW, KV8, true>(a, bt_all, (lds_char*)lds + zero, (const lds_char*)lds, active);
  else
    prefill_bf16_items<D, HW, KV8, false>(a, bt_all, (lds_char*)lds + zero, (const lds_char*)lds, active);
}

// ---------------------------------------------------------------- fp32 ----
// Also serves 8-bit pools (KV8): q and out are bf16 there, and each K/V
// element is widened from its E4M3 code (exact) while staging; k_scale
// joins the score scale and v_scale the output normalisation.
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D, int HW, bool KV8>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(AttnArgs a, int beside, int fold_reduce) {
  // beside the decode kernel only the plan kernel's share of workgroups take items
  if (beside && static_cast<int>(blockIdx.x) >= min(a.work_counter[1], static_cast<int>(gridDim.x))) return;
  // After the decode on the same stream: first the decode's partition reduce
  // (q and out are bf16 over an 8-bit pool, fp32 otherwise).
  if (fold_reduce) {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t it = int64_t(blockIdx.x) * kWaves + wv; it < a.S * a.Hq; it += int64_t(gridDim.x) * kWaves)
      reduce_partitions<KV8, D>(a, it, threadIdx.x & 63);
  }
  constexpr int KT = 32;        // keys per LDS stage
  constexpr int KROW = D + 4;   // floats per K tile row
  constexpr int VROW = KT + 4;  // floats per V^T tile row
  constexpr int QTB = tile_tokens(HW);
  constexpr int VPR = D / 4;    // 16-byte vectors per K/V row
  __shared__ __attribute__((aligned(16))) float ks[KT * KROW];
  __shared__ __attribute__((aligned(16))) float vt[D * VROW];
  __shared__ int item_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave % HW, tw = wave / HW;
  const int G = static_cast<int>(a.Hq / a.Hkv);
  const int n_hg = G / HW;
  const int64_t total_tiles = a.tile_start[a.S];
  const int64_t n_items = total_tiles * a.Hkv * n_hg;
  const float c_scale = a.scale * kLog2e * (KV8 ? a.k_scale : 1.f);
  const float o_scale = KV8 ? a.v_scale : 1.f;
  const uint32_t NB = static_cast<uint32_t>(min(a.NB, int64_t(0x7fffffff)));

  for (int64_t item = next_item(a, &item_sh); item < n_items; item = next_item(a, &item_sh)) {
    const TileRef tr = locate(a, item, n_hg, total_tiles);
    const int64_t s = tr.s, lt = tr.lt, g = tr.g, hg = tr.hg;
    const int64_t q0 = min(max(static_cast<int64_t>(a.qsl[s]), int64_t(0)), a.T);
    const int64_t n = min(max(static_cast<int64_t>(a.qsl[s + 1]), q0), a.T) - q0;
    const int64_t C = max(static_cast<int64_t>(a.ctx_lens[s]), int64_t(0));
    const int64_t Lc = min(max(static_cast<int64_t>(a.seq_lens[s]), int64_t(0)), a.MB * kBlockTokens);
    const int64_t h = g * G + hg * HW + hw;
    const int64_t i0 = lt * QTB + tw * kWaveTokens;
    const bool wave_active = i0 < n;
    const int64_t blk_last = min(n, (lt + 1) * QTB) - 1;
    const int64_t kend = min(C + blk_last + 1, Lc);
    const int64_t wave_kend = wave_active ? min(C + min(n, i0 + kWaveTokens), Lc) : 0;
    const int64_t my_i = min(i0 + col, n - 1);
    const int64_t my_pos = C + my_i;

    float qf[D / 2];  // Q^T: token col, d = 2 st + hh
    if constexpr (KV8) {
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q + (q0 + my_i) * a.q_st + h * a.q_sh);
#pragma unroll
      for (int st = 0; st < D / 2; ++st) qf[st] = __uint_as_float(static_cast<uint32_t>(qrow[2 * st + hh]) << 16);
    } else {
      const float* qrow = reinterpret_cast<const float*>(a.q + (q0 + my_i) * a.q_st + h * a.q_sh);
#pragma unroll
      for (int st = 0; st < D / 2; ++st) qf[st] = qrow[2 * st + hh];
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int32_t* bt = a.block_tables + s * a.bt_row;
    const char* kc = a.kc + g * a.kc_sh;
    const char* vc = a.vc + g * a.vc_sh;
    for (int64_t k0 = 0; k0 < kend; k0 += KT) {
      __syncthreads();  // previous tile fully consumed
      for (int v = tid; v < KT * VPR; v += kThreads) {
        const int key = v / VPR, c = v % VPR;
        const int64_t j = k0 + key;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (j < kend) {
          const uint32_t id32 = static_cast<uint32_t>(bt[j / kBlockTokens]);
          const int64_t pid = id32 < NB ? int64_t(id32) : 0;
          if constexpr (KV8) {  // 4 codes per vector
            const uint32_t kw = *reinterpret_cast<const uint32_t*>(kc + pid * a.kc_sb + (j % kBlockTokens) * a.kc_sr + 4 * c);
            const uint32_t vw = *reinterpret_cast<const uint32_t*>(vc + pid * a.vc_sb + (j % kBlockTokens) * a.vc_sr + 4 * c);
            const f32x2 k01 = __builtin_amdgcn_cvt_pk_f32_fp8(kw, false), k23 = __builtin_amdgcn_cvt_pk_f32_fp8(kw, true);
            const f32x2 v01 = __builtin_amdgcn_cvt_pk_f32_fp8(vw, false), v23 = __builtin_amdgcn_cvt_pk_f32_fp8(vw, true);
            kv = make_float4(k01.x, k01.y, k23.x, k23.y);
            vv = make_float4(v01.x, v01.y, v23.x, v23.y);
          } else {
            kv = *reinterpret_cast<const float4*>(kc + pid * a.kc_sb + (j % kBlockTokens) * a.kc_sr + 16 * c);
            vv = *reinterpret_cast<const float4*>(vc + pid * a.vc_sb + (j % kBlockTokens) * a.vc_sr + 16 * c);
          }
        }
        *reinterpret_cast<float4*>(ks + key * KROW + 4 * c) = kv;
        vt[(4 * c + 0) * VROW + key] = vv.x;
        vt[(4 * c + 1) * VROW + key] = vv.y;
        vt[(4 * c + 2) * VROW + key] = vv.z;
        vt[(4 * c + 3) * VROW + key] = vv.w;
      }
      __syncthreads();
      if (!wave_active || k0 >= wave_kend) continue;
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
      for (int st = 0; st < D / 2; ++st)
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[col * KROW + 2 * st + hh], qf[st], sacc, 0, 0, 0);
      float sc[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t key = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        sc[i] = (key <= my_pos && key < kend) ? sacc[i] : -INFINITY;
        tmax = fmaxf(tmax, sc[i]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * c_scale;
      if (__any(tmax > m_run + kRescaleThreshold)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sc[i], c_scale, -m_run));
        l_run += p;
        const int key = 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[(32 * dt + col) * VROW + key], p, o[dt], 0, 0, 0);
      }
    }

    if (wave_active) {
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const int64_t my_tok = i0 + col;
      if (my_tok < n) {
        const float inv = o_scale / l_tot;
        char* dst = a.out + (q0 + my_tok) * a.out_st + h * a.out_sh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d = 32 * dt + 8 * q + 4 * hh;
            const float4 r = make_float4(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv, o[dt][4 * q + 2] * inv,
                                         o[dt][4 * q + 3] * inv);
            if constexpr (KV8) {
              const bf16x2 lo = {static_cast<__bf16>(r.x), static_cast<__bf16>(r.y)};
              const bf16x2 hi = {static_cast<__bf16>(r.z), static_cast<__bf16>(r.w)};
              *reinterpret_cast<uint2*>(dst + 2 * d) =
                  make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
            } else {
              *reinterpret_cast<float4*>(dst + 4 * d) = r;
            }
          }
      }
    }
  }
}

// Prefill workgroups to launch: enough to fill every CU (bf16: one 8-wave
// workgroup per CU; fp32: four 4-wave), none when an upper bound on the items
// that needs no lengths (every prefill sequence has more than 16 / G tokens)
// is zero. The fp32 kernel launches at most that many; the bf16 kernel always
// fills the CUs, because its schedule may cut a few long items into pieces
// for all of them (with the queue, workgroups past the last item exit).
template <bool BF16, int D, int HW>
int64_t prefill_slots(const AttnArgs& a) {
  constexpr int QTB = BF16 ? bf16_tile_tokens(HW) : tile_tokens(HW);
  const int64_t G = a.Hq / a.Hkv;
  const int64_t tiles_ub = a.T / QTB + std::min<int64_t>(a.S, a.T / (kMaxDecodeColumns / G + 1));
  const int64_t items_ub = tiles_ub * a.Hkv * (G / HW);
  if (items_ub <= 0) return 0;
  return BF16 ? int64_t(kMaxPrefillWorkgroups) : std::min<int64_t>(items_ub, 1024);
}

template <bool BF16, int D, int HW>
PlanArgs plan_args(const AttnArgs& a, int64_t slots, bool beside) {
  PlanArgs p{};
  p.qsl = a.qsl;
  p.ctx_lens = a.ctx_lens;
  p.seq_lens = a.seq_lens;
  p.block_tables = a.block_tables;
  p.bt_row = a.bt_row;
  p.S = a.S;
  p.T = a.T;
  p.MB = a.MB;
  p.G = a.Hq / a.Hkv;
  p.qtile = BF16 ? bf16_tile_tokens(HW) : tile_tokens(HW);
  p.Hq = a.Hq;
  p.D = a.D;
  p.kv_token_bytes = 2 * a.Hkv * a.D * (a.kv8 ? 1 : (a.elem == Elem::BF16 ? 2 : 4));
  p.items_per_tile = static_cast<int>(a.Hkv * (a.Hq / a.Hkv / HW));
  p.slots = static_cast<int>(slots);
  p.beside = beside ? 1 : 0;
  // (the share beside the decode: bf16 kernel only)
  p.flop_per_cu_us = kPrefillFlopPerCuUs;
  p.wg_per_cu = 1;
  p.ratio = kBesideRatio;
  p.tile_start = a.tile_start;
  p.tile_order = a.tile_order;
  p.counter = a.work_counter;
  p.sched = BF16 ? a.sched : nullptr;
  return p;
}

// What one call of the prefill launcher puts on the stream: the plan (alone,
// or with the KV write `write` in one launch), then the prefill kernel
// (folding in the decode's partition reduce when asked).
struct Launch {
  bool plan, prefill, beside, fold_reduce;
  const WriteArgs* write;
};

template <bool BF16, int D, int HW, bool KV8 = false>
hipError_t launch_typed(const AttnArgs& a, hipStream_t stream, const Launch& l) {
  const int64_t grid = prefill_slots<BF16, D, HW>(a);
  if (l.write) {
    const WriteArgs& w = *l.write;
    const int vec_per_head = static_cast<int>(w.kv8 ? w.D / 16 : w.D * w.es / 16);
    const int vec_per_tok = 2 * static_cast<int>(w.Hkv) * vec_per_head;
    const int tpb = vec_per_tok >= 1024 ? 1 : 1024 / vec_per_tok;
    const int64_t blocks = 1 + (w.T + tpb - 1) / tpb;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    ProfileScope ps(kWritePlan, stream);
    hipLaunchKernelGGL(write_plan_kernel, dim3(static_cast<unsigned>(blocks)), dim3(1024), 0, stream, w,
                       vec_per_head, tpb, plan_args<BF16, D, HW>(a, grid, l.beside));
  } else if (l.plan) {
    ProfileScope ps(kPlan, stream);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, plan_args<BF16, D, HW>(a, grid, l.beside));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !l.prefill || grid == 0) return e;
  // bf16: each workgroup takes its share of the static schedule; fp32:
  // workgroups pull items from the queue until it is empty.
  {
    ProfileScope ps(kPrefill, stream);
    if constexpr (BF16) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, HW, KV8>), dim3(static_cast<unsigned>(grid)), dim3(kPThreads),
                         bf16_lds_bytes<D>(), stream, a, a.block_tables, l.beside ? 1 : 0, l.fold_reduce ? 1 : 0);
    } else {
      hipLaunchKernelGGL((prefill_f32_kernel<D, HW, KV8>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                         stream, a, l.beside ? 1 : 0, l.fold_reduce ? 1 : 0);
    }
  }
  return hipGetLastError();
}

// KV8: an 8-bit pool, attended by the fp32-MFMA kernel (the f32 work layout).
template <bool BF16, int D, bool KV8 = false>
hipError_t launch_heads(const AttnArgs& a, hipStream_t stream, const Launch& l) {
  const int64_t G = a.Hq / a.Hkv;
  if (G % 4 == 0) return launch_typed<BF16, D, 4, KV8>(a, stream, l);
  if (G % 2 == 0) return launch_typed<BF16, D, 2, KV8>(a, stream, l);
  return launch_typed<BF16, D, 1, KV8>(a, stream, l);
}

template <bool BF16, int D>
int64_t slots_heads(const AttnArgs& a) {
  const int64_t G = a.Hq / a.Hkv;
  if (G % 4 == 0) return prefill_slots<BF16, D, 4>(a);
  if (G % 2 == 0) return prefill_slots<BF16, D, 2>(a);
  return prefill_slots<BF16, D, 1>(a);
}

template <int D, int HW, bool KV8 = false>
hipError_t allow_lds() {
  // The four bf16 K and V stages take 128 KB of dynamic LDS at D = 128.
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_bf16_kernel<D, HW, KV8>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bf16_lds_bytes<D>()));
}

}  // namespace

namespace {

hipError_t run_launch(const AttnArgs& a, hipStream_t stream, const Launch& l) {
  static const hipError_t lds_ok = [] {
    hipError_t e = hipSuccess;
    for (hipError_t r : {allow_lds<64, 1>(), allow_lds<64, 2>(), allow_lds<64, 4>(), allow_lds<128, 1>(),
                         allow_lds<128, 2>(), allow_lds<128, 4>(), allow_lds<128, 1, true>(),
                         allow_lds<128, 2, true>(), allow_lds<128, 4, true>()})
      if (r != hipSuccess) e = r;
    return e;
  }();
  if (lds_ok != hipSuccess) return lds_ok;
  // 8-bit pools: the bf16-MFMA kernel widens the codes at head size 128; the
  // fp32-MFMA kernel serves head size 64
  if (a.kv8) return a.D == 64 ? launch_heads<false, 64, true>(a, stream, l) : launch_heads<true, 128, true>(a, stream, l);
  const bool bf16 = a.elem == Elem::BF16;
  if (a.D == 64) return bf16 ? launch_heads<true, 64>(a, stream, l) : launch_heads<false, 64>(a, stream, l);
  return bf16 ? launch_heads<true, 128>(a, stream, l) : launch_heads<false, 128>(a, stream, l);
}

}  // namespace

hipError_t launch_plan(const AttnArgs& a, hipStream_t stream, bool beside) {
  return run_launch(a, stream, Launch{true, false, beside, false, nullptr});
}

hipError_t launch_write_plan(const WriteArgs& w, const AttnArgs& a, hipStream_t stream) {
  return run_launch(a, stream, Launch{false, false, false, false, &w});
}

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream, bool beside, bool fold_reduce) {
  return run_launch(a, stream, Launch{false, true, beside, fold_reduce, nullptr});
}

bool prefill_launches(const AttnArgs& a) {
  if (a.kv8) return (a.D == 64 ? slots_heads<false, 64>(a) : slots_heads<true, 128>(a)) > 0;
  const bool bf16 = a.elem == Elem::BF16;
  if (a.D == 64) return (bf16 ? slots_heads<true, 64>(a) : slots_heads<false, 64>(a)) > 0;
  return (bf16 ? slots_heads<true, 128>(a) : slots_heads<false, 128>(a)) > 0;
}

}  // namespace pa
