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
//    resets a work-queue head, so the host never reads lengths. Workgroups
//    take tiles from the queue until it is empty: longest-first greedy
//    assignment keeps the 9x spread of chunk contexts from leaving a tail.
//  - A workgroup of 4 waves owns one (q-tile, KV head, group of HW query
//    heads); wave w takes query head hw = w % HW and 32 tokens of sub-tile
//    w / HW. The waves share K/V tiles of 64 keys in LDS.
//  - bf16: K and V tiles are staged row-major in LDS with a 16-byte XOR
//    swizzle (row r, chunk c at c ^ (r mod chunks)), double buffered: the
//    next tile's global loads are in flight while the current tile is
//    computed, with one barrier per tile.
//  - S^T = K . Q^T on 32x32x16 bf16 MFMA (keys as rows): each lane owns one
//    query token, so the row max needs one cross-lane exchange and the output
//    rescale none. The scores are already the B operand of O^T = V^T . P^T; the
//    V^T operand comes straight from the row-major tile through gfx950's
//    transposing LDS read (ds_read_b64_tr_b16), two per MFMA.
//  - Online softmax in log2 units with the scale folded into one FMA before
//    exp2, the same lazy rescale as decode, and the causal mask only on tiles
//    that cross the diagonal or the sequence end.
//  - fp32 inputs take a simpler exact kernel (fp32 MFMA, V transposed while
//    staging); it exists for accuracy, not speed.
#include <algorithm>
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) const uint4 lds_u4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;
// The bf16 kernel keeps its reference maximum while a slice's weights (16
// per lane) sum to at most 2^8; each weight is then at most 2^8 as well.
constexpr float kRescaleBound = 256.0f;
// Word 3 of a raw (unformatted, unswizzled) buffer resource on gfx9-family
// parts: 32-bit data format, no index stride.
constexpr int kBufferFlags = 0x00020000;
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

// One block of 1024 threads: per-sequence tile counts, exclusive scan into
// tile_start, cost-sorted tile order (if it fits), queue head reset.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* qsl, const int32_t* ctx_lens,
                                                    const int32_t* seq_lens, int64_t S, int64_t T, int64_t MB,
                                                    int64_t G, int qtile, int32_t* tile_start, int32_t* tile_order,
                                                    int32_t* counter) {
  __shared__ int32_t part[1024];
  __shared__ uint64_t keys[kMaxSortedTiles];
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
  for (int64_t s = s0; s < s1; ++s) sum += tiles(qlen(s));
  part[tid] = sum;
  __syncthreads();
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
      }
    }
    run += nt;
  }
  if (tid == 1023) tile_start[S] = total;
  if (tid == 0) *counter = 0;
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
  for (int i = tid; i < total; i += 1024) tile_order[i] = static_cast<int32_t>(0xffffffffu - uint32_t(keys[i]));
}

// Which sequence and local tile a queue item names.
struct TileRef {
  int64_t s, lt, g, hg;
};

__device__ inline TileRef locate(const AttnArgs& a, int64_t item, int n_hg, int64_t total_tiles) {
  TileRef r;
  r.g = item % a.Hkv;
  const int64_t rest = item / a.Hkv;
  r.hg = rest % n_hg;
  const int64_t rank = rest / n_hg;
  const int64_t t = total_tiles <= kMaxSortedTiles ? int64_t(a.tile_order[rank]) : rank;
  int64_t lo = 0, hi = a.S - 1;  // last s with tile_start[s] <= t
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (a.tile_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  r.s = lo;
  r.lt = t - a.tile_start[lo];
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

// 16 bytes at byte offset off of a block's head slice. The block base is
// wave-uniform, so the load goes through a buffer resource built in scalar
// registers and the per-lane offset is the only vector operand; reads at or
// past rec bytes return zero.
__device__ inline uint4 load_row16(const char* base, uint32_t rec, uint32_t off) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, static_cast<int>(rec), kBufferFlags);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

// ---------------------------------------------------------------- bf16 ----
template <int D>
struct Bf16Tile {
  static constexpr int KT = 64;                    // keys per stage
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int CHUNKS = KT * CPR;          // per K or V tile
  static constexpr int LOADS = CHUNKS / kPThreads;  // 16-byte loads per thread per tile (K and V each)
  // Chunk c of row r sits at r * CPR + (c ^ swz(r)). LDS has 64 banks of 4
  // bytes, so a 256-byte span is one pass. swz depends on r mod 16 only and
  // keeps all three access patterns to one pass per 256 bytes: 16 rows read
  // at one chunk (K fragments), 4 consecutive rows x 4 consecutive chunks
  // (transposing V reads), and whole rows written by consecutive lanes.
  __device__ static int swz(int r) {
    return CPR == 16 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  __device__ static int chunk(int r, int c) { return r * CPR + (c ^ swz(r)); }
  static_assert(CPR == 8 || CPR == 16, "head size 64 or 128");
};

// block_tables comes in again as a restrict pointer: nothing in the kernel
// writes it, so its wave-uniform entries are read with scalar loads.
template <int D, int HW>
__global__ __launch_bounds__(kPThreads) void prefill_bf16_kernel(AttnArgs a, const int32_t* __restrict__ bt_all) {
  using Tl = Bf16Tile<D>;
  constexpr int KT = Tl::KT, CPR = Tl::CPR, LOADS = Tl::LOADS;
  constexpr int QTB = bf16_tile_tokens(HW);
  constexpr int QS = D / 16;  // k-steps of S^T
  // [stage 2][K | V][CHUNKS], then the queue slot. No static LDS: the
  // dynamic array starts at address 0, so fragment addresses are a per-lane
  // base plus an immediate offset.
  extern __shared__ uint4 lds[];
  int* item_sh = reinterpret_cast<int*>(lds + 2 * 2 * Tl::CHUNKS);

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
  const float c_scale = a.scale * kLog2e;
  const uint32_t NB = static_cast<uint32_t>(min(a.NB, int64_t(0x7fffffff)));

  for (int64_t item = next_item(a, item_sh); item < n_items; item = next_item(a, item_sh)) {
    const TileRef tr = locate(a, item, n_hg, total_tiles);
    // Positions fit in 32 bits: keys are bounded by MB * 16 (checked on the host).
    const int64_t s = tr.s, g = tr.g;
    const int lt = static_cast<int>(tr.lt), hg = static_cast<int>(tr.hg);
    const int64_t q0 = min(max(static_cast<int64_t>(a.qsl[s]), int64_t(0)), a.T);
    const int n = static_cast<int>(min(max(static_cast<int64_t>(a.qsl[s + 1]), q0), a.T) - q0);
    const int Lc = static_cast<int>(min(max(static_cast<int64_t>(a.seq_lens[s]), int64_t(0)), a.MB * kBlockTokens));
    const int C = min(max(a.ctx_lens[s], 0), Lc);
    const int64_t h = g * G + hg * HW + hw;
    const int i0 = lt * QTB + tw * kWaveTokens;  // first token of this wave
    const bool wave_active = i0 < n;
    const int blk_last = min(n, (lt + 1) * QTB) - 1;  // last token of the tile
    const int kend = min(C + blk_last + 1, Lc);       // keys [0, kend) needed by the tile
    const int wave_kend = wave_active ? min(C + min(n, i0 + kWaveTokens), Lc) : 0;
    const int wave_first = C + i0;                    // smallest position among the wave's tokens
    const int my_i = min(i0 + col, n - 1);            // clamped token of this lane
    const int my_pos = C + my_i;                      // last key this lane sees
    const int nkt = (kend + KT - 1) / KT;

    bf16x8 qf[QS];  // Q^T (B operand): token col, d = 16 st + 8 hh .. +8
    {
      const char* qrow = a.q + (q0 + my_i) * a.q_st + h * a.q_sh + 16 * hh;
#pragma unroll
      for (int st = 0; st < QS; ++st)
        qf[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 32 * st));
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // Per-lane byte offsets of the fragments inside a 32-row slice of a tile;
    // the swizzle term depends only on the row modulo 16, which the slice
    // start does not change, so these hold for every slice and stage.
    // They are LDS byte addresses; the empty asm keeps each one in a register
    // (otherwise the compiler re-adds the LDS base before every read) so the
    // slice, stage and K/V offsets fold into the reads' immediate offsets.
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    uint32_t k_rd[QS];
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      k_rd[st] = lds0 + 16u * Tl::chunk(col, 2 * st + hh);
      asm volatile("" : "+v"(k_rd[st]));
    }
    uint32_t v_rd[D / 32][2];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        // lane j16 of 16-lane group g16 points at V[row][d .. d + 3]; the
        // transposing read hands it V[row0 + e][32 dt + 16 (g16 & 1) + j16], e = 0..3
        const int row = 4 * hh + (j16 >> 2) + 8 * w;
        const int d = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3);
        v_rd[dt][w] = lds0 + 16u * Tl::CHUNKS + 16u * Tl::chunk(row, d >> 3) + 2u * (d & 7);  // V follows K
        asm volatile("" : "+v"(v_rd[dt][w]));
      }
    const int32_t* bt = bt_all + s * a.bt_row;
    const char* kc = a.kc + g * a.kc_sh;
    const char* vc = a.vc + g * a.vc_sh;
    uint4 kreg[LOADS], vreg[LOADS];
    // Load i of a thread covers tile row r = (tid + 512 i) / CPR, chunk
    // c = tid % CPR. A wave's rows of one load lie in a single 16-token
    // block, so the block-table entry and the block's base address are
    // wave-uniform (scalar); only the in-block offset is per lane, and it is
    // the same for every tile.
    uint32_t k_off[LOADS], v_off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int id = tid + i * kPThreads, r = id / CPR, c = id % CPR;
      k_off[i] = static_cast<uint32_t>((r % kBlockTokens) * a.kc_sr + 16 * c);
      v_off[i] = static_cast<uint32_t>((r % kBlockTokens) * a.vc_sr + 16 * c);
    }
    // Rows at or past kend (only in the last tile) are loaded from the last
    // block the tile needs, so that every address is inside the pool, and
    // are zeroed when stashed.
    const int last_blk = (kend - 1) / kBlockTokens;
    // bytes of one block's head slice, from its first row
    const uint32_t k_rec = static_cast<uint32_t>((kBlockTokens - 1) * a.kc_sr + a.D * 2);
    const uint32_t v_rec = static_cast<uint32_t>((kBlockTokens - 1) * a.vc_sr + a.D * 2);
    auto fetch = [&](int kt) {
      uint32_t id32[LOADS];
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        // block of the wave's rows in load i (lane 0's row / 16; the same for every lane)
        const int blk = kt * (KT / kBlockTokens) + ((wave * 64 + i * kPThreads) / CPR) / kBlockTokens;
        id32[i] = static_cast<uint32_t>(bt[min(blk, last_blk)]);
      }
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int64_t pid = id32[i] < NB ? int64_t(id32[i]) : 0;
        kreg[i] = load_row16(kc + pid * a.kc_sb, k_rec, k_off[i]);
        vreg[i] = load_row16(vc + pid * a.vc_sb, v_rec, v_off[i]);
      }
    };
    auto stash = [&](int stage, int kt) {
      uint4* k_l = lds + stage * 2 * Tl::CHUNKS;
      uint4* v_l = k_l + Tl::CHUNKS;
      if ((kt + 1) * KT <= kend) {  // uniform: every row is a real key
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int id = tid + i * kPThreads, r = id / CPR, c = id % CPR;
          k_l[Tl::chunk(r, c)] = kreg[i];
          v_l[Tl::chunk(r, c)] = vreg[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int id = tid + i * kPThreads, r = id / CPR, c = id % CPR;
          const bool real = kt * KT + r < kend;
          k_l[Tl::chunk(r, c)] = real ? kreg[i] : make_uint4(0, 0, 0, 0);
          v_l[Tl::chunk(r, c)] = real ? vreg[i] : make_uint4(0, 0, 0, 0);
        }
      }
    };

    fetch(0);
    stash(0, 0);
    // Everything loaded so far (Q fragments, tile 0) has landed. Without this
    // explicit wait the compiler cannot tell at the loop head and waits on the
    // vector-memory counter inside the MFMA chain, which also stalls on the
    // prefetch of the next tile.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // One key tile: the loads of the next tile are issued first and stashed
    // into the other stage after this tile's MFMAs. The stage is a
    // compile-time constant (the loop below runs tiles in pairs), so every
    // LDS address is a per-lane base plus an immediate offset.
    auto tile_step = [&](auto stage_c, int kt) {
      constexpr int stage = decltype(stage_c)::value;
      if (kt + 1 < nkt) fetch(kt + 1);
      const int k0 = kt * KT;
      if (wave_active && k0 < wave_kend) {
        constexpr uint32_t stage_off = stage * 2 * Tl::CHUNKS * 16;  // bytes
        // K fragments of a slice: K[32 half + col][16 st + 8 hh .. +8]. Slice
        // 0's are read before its chain (only the first MFMA waits for LDS);
        // slice 1's are read right after slice 0's chain and land during
        // slice 0's softmax.
        bf16x8 kf[QS];
#pragma unroll
        for (int st = 0; st < QS; ++st) kf[st] = __builtin_bit_cast(bf16x8, *(lds_u4*)(uintptr_t)(k_rd[st] + stage_off));
        static_assert(KT == 64, "two 32-key slices per stage");
        auto slice = [&](auto half_c) {
          constexpr int half = decltype(half_c)::value;
          const int kh0 = k0 + 32 * half;
          f32x16 sacc;
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
          // Raised priority while a wave feeds the matrix core: the other wave
          // on the SIMD fills the gaps with its softmax instead of delaying
          // the MFMA issue.
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int st = 0; st < QS; ++st) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], sacc, 0, 0, 0);
          if constexpr (half == 0) {
            const uint32_t k_n = stage_off + 32 * CPR * 16;  // slice 1 of K
#pragma unroll
            for (int st = 0; st < QS; ++st) kf[st] = __builtin_bit_cast(bf16x8, *(lds_u4*)(uintptr_t)(k_rd[st] + k_n));
            __builtin_amdgcn_sched_group_barrier(0x100, QS, 0);  // slice 0's reads,
            __builtin_amdgcn_sched_group_barrier(0x008, QS, 0);  // its chain,
            __builtin_amdgcn_sched_group_barrier(0x100, QS, 0);  // slice 1's reads
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, QS, 0);  // slice 1's chain
          }
          __builtin_amdgcn_s_setprio(0);
          // S^T[key kh0 + 8q + 4hh + r][token col] in sacc[4q + r]
          float sc[16];
          if ((kh0 + 31 > wave_first) || (kh0 + 31 >= kend)) {  // slice crosses the diagonal or the end
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kh0 + 8 * (i >> 2) + 4 * hh + (i & 3);
              sc[i] = (key <= my_pos && key < kend) ? sacc[i] : -INFINITY;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[i] = sacc[i];
          }
          // Weights against the running reference m_run. While no weight of
          // the slice exceeds 2^8 (checked through the lane's sum, which also
          // catches inf and NaN) the reference stands; otherwise the slice's
          // true maximum is taken across the two lane halves of each token,
          // the accumulators are rescaled and the weights recomputed. The
          // first slice always takes that path (m_run starts at -inf).
          // four partial sums: the adds do not form one serial chain
          auto weights = [&](float (&w)[16]) {
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              w[i] = fast_exp2(__builtin_fmaf(sc[i], c_scale, -m_run));
              part[i & 3] += w[i];
            }
            return (part[0] + part[1]) + (part[2] + part[3]);
          };
          float pv[16];
          float lsum = weights(pv);
          if (__any(!(lsum <= kRescaleBound))) {
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[i]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * c_scale;
            const float m_new = fmaxf(m_run, tmax);
            if (m_new > m_run) {
              const float alpha = fast_exp2(m_run - m_new);
              l_run *= alpha;
#pragma unroll
              for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
              m_run = m_new;
            }
            lsum = weights(pv);
          }
          l_run += lsum;
          // O^T[d][token] += V^T[d][key] P^T[key][token]; key slots of lane half hh:
          // e < 4 -> 16 q2 + 4 hh + e, e >= 4 -> 16 q2 + 8 + 4 hh + (e - 4)
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(pv[8 * q2 + e]);
            // rows 32 half + 16 q2 + [4 hh, 4 hh + 4) and the same + 8; all
            // fragments of the 16 keys are read before their MFMAs
            const uint32_t v_q = stage_off + (32 * half + 16 * q2) * CPR * 16;
            bf16x8 va[D / 32];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
              const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(v_rd[dt][0] + v_q));
              const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(v_rd[dt][1] + v_q));
              const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
              va[dt] = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
            }
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], pb, o[dt], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 1);  // the reads first,
            __builtin_amdgcn_sched_group_barrier(0x008, D / 32, 1);  // then the MFMAs
          }
          __builtin_amdgcn_s_setprio(0);
        };
        slice(std::integral_constant<int, 0>{});
        if (k0 + 32 < wave_kend) slice(std::integral_constant<int, 1>{});
      }
      if (kt + 1 < nkt) stash(stage ^ 1, kt + 1);
      __syncthreads();
    };
    for (int kt = 0; kt < nkt; kt += 2) {
      tile_step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < nkt) tile_step(std::integral_constant<int, 1>{}, kt + 1);
    }

    if (wave_active) {
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const int my_tok = i0 + col;
      if (my_tok < n) {
        const float inv = 1.f / l_tot;
        char* dst = a.out + (q0 + my_tok) * a.out_st + h * a.out_sh;
        // lane holds O^T[d = 32 dt + 8 q + 4 hh + r][token col]
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d = 32 * dt + 8 * q + 4 * hh;
            *reinterpret_cast<uint2*>(dst + 2 * d) =
                make_uint2(pack_bf16(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv),
                           pack_bf16(o[dt][4 * q + 2] * inv, o[dt][4 * q + 3] * inv));
          }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 ----
template <int D, int HW>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(AttnArgs a) {
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
  const float c_scale = a.scale * kLog2e;
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
    {
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
          kv = *reinterpret_cast<const float4*>(kc + pid * a.kc_sb + (j % kBlockTokens) * a.kc_sr + 16 * c);
          vv = *reinterpret_cast<const float4*>(vc + pid * a.vc_sb + (j % kBlockTokens) * a.vc_sr + 16 * c);
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
        const float inv = 1.f / l_tot;
        char* dst = a.out + (q0 + my_tok) * a.out_st + h * a.out_sh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d = 32 * dt + 8 * q + 4 * hh;
            *reinterpret_cast<float4*>(dst + 4 * d) =
                make_float4(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv, o[dt][4 * q + 2] * inv,
                            o[dt][4 * q + 3] * inv);
          }
      }
    }
  }
}

template <int D>
constexpr size_t bf16_lds_bytes() {
  return sizeof(uint4) * (2 * 2 * Bf16Tile<D>::CHUNKS + 1);
}

template <bool BF16, int D, int HW>
hipError_t launch_typed(const AttnArgs& a, hipStream_t stream) {
  constexpr int QTB = BF16 ? bf16_tile_tokens(HW) : tile_tokens(HW);
  {
    ProfileScope ps(kPlan, stream);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a.qsl, a.ctx_lens, a.seq_lens, a.S, a.T, a.MB,
                       a.Hq / a.Hkv, QTB, a.tile_start, a.tile_order, a.work_counter);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Upper bound on work without reading lengths: every prefill sequence has
  // more than 16 / G tokens.
  const int64_t G = a.Hq / a.Hkv;
  const int64_t tiles_ub = a.T / QTB + std::min<int64_t>(a.S, a.T / (kMaxDecodeColumns / G + 1));
  const int64_t items_ub = tiles_ub * a.Hkv * (G / HW);
  if (items_ub == 0) return hipSuccess;
  // Workgroups pull items from the queue until it is empty: enough of them
  // to fill every CU (bf16: one 8-wave workgroup per CU; fp32: four 4-wave).
  const int64_t grid = std::min<int64_t>(items_ub, BF16 ? 512 : 1024);
  {
    ProfileScope ps(kPrefill, stream);
    if constexpr (BF16) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, HW>), dim3(static_cast<unsigned>(grid)), dim3(kPThreads),
                         bf16_lds_bytes<D>(), stream, a, a.block_tables);
    } else {
      hipLaunchKernelGGL((prefill_f32_kernel<D, HW>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                         a);
    }
  }
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_heads(const AttnArgs& a, hipStream_t stream) {
  const int64_t G = a.Hq / a.Hkv;
  if (G % 4 == 0) return launch_typed<BF16, D, 4>(a, stream);
  if (G % 2 == 0) return launch_typed<BF16, D, 2>(a, stream);
  return launch_typed<BF16, D, 1>(a, stream);
}

template <int D, int HW>
hipError_t allow_lds() {
  // The double-buffered bf16 tiles take 64 KB of dynamic LDS at D = 128.
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_bf16_kernel<D, HW>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bf16_lds_bytes<D>()));
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  static const hipError_t lds_ok = [] {
    hipError_t e = hipSuccess;
    for (hipError_t r : {allow_lds<64, 1>(), allow_lds<64, 2>(), allow_lds<64, 4>(), allow_lds<128, 1>(),
                         allow_lds<128, 2>(), allow_lds<128, 4>()})
      if (r != hipSuccess) e = r;
    return e;
  }();
  if (lds_ok != hipSuccess) return lds_ok;
  const bool bf16 = a.elem == Elem::BF16;
  if (a.D == 64) return bf16 ? launch_heads<true, 64>(a, stream) : launch_heads<false, 64>(a, stream);
  return bf16 ? launch_heads<true, 128>(a, stream) : launch_heads<false, 128>(a, stream);
}

}  // namespace pa
