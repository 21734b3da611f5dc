// Decode attention: sequences whose new tokens times the query heads per KV
// head fit 16 MFMA columns (every decode, and short queries such as
// speculative-decode verification) read all of their cached K/V through the
// block table; HBM-bound ("Inside vLLM", section "Scheduler": decode steps
// are memory-bandwidth-bound; "Serving models at scale with vLLM", section
// "Speculative decoding": a decode pass is limited by moving data, not math).
//
// Design for gfx950 (the pages give no kernel design):
//  - A workgroup of 8 waves owns (sequence s, group of hw KV heads, partition
//    p), the keys [p * PT, min((p + 1) * PT, L)). With 8 KV heads each wave
//    streams one head through every block of the partition, so the 8 head
//    slices of a pool block (one contiguous block of all heads) are read by
//    one workgroup at about the same time; with fewer heads the 8 / hw waves
//    of a head split the blocks round-robin and merge through LDS at the end.
//    All G = Hq / Hkv query heads of a KV head share each K/V read.
//  - Each lane loads the 16-byte chunks of a block's K and V head slices it
//    needs with non-temporal buffer loads (one block in flight per wave), then
//    stages them through a per-wave LDS tile into the MFMA operand layouts
//    (8-bit codes are widened to bf16 on the way into LDS).
//  - Scores use MFMA with the key rows as the A operand: S^T = K . Q^T; the
//    16 columns are (new token, query head) pairs, each with its own causal
//    limit. In the score layout a lane holds one column and 4 consecutive
//    keys, which is already the P^T operand of the 16x16x16 bf16 MFMA; V^T
//    comes from the row-major V slice through the transposing LDS read, so
//    O^T = V^T . P^T needs no lane exchange and rescaling touches one column
//    per lane. fp32 inputs keep an exact path on the fp32 MFMA.
//  - Online softmax in log2 units with a lazy rescale: the running maximum is
//    only raised (and the accumulators rescaled) when a block's maximum beats
//    it by more than 2^8, so weights stay <= 256 and rescales are rare.
//  - Sequences longer than one partition write (unnormalised output, max,
//    weight sum) per partition; the partitions are combined in a fixed order
//    (deterministic) by a reduce kernel, or by the prefill kernel's waves
//    when it runs after the decode on the same stream. Single-partition
//    sequences write the output directly.
#include <cstdlib>
#include <type_traits>

#include "pa_internal.h"
#include "step_parts.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr size_t kDecodeMaxLds = 80 * 1024;  // dynamic LDS a decode workgroup may ask for

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Word 3 of a raw (unformatted, unswizzled) buffer resource on gfx9-family
// parts: 32-bit data format, no index stride.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the K/V loads: non-temporal. Each K/V byte is read once per
// step; streaming it past the caches instead of allocating it there raises
// the sustained read rate (measured: about 7.2 vs 6.2 TB/s for a plain read).
constexpr int kStreamPolicy = 2;

// A block's head slice as a buffer resource: the base is wave-uniform, so it
// lives in scalar registers and the loads take only a per-lane offset.
__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, static_cast<int>(bytes), kBufferFlags);
}

template <int VW>
__device__ inline void load_words(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff, uint32_t (&w)[VW]) {
  if constexpr (VW == 2) {
    const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, soff, kStreamPolicy));
    w[0] = u.x;
    w[1] = u.y;
  } else {
#pragma unroll
    for (int i = 0; i < VW / 4; ++i) {
      const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, soff, kStreamPolicy));
      w[4 * i] = u.x;
      w[4 * i + 1] = u.y;
      w[4 * i + 2] = u.z;
      w[4 * i + 3] = u.w;
    }
  }
}

template <bool BF16, int D>
struct DecodeShape {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int KC = D * ES / 64;           // 16-byte K chunks per lane per block
  static constexpr int VE = D / 16;                // V elements per lane per row
  static constexpr int VW = VE * ES / 4;           // 32-bit words per lane per V row
  static constexpr int NACC = BF16 ? D / 16 : VE;  // 16x16 accumulator tiles
  static constexpr int LPR = D * ES / 16;          // lanes per K row when loading (16 bytes each)
  static constexpr int RPI = 64 / LPR;             // K rows per load instruction
  static constexpr int KT_BYTES = kBlockTokens * D * ES;  // per-wave K tile (one block)
  static constexpr int VT_BYTES = BF16 ? kBlockTokens * D * 2 : 0;  // per-wave V tile (one block)
  static constexpr int TILE_BYTES = KT_BYTES + VT_BYTES;
  // K tile: row-major, chunk c of row r at c ^ swzk(r). Fragment reads (16
  // rows at one chunk per 16 lanes) and row writes both stay one pass per 256
  // bytes.
  __device__ static int swzk(int r) { return LPR == 8 ? (r >> 1) & 7 : r & 15; }
  __device__ static int kt_off(int r, int c) { return r * D * ES + 16 * (c ^ swzk(r)); }
  // The V tile is row-major (key, d) with its 16-byte chunks permuted within
  // each row: chunk c of row r sits at c ^ swz(r). LDS has 64 banks of 4
  // bytes; with this permutation the transposing reads (8 rows x 2 chunks per
  // 32 lanes) touch every bank once, and the row writes stay conflict-free
  // at D = 128 (two rows share a pass at D = 64: 2-way on writes only).
  __device__ static int swz(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
  __device__ static int vt_off(int r, int elem) {
    return r * D * 2 + 16 * ((elem >> 3) ^ swz(r)) + 2 * (elem & 7);
  }
};

template <bool BF16, int D>
struct BlockRegs {
  using Sh = DecodeShape<BF16, D>;
  uint4 k[Sh::KC];
  uint32_t v[4][Sh::VW];
};

// One block of an 8-bit (OCP FP8 E4M3) pool in registers, as loaded: K load
// i of a lane covers row RPI8 i + lane / LPR8, codes 16 (lane % LPR8) ..
// +15; V: rows 4kg + j, codes VB n .. VB n + VB - 1 (the same elements the
// bf16 layout gives the lane).
template <int D>
struct BlockRegs8 {
  static constexpr int LPR8 = D / 16;  // lanes per K row (16 codes each)
  static constexpr int RPI8 = 64 / LPR8;
  static constexpr int KC8 = D / 64;   // K loads per lane per block
  static constexpr int VB = D / 16;    // V codes per lane per row
  static constexpr int VW8 = VB / 4;   // 32-bit words of them
  uint4 k[KC8];
  uint32_t v[4][VW8];
};

// Codes 2 SEL, 2 SEL + 1 of w as two bf16 values (exact: every E4M3 value is
// a bf16 value), low half first.
template <bool SEL>
__device__ inline uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, SEL));
}

// K: load i of a lane covers row RPI i + lane / LPR, bytes k_off = 16 (lane %
// LPR) of it (whole 128-byte lines per instruction); V: rows 4kg + j, bytes
// v_off.
template <bool BF16, int D>
__device__ inline void load_block(BlockRegs<BF16, D>& r, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                  uint32_t k_off, uint32_t kc_sr, uint32_t v_off, uint32_t vc_sr) {
  using Sh = DecodeShape<BF16, D>;
#pragma unroll
  for (int i = 0; i < Sh::KC; ++i)
    r.k[i] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off, i * Sh::RPI * kc_sr, kStreamPolicy));
#pragma unroll
  for (int j = 0; j < 4; ++j) load_words<Sh::VW>(vr, v_off, j * vc_sr, r.v[j]);
}

template <int D>
__device__ inline void load_block8(BlockRegs8<D>& r, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                   uint32_t k_off, uint32_t kc_sr, uint32_t v_off, uint32_t vc_sr) {
  using R = BlockRegs8<D>;
#pragma unroll
  for (int i = 0; i < R::KC8; ++i)
    r.k[i] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off, i * R::RPI8 * kc_sr, kStreamPolicy));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (R::VW8 == 2) {
      const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vr, v_off, j * vc_sr, kStreamPolicy));
      r.v[j][0] = u.x;
      r.v[j][1] = u.y;
    } else {
      r.v[j][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, v_off, j * vc_sr, kStreamPolicy);
    }
  }
}

// Consume one block: scores, online softmax, P.V. `blk` is the block's index
// within the sequence; rows at or past `end` (the partition's end) are
// zeroed, and this lane's column sees keys below `lim` only. Lane (kg, n) holds
// K row n and V rows 4kg..4kg+3 (elements VE*n..VE*n+VE-1) of the block.
// Accumulators: bf16 path O^T[d = 16t + 4kg + r][head n] in o[t][r];
// fp32 path O[head 4kg + r][d = VE*n + e] in o[e][r].
template <bool BF16, int D, bool KV8>
using RawBlock = std::conditional_t<KV8, BlockRegs8<D>, BlockRegs<BF16, D>>;

template <bool BF16, int D, bool KV8>
__device__ inline void attend_block(RawBlock<BF16, D, KV8>& raw, const uint4 (&qv)[DecodeShape<BF16, D>::KC],
                                    f32x4 (&o)[DecodeShape<BF16, D>::NACC], float& m_run, float& l_run,
                                    char* tile, int blk, int end, int lim, int lane, float qk_scale) {
  using Sh = DecodeShape<BF16, D>;
  constexpr int KC = Sh::KC, VE = Sh::VE, VW = Sh::VW;
  const int n = lane & 15, kg = lane >> 4;
  // Stage K row-major, then read the MFMA A fragments: lane (kg, n) takes row
  // n, bytes 64 c + 16 kg (chunk 4c + kg) for k-step c. An 8-bit block is
  // widened to bf16 on the way: a lane's 16 codes become chunks 2c, 2c + 1.
  BlockRegs<BF16, D> conv;
  BlockRegs<BF16, D>& cur = [&]() -> BlockRegs<BF16, D>& {
    if constexpr (KV8) return conv;
    else return raw;
  }();
  if constexpr (KV8) {
    using R = BlockRegs8<D>;
#pragma unroll
    for (int i = 0; i < R::KC8; ++i) {
      const uint32_t w[4] = {raw.k[i].x, raw.k[i].y, raw.k[i].z, raw.k[i].w};
      const int row = R::RPI8 * i + lane / R::LPR8, c = 2 * (lane % R::LPR8);
      *reinterpret_cast<uint4*>(tile + Sh::kt_off(row, c)) =
          make_uint4(fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]), fp8x2_to_bf16x2<false>(w[1]),
                     fp8x2_to_bf16x2<true>(w[1]));
      *reinterpret_cast<uint4*>(tile + Sh::kt_off(row, c + 1)) =
          make_uint4(fp8x2_to_bf16x2<false>(w[2]), fp8x2_to_bf16x2<true>(w[2]), fp8x2_to_bf16x2<false>(w[3]),
                     fp8x2_to_bf16x2<true>(w[3]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < R::VW8; ++w) {
        conv.v[j][2 * w] = fp8x2_to_bf16x2<false>(raw.v[j][w]);
        conv.v[j][2 * w + 1] = fp8x2_to_bf16x2<true>(raw.v[j][w]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < KC; ++i)
      *reinterpret_cast<uint4*>(tile + Sh::kt_off(Sh::RPI * i + lane / Sh::LPR, lane % Sh::LPR)) = cur.k[i];
  }
  __builtin_amdgcn_wave_barrier();
  // scores S^T[token 4kg + r][head n]
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const uint4 kc = *reinterpret_cast<const uint4*>(tile + Sh::kt_off(n, 4 * c + kg));
    if constexpr (BF16) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc),
                                                     __builtin_bit_cast(bf16x8, qv[c]), acc, 0, 0, 0);
    } else {
      const float4 kf = __builtin_bit_cast(float4, kc);
      const float4 qf = __builtin_bit_cast(float4, qv[c]);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.x, qf.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.y, qf.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.z, qf.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.w, qf.w, acc, 0, 0, 0);
    }
  }
  float sc[4];
  const int tok0 = blk * kBlockTokens + 4 * kg;
#pragma unroll
  for (int r = 0; r < 4; ++r) sc[r] = (tok0 + r < lim) ? acc[r] * qk_scale : -INFINITY;
  float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  // A column can have no visible key yet (a later token of a short query in
  // a partition that starts past its position): its maximum stays -inf and
  // its weights and accumulators stay 0, never NaN.
  if (__any(mloc > m_run + kRescaleThreshold)) {
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = m_new == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
    l_run *= alpha;
    if constexpr (BF16) {
#pragma unroll
      for (int t = 0; t < Sh::NACC; ++t) o[t] *= alpha;  // this lane's head column
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * kg + r);  // output row r holds head 4kg + r
#pragma unroll
        for (int e = 0; e < VE; ++e) o[e][r] *= ar;
      }
    }
    m_run = m_new;
  }
  float pr[4];
  const float m_ref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pr[r] = fast_exp2(sc[r] - m_ref);
    l_run += pr[r];
  }
  // Rows past the sequence end carry weight 0 but arbitrary bits (0 * NaN is
  // NaN), so they are zeroed before the product.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (tok0 + j >= end) {
#pragma unroll
      for (int w = 0; w < VW; ++w) cur.v[j][w] = 0u;
    }
  }
  if constexpr (BF16) {
    // Stage the block's V rows (this lane: rows 4kg + j, elements VE n ..)
    // and read V^T fragments back with the transposing LDS read.
    char* vtb = tile + Sh::KT_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      char* dst = vtb + Sh::vt_off(4 * kg + j, VE * n);
      if constexpr (VW == 4)
        *reinterpret_cast<uint4*>(dst) = make_uint4(cur.v[j][0], cur.v[j][1], cur.v[j][2], cur.v[j][3]);
      else
        *reinterpret_cast<uint2*>(dst) = make_uint2(cur.v[j][0], cur.v[j][1]);
    }
    __builtin_amdgcn_wave_barrier();
    const i16x4 pb = __builtin_bit_cast(i16x4, make_uint2(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])));
#pragma unroll
    for (int t = 0; t < Sh::NACC; ++t) {
      // lane (kg, n) points at V[4kg + n/4][16t + 4(n%4) ..] and receives
      // V[4kg + e][16t + n], e = 0..3: the A operand V^T[d][key] of tile t
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vtb + Sh::vt_off(4 * kg + (n >> 2), 16 * t + 4 * (n & 3))));
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[t], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  } else {
    // O[head][d = VE * n + e] += sum over the 4 lane groups of P[head][token] V[token][d]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < VE; ++e)
        o[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[j], __uint_as_float(cur.v[j][e]), o[e], 0, 0, 0);
    }
  }
}

// The waves of each head have left (max, weight sum, unnormalised output)
// per column in LDS, [wave][m: 16][l: 16][o: ncol * D]; combine those of
// the same head (waves hl, hl + hw, ...) and store the result: normalised
// into out for a one-partition sequence, else as the partition's partial.
template <bool BF16, int D, bool KV8>
__device__ inline void combine_waves(const AttnArgs& a, const float* smem, int wstride, int hw, int wph, int ncol,
                                     uint32_t hg, int G, int q0, int nparts, int p) {
  constexpr int ES = BF16 ? 2 : 4;
  const int per_head = ncol * (D / 4);
  for (int idx = threadIdx.x; idx < hw * per_head; idx += kDecodeThreads) {
    const int hl = idx / per_head, rest = idx - hl * per_head;
    const int h = rest / (D / 4), d = 4 * (rest - h * (D / 4));  // h: column
    float m = -INFINITY;
    for (int ph = 0; ph < wph; ++ph) m = fmaxf(m, smem[(hl + hw * ph) * wstride + h]);
    float lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int ph = 0; ph < wph; ++ph) {
      const float* wsw = smem + (hl + hw * ph) * wstride;
      // 0 for a wave that saw no block or no visible key of this column
      const float sw = m == -INFINITY ? 0.f : fast_exp2(wsw[h] - m);
      lsum += sw * wsw[16 + h];
      const float4 x = *reinterpret_cast<const float4*>(wsw + 32 + h * D + d);
      acc.x += sw * x.x;
      acc.y += sw * x.y;
      acc.z += sw * x.z;
      acc.w += sw * x.w;
    }
    if constexpr (KV8) {  // values read back as value(code) * v_scale
      acc.x *= a.v_scale;
      acc.y *= a.v_scale;
      acc.z *= a.v_scale;
      acc.w *= a.v_scale;
    }
    const int64_t hq = int64_t(hg * hw + hl) * G + h % G;
    const int64_t t = q0 + h / G;  // the column's token
    if (nparts == 1) {
      const float inv = 1.f / lsum;
      char* dst = a.out + t * a.out_st + hq * a.out_sh + d * ES;
      if constexpr (BF16) {
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      }
    } else {
      const int64_t slot = (t * a.Hq + hq) * a.max_parts + p;
      *reinterpret_cast<float4*>(a.ws_o + slot * D + d) = acc;
      if (d == 0) a.ws_ml[slot] = make_float2(m, lsum);
    }
  }
}

// Workgroup: 8 waves, (sequence s, group of HW KV heads, partition p); grid
// x = s * (Hkv / HW) + head group, y = p, or, for a launch with a work order,
// one workgroup per unit of a 1-D grid (below). Wave w serves KV head w % HW and,
// of the partition's blocks, those with index = w / HW modulo 8 / HW. With
// HW = 8 every wave streams one head through all blocks, so the 8 head
// slices of each pool block (one contiguous block of all heads) are read by
// one workgroup at the same time. Dynamic LDS: per-wave V tiles during the
// sweep, then each wave's (max, sum, output) for the merge.
template <bool BF16, int D, int NPF, bool KV8>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(AttnArgs a, const int32_t* __restrict__ bt_all,
                                                                int hw, int first_round) {
  static_assert(!KV8 || BF16, "8-bit pools compute in bf16");
  using Sh = DecodeShape<BF16, D>;
  constexpr int ES = Sh::ES, KC = Sh::KC, VE = Sh::VE;
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;   // K row (token) for the A operand; head column of scores
  const int kg = lane >> 4;  // lane group: token rows 4kg..4kg+3 of scores
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wph = kDecodeWaves / hw;  // waves per KV head
  const uint32_t n_hg = static_cast<uint32_t>(a.Hkv / hw);
  // The workgroup's unit x = s * n_hg + hg and partition p, with the
  // sequence's query rows [q0, q1), length and cached context: a record of
  // the work order (longest first) when the launch has one, else the grid
  // position. Of an ordered launch (a 1-D grid), the first round of
  // workgroups, which start together, take records 0 .. first_round - 1;
  // each later one claims the next record as it starts. Workgroup b runs on
  // XCD b mod 8, and the XCDs stream at different rates (in the 70B batch,
  // one round of equal units, their mean finish times spread over 8%): with
  // a fixed assignment every XCD gets an equal share of the order and the
  // slowest ends last; with claims, the CUs of a slower XCD free up later
  // and draw the shorter units at the end of the order.
  uint32_t x;
  int p, q0, q1, len_s, ctx_s;
  if (a.dorder != nullptr) {
    uint32_t b = blockIdx.x;
    if (static_cast<int>(b) >= first_round) {
      __shared__ int claimed;
      if (threadIdx.x == 0) claimed = atomicAdd(a.dorder + 1, 1);
      __syncthreads();
      b = static_cast<uint32_t>(first_round + __builtin_amdgcn_readfirstlane(claimed));
    }
    const int4* rec = reinterpret_cast<const int4*>(a.dorder + kDecodeOrderHeader) + 2 * b;
    const int n_work = a.dorder[0];
    const int4 r0 = rec[0], r1 = rec[1];
    // every value taken here, so that the compiler issues the loads together
    // (one round trip) instead of waiting for the count before the record
    asm volatile("" ::"s"(n_work), "s"(r0.x), "s"(r0.y), "s"(r0.z), "s"(r0.w), "s"(r1.x), "s"(r1.y));
    if (static_cast<int64_t>(b) >= n_work) return;  // whole workgroup
    x = static_cast<uint32_t>(r0.x);
    p = r0.y;
    q0 = r0.z;
    q1 = r0.w;
    len_s = r1.x;
    ctx_s = r1.y;
  } else {
    x = blockIdx.x;
    p = blockIdx.y;
    const uint32_t s0 = x / n_hg;
    q0 = a.qsl[s0];
    q1 = a.qsl[s0 + 1];
    len_s = a.seq_lens[s0];
    ctx_s = a.ctx_lens[s0];
  }
  const uint32_t s = x / n_hg, hg = x - s * n_hg;
  const uint32_t g = hg * hw + wave % hw;
  const int phase = wave / hw;
  const int G = static_cast<int>(a.Hq / a.Hkv);
  const int nq = q1 - q0;  // new tokens of the sequence
  // this kernel's sequences only (whole workgroup); the rows must lie in [0, T)
  if (!decode_path(nq, G) || q0 < 0 || q1 > a.T) return;
  const int PT = static_cast<int>(a.part_tokens);
  const int L = static_cast<int>(min(max(static_cast<int64_t>(len_s), int64_t(0)), a.MB * kBlockTokens));
  const int start = p * PT;
  if (start >= L) return;  // whole workgroup
  const int end = min(start + PT, L);
  const int nparts = (L + PT - 1) / PT;
  const int ncol = nq * G;  // columns (token i, head h) = i * G + h
  // Column n is new token n / G at position C + n / G: it sees keys up to there.
  const int C = min(max(ctx_s, 0), L);
  const int lim = min(end, C + n / G + 1);
  const float qk_scale = a.scale * kLog2e * (KV8 ? a.k_scale : 1.f);
  const int b0 = start / kBlockTokens;
  const int nblk = (end - start + kBlockTokens - 1) / kBlockTokens;
  const int nbw = nblk > phase ? (nblk - phase + wph - 1) / wph : 0;  // blocks b0 + phase + wph i

  // Q^T as the B operand: lane (kg, n) holds column n = (token n / G, head
  // n % G), the same d positions its K chunks cover. Columns >= ncol are zero.
  uint4 qv[KC];
  {
    const int qi = n < ncol ? n / G : 0, qh = n < ncol ? n % G : 0;
    const char* qrow = a.q + int64_t(q0 + qi) * a.q_st + int64_t(g * G + qh) * a.q_sh + 16 * kg;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qv[c] = n < ncol ? *reinterpret_cast<const uint4*>(qrow + 64 * c) : make_uint4(0, 0, 0, 0);
  }

  const int32_t* bt = bt_all + int64_t(s) * a.bt_row;
  const char* kbase = a.kc + int64_t(g) * a.kc_sh;
  const char* vbase = a.vc + int64_t(g) * a.vc_sh;
  // cache element bytes: 1 for an 8-bit pool
  constexpr int CES = KV8 ? 1 : ES;
  constexpr int KLPR = KV8 ? BlockRegs8<D>::LPR8 : Sh::LPR;
  const uint32_t k_off = static_cast<uint32_t>((lane / KLPR) * a.kc_sr + 16 * (lane % KLPR));
  const uint32_t kc_sr = static_cast<uint32_t>(a.kc_sr);
  const uint32_t v_off = static_cast<uint32_t>(4 * kg * a.vc_sr + VE * CES * n);
  const uint32_t k_rec = static_cast<uint32_t>((kBlockTokens - 1) * a.kc_sr + D * CES);
  const uint32_t v_rec = static_cast<uint32_t>((kBlockTokens - 1) * a.vc_sr + D * CES);
  const uint32_t vc_sr = static_cast<uint32_t>(a.vc_sr);
  const uint32_t NB = static_cast<uint32_t>(min(a.NB, int64_t(0x7fffffff)));
  auto load = [&](RawBlock<BF16, D, KV8>& r, int i) {
    const uint32_t id = static_cast<uint32_t>(bt[b0 + phase + wph * i]);
    const int64_t pid = id < NB ? int64_t(id) : 0;
    const __amdgpu_buffer_rsrc_t kr = block_rsrc(kbase + pid * a.kc_sb, k_rec);
    const __amdgpu_buffer_rsrc_t vr = block_rsrc(vbase + pid * a.vc_sb, v_rec);
    if constexpr (KV8) load_block8<D>(r, kr, vr, k_off, kc_sr, v_off, vc_sr);
    else load_block<BF16, D>(r, kr, vr, k_off, kc_sr, v_off, vc_sr);
  };
  char* tile = reinterpret_cast<char*>(smem) + wave * Sh::TILE_BYTES;

  f32x4 o[Sh::NACC];
#pragma unroll
  for (int t = 0; t < Sh::NACC; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  RawBlock<BF16, D, KV8> ring[NPF];
#pragma unroll
  for (int j = 0; j < NPF; ++j)
    if (j < nbw) load(ring[j], j);
  for (int i = 0; i < nbw; i += NPF) {
#pragma unroll
    for (int j = 0; j < NPF; ++j) {
      const int ib = i + j;
      if (ib < nbw) {
        attend_block<BF16, D, KV8>(ring[j], qv, o, m_run, l_run, tile, b0 + phase + wph * ib, end, lim, lane,
                                   qk_scale);
        if (ib + NPF < nbw) load(ring[j], ib + NPF);
      }
    }
  }

  // With one wave per head (hw = 8) there is nothing to merge: the wave
  // stores its own columns and ends, so that the waves which finish first
  // free their slots for the next workgroup instead of waiting for the
  // slowest. The values are those of the merge below for one wave (its
  // weight is exp2(0) = 1).
  if constexpr (BF16) {
    if (wph == 1) {
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      if (n >= ncol) return;
      const int64_t hq = int64_t(g) * G + n % G;
      const int64_t t = q0 + n / G;  // the column's token
      const float vs = KV8 ? a.v_scale : 1.f;
      if (nparts == 1) {
        const float inv = 1.f / l_tot;
        char* dst = a.out + t * a.out_st + hq * a.out_sh;
#pragma unroll
        for (int u = 0; u < Sh::NACC; ++u) {
          const int d = 16 * u + 4 * kg;
          f32x4 v = o[u];
          if constexpr (KV8) v *= vs;
          *reinterpret_cast<uint2*>(dst + 2 * d) =
              make_uint2(pack_bf16(v[0] * inv, v[1] * inv), pack_bf16(v[2] * inv, v[3] * inv));
        }
      } else {
        const int64_t slot = (t * a.Hq + hq) * a.max_parts + p;
#pragma unroll
        for (int u = 0; u < Sh::NACC; ++u) {
          f32x4 v = o[u];
          if constexpr (KV8) v *= vs;
          *reinterpret_cast<float4*>(a.ws_o + slot * D + 16 * u + 4 * kg) = make_float4(v[0], v[1], v[2], v[3]);
        }
        if (kg == 0) a.ws_ml[slot] = make_float2(m_run, l_tot);
      }
      return;
    }
  }

  // merge the waves of each head: LDS layout [wave][m: 16][l: 16][o: ncol * D]
  __syncthreads();  // K/V tiles are no longer in use
  const int wstride = 32 + ncol * D;
  float* ws = smem + wave * wstride;
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (kg == 0) {
    ws[n] = m_run;
    ws[16 + n] = l_tot;
  }
  if constexpr (BF16) {
    if (n < ncol) {
#pragma unroll
      for (int t = 0; t < Sh::NACC; ++t)
        *reinterpret_cast<float4*>(ws + 32 + n * D + 16 * t + 4 * kg) =
            make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * kg + r;
      if (h < ncol) {
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<float4*>(ws + 32 + h * D + VE * n + e) =
              make_float4(o[e][r], o[e + 1][r], o[e + 2][r], o[e + 3][r]);
      }
    }
  }
  __syncthreads();
  combine_waves<BF16, D, KV8>(a, smem, wstride, hw, wph, ncol, hg, G, q0, nparts, p);
}

// The decode's work order. Workgroups start in grid order as CUs free up, so
// a launch of several rounds that happens to dispatch long partitions last
// ends with a few CUs streaming them alone, each at the rate of its waves'
// few loads in flight, while the rest of the GPU idles. One workgroup sorts
// the launch's (sequence, head group, partition) units by the partition's
// token count, longest first (a counting sort over kOrderBuckets length
// classes; the order within a class is whatever the LDS atomics give, which
// no result depends on), and writes one record per unit for the decode
// kernel: [0] of dorder gets the count. Units are exactly those the decode
// kernel would attend from its grid position.
constexpr int kOrderBuckets = 256;
constexpr int kOrderThreads = 1024;
constexpr int kOrderKeep = 8;  // sequences per thread kept in registers (all of them up to 8,192)

__global__ __launch_bounds__(kOrderThreads) void decode_order_kernel(AttnArgs a, int hw) {
  __shared__ int32_t count[kOrderBuckets];
  __shared__ int32_t next[kOrderBuckets];
  const int tid = threadIdx.x;
  const int n_hg = static_cast<int>(a.Hkv / hw);
  const int64_t G = a.Hq / a.Hkv;
  const int PT = static_cast<int>(a.part_tokens);
  const int64_t max_len = a.MB * kBlockTokens;
  for (int i = tid; i < kOrderBuckets; i += kOrderThreads) count[i] = 0;
  // Sequence tid + k * kOrderThreads's query rows, length and cached context:
  // the first kOrderKeep in registers, loaded together (one round trip for
  // both passes), any further ones loaded where they are used.
  int rq0[kOrderKeep], rq1[kOrderKeep], rlen[kOrderKeep], rctx[kOrderKeep];
#pragma unroll
  for (int k = 0; k < kOrderKeep; ++k) {
    const int64_t s = tid + int64_t(k) * kOrderThreads;
    const bool in = s < a.S;
    rq0[k] = in ? a.qsl[s] : 0;
    rq1[k] = in ? a.qsl[s + 1] : 0;
    rlen[k] = in ? a.seq_lens[s] : 0;
    rctx[k] = in ? a.ctx_lens[s] : 0;
  }
  __syncthreads();
  // Partitions of a sequence that the decode kernel attends (0 if none), and
  // its clamped length.
  auto parts_of = [&](int q0, int q1, int len_raw, int& len) {
    if (!decode_path(q1 - q0, G) || q0 < 0 || q1 > a.T) return 0;
    len = static_cast<int>(min(max(static_cast<int64_t>(len_raw), int64_t(0)), max_len));
    return (len + PT - 1) / PT;
  };
  // class of a partition of `tok` tokens (1 .. PT): 0 for the longest
  auto bucket = [&](int tok) { return kOrderBuckets - 1 - (tok - 1) * kOrderBuckets / PT; };
  // f(s, q0, q1, len_raw, ctx) for every sequence of this thread
  auto each_seq = [&](auto f) {
#pragma unroll
    for (int k = 0; k < kOrderKeep; ++k) {
      const int64_t s = tid + int64_t(k) * kOrderThreads;
      if (s < a.S) f(s, rq0[k], rq1[k], rlen[k], rctx[k]);
    }
    for (int64_t s = tid + int64_t(kOrderKeep) * kOrderThreads; s < a.S; s += kOrderThreads)
      f(s, a.qsl[s], a.qsl[s + 1], a.seq_lens[s], a.ctx_lens[s]);
  };
  each_seq([&](int64_t, int q0, int q1, int len_raw, int) {
    int len = 0;
    const int np = parts_of(q0, q1, len_raw, len);
    for (int p = 0; p < np; ++p) atomicAdd(&count[bucket(min(PT, len - p * PT))], n_hg);
  });
  __syncthreads();
  // Each class's first place: an exclusive scan of the counts, in place over
  // kOrderBuckets threads (Hillis-Steele: every round reads before any
  // thread writes).
  const int own = tid < kOrderBuckets ? count[tid] : 0;
  for (int off = 1; off < kOrderBuckets; off <<= 1) {
    const int add = tid < kOrderBuckets && tid >= off ? count[tid - off] : 0;
    __syncthreads();
    if (tid < kOrderBuckets) count[tid] += add;
    __syncthreads();
  }
  if (tid < kOrderBuckets) next[tid] = count[tid] - own;
  if (tid == kOrderBuckets - 1) {
    a.dorder[0] = count[tid];  // units in all
    a.dorder[1] = 0;           // the decode's claim counter
  }
  __syncthreads();
  int4* const rec = reinterpret_cast<int4*>(a.dorder + kDecodeOrderHeader);
  each_seq([&](int64_t s, int q0, int q1, int len_raw, int ctx) {
    int len = 0;
    const int np = parts_of(q0, q1, len_raw, len);
    for (int p = 0; p < np; ++p) {
      const int at = atomicAdd(&next[bucket(min(PT, len - p * PT))], n_hg);
      for (int hg = 0; hg < n_hg; ++hg) {
        rec[2 * (at + hg)] = make_int4(static_cast<int>(s) * n_hg + hg, p, q0, q1);
        rec[2 * (at + hg) + 1] = make_int4(len_raw, ctx, 0, 0);
      }
    }
  });
}

// Whether a decode launch takes the work order: more units than one round of
// workgroups, units that can be long enough for a late one to matter (the
// order costs a launch and about 25 us for 4,000 sequences; a 1024-token
// unit streamed alone at the end takes longer), no more units than the
// workspace holds records for, and not switched off with PA_DECODE_ORDER=0
// in the environment (read at each launch).
constexpr int64_t kOrderMinTokens = 1024;

bool decode_ordered(const AttnArgs& a, int hw, int per_cu) {
  if (a.dorder == nullptr) return false;
  const int64_t units = a.S * (a.Hkv / hw) * a.max_parts;
  if (units <= int64_t(256) * (per_cu > 0 ? per_cu : 1) || units > kMaxOrderedUnits) return false;
  if (std::min(a.part_tokens, a.MB * kBlockTokens) < kOrderMinTokens) return false;
  const char* e = std::getenv("PA_DECODE_ORDER");
  return !(e && e[0] == '0' && e[1] == 0);
}

// Combine the partitions of multi-partition sequences of the decode kernel
// (step_parts.h): one wave per (sequence, query head), in fixed partition
// order.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void reduce_kernel(AttnArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  reduce_partitions<BF16, D>(a, static_cast<int64_t>(blockIdx.x) * kWaves + wave, threadIdx.x & 63);
}

hipError_t reduce_launch(const AttnArgs& a, hipStream_t stream) {
  if (a.max_parts <= 1) return hipSuccess;
  const bool bf16 = a.elem == Elem::BF16;  // bf16 out (also over an 8-bit pool)
  const dim3 grid(static_cast<unsigned>((a.S * a.Hq + kWaves - 1) / kWaves));
  ProfileScope ps(kReduce, stream);
  if (a.D == 64) {
    if (bf16) hipLaunchKernelGGL((reduce_kernel<true, 64>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((reduce_kernel<false, 64>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (bf16) hipLaunchKernelGGL((reduce_kernel<true, 128>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((reduce_kernel<false, 128>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

// Dynamic LDS of a decode workgroup: the per-wave K/V tiles during the sweep,
// then the merge area (up to 16 columns per wave).
template <bool BF16, int D>
constexpr size_t decode_lds_bytes() {
  constexpr size_t merge = sizeof(float) * kDecodeWaves * (32 + kMaxDecodeColumns * D);
  constexpr size_t tiles = size_t(kDecodeWaves) * DecodeShape<BF16, D>::TILE_BYTES;
  return merge > tiles ? merge : tiles;
}

// 16 query heads per KV head at D = 128 need 65 KB for the merge, past the
// default dynamic-LDS limit.
template <bool BF16, int D, bool KV8>
hipError_t allow_decode_lds() {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<BF16, D, 1, KV8>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kDecodeMaxLds));
  return attr;
}

// Workgroups of this decode kernel one CU holds at once (its registers and
// LDS, through the HIP occupancy query), or 0 when the query fails.
template <bool BF16, int D, bool KV8>
int decode_occupancy() {
  static const int n = [] {
    int blocks = 0;
    if (allow_decode_lds<BF16, D, KV8>() != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void*>(&decode_kernel<BF16, D, 1, KV8>),
                                                     kDecodeThreads, decode_lds_bytes<BF16, D>()) != hipSuccess)
      return 0;
    return blocks;
  }();
  return n;
}

template <bool BF16, int D, bool KV8>
hipError_t launch_staged(const AttnArgs& a, hipStream_t stream, bool with_reduce) {
  const int hw = decode_heads_per_workgroup(a.Hkv);
  constexpr size_t lds = decode_lds_bytes<BF16, D>();
  static_assert(lds <= kDecodeMaxLds, "decode LDS");
  const dim3 grid(static_cast<unsigned>(a.S * (a.Hkv / hw)), static_cast<unsigned>(a.max_parts));
  const hipError_t attr = allow_decode_lds<BF16, D, KV8>();
  if (attr != hipSuccess) return attr;
  // An ordered launch takes its units from the work order, one per
  // workgroup of a 1-D grid of the same size.
  AttnArgs b = a;
  dim3 g = grid;
  const int per_cu = decode_occupancy<BF16, D, KV8>();
  // workgroups that start together: 256 CUs times the kernel's occupancy
  const int first_round = 256 * (per_cu > 0 ? per_cu : 1);
  if (decode_ordered(a, hw, per_cu)) {
    ProfileScope ps(kDecodeOrder, stream);
    hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, b, hw);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    g = dim3(grid.x * grid.y);
  } else {
    b.dorder = nullptr;
  }
  {
    ProfileScope ps(kDecode, stream);
    hipLaunchKernelGGL((decode_kernel<BF16, D, 1, KV8>), g, dim3(kDecodeThreads), lds, stream, b, b.block_tables,
                       hw, first_round);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !with_reduce) return e;
  return reduce_launch(a, stream);
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, hipStream_t stream, bool with_reduce) {
  const bool r = with_reduce;
  if (a.elem != Elem::BF16)
    return a.D == 64 ? launch_staged<false, 64, false>(a, stream, r) : launch_staged<false, 128, false>(a, stream, r);
  if (a.kv8) return a.D == 64 ? launch_staged<true, 64, true>(a, stream, r) : launch_staged<true, 128, true>(a, stream, r);
  return a.D == 64 ? launch_staged<true, 64, false>(a, stream, r) : launch_staged<true, 128, false>(a, stream, r);
}

hipError_t launch_reduce(const AttnArgs& a, hipStream_t stream) { return reduce_launch(a, stream); }

int decode_workgroups_per_cu(Elem elem, bool kv8, int64_t D) {
  if (D != 64 && D != 128) return 0;
  if (elem != Elem::BF16) return D == 64 ? decode_occupancy<false, 64, false>() : decode_occupancy<false, 128, false>();
  if (kv8) return D == 64 ? decode_occupancy<true, 64, true>() : decode_occupancy<true, 128, true>();
  return D == 64 ? decode_occupancy<true, 64, false>() : decode_occupancy<true, 128, false>();
}

}  // namespace pa
