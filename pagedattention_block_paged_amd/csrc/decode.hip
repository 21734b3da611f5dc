// Decode attention: sequences with exactly one new token read all of their
// cached K/V through the block table; HBM-bound ("Inside vLLM", section
// "Scheduler": decode steps are memory-bandwidth-bound; ngrok "Serving models
// at scale with vLLM", section "Speculative decoding": a decode pass is
// limited by moving data, not by math).
//
// Design for gfx950 (the pages give no kernel design):
//  - One wave owns (sequence s, KV head g, partition p): the keys
//    [p * PT, min((p + 1) * PT, L)). All G = Hq / Hkv query heads of the group
//    share each K/V read. A workgroup is 4 such waves; with the pool layout
//    [block][K|V][16 rows][Hkv][D] the 4 waves of a workgroup read adjacent
//    head slices of the same rows.
//  - Scores use MFMA with the key rows as the A operand: S^T = K . Q^T. Each
//    lane loads the 16-byte K chunk it feeds the matrix core straight from
//    HBM; no LDS staging, no shuffles. Query heads fill the 16 columns (G <= 16;
//    unused columns are zero and cost nothing in an HBM-bound kernel).
//  - The score layout (lane = head column, 4 token rows per lane) is exactly
//    the A operand of the fp32 16x16x4 MFMA, and a V row loaded as VE = D/16
//    consecutive elements per lane is its B operand, so P.V also runs on the
//    matrix core with no data movement between lanes. V is widened to fp32.
//  - Online softmax in log2 units with a lazy rescale: the running maximum is
//    only raised (and the accumulators rescaled) when a block's maximum beats
//    it by more than 2^8, so weights stay <= 256 and rescales are rare.
//  - The next block's K and V are loaded while the current one is computed.
//  - Sequences longer than one partition write (unnormalised output, max,
//    weight sum) per partition; a second kernel combines partitions in a fixed
//    order (deterministic). Single-partition sequences write the output
//    directly.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

__device__ inline float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Widen VE elements of one V row (raw 32-bit words) to fp32.
template <bool BF16, int VE, int VW>
__device__ inline void widen(const uint32_t (&w)[VW], float (&f)[VE]) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < VW; ++i) {
      f[2 * i] = lo_bf16(w[i]);
      f[2 * i + 1] = hi_bf16(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VW; ++i) f[i] = __uint_as_float(w[i]);
  }
}

template <int VW>
__device__ inline void load_words(const char* p, uint32_t (&w)[VW]) {
  if constexpr (VW == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    w[0] = u.x;
    w[1] = u.y;
  } else {
#pragma unroll
    for (int i = 0; i < VW / 4; ++i) {
      const uint4 u = *reinterpret_cast<const uint4*>(p + 16 * i);
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
  static constexpr int KC = D * ES / 64;  // 16-byte K chunks per lane per block
  static constexpr int VE = D / 16;       // V elements per lane per row
  static constexpr int VW = VE * ES / 4;  // 32-bit words per lane per V row
};

template <bool BF16, int D>
struct BlockRegs {
  using Sh = DecodeShape<BF16, D>;
  uint4 k[Sh::KC];
  uint32_t v[4][Sh::VW];
};

template <bool BF16, int D>
__device__ inline void load_block(BlockRegs<BF16, D>& r, const char* kp, const char* vp, int64_t vc_sr) {
  using Sh = DecodeShape<BF16, D>;
#pragma unroll
  for (int c = 0; c < Sh::KC; ++c) r.k[c] = *reinterpret_cast<const uint4*>(kp + 64 * c);
#pragma unroll
  for (int j = 0; j < 4; ++j) load_words<Sh::VW>(vp + j * vc_sr, r.v[j]);
}

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(AttnArgs a) {
  using Sh = DecodeShape<BF16, D>;
  constexpr int ES = Sh::ES, KC = Sh::KC, VE = Sh::VE;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;   // K row (token) for the A operand; head column of scores
  const int kg = lane >> 4;  // lane group: token rows 4kg..4kg+3 of scores
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int64_t g = item % a.Hkv;
  const int64_t sp = item / a.Hkv;
  const int64_t p = sp % a.max_parts;
  const int64_t s = sp / a.max_parts;
  if (s >= a.S) return;
  const int64_t q0 = a.qsl[s], q1 = a.qsl[s + 1];
  if (q1 - q0 != 1 || q0 < 0 || q0 >= a.T) return;  // decode sequences only
  const int64_t PT = a.part_tokens;
  const int64_t L = min(max(static_cast<int64_t>(a.seq_lens[s]), int64_t(0)), a.MB * kBlockTokens);
  const int64_t start = p * PT;
  if (start >= L) return;
  const int64_t end = min(start + PT, L);
  const int64_t nparts = (L + PT - 1) / PT;
  const int G = static_cast<int>(a.Hq / a.Hkv);
  const float qk_scale = a.scale * kLog2e;

  // Q^T as the B operand: lane (kg, n) holds head n, the same d positions its
  // K chunks cover. Columns n >= G are zero.
  uint4 qv[KC];
  {
    const char* qrow = a.q + q0 * a.q_st + (g * G + n) * a.q_sh + 16 * kg;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qv[c] = n < G ? *reinterpret_cast<const uint4*>(qrow + 64 * c) : make_uint4(0, 0, 0, 0);
  }

  const int32_t* bt = a.block_tables + s * a.bt_row;
  const char* kbase = a.kc + g * a.kc_sh + n * a.kc_sr + 16 * kg;
  const char* vbase = a.vc + g * a.vc_sh + (4 * kg) * a.vc_sr + VE * ES * n;
  auto phys = [&](int64_t b) -> int64_t {
    const int64_t id = bt[b];
    return static_cast<uint64_t>(id) < static_cast<uint64_t>(a.NB) ? id : 0;
  };

  const int64_t b0 = start / kBlockTokens, b1 = (end + kBlockTokens - 1) / kBlockTokens;
  BlockRegs<BF16, D> cur;
  {
    const int64_t id = phys(b0);
    load_block<BF16, D>(cur, kbase + id * a.kc_sb, vbase + id * a.vc_sb, a.vc_sr);
  }
  f32x4 o[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int64_t b = b0; b < b1; ++b) {
    BlockRegs<BF16, D> nxt;
    if (b + 1 < b1) {
      const int64_t id = phys(b + 1);
      load_block<BF16, D>(nxt, kbase + id * a.kc_sb, vbase + id * a.vc_sb, a.vc_sr);
    }
    // scores S^T[token 4kg + r][head n]
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if constexpr (BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[c]),
                                                       __builtin_bit_cast(bf16x8, qv[c]), acc, 0, 0, 0);
      } else {
        const float4 kf = __builtin_bit_cast(float4, cur.k[c]);
        const float4 qf = __builtin_bit_cast(float4, qv[c]);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.x, qf.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.y, qf.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.z, qf.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.w, qf.w, acc, 0, 0, 0);
      }
    }
    float sc[4];
    const int64_t tok0 = b * kBlockTokens + 4 * kg;
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (tok0 + r < end) ? acc[r] * qk_scale : -INFINITY;
    float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    if (__any(mloc > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * kg + r);  // output row r holds head 4kg + r
#pragma unroll
        for (int e = 0; e < VE; ++e) o[e][r] *= ar;
      }
      m_run = m_new;
    }
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = fast_exp2(sc[r] - m_run);
      l_run += pr[r];
    }
    // O[head][d = VE * n + e] += sum over the 4 lane groups of P[head][token] V[token][d].
    // Rows past the sequence end carry weight 0 but arbitrary bits (0 * NaN is
    // NaN), so they are zeroed before the product.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (tok0 + j >= end) {
#pragma unroll
        for (int w = 0; w < Sh::VW; ++w) cur.v[j][w] = 0u;
      }
      float vf[VE];
      widen<BF16, VE, Sh::VW>(cur.v[j], vf);
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[j], vf[e], o[e], 0, 0, 0);
    }
    if (b + 1 < b1) cur = nxt;
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  // lane (kg, n) holds O[head 4kg + r][d = VE * n + e]
  if (nparts == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lt = __shfl(l_tot, 4 * kg + r);
      const int h = 4 * kg + r;
      if (h < G) {
        const float inv = 1.f / lt;
        char* dst = a.out + q0 * a.out_st + (g * G + h) * a.out_sh + VE * ES * n;
        if constexpr (BF16) {
          uint32_t w[VE / 2];
#pragma unroll
          for (int e = 0; e < VE / 2; ++e) w[e] = pack_bf16(o[2 * e][r] * inv, o[2 * e + 1][r] * inv);
          if constexpr (VE == 8) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
          } else {
            *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < VE; e += 4)
            *reinterpret_cast<float4*>(dst + 4 * e) =
                make_float4(o[e][r] * inv, o[e + 1][r] * inv, o[e + 2][r] * inv, o[e + 3][r] * inv);
        }
      }
    }
  } else {
    const int64_t hbase = s * a.Hq + g * G;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * kg + r;
      if (h < G) {
        float* dst = a.ws_o + ((hbase + h) * a.max_parts + p) * D + VE * n;
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<float4*>(dst + e) = make_float4(o[e][r], o[e + 1][r], o[e + 2][r], o[e + 3][r]);
      }
    }
    if (kg == 0 && n < G) a.ws_ml[(hbase + n) * a.max_parts + p] = make_float2(m_run, l_tot);
  }
}

// Combine the partitions of multi-partition decode sequences: one wave per
// (sequence, query head), fixed partition order.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void reduce_kernel(AttnArgs a) {
  constexpr int DPL = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int64_t s = item / a.Hq, hq = item % a.Hq;
  if (s >= a.S) return;
  const int64_t q0 = a.qsl[s], q1 = a.qsl[s + 1];
  if (q1 - q0 != 1 || q0 < 0 || q0 >= a.T) return;
  const int64_t L = min(max(static_cast<int64_t>(a.seq_lens[s]), int64_t(0)), a.MB * kBlockTokens);
  const int64_t nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const float2* ml = a.ws_ml + (s * a.Hq + hq) * a.max_parts;
  const float* po = a.ws_o + (s * a.Hq + hq) * a.max_parts * D + DPL * lane;
  float m = -INFINITY;
  for (int64_t p = 0; p < nparts; ++p) m = fmaxf(m, ml[p].x);
  float acc[DPL] = {};
  float lsum = 0.f;
  for (int64_t p = 0; p < nparts; ++p) {
    const float2 v = ml[p];
    const float w = fast_exp2(v.x - m);
    lsum += w * v.y;
    if constexpr (DPL == 2) {
      const float2 x = *reinterpret_cast<const float2*>(po + p * D);
      acc[0] += w * x.x;
      acc[1] += w * x.y;
    } else {
      acc[0] += w * po[p * D];
    }
  }
  const float inv = 1.f / lsum;
  char* dst = a.out + q0 * a.out_st + hq * a.out_sh;
  if constexpr (BF16) {
    if constexpr (DPL == 2) {
      *reinterpret_cast<uint32_t*>(dst + 4 * lane) = pack_bf16(acc[0] * inv, acc[1] * inv);
    } else {
      reinterpret_cast<__bf16*>(dst)[lane] = static_cast<__bf16>(acc[0] * inv);
    }
  } else {
#pragma unroll
    for (int i = 0; i < DPL; ++i) reinterpret_cast<float*>(dst)[DPL * lane + i] = acc[i] * inv;
  }
}

template <bool BF16, int D>
hipError_t launch_typed(const AttnArgs& a, hipStream_t stream) {
  const int64_t items = a.S * a.max_parts * a.Hkv;
  const int64_t blocks = (items + kWaves - 1) / kWaves;
  {
    ProfileScope ps(kDecode, stream);
    hipLaunchKernelGGL((decode_kernel<BF16, D>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  const int64_t rblocks = (a.S * a.Hq + kWaves - 1) / kWaves;
  {
    ProfileScope ps(kReduce, stream);
    hipLaunchKernelGGL((reduce_kernel<BF16, D>), dim3(static_cast<unsigned>(rblocks)), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, hipStream_t stream) {
  const bool bf16 = a.elem == Elem::BF16;
  if (a.D == 64) return bf16 ? launch_typed<true, 64>(a, stream) : launch_typed<false, 64>(a, stream);
  return bf16 ? launch_typed<true, 128>(a, stream) : launch_typed<false, 128>(a, stream);
}

}  // namespace pa
